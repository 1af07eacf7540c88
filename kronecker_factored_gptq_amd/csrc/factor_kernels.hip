// Factor kernels (float64) for gfx950.
//
// The solver needs L = Cholesky(A^-1) with columns divided by their
// diagonal ("BaKron: Efficient Quantization with Kronecker-Factored
// Hessians", arXiv 2608.06291, §3.2 Algorithm 2, first two steps; Cholesky
// and RevCholesky as defined in §3.1). We never form A^-1: with J the
// reversal permutation and C = Cholesky(J A J), A = (J C J)(J C J)^T, so
// A^-1 = (J C^-T J)(J C^-T J)^T and J C^-T J is lower triangular with a
// positive diagonal, i.e. it IS Cholesky(A^-1). Steps:
//   X = J A J (lower triangle)        load_reversed_kernel
//   Y = Cholesky(X)^-1                recursive: for X = [X11 .; X21 X22],
//       (Y11 from X11)                  C11 and Y11 = C11^-1 recursively,
//       C21 = X21 Y11^T                 the panel of the Cholesky factor,
//       X22 -= C21 C21^T                the Schur complement,
//       (Y22 from X22)                  recursively,
//       Y21 = -Y22 (C21 Y11)            the off-diagonal block of the inverse;
//                                     64 x 64 leaves in LDS, everything else
//                                     float64 MFMA GEMMs (gemm64)
//   L[i][j] = Y[n-1-j][n-1-i], normalised by its diagonal  store_normalized
#include <climits>

#include "device.hpp"
#include "launch.hpp"

namespace bk {

namespace {
constexpr int NB = 64;  // Cholesky panel width
constexpr int kLeafCols = 4;  // columns per barrier step of the leaf (8: spills, 6.90 ms factor against 6.69)
constexpr int kLeafPatchCols = 2;  // columns of a thread's patch: 4 x 2 patches, 512 threads
}

// X[i][j] = A[n-1-j][n-1-i] for i >= j (the lower triangle of J A J read from
// the lower triangle of A), 0 above the diagonal. 32 x 32 tiles through LDS.
template <typename R>
__global__ __launch_bounds__(256) void load_reversed_kernel(int64_t n, const R* __restrict__ A,
                                                            int64_t lda, int64_t sA,
                                                            double* __restrict__ X, int64_t sX) {
  __shared__ double tile[32][33];
  A += (int64_t)blockIdx.z * sA;  // matrix blockIdx.z of a batch
  X += (int64_t)blockIdx.z * sX;
  const int64_t i0 = (int64_t)blockIdx.y * 32, j0 = (int64_t)blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // ty 0..7
  const bool lower_tile = i0 + 31 >= j0;
  if (lower_tile) {
    // tile[jj][ii] = A[n-1-(j0+jj)][n-1-(i0+ii)]
    for (int jj = ty; jj < 32; jj += 8) {
      const int64_t sr = n - 1 - (j0 + jj), sc = n - 1 - (i0 + tx);
      double v = 0.0;
      if (j0 + jj < n && i0 + tx < n && sc <= sr) v = (double)A[sr * lda + sc];
      tile[jj][tx] = v;
    }
  }
  __syncthreads();
  for (int ii = ty; ii < 32; ii += 8) {
    const int64_t i = i0 + ii, j = j0 + tx;
    if (i < n && j < n) X[i * n + j] = (lower_tile && i >= j) ? tile[tx][ii] : 0.0;
  }
}

// Leaf of the recursion: the Cholesky factor C of the bs x bs diagonal block
// X[off.., off..] (bs <= 64) and its inverse Y = C^-1; Y[off.., off..]
// receives C^-1 (zeros above the diagonal). Thread (ty, tx) of a 16 x 16
// grid keeps the 4 x 4 patch rows 4ty.., columns 4tx.. of both C and Y in
// registers; rows and columns past bs are padded with the identity.
// Right-looking, NC columns j .. j+NC-1 per step (whole patch columns) and
// one barrier per step: the owners publish the raw columns j.. and the raw
// rows j.. of Y (and the next step's pivot block as it stands); the pivot
// factor l (NC x NC lower; reciprocal square roots by one Newton step from
// the hardware estimate) of each step comes from one extra wave, which
// forms it during the step before (applying that step's update to the pivot
// block itself). After the barrier every patch thread reads l and, by
// forward substitution, forms
//   C[i][j+q] = (X[i][j+q] - sum_{p<q} C[i][j+p] l[q][p]) / l[q][q],
//   Y[j+q]    = (Y[j+q]    - sum_{p<q} l[q][p] Y[j+p]) / l[q][q]   (rows),
// then updates its patch with the rank-NC terms
//   C[i][c] -= sum_q C[i][j+q] C[c][j+q]   (j + NC <= c <= i),
//   Y[i][c] -= sum_q C[i][j+q] Y[j+q][c]   (i >= j + NC).
// Published values are double-buffered by the parity of the step. A pivot
// that is not positive and finite records off + j + q in *info (smallest
// wins) and the factorisation continues with NaN.
// Cholesky factor l (NC x NC, lower) of the pivot block blk and the
// reciprocals dinv of its diagonal; bad = the first pivot that is not
// positive and finite (-1 if none), whose dinv becomes NaN.
template <int NC>
__device__ __forceinline__ void pivot_factor(const double (&blk)[NC][NC], double (&l)[NC][NC],
                                             double (&dinv)[NC], int& bad) {
  bad = -1;
#pragma unroll
  for (int q = 0; q < NC; ++q) {
#pragma unroll
    for (int p = 0; p < NC; ++p) {
      if (p > q) continue;
      double v = blk[q][p];
#pragma unroll
      for (int r = 0; r < NC; ++r)
        if (r < p) v -= l[q][r] * l[p][r];
      if (p < q) {
        l[q][p] = v * dinv[p];
      } else {
        const bool ok = v > 0.0 && v < INFINITY;
        if (!ok && bad < 0) bad = q;
        // 1/sqrt(v) from the hardware estimate and one Newton step
        // (y += y (1 - v y^2) / 2), then sqrt(v) = v / sqrt(v): a short
        // dependent chain instead of a rounded square root and a division
        const double y0 = __builtin_amdgcn_rsq(v);
        const double r = __builtin_fma(-v * y0, y0, 1.0);
        const double y = __builtin_fma(0.5 * y0, r, y0);
        dinv[q] = ok ? y : __builtin_nan("");
        l[q][q] = v * dinv[q];
      }
    }
  }
}

template <int NC, int PCW>
__global__ __launch_bounds__(16 * (64 / PCW) + 64) void chol_inv_leaf_kernel(FactorSet set,
                                                                            int64_t n, int64_t off,
                                                                            int bs) {
  static_assert(NC % 4 == 0 && NC % PCW == 0, "whole patch rows and columns per step");
  constexpr int PRS = NC / 4;  // patch rows per step
  constexpr int TX = 64 / PCW;  // thread columns; 16 thread rows of 4 rows each
  constexpr int NCT = 16 * TX;  // patch threads; one more wave factors the pivot blocks
  __shared__ double pnext[2][NC][NC];     // next step's pivot block before this step's update
  __shared__ double lpub[2][NC][NC + 1];  // a step's pivot factor l, and dinv in column NC
  __shared__ double colp[2][NC][64];
  __shared__ double rowp[2][NC][64];
  const FactorSide S = factor_side(set, (int)blockIdx.x);  // one matrix per workgroup
  const int tid = threadIdx.x;
  const int steps = (bs + NC - 1) / NC;
  if (tid >= NCT) {
    // Pivot wave: during step st it applies step st's update to the pivot
    // block of step st + 1 (with the same operations the patch threads use
    // for those entries), factors it and publishes l and dinv for step
    // st + 1, so that the patch threads never wait for a pivot factor.
    const bool lead = tid == NCT;
    double l[NC][NC], dinv[NC];
    {
      double blk[NC][NC];
#pragma unroll
      for (int q = 0; q < NC; ++q)
#pragma unroll
        for (int p = 0; p < NC; ++p) {
          double v = 0.0;
          if (q < bs && p < bs) v = p <= q ? S.X[(off + q) * n + off + p] : 0.0;
          else if (q == p) v = 1.0;
          blk[q][p] = v;
        }
      int bad;
      pivot_factor<NC>(blk, l, dinv, bad);
      if (lead && bad >= 0 && bad < bs) atomicMin(S.info, (int32_t)(off + bad));
      if (lead) {
#pragma unroll
        for (int q = 0; q < NC; ++q) {
#pragma unroll
          for (int p = 0; p < NC; ++p) lpub[0][q][p] = l[q][p];
          lpub[0][q][NC] = dinv[q];
        }
      }
    }
    for (int st = 0; st < steps; ++st) {
      const int pb = st & 1;
      __syncthreads();
      if (st + 1 >= steps) continue;
      const int j1 = NC * (st + 1);
      double ci[NC][NC];  // step st's panel C[j1 + a][j + q]
#pragma unroll
      for (int a = 0; a < NC; ++a) {
#pragma unroll
        for (int q = 0; q < NC; ++q) {
          double vi = colp[pb][q][j1 + a];
#pragma unroll
          for (int p = 0; p < NC; ++p)
            if (p < q) vi -= ci[a][p] * l[q][p];
          ci[a][q] = vi * dinv[q];
        }
      }
      double blk[NC][NC];
#pragma unroll
      for (int a = 0; a < NC; ++a)
#pragma unroll
        for (int b = 0; b < NC; ++b) {
          double dl = 0.0;
#pragma unroll
          for (int q = 0; q < NC; ++q) dl += ci[a][q] * ci[b][q];
          double v = pnext[pb][a][b];
          if (b <= a) v -= dl;
          blk[a][b] = v;
        }
      int bad;
      pivot_factor<NC>(blk, l, dinv, bad);
      if (lead && bad >= 0 && j1 + bad < bs) atomicMin(S.info, (int32_t)(off + j1 + bad));
      if (lead) {
#pragma unroll
        for (int q = 0; q < NC; ++q) {
#pragma unroll
          for (int p = 0; p < NC; ++p) lpub[pb ^ 1][q][p] = l[q][p];
          lpub[pb ^ 1][q][NC] = dinv[q];
        }
      }
    }
    return;
  }
  const int ty = tid / TX, tx = tid % TX;
  double Lr[4][PCW], Yr[4][PCW];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < PCW; ++b) {
      const int i = 4 * ty + a, c = PCW * tx + b;
      double v = 0.0;
      if (i < bs && c < bs) v = c <= i ? S.X[(off + i) * n + off + c] : 0.0;
      else if (i == c) v = 1.0;
      Lr[a][b] = v;
      Yr[a][b] = (i == c) ? 1.0 : 0.0;
    }
  for (int st = 0; st < steps; ++st) {
    const int j = NC * st, pb = st & 1;
    // owners of columns j..j+NC-1 and of rows j..j+NC-1
    const bool ownc = tx >= j / PCW && tx < (j + NC) / PCW;
    const bool ownr = ty >= PRS * st && ty < PRS * (st + 1);
    const int rq = 4 * (ty - PRS * st);  // first pivot row of this thread row
    // publish the next step's pivot block, columns j..j+NC-1 and rows
    // j..j+NC-1 of Y
    if (tx >= (j + NC) / PCW && tx < (j + 2 * NC) / PCW && ty >= PRS * (st + 1) &&
        ty < PRS * (st + 2)) {
      const int rn = 4 * (ty - PRS * (st + 1));
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < PCW; ++b) pnext[pb][rn + a][PCW * tx + b - j - NC] = Lr[a][b];
    }
    if (ownc) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < PCW; ++b) colp[pb][PCW * tx + b - j][4 * ty + a] = Lr[a][b];
    }
    if (ownr) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < PCW; ++b) rowp[pb][rq + a][PCW * tx + b] = Yr[a][b];
    }
    __syncthreads();
    // A thread whose rows all lie above the pivot block is done with them:
    // its rows of Y are final and its rows of C are never read again (its
    // entries of C in later columns are exact zeros, published as such).
    if (ty < PRS * st) continue;
    // this step's pivot factor, from the pivot wave
    double l[NC][NC], dinv[NC];
#pragma unroll
    for (int q = 0; q < NC; ++q) {
#pragma unroll
      for (int p = 0; p < NC; ++p) l[q][p] = lpub[pb][q][p];
      dinv[q] = lpub[pb][q][NC];
    }
    // columns j.. of C at this thread's rows i and at its columns c taken as
    // rows, and rows j.. of Y at its columns c (final after this step). No
    // masks: above the pivot block these are exact zeros (C and Y keep exact
    // zeros above their diagonals, and 0 * dinv = 0); the pivot block's own
    // rows of C only reach entries of C in columns < j + NC, which no later
    // step reads, and its rows of Y are overwritten with yq after the update
    double ci[4][NC], cc[PCW][NC], yq[NC][PCW];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int i = 4 * ty + a;
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        double vi = colp[pb][q][i];
#pragma unroll
        for (int p = 0; p < NC; ++p)
          if (p < q) vi -= ci[a][p] * l[q][p];
        ci[a][q] = vi * dinv[q];
      }
    }
#pragma unroll
    for (int b = 0; b < PCW; ++b) {
      const int c = PCW * tx + b;
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        double vc = colp[pb][q][c];
#pragma unroll
        for (int p = 0; p < NC; ++p)
          if (p < q) vc -= cc[b][p] * l[q][p];
        cc[b][q] = vc * dinv[q];
      }
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        double v = rowp[pb][q][c];
#pragma unroll
        for (int p = 0; p < NC; ++p)
          if (p < q) v -= l[q][p] * yq[p][b];
        yq[q][b] = v * dinv[q];
      }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < PCW; ++b) {
        const int i = 4 * ty + a, c = PCW * tx + b;
        double dl = 0.0, dy = 0.0;
#pragma unroll
        for (int q = 0; q < NC; ++q) {
          dl += ci[a][q] * cc[b][q];
          dy += ci[a][q] * yq[q][b];
        }
        if (c <= i) Lr[a][b] -= dl;  // C keeps exact zeros above its diagonal
        Yr[a][b] -= dy;
      }
    if (ownr) {  // rows j.. of Y are final now
#pragma unroll
      for (int pr = 0; pr < PRS; ++pr)
        if (rq == 4 * pr) {
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < PCW; ++b) Yr[a][b] = yq[4 * pr + a][b];
        }
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < PCW; ++b) {
      const int i = 4 * ty + a, c = PCW * tx + b;
      if (i < bs && c < bs) S.Y[(off + i) * n + off + c] = c <= i ? Yr[a][b] : 0.0;
    }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t count, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = v;
}

// L[i][j] = Y[n-1-j][n-1-i] / Y[n-1-j][n-1-j] for i > j, 1 on the diagonal,
// 0 above; d[j] = Y[n-1-j][n-1-j]. 32 x 32 tiles through LDS.
template <typename R>
__global__ __launch_bounds__(256) void store_normalized_kernel(int64_t n,
                                                               const double* __restrict__ Y,
                                                               int64_t sY, R* __restrict__ L,
                                                               int64_t ldl, int64_t sL,
                                                               R* __restrict__ d, int64_t sd) {
  __shared__ double tile[32][33];
  __shared__ double diag[32];
  Y += (int64_t)blockIdx.z * sY;  // matrix blockIdx.z of a batch
  L += (int64_t)blockIdx.z * sL;
  if (d) d += (int64_t)blockIdx.z * sd;
  const int64_t i0 = (int64_t)blockIdx.y * 32, j0 = (int64_t)blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const bool lower_tile = i0 + 31 >= j0;
  if (lower_tile) {
    // tile[jj][ii] = Y[n-1-(j0+jj)][n-1-(i0+ii)]
    for (int jj = ty; jj < 32; jj += 8) {
      const int64_t sr = n - 1 - (j0 + jj), sc = n - 1 - (i0 + tx);
      double v = 0.0;
      if (j0 + jj < n && i0 + tx < n && sc <= sr) v = Y[sr * n + sc];
      tile[jj][tx] = v;
    }
    if (ty == 0) {
      const int64_t j = j0 + tx;
      diag[tx] = j < n ? Y[(n - 1 - j) * n + (n - 1 - j)] : 1.0;
    }
  }
  __syncthreads();
  for (int ii = ty; ii < 32; ii += 8) {
    const int64_t i = i0 + ii, j = j0 + tx;
    if (i < n && j < n) {
      double v = 0.0;
      if (lower_tile) {
        if (i == j) v = 1.0;
        else if (i > j) v = tile[tx][ii] / diag[tx];
      }
      L[i * ldl + j] = (R)v;
    }
  }
  if (d && blockIdx.y == blockIdx.x && ty == 0) {
    const int64_t j = j0 + tx;
    if (j < n) d[j] = (R)diag[tx];
  }
}

// ---------------------------------------------------------------------------
template <typename R>
hipError_t launch_load_reversed(int64_t n, const R* A, int64_t lda, int64_t sA, double* X,
                                int64_t sX, int batch, hipStream_t s) {
  if (n <= 0 || batch <= 0) return hipSuccess;
  const unsigned nb = (unsigned)((n + 31) / 32);
  hipLaunchKernelGGL((load_reversed_kernel<R>), dim3(nb, nb, (unsigned)batch), dim3(256), 0, s, n,
                     A, lda, sA, X, sX);
  return hipGetLastError();
}

template <typename R>
hipError_t launch_store_normalized(int64_t n, const double* Y, int64_t sY, R* L, int64_t ldl,
                                   int64_t sL, R* d, int64_t sd, int batch, hipStream_t s) {
  if (n <= 0 || batch <= 0) return hipSuccess;
  const unsigned nb = (unsigned)((n + 31) / 32);
  hipLaunchKernelGGL((store_normalized_kernel<R>), dim3(nb, nb, (unsigned)batch), dim3(256), 0, s,
                     n, Y, sY, L, ldl, sL, d, sd);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t count, int32_t v, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, p,
                     count, v);
  return hipGetLastError();
}

// Recursive split point: about half, a multiple of 64, strictly inside.
static inline int64_t split_point(int64_t n) {
  int64_t n1 = (n / 2 + 63) / 64 * 64;
  if (n1 >= n) n1 = n - 64;
  return n1;
}

// Size class of a node of order len: the smallest c with len <= 128 << c.
static inline int tmp_class(int64_t len) {
  int c = 0;
  while (c + 1 < kTmpClasses && len > ((int64_t)128 << c)) ++c;
  return c;
}

static void tmp_need(int64_t len, int64_t* need) {
  if (len <= NB) return;
  const int64_t n1 = split_point(len), n2 = len - n1;
  const int c = tmp_class(len);
  if (n2 * n1 > need[c]) need[c] = n2 * n1;
  tmp_need(n1, need);
  tmp_need(n2, need);
}

int64_t factor_tmp_layout(int64_t n, int64_t* off) {
  int64_t need[kTmpClasses] = {0};
  if (n > 0) tmp_need(n, need);
  int64_t total = 0;
  for (int c = 0; c < kTmpClasses; ++c) {
    if (off) off[c] = total;
    total += (need[c] + 31) / 32 * 32;  // 256-byte aligned buffers
  }
  return total;
}

// Nodes above this order form Tmp = C21 Y11 on the helper stream (when there
// is one), concurrently with the recursion into X22; smaller nodes form it
// in the same launch as the Schur update.
constexpr int64_t kPairMaxOrder = 1024;

static int64_t large_nodes(int64_t len) {
  if (len <= kPairMaxOrder) return 0;
  const int64_t n1 = split_point(len);
  return 1 + large_nodes(n1) + large_nodes(len - n1);
}
int64_t factor_helper_events(int64_t n) { return n > 0 ? 2 * large_nodes(n) : 0; }

static hipError_t chol_inv_rec(int64_t n, const FactorSet& sd, int64_t off, int64_t len,
                               hipStream_t s, FactorAux* aux, const int64_t* toff) {
  hipError_t err;
  const int ns = sd.count;
  const FactorSide& f0 = sd.first;
  const int64_t zs = sd.stride;
  if (len <= NB) {
    hipLaunchKernelGGL((chol_inv_leaf_kernel<kLeafCols, kLeafPatchCols>), dim3(ns),
                       dim3(16 * (64 / kLeafPatchCols) + 64), 0, s, sd, n, off, (int)len);
    return hipGetLastError();
  }
  const int64_t n1 = split_point(len), n2 = len - n1;
  if ((err = chol_inv_rec(n, sd, off, n1, s, aux, toff)) != hipSuccess) return err;
  const int64_t o11 = off * n + off;            // (off, off)
  const int64_t o21 = (off + n1) * n + off;     // (off + n1, off)
  const int64_t o22 = (off + n1) * n + off + n1;
  // C21 = X21 Y11^T, written where Y21 will go (that block of Y is free until then)
  Gemm64Args g{};
  g.M = n2; g.N = n1; g.K = n1; g.batch = ns;
  g.A = f0.X + o21; g.B = f0.Y + o11; g.C = f0.Y + o21; g.sA = g.sB = g.sC = zs;
  g.lda = n; g.ldb = n; g.ldc = n; g.transB = 1; g.b_lower = 1; g.alpha = 1.0; g.beta = 0.0;
  if ((err = launch_gemm64(g, s)) != hipSuccess) return err;
  // X22 -= C21 C21^T (lower blocks)
  Gemm64Args h{};
  h.M = n2; h.N = n2; h.K = n1; h.batch = ns;
  h.A = f0.Y + o21; h.B = f0.Y + o21; h.C = f0.X + o22; h.sA = h.sB = h.sC = zs;
  h.lda = n; h.ldb = n; h.ldc = n; h.transB = 1; h.lower_out = 1; h.alpha = -1.0; h.beta = 1.0;
  // Tmp = C21 Y11 (Y11 lower: column block c needs k >= c * 64), into the
  // buffer of this node's size class: the nodes inside the X22 recursion are
  // of smaller classes, and the previous node of this class finished with
  // its buffer before this node's C21 was formed
  Gemm64Args t{};
  t.M = n2; t.N = n1; t.K = n1; t.batch = ns;
  t.lda = n; t.ldb = n; t.ldc = n1; t.transB = 0; t.b_lower = 1; t.alpha = 1.0; t.beta = 0.0;
  t.A = f0.Y + o21; t.B = f0.Y + o11; t.C = f0.Tmp + toff[tmp_class(len)];
  t.sA = t.sB = t.sC = zs;
  if (len <= kPairMaxOrder || !aux || !aux->ts) {
    if ((err = launch_gemm64_pair(h, t, s)) != hipSuccess) return err;
    if ((err = chol_inv_rec(n, sd, off + n1, n2, s, aux, toff)) != hipSuccess) return err;
  } else {
    // t only has to be done before Y21 below: on the helper stream, while
    // this stream updates X22 and recurses into it
    hipEvent_t eg = aux->event(), et = aux->event();
    if (!eg || !et) return hipErrorOutOfMemory;
    if ((err = hipEventRecord(eg, s)) != hipSuccess) return err;
    if ((err = hipStreamWaitEvent(aux->ts, eg, 0)) != hipSuccess) return err;
    if ((err = launch_gemm64(t, aux->ts)) != hipSuccess) return err;
    if ((err = hipEventRecord(et, aux->ts)) != hipSuccess) return err;
    if ((err = launch_gemm64(h, s)) != hipSuccess) return err;
    if ((err = chol_inv_rec(n, sd, off + n1, n2, s, aux, toff)) != hipSuccess) return err;
    if ((err = hipStreamWaitEvent(s, et, 0)) != hipSuccess) return err;
  }
  // Y21 = -Y22 Tmp (Y22 lower)
  Gemm64Args u{};
  u.M = n2; u.N = n1; u.K = n2; u.batch = ns;
  u.A = f0.Y + o22; u.B = t.C; u.C = f0.Y + o21; u.sA = u.sB = u.sC = zs;
  u.lda = n; u.ldb = n1; u.ldc = n; u.transB = 0; u.a_lower = 1; u.alpha = -1.0; u.beta = 0.0;
  return launch_gemm64(u, s);
}

hipError_t factor_cholesky_inverse(int64_t n, const FactorSet& set, hipStream_t s,
                                   FactorAux* aux) {
  if (n <= 0 || set.count <= 0) return hipSuccess;
  if (set.count > kMaxGemmBatch) return hipErrorInvalidValue;
  int64_t toff[kTmpClasses];
  factor_tmp_layout(n, toff);
  return chol_inv_rec(n, set, 0, n, s, aux, toff);
}

template hipError_t launch_load_reversed<float>(int64_t, const float*, int64_t, int64_t, double*,
                                                int64_t, int, hipStream_t);
template hipError_t launch_load_reversed<double>(int64_t, const double*, int64_t, int64_t, double*,
                                                 int64_t, int, hipStream_t);
template hipError_t launch_store_normalized<float>(int64_t, const double*, int64_t, float*, int64_t,
                                                   int64_t, float*, int64_t, int, hipStream_t);
template hipError_t launch_store_normalized<double>(int64_t, const double*, int64_t, double*,
                                                    int64_t, int64_t, double*, int64_t, int,
                                                    hipStream_t);

}  // namespace bk
