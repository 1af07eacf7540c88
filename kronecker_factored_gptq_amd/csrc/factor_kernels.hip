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
//                                     nodes of order <= 128 in one workgroup
//                                     (two 64 x 64 leaves and the node's four
//                                     products in LDS), everything above on
//                                     float64 MFMA GEMMs (gemm64)
//   L[i][j] = Y[n-1-j][n-1-i], normalised by its diagonal  store_normalized
#include <climits>

#include "device.hpp"
#include "launch.hpp"

namespace bk {

namespace {
constexpr int NB = 64;  // Cholesky panel width
// columns per barrier step of the leaf (8: the panel wave's 8 x 8 pivot chain
// makes each step longer than two steps of 4; factor 5.81 ms against 5.26)
constexpr int kLeafCols = 4;
// columns of a patch thread's patch: 4 x 2 patches, 512 threads (4 x 4 on 256
// threads: 5.60 ms against 5.26, one wave per SIMD hides too little latency)
constexpr int kLeafPatchCols = 2;
// issue priority of the panel wave (its chain is every leaf step's critical
// path; factor 5.01 -> 4.94 ms at 4096)
constexpr int kPanelPrio = 3;
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

// Lane l's value of x (l uniform across the wave).
__device__ __forceinline__ double lane_f64(double x, int l) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane((int)b, l);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Leaf of the recursion: the Cholesky factor C of a bs x bs diagonal block
// (bs <= 64, padded with the identity) and its inverse Y = C^-1, in one
// workgroup. Right-looking, NC columns per barrier step. Patch thread
// (ty, tx) of a 16 x (64 / PCW) grid keeps rows 4 ty .., columns PCW tx .. of
// both C and Y in registers. Step st (columns j .. j + NC - 1) needs the
// panel C[i][j + q] of every row i and the final rows Y[j + q][c] of every
// column c; one extra wave (lane i: row i of the panel, column i of the rows
// of Y) forms the panel of step st + 1 during step st: it takes the columns
// j + NC .. of C and rows j + NC .. of Y as they stand before step st
// (published by their owners), applies step st's rank-NC update to them
// itself (it holds step st's panel), factors the pivot block it finds on
// rows j + NC .. (pivot_factor) and substitutes:
//   C[i][j+q] = (X[i][j+q] - sum_{p<q} C[i][j+p] l[q][p]) / l[q][q]   (i >= j+q, else 0)
//   Y[j+q][c] = (Y[j+q][c] - sum_{p<q} l[q][p] Y[j+p][c]) / l[q][q]
// The patch threads only read the panel and apply the rank-NC terms
//   C[i][c] -= sum_q C[i][j+q] C[c][j+q]   (c <= i),
//   Y[i][c] -= sum_q C[i][j+q] Y[j+q][c]   (rows below the pivot block),
// and the rows of the pivot block take their final rows of Y from the
// panel. Entries of C above the diagonal stay exact zeros (masked), so the
// upper parts of Y's rows do too. Published values are double-buffered by
// the parity of the step. A pivot that is not positive and finite records
// base + its index in *info (smallest wins) and the factorisation continues
// with NaN.
template <int NC>
struct PanelLds {
  double pc[2][NC][64];  // a step's panel C[i][j + q] (i = 0..63)
  double py[2][NC][64];  // a step's final rows Y[j + q][c] (c = 0..63)
  double rc[2][NC][64];  // the next step's columns of C before this step
  double ry[2][NC][64];  // the next step's rows of Y before this step
};

// One 64 x 64 leaf (bs x bs, padded with the identity) by the whole
// workgroup: 16 * (64 / PCW) patch threads and one panel wave. x(i, c)
// returns the leaf's input for i, c < bs, c <= i. Patch thread (ty, tx)
// returns its patch of Y = C^-1 (rows 4 ty.., columns PCW tx..) in Yr; the
// panel wave's Yr is untouched. Every thread passes the same barriers.
template <int NC, int PCW, typename XF>
__device__ __forceinline__ void leaf64(int bs, const XF& x, double (&Yr)[4][PCW],
                                       PanelLds<NC>& L, int32_t* info, int64_t base) {
  static_assert(NC % 4 == 0 && NC % PCW == 0, "whole patch rows and columns per step");
  constexpr int PRS = NC / 4;   // patch rows per step
  constexpr int TX = 64 / PCW;  // thread columns; 16 thread rows of 4 rows each
  constexpr int NCT = 16 * TX;  // patch threads; one more wave forms the panels
  const int tid = threadIdx.x;
  const int steps = (bs + NC - 1) / NC;
  auto input = [&](int i, int c) {
    if (i < bs && c < bs) return c <= i ? x(i, c) : 0.0;
    return i == c ? 1.0 : 0.0;
  };
  if (tid >= NCT) {
    // the panel chain is each step's critical path: its instructions go
    // first when the patch waves on its SIMD are ready too
    __builtin_amdgcn_s_setprio(kPanelPrio);
    const int i = tid - NCT;  // row of the panel, column of the rows of Y
    double cp[NC], yp[NC];    // this step's panel at row i / column i
    // the panel of step j1 / NC from raw columns v and raw rows w (lane i),
    // published into buffer b
    auto panel = [&](int j1, const double (&v)[NC], const double (&w)[NC], int b) {
      double blk[NC][NC], l[NC][NC], dinv[NC];
#pragma unroll
      for (int q = 0; q < NC; ++q)
#pragma unroll
        for (int p = 0; p < NC; ++p) blk[q][p] = p <= q ? lane_f64(v[p], j1 + q) : 0.0;
      int bad;
      pivot_factor<NC>(blk, l, dinv, bad);
      if (i == 0 && bad >= 0 && j1 + bad < bs) atomicMin(info, (int32_t)(base + j1 + bad));
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        double c = v[q], y = w[q];
#pragma unroll
        for (int p = 0; p < NC; ++p)
          if (p < q) {
            c -= cp[p] * l[q][p];
            y -= l[q][p] * yp[p];
          }
        cp[q] = i >= j1 + q ? c * dinv[q] : 0.0;
        yp[q] = y * dinv[q];
        L.pc[b][q][i] = cp[q];
        L.py[b][q][i] = yp[q];
      }
    };
    {
      double v[NC], w[NC];
#pragma unroll
      for (int a = 0; a < NC; ++a) {
        v[a] = input(i, a);
        w[a] = i == a ? 1.0 : 0.0;
      }
      panel(0, v, w, 0);
    }
    for (int st = 0; st < steps; ++st) {
      const int pb = st & 1;
      __syncthreads();
      if (st + 1 >= steps) continue;
      const int j1 = NC * (st + 1);
      // step st's update of the next columns and rows:
      //   C[i][j1+a] -= sum_q C[i][j+q] C[j1+a][j+q],  Y[j1+a][i] -= sum_q C[j1+a][j+q] Y[j+q][i]
      double cq[NC][NC], v[NC], w[NC];
#pragma unroll
      for (int a = 0; a < NC; ++a)
#pragma unroll
        for (int q = 0; q < NC; ++q) cq[a][q] = lane_f64(cp[q], j1 + a);
#pragma unroll
      for (int a = 0; a < NC; ++a) {
        double c = L.rc[pb][a][i], y = L.ry[pb][a][i];
#pragma unroll
        for (int q = 0; q < NC; ++q) {
          c -= cp[q] * cq[a][q];
          y -= cq[a][q] * yp[q];
        }
        v[a] = i >= j1 + a ? c : 0.0;
        w[a] = y;
      }
      panel(j1, v, w, pb ^ 1);
    }
    __builtin_amdgcn_s_setprio(0);
    return;
  }
  const int ty = tid / TX, tx = tid % TX;
  double Lr[4][PCW];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < PCW; ++b) {
      const int i = 4 * ty + a, c = PCW * tx + b;
      Lr[a][b] = input(i, c);
      Yr[a][b] = (i == c) ? 1.0 : 0.0;
    }
  for (int st = 0; st < steps; ++st) {
    const int j = NC * st, j1 = j + NC, pb = st & 1;
    // publish the next step's columns of C and rows of Y as they stand
    if (tx >= j1 / PCW && tx < (j1 + NC) / PCW) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < PCW; ++b) L.rc[pb][PCW * tx + b - j1][4 * ty + a] = Lr[a][b];
    }
    if (ty >= PRS * (st + 1) && ty < PRS * (st + 2)) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < PCW; ++b)
          L.ry[pb][4 * (ty - PRS * (st + 1)) + a][PCW * tx + b] = Yr[a][b];
    }
    __syncthreads();
    // rows above the pivot block are final
    if (ty < PRS * st) continue;
    double ci[4][NC], cc[PCW][NC], yq[NC][PCW];
#pragma unroll
    for (int q = 0; q < NC; ++q) {
#pragma unroll
      for (int a = 0; a < 4; ++a) ci[a][q] = L.pc[pb][q][4 * ty + a];
#pragma unroll
      for (int b = 0; b < PCW; ++b) {
        cc[b][q] = L.pc[pb][q][PCW * tx + b];
        yq[q][b] = L.py[pb][q][PCW * tx + b];
      }
    }
    if (ty < PRS * (st + 1)) {
      // rows of the pivot block: their rows of Y are final now
      const int rq = 4 * (ty - PRS * st);
#pragma unroll
      for (int pr = 0; pr < PRS; ++pr)
        if (rq == 4 * pr) {
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < PCW; ++b) Yr[a][b] = yq[4 * pr + a][b];
        }
      continue;
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
  }
}

template <int NC, int PCW>
__global__ __launch_bounds__(16 * (64 / PCW) + 64) void chol_inv_leaf_kernel(FactorSet set,
                                                                                  int64_t n,
                                                                                  int64_t off,
                                                                                  int bs) {
  __shared__ PanelLds<NC> L;
  const FactorSide S = factor_side(set, (int)blockIdx.x);  // one matrix per workgroup
  const double* X = S.X + off * n + off;
  double Yr[4][PCW];
  leaf64<NC, PCW>(bs, [&](int i, int c) { return X[(int64_t)i * n + c]; }, Yr, L, S.info, off);
  if ((int)threadIdx.x >= 16 * (64 / PCW)) return;
  const int ty = threadIdx.x / (64 / PCW), tx = threadIdx.x % (64 / PCW);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < PCW; ++b) {
      const int i = 4 * ty + a, c = PCW * tx + b;
      if (i < bs && c < bs) S.Y[(off + i) * n + off + c] = c <= i ? Yr[a][b] : 0.0;
    }
}

// A 64 x 64 LDS matrix, padded against bank conflicts.
constexpr int kNodeLd = 66;
typedef double NodeMat[64][kNodeLd];

// Two 16 x 16 output tiles of one wave, rows r0 .., columns c0 .. and
// c0 + 16 ..: acc[u] += A[r0 .., k] B[k, c0 + 16 u ..] over k in [k0, k1)
// (multiples of 16), a(r, k) and b(k, c) reading LDS; the two chains share
// the A operand and interleave on the matrix unit.
template <typename FA, typename FB>
__device__ __forceinline__ void node_tiles(v4d (&acc)[2], int r0, int c0, int k0, int k1,
                                           const FA& a, const FB& b) {
  const int l = threadIdx.x & 63, r = l & 15, q = l >> 4;
  for (int k = k0; k < k1; k += 16) {
    double av[4], b0[4], b1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      av[u] = a(r0 + r, k + 4 * u + q);
      b0[u] = b(k + 4 * u + q, c0 + r);
      b1[u] = b(k + 4 * u + q, c0 + 16 + r);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[0] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[u], b0[u], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[u], b1[u], acc[1], 0, 0, 0);
    }
  }
}

// A whole node of order len in (64, 128] (children: leaves of 64 and
// len - 64) in one workgroup per matrix, every intermediate in LDS:
//   Y11 = C11^-1 (leaf of X11), C21 = X21 Y11^T, X22 -= C21 C21^T,
//   Tmp = C21 Y11, Y22 = C22^-1 (leaf of X22), Y21 = -Y22 Tmp.
// The four products run on v_mfma_f64_16x16x4; each of the eight patch
// waves takes two adjacent 16 x 16 output tiles (tile row ti, tile columns
// tj0, tj0 + 1), with K ranges cut at the triangular operands' zero blocks
// (16-granular; the extra terms are exact zeros). The wave-to-tile map
// pairs heavy and light tile rows on each SIMD (waves w and w + 4 share
// one). X21 and X22 are loaded into registers early, so no global load
// latency sits between the phases.
template <int NC, int PCW>
__global__ __launch_bounds__(16 * (64 / PCW) + 64) void chol_inv_node_kernel(FactorSet set,
                                                                            int64_t n,
                                                                            int64_t off,
                                                                            int len) {
  constexpr int TX = 64 / PCW, NCT = 16 * TX;
  static_assert(NCT == 512, "eight patch waves");
  __shared__ PanelLds<NC> L;
  __shared__ NodeMat S1, S2, S3;
  const FactorSide S = factor_side(set, (int)blockIdx.x);
  const int n2 = len - 64;
  const int tid = threadIdx.x, w = tid >> 6;
  const int ty = tid / TX, tx = tid % TX;
  const bool patch = tid < NCT;
  const double* X11 = S.X + off * n + off;
  const double* X21 = S.X + (off + 64) * n + off;
  const double* X22 = S.X + (off + 64) * n + off + 64;
  double* Y11 = S.Y + off * n + off;
  double* Y21 = S.Y + (off + 64) * n + off;
  double* Y22 = S.Y + (off + 64) * n + off + 64;
  // this thread's patch of X21 (zero rows past n2), kept until the leaf is done
  double x21[4][PCW];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < PCW; ++b) {
      const int i = 4 * ty + a, c = PCW * tx + b;
      x21[a][b] = (patch && i < n2) ? X21[(int64_t)i * n + c] : 0.0;
    }
  double Yr[4][PCW];
  leaf64<NC, PCW>(64, [&](int i, int c) { return X11[(int64_t)i * n + c]; }, Yr, L, S.info, off);
  // X22's lower triangle (rows and columns below n2) for the second leaf
  double x22[4][PCW];
  if (patch) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < PCW; ++b) {
        const int i = 4 * ty + a, c = PCW * tx + b;
        x22[a][b] = (c <= i && i < n2) ? X22[(int64_t)i * n + c] : 0.0;
        const double y = c <= i ? Yr[a][b] : 0.0;
        Y11[(int64_t)i * n + c] = y;
        S1[i][c] = y;
        S2[i][c] = x21[a][b];
      }
  }
  __syncthreads();
  constexpr int kRow[8] = {1, 2, 3, 0, 0, 1, 2, 3};
  const int ti = kRow[w & 7], tj0 = w < 4 ? 0 : 2;
  const int lane = tid & 63, r16 = lane & 15, q4 = lane >> 4;
  if (patch) {
    // C21 = X21 Y11^T into S3 (Y11[c][k] = 0 for k > c)
    v4d acc[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
    node_tiles(acc, 16 * ti, 16 * tj0, 0, 16 * tj0 + 32, [&](int r, int k) { return S2[r][k]; },
               [&](int k, int c) { return S1[c][k]; });
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) S3[16 * ti + q4 + 4 * r][16 * (tj0 + u) + r16] = acc[u][r];
  }
  __syncthreads();
  v4d tmp[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
  if (patch) {
    // X22's update C21 C21^T on the lower tiles into S2 (X21 is done with),
    // and Tmp = C21 Y11 (Y11[k][c] = 0 for k < c) in registers
    if (tj0 <= ti) {
      v4d acc[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
      node_tiles(acc, 16 * ti, 16 * tj0, 0, 64, [&](int r, int k) { return S3[r][k]; },
                 [&](int k, int c) { return S3[c][k]; });
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) S2[16 * ti + q4 + 4 * r][16 * (tj0 + u) + r16] = acc[u][r];
    }
    node_tiles(tmp, 16 * ti, 16 * tj0, 16 * tj0, 64, [&](int r, int k) { return S3[r][k]; },
               [&](int k, int c) { return S1[k][c]; });
  }
  __syncthreads();
  if (patch) {
    // Tmp into S1 (Y11 is done with); the second leaf's input X22 - C21 C21^T
    // into S2 (lower triangle; the leaf reads nothing else)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) S1[16 * ti + q4 + 4 * r][16 * (tj0 + u) + r16] = tmp[u][r];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < PCW; ++b) {
        const int i = 4 * ty + a, c = PCW * tx + b;
        if (c <= i) S2[i][c] = x22[a][b] - S2[i][c];
      }
  }
  __syncthreads();
  leaf64<NC, PCW>(n2, [&](int i, int c) { return S2[i][c]; }, Yr, L, S.info, off + 64);
  if (patch) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < PCW; ++b) {
        const int i = 4 * ty + a, c = PCW * tx + b;
        const double y = (c <= i && i < n2 && c < n2) ? Yr[a][b] : 0.0;
        if (i < n2 && c < n2) Y22[(int64_t)i * n + c] = y;
        S2[i][c] = y;
      }
  }
  __syncthreads();
  if (patch) {
    // Y21 = -Y22 Tmp (Y22[r][k] = 0 for k > r)
    v4d acc[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
    node_tiles(acc, 16 * ti, 16 * tj0, 0, 16 * ti + 16, [&](int r, int k) { return S2[r][k]; },
               [&](int k, int c) { return S1[k][c]; });
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + q4 + 4 * r;
        if (i < n2) Y21[(int64_t)i * n + 16 * (tj0 + u) + r16] = -acc[u][r];
      }
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
  if (len <= 2 * NB) return;  // nodes of order <= 128 keep Tmp in LDS
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
  if (len <= 2 * NB) {
    // split_point gives 64 here: both children are leaves
    hipLaunchKernelGGL((chol_inv_node_kernel<kLeafCols, kLeafPatchCols>), dim3(ns),
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
