// BaKron solve kernels for gfx950.
//
// The solve follows "BaKron: Efficient Quantization with Kronecker-Factored
// Hessians" (arXiv 2608.06291), §3.5 Algorithm 6, applied to a tiling of W
// into T x T tiles: the recursion runs over ranges of *tile* anti-diagonals
// K = P + Q. Tiles on one tile anti-diagonal never influence each other (an
// error at (i, j) only reaches (p, q) with p >= i and q >= j, §3.3), so a leaf
// processes all of them in parallel, each tile running the entry-level
// anti-diagonal sweep of §3.3 (Algorithm 3 restricted to the tile). An
// internal node [k, l) split at mid adds, to every tile on tile
// anti-diagonals [mid, l), the update L^B E L^A^T of the errors E recorded on
// [k, mid) — the "restricted band products" of Appendix C — as two products:
// M = L^B E on the band, then W += M L^A^T on the second half.
//
// Workspace layout (HBM): W as Mt x Nt tiles, tile (P,Q) contiguous and
// row-major; after a tile is processed its slot holds its errors
// E = s*code - (value at rounding), which is what the band products read.
// L^A, L^B as packed lower-triangular tile arrays (tile (P,I), I <= P, at
// P(P+1)/2 + I), unit diagonal, zero above it and on padding.
#include "device.hpp"
#include "launch.hpp"

namespace bk {

// ---------------------------------------------------------------------------
// Pack W (row-major, ldw) into tiles; padding is zero.
// ---------------------------------------------------------------------------
template <typename R, int T>
__global__ __launch_bounds__(256) void pack_w_kernel(int64_t m, int64_t n, int Nt,
                                                     const R* __restrict__ W, int64_t ldw,
                                                     R* __restrict__ Wk) {
  const int64_t tile = blockIdx.x;
  const int64_t P = tile / Nt, Q = tile % Nt;
  R* dst = Wk + tile * T * T;
  for (int e = threadIdx.x; e < T * T; e += blockDim.x) {
    const int64_t i = P * T + e / T, j = Q * T + e % T;
    dst[e] = (i < m && j < n) ? W[i * ldw + j] : R(0);
  }
}

// Pack the strict lower triangle of a normalised factor into lower tiles;
// the diagonal is 1 (normalised factor), everything above it and on padding 0.
template <typename R, int T>
__global__ __launch_bounds__(256) void pack_l_kernel(int64_t dim, const R* __restrict__ L,
                                                     int64_t ld, R* __restrict__ Lp) {
  const int64_t t = blockIdx.x;
  int64_t P = (int64_t)((__builtin_sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while (P * (P + 1) / 2 > t) --P;
  while ((P + 1) * (P + 2) / 2 <= t) ++P;
  const int64_t I = t - P * (P + 1) / 2;
  R* dst = Lp + t * T * T;
  for (int e = threadIdx.x; e < T * T; e += blockDim.x) {
    const int64_t i = P * T + e / T, j = I * T + e % T;
    R v = R(0);
    if (i == j) v = R(1);
    else if (j < i && i < dim) v = L[i * ld + j];
    dst[e] = v;
  }
}

// ---------------------------------------------------------------------------
// Leaf: one tile anti-diagonal K. One workgroup per tile, one thread per entry.
// Entry (p, q) of the tile is rounded at in-tile step t = p + q; after each
// step the errors of that in-tile anti-diagonal are added to the tile with
// the rank-d update of §3.3, L^B[:, i] e_i L^A[:, t-i]^T summed over the
// step's entries (i, t-i). Rows p of the diagonal factor tiles live in
// registers; entries with i > p or t-i > q meet exact zeros of the
// triangular factors, so every thread runs the same unrolled update.
// ---------------------------------------------------------------------------
template <typename R, int T>
__global__ __launch_bounds__(T * T) void leaf_kernel(int K, int Mt, int Nt, int64_t m, int64_t n,
                                                     R* __restrict__ Wk,
                                                     const R* __restrict__ LBp,
                                                     const R* __restrict__ LAp, LeafParams<R> lp) {
  __shared__ R ebuf[2][T];
  const int tid = threadIdx.x;
  const int p = tid / T, q = tid % T;
  const int P = (K - (Nt - 1) > 0 ? K - (Nt - 1) : 0) + (int)blockIdx.x;
  const int Q = K - P;
  R* tileW = Wk + ((int64_t)P * Nt + Q) * T * T;
  const R* tB = LBp + tri_index(P, P) * T * T + p * T;  // row p of L^B[P,P]
  const R* tA = LAp + tri_index(Q, Q) * T * T + q * T;  // row q of L^A[Q,Q]

  R lb[T], la[T];
#pragma unroll
  for (int i = 0; i < T; ++i) {
    lb[i] = tB[i];
    la[i] = tA[i];
  }
  R x = tileW[p * T + q];
  const int64_t gi = (int64_t)P * T + p, gj = (int64_t)Q * T + q;
  const bool valid = gi < m && gj < n;
  R s = R(1);
  if (lp.scale_mode == 1) s = gi < m ? lp.scales[gi] : R(1);
  else if (lp.scale_mode == 2) s = gj < n ? lp.scales[gj] : R(1);
  const bool unb = lp.unbounded != 0;

  R code = R(0), xt = R(0), eout = R(0);
#pragma unroll
  for (int t = 0; t < 2 * T - 1; ++t) {
    if (p + q == t) {
      const R c = quant_code(x, s, lp.lo, lp.hi, unb);
      const R e = valid ? s * c - x : R(0);
      code = c;
      xt = x;
      eout = e;
      ebuf[t & 1][p] = e;
    }
    __syncthreads();
    const int ilo = t - (T - 1) > 0 ? t - (T - 1) : 0;
    const int ihi = t < T - 1 ? t : T - 1;
    R acc0 = R(0), acc1 = R(0);
#pragma unroll
    for (int i = ilo; i <= ihi; ++i) {
      const R g = lb[i] * ebuf[t & 1][i];
      if ((i - ilo) & 1) acc1 = __builtin_fma(g, la[t - i], acc1);
      else acc0 = __builtin_fma(g, la[t - i], acc0);
    }
    x += acc0 + acc1;
  }
  tileW[p * T + q] = eout;
  if (valid) {
    lp.V[gi * lp.ldv + gj] = (int32_t)code;
    if (lp.Wt) lp.Wt[gi * lp.ldwt + gj] = xt;
  }
}

// ---------------------------------------------------------------------------
// Small internal node (q = l - k <= kSmallNodeMaxQ): one wave per target tile
// (P, Q) on tile anti-diagonals [mid, l), computing
//   sum_J (sum_I L^B[P,I] E[I,J]) L^A[Q,J]^T
// over source tiles (I, J) on [k, mid) with I <= P, J <= Q, in one launch.
// T must be 16: a tile is one 16x16 MFMA block.
// ---------------------------------------------------------------------------
struct SmallNodeDiags {
  int count;        // number of target tile anti-diagonals (l - mid)
  int first[9];     // first[d] = linear index of the first tile of diagonal mid + d
};

template <typename R>
__global__ __launch_bounds__(64) void node_small_kernel(int k, int mid, int l, int Mt, int Nt,
                                                        R* __restrict__ Wk,
                                                        const R* __restrict__ LBp,
                                                        const R* __restrict__ LAp,
                                                        SmallNodeDiags dg) {
  constexpr int T = 16;
  typedef Mfma<R> MF;
  typedef typename MF::acc_t acc_t;
  __shared__ R ms[T][T + 2];
  const int lane = threadIdx.x;
  const int idx = blockIdx.x;
  int d = 0;
  while (d + 1 < dg.count && idx >= dg.first[d + 1]) ++d;
  const int Kt = mid + d;
  const int Plo = Kt - (Nt - 1) > 0 ? Kt - (Nt - 1) : 0;
  const int P = Plo + (idx - dg.first[d]);
  const int Q = Kt - P;
  const int r16 = lane & 15, kg = lane >> 4;

  acc_t acc = MF::zero();
  const int Jlo = k - P > 0 ? k - P : 0;
  const int Jhi = Q < mid - 1 ? Q : mid - 1;
  for (int J = Jlo; J <= Jhi; ++J) {
    const int Ilo = k - J > 0 ? k - J : 0;
    const int Ihi = P < mid - 1 - J ? P : mid - 1 - J;
    if (Ilo > Ihi) continue;
    acc_t macc = MF::zero();
    for (int I = Ilo; I <= Ihi; ++I) {
      const R* a = LBp + tri_index(P, I) * T * T;   // [r][k]
      const R* b = Wk + ((int64_t)I * Nt + J) * T * T;  // E[I,J] [k][c]
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int kk = 4 * kg + st;
        macc = MF::mma(a[r16 * T + kk], b[kk * T + r16], macc);
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) ms[MF::row(lane, r)][r16] = macc[r];
    __syncthreads();
    const R* la = LAp + tri_index(Q, J) * T * T;  // B[k][c] = L^A[Q,J][c][k]
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kk = 4 * kg + st;
      acc = MF::mma(ms[r16][kk], la[r16 * T + kk], acc);
    }
  }
  R* w = Wk + ((int64_t)P * Nt + Q) * T * T;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = MF::row(lane, r);
    w[row * T + r16] += acc[r];
  }
}

// ---------------------------------------------------------------------------
// Large internal node: the two restricted band products as MFMA GEMMs over
// macro tiles of MB x MB solver tiles (MB*T elements square), 4 waves in a
// 2 x 2 arrangement, K stepped one solver tile at a time through
// double-buffered LDS. Masks are per solver tile.
//   stage 1: M[P,J]  = sum_I L^B[P,I] E[I,J],   I <= P, k <= I+J < mid
//   stage 2: W[P,Q] += sum_J M[P,J] L^A[Q,J]^T, J <= Q, J < mid,
//            k <= P+J <= l-1, written only where mid <= P+Q <= l-1.
// ---------------------------------------------------------------------------
template <typename R> struct BandCfg;
template <> struct BandCfg<float> { static constexpr int MB = 8; static constexpr int PAD = 4; };
template <> struct BandCfg<double> { static constexpr int MB = 4; static constexpr int PAD = 2; };

template <typename R, int STAGE>
__global__ __launch_bounds__(256) void band_kernel(int k, int mid, int l, int Mt, int Nt,
                                                   R* __restrict__ Wk, const R* __restrict__ LBp,
                                                   const R* __restrict__ LAp, R* __restrict__ Mb) {
  constexpr int T = kTile;
  constexpr int MB = BandCfg<R>::MB;
  constexpr int BM = MB * T;       // macro tile edge in elements
  constexpr int LDS_LD = T + BandCfg<R>::PAD;
  constexpr int WT = BM / 2;       // wave tile edge
  constexpr int NBW = WT / 16;     // 16x16 blocks per wave edge
  constexpr int PER = MB * T * T / 256;  // elements per thread per operand per K step
  typedef Mfma<R> MF;
  typedef typename MF::acc_t acc_t;

  __shared__ R As[2][BM][LDS_LD];
  __shared__ R Bs[2][BM][LDS_LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int r16 = lane & 15, kg = lane >> 4;

  const int pb = blockIdx.y;
  const int P0 = pb * MB;
  // column-block range of this macro row
  int Clo, Chi;
  if (STAGE == 1) {
    Clo = k - (P0 + MB - 1); if (Clo < 0) Clo = 0;
    Chi = Nt - 1; if (mid - 1 < Chi) Chi = mid - 1; if (l - 1 - P0 < Chi) Chi = l - 1 - P0;
  } else {
    Clo = mid - (P0 + MB - 1); if (Clo < 0) Clo = 0;
    Chi = Nt - 1; if (l - 1 - P0 < Chi) Chi = l - 1 - P0;
  }
  if (Clo > Chi) return;
  const int cb = Clo / MB + (int)blockIdx.x;
  if (cb > Chi / MB) return;
  const int C0 = cb * MB;

  int Klo, Khi;
  if (STAGE == 1) {
    Klo = k - (C0 + MB - 1); if (Klo < 0) Klo = 0;
    Khi = P0 + MB - 1; if (mid - 1 - C0 < Khi) Khi = mid - 1 - C0; if (Mt - 1 < Khi) Khi = Mt - 1;
  } else {
    Klo = k - (P0 + MB - 1); if (Klo < 0) Klo = 0;
    Khi = C0 + MB - 1; if (mid - 1 < Khi) Khi = mid - 1; if (Nt - 1 < Khi) Khi = Nt - 1;
  }

  acc_t acc[NBW][NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = MF::zero();

  R ra[PER], rb[PER];
  auto gload = [&](int kk) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = u * 256 + tid;
      const int t = e / (T * T);          // which tile of the macro row / column
      const int w = e % (T * T);
      const int P = P0 + t, C = C0 + t;
      R va = R(0), vb = R(0);
      if (STAGE == 1) {
        if (P < Mt && kk <= P) va = LBp[tri_index(P, kk) * T * T + w];
        const int s = kk + C;
        if (C < Nt && s >= k && s < mid) vb = Wk[((int64_t)kk * Nt + C) * T * T + w];
      } else {
        const int s = P + kk;
        if (P < Mt && kk <= mid - 1 && s >= k && s <= l - 1) va = Mb[((int64_t)P * Nt + kk) * T * T + w];
        if (C < Nt && kk <= C) vb = LAp[tri_index(C, kk) * T * T + w];
      }
      ra[u] = va;
      rb[u] = vb;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = u * 256 + tid;
      const int t = e / (T * T);
      const int w = e % (T * T);
      const int r = w / T, c = w % T;
      As[buf][t * T + r][c] = ra[u];               // A[row][k]
      if (STAGE == 1) Bs[buf][t * T + c][r] = rb[u];  // E[k=r][col=c] -> Bs[col][k]
      else Bs[buf][t * T + r][c] = rb[u];           // L^A[col=r][k=c] -> Bs[col][k]
    }
  };

  if (Klo <= Khi) {
    gload(Klo);
    sstore(0);
    __syncthreads();
    for (int kk = Klo; kk <= Khi; ++kk) {
      const int buf = (kk - Klo) & 1;
      if (kk < Khi) gload(kk + 1);
#pragma unroll
      for (int st = 0; st < T / 4; ++st) {
        R af[NBW], bf[NBW];
#pragma unroll
        for (int i = 0; i < NBW; ++i) af[i] = As[buf][wr * WT + i * 16 + r16][4 * kg + st];
#pragma unroll
        for (int j = 0; j < NBW; ++j) bf[j] = Bs[buf][wc * WT + j * 16 + r16][4 * kg + st];
#pragma unroll
        for (int i = 0; i < NBW; ++i)
#pragma unroll
          for (int j = 0; j < NBW; ++j) acc[i][j] = MF::mma(af[i], bf[j], acc[i][j]);
      }
      if (kk < Khi) sstore(buf ^ 1);
      __syncthreads();
    }
  }

  // epilogue
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wr * WT + i * 16 + MF::row(lane, r);
        const int col = wc * WT + j * 16 + r16;
        const int P = P0 + row / T, C = C0 + col / T;
        if (P >= Mt || C >= Nt) continue;
        const int64_t off = ((int64_t)P * Nt + C) * T * T + (row % T) * T + (col % T);
        if (STAGE == 1) {
          Mb[off] = acc[i][j][r];
        } else {
          const int s = P + C;
          if (s >= mid && s <= l - 1) Wk[off] += acc[i][j][r];
        }
      }
}

// ---------------------------------------------------------------------------
// Host wrappers
// ---------------------------------------------------------------------------
template <typename R>
hipError_t launch_pack_w(const SolveGeom& g, const R* W, int64_t ldw, R* Wk, hipStream_t s) {
  const int64_t nt = (int64_t)g.Mt * g.Nt;
  if (nt == 0) return hipSuccess;
  hipLaunchKernelGGL((pack_w_kernel<R, kTile>), dim3((unsigned)nt), dim3(256), 0, s, g.m, g.n,
                     g.Nt, W, ldw, Wk);
  return hipGetLastError();
}

template <typename R>
hipError_t launch_pack_l(int64_t dim, int Dt, const R* L, int64_t ld, R* Lp, hipStream_t s) {
  const int64_t nt = (int64_t)Dt * (Dt + 1) / 2;
  if (nt == 0) return hipSuccess;
  hipLaunchKernelGGL((pack_l_kernel<R, kTile>), dim3((unsigned)nt), dim3(256), 0, s, dim, L, ld,
                     Lp);
  return hipGetLastError();
}

static inline void diag_range(const SolveGeom& g, int K, int* lo, int* hi) {
  *lo = K - (g.Nt - 1) > 0 ? K - (g.Nt - 1) : 0;
  *hi = K < g.Mt - 1 ? K : g.Mt - 1;
}

template <typename R>
hipError_t launch_leaf(const SolveGeom& g, int K, R* Wk, const R* LBp, const R* LAp,
                       const LeafParams<R>& lp, hipStream_t s) {
  int lo, hi;
  diag_range(g, K, &lo, &hi);
  if (hi < lo) return hipSuccess;
  hipLaunchKernelGGL((leaf_kernel<R, kTile>), dim3(hi - lo + 1), dim3(kTile * kTile), 0, s, K,
                     g.Mt, g.Nt, g.m, g.n, Wk, LBp, LAp, lp);
  return hipGetLastError();
}

template <typename R>
hipError_t launch_node_small(const SolveGeom& g, int k, int mid, int l, R* Wk, const R* LBp,
                             const R* LAp, hipStream_t s) {
  static_assert(kTile == 16, "small-node kernel assumes 16x16 tiles");
  SmallNodeDiags dg;
  dg.count = l - mid;
  if (dg.count > 8 || dg.count < 1) return hipErrorInvalidValue;
  int total = 0;
  for (int d = 0; d < dg.count; ++d) {
    dg.first[d] = total;
    int lo, hi;
    diag_range(g, mid + d, &lo, &hi);
    total += hi >= lo ? hi - lo + 1 : 0;
  }
  for (int d = dg.count; d < 9; ++d) dg.first[d] = total;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((node_small_kernel<R>), dim3(total), dim3(64), 0, s, k, mid, l, g.Mt, g.Nt,
                     Wk, LBp, LAp, dg);
  return hipGetLastError();
}

template <typename R>
hipError_t launch_node_band(const SolveGeom& g, int k, int mid, int l, int stage, R* Wk,
                            const R* LBp, const R* LAp, R* Mb, hipStream_t s) {
  constexpr int MB = BandCfg<R>::MB;
  const int nPb = (g.Mt + MB - 1) / MB;
  int maxw = 0;
  for (int pb = 0; pb < nPb; ++pb) {
    const int P0 = pb * MB;
    int Clo, Chi;
    if (stage == 1) {
      Clo = k - (P0 + MB - 1); if (Clo < 0) Clo = 0;
      Chi = g.Nt - 1; if (mid - 1 < Chi) Chi = mid - 1; if (l - 1 - P0 < Chi) Chi = l - 1 - P0;
    } else {
      Clo = mid - (P0 + MB - 1); if (Clo < 0) Clo = 0;
      Chi = g.Nt - 1; if (l - 1 - P0 < Chi) Chi = l - 1 - P0;
    }
    if (Clo > Chi) continue;
    const int w = Chi / MB - Clo / MB + 1;
    if (w > maxw) maxw = w;
  }
  if (maxw == 0) return hipSuccess;
  if (stage == 1)
    hipLaunchKernelGGL((band_kernel<R, 1>), dim3(maxw, nPb), dim3(256), 0, s, k, mid, l, g.Mt,
                       g.Nt, Wk, LBp, LAp, Mb);
  else
    hipLaunchKernelGGL((band_kernel<R, 2>), dim3(maxw, nPb), dim3(256), 0, s, k, mid, l, g.Mt,
                       g.Nt, Wk, LBp, LAp, Mb);
  return hipGetLastError();
}

#define BK_INST(R)                                                                              \
  template hipError_t launch_pack_w<R>(const SolveGeom&, const R*, int64_t, R*, hipStream_t);  \
  template hipError_t launch_pack_l<R>(int64_t, int, const R*, int64_t, R*, hipStream_t);      \
  template hipError_t launch_leaf<R>(const SolveGeom&, int, R*, const R*, const R*,             \
                                     const LeafParams<R>&, hipStream_t);                        \
  template hipError_t launch_node_small<R>(const SolveGeom&, int, int, int, R*, const R*,       \
                                           const R*, hipStream_t);                              \
  template hipError_t launch_node_band<R>(const SolveGeom&, int, int, int, int, R*, const R*,   \
                                          const R*, R*, hipStream_t);
BK_INST(float)
BK_INST(double)
#undef BK_INST

}  // namespace bk
