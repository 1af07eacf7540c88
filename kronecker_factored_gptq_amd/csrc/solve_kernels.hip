// BaKron solve kernels for gfx950.
//
// The solve follows "BaKron: Efficient Quantization with Kronecker-Factored
// Hessians" (arXiv 2608.06291), §3.5 Algorithm 6, applied to a tiling of W
// into T x T tiles: the recursion runs over ranges of *tile* anti-diagonals
// K = P + Q. Tiles on one tile anti-diagonal never influence each other (an
// error at (i, j) only reaches (p, q) with p >= i and q >= j, §3.3), so a leaf
// processes all of them in parallel, each tile running the entry-level
// anti-diagonal sweep of §3.3 (Algorithm 3 restricted to the tile). The
// recursion runs over blocks of G consecutive tile anti-diagonals; inside a
// block, each leaf first applies the updates from the block's earlier tile
// anti-diagonals (left-looking), and an internal node [k, l) split at mid
// (block boundaries) adds to every tile on [mid, l) the update L^B E L^A^T of
// the errors E recorded on [k, mid) — the "restricted band products" of
// Appendix C, in band_kernels.hip.
//
// Code units. With per-row scales s (S = diag(s)) the solve runs on
// U = S^-1 W, whose entries are rounded by a plain rint: the update
// W += e (L^B e_i)(L^A e_j)^T of §3.3 with e = s_i (c - u) is, divided by the
// row scales, U += (c - u) (S^-1 L^B S e_i)(L^A e_j)^T. So the packed L^B is
// S^-1 L^B S (still unit lower triangular) and every error is c - u, in units
// of its row's scale; per-column scales scale L^A the same way; without
// scales nothing changes. Exact arithmetic gives the same codes (the
// quotient x / s at rounding time equals u), with no division in the sweep.
//
// Workspace layout (HBM): U as Mt x Nt tiles, tile (P,Q) contiguous and
// row-major; after a tile is processed its slot holds its errors c - u
// (code units), which is what the band products read. The scaled L^A, L^B as
// packed lower-triangular tile arrays (tile (P,I), I <= P, at P(P+1)/2 + I),
// unit diagonal, zero above it and on padding.
#include <hip/hip_ext.h>

#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace bk {

// ---------------------------------------------------------------------------
// Pack U = W / s (row-major W, ldw) into tiles; padding is zero. mode: 0 no
// scales, 1 per-row, 2 per-column.
// ---------------------------------------------------------------------------
template <typename R, int T>
__global__ __launch_bounds__(256) void pack_w_kernel(int64_t m, int64_t n, int Nt,
                                                     const R* __restrict__ W, int64_t ldw,
                                                     const R* __restrict__ sc, int mode,
                                                     R* __restrict__ Wk, BatchStrides bs) {
  // problem blockIdx.y of a batch
  const int64_t b = blockIdx.y;
  W += b * bs.w;
  if (sc) sc += b * bs.s;
  Wk += b * bs.ws;
  const int64_t tile = blockIdx.x;
  const int64_t P = tile / Nt, Q = tile % Nt;
  R* dst = Wk + tile * T * T;
  for (int e = threadIdx.x; e < T * T; e += blockDim.x) {
    const int64_t i = P * T + e / T, j = Q * T + e % T;
    R v = R(0);
    if (i < m && j < n) {
      v = W[i * ldw + j];
      if (mode == 1) v = v / sc[i];
      else if (mode == 2) v = v / sc[j];
    }
    dst[e] = v;
  }
}

// Pack the strict lower triangle of a normalised factor into lower tiles,
// scaled to code units when sc is given (entry (i, j) times s_j / s_i); the
// diagonal is 1, everything above it and on padding 0.
template <typename R, int T>
__global__ __launch_bounds__(256) void pack_l_kernel(int64_t dim, const R* __restrict__ L,
                                                     int64_t ld, int64_t sL,
                                                     const R* __restrict__ sc, int64_t sS,
                                                     R* __restrict__ Lp, int64_t sLp) {
  const int64_t b = blockIdx.y;  // problem of a batch
  L += b * sL;
  if (sc) sc += b * sS;
  Lp += b * sLp;
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
    else if (j < i && i < dim) {
      v = L[i * ld + j];
      if (sc) v = v * sc[j] / sc[i];
    }
    dst[e] = v;
  }
}

// ---------------------------------------------------------------------------
// Leaf: tile anti-diagonal K, the (K - K0)-th of the block [K0, K0 + G) of
// tile anti-diagonals. One workgroup per tile (P, Q); T = 16.
//
// 1. Prologue (four waves): add the errors of the tiles (I, J) of the same
//    block on earlier tile anti-diagonals, I <= P, J <= Q, as
//    sum_J (sum_I L^B[P,I] E[I,J]) L^A[Q,J]^T — the updates between tile
//    anti-diagonals of one block are done here, left-looking, instead of by
//    internal nodes (any grouping of the updates gives the same codes,
//    Appendix B). The inner sums M[P][J] of row P are carried from leaf to
//    leaf of the block (only two columns change per leaf); each wave takes
//    every fourth J and a quarter of the new column's terms. The inner sum is
//    computed transposed, M^T = E^T L^B^T, because the MFMA result layout of
//    M^T is exactly the A-operand layout of the outer product with k = its
//    row index: no data movement between the two products.
// 2. Sweep (wave 0): the tile lives in the MFMA accumulator. In-tile step t
//    rounds the entries (p, t - p) (one per column, §3.3's anti-diagonal
//    order) to c = clamp(rint(u)) and adds L^B e L^A^T for the step's errors
//    e = c - u as one 16x16x16 MFMA product: A[p][k] = L^B[p][k] e_k,
//    B[k][q] = L^A[q][t - k]. Entries already rounded, or with (k, t - k)
//    outside the tile, meet exact zeros of the triangular factors. Each step
//    records the value at rounding in LDS; codes and errors are formed from
//    it again (same operations) when the tile is written back.
// ---------------------------------------------------------------------------
template <typename R> struct EVec;
template <> struct EVec<float> {
  __device__ static inline void load4(const float* p, float* out) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
  __device__ static inline void store4(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct EVec<double> {
  __device__ static inline void load4(const double* p, double* out) {
    const double2 v0 = reinterpret_cast<const double2*>(p)[0];
    const double2 v1 = reinterpret_cast<const double2*>(p)[1];
    out[0] = v0.x; out[1] = v0.y; out[2] = v1.x; out[3] = v1.y;
  }
  __device__ static inline void store4(double* p, const double* v) {
    reinterpret_cast<double2*>(p)[0] = make_double2(v[0], v[1]);
    reinterpret_cast<double2*>(p)[1] = make_double2(v[2], v[3]);
  }
};

// Sweep error exchange. MFMA s of a sweep step takes, in lane row kg
// (lanes 16 kg .. 16 kg + 15), the in-tile row k = KA kg + KB s. The choice
// makes the error e_k come from the same lane row that consumes it: the float
// accumulator holds tile row 4 kg + r in lane row kg, the double one row
// kg + 4 r. The producing lane sits at column t - k; skewing lane row kg by
// KA kg columns (two masked row rotations) moves every producer of MFMA s to
// column (t - KB s) mod 16, and one row broadcast hands e_k to the row.
template <typename R> struct SweepK;
template <> struct SweepK<float> { static constexpr int KA = 4, KB = 1; };
template <> struct SweepK<double> { static constexpr int KA = 1, KB = 4; };

// gfx9 DPP controls: rotate right inside each row of 16 lanes (lane c reads
// lane c - n), and broadcast lane n of each row to that row (gfx90a on).
constexpr int kDppRowRor = 0x120;
constexpr int kDppRowNewBcast = 0x150;

template <int CTRL, int ROWS>
__device__ inline float dpp_mov(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROWS, 0xF, false));
}
template <int CTRL, int ROWS>
__device__ inline double dpp_mov(double old, double v) {
  const int2 o = __builtin_bit_cast(int2, old), x = __builtin_bit_cast(int2, v);
  int2 r;
  r.x = __builtin_amdgcn_update_dpp(o.x, x.x, CTRL, ROWS, 0xF, false);
  r.y = __builtin_amdgcn_update_dpp(o.y, x.y, CTRL, ROWS, 0xF, false);
  return __builtin_bit_cast(double, r);
}

// Broadcast of lane n of each row to its row. Float: written with an old
// value of 0 so that the compiler folds it into the multiply that uses it;
// double: two full-row moves (every lane written, no old value needed).
template <int N>
__device__ inline float row_bcast(float v) {
  return dpp_mov<kDppRowNewBcast + N, 0xF>(0.0f, v);
}
template <int N>
__device__ inline double row_bcast(double v) {
  const int2 x = __builtin_bit_cast(int2, v);
  int2 r;
  r.x = __builtin_amdgcn_mov_dpp(x.x, kDppRowNewBcast + N, 0xF, 0xF, false);
  r.y = __builtin_amdgcn_mov_dpp(x.y, kDppRowNewBcast + N, 0xF, 0xF, false);
  return __builtin_bit_cast(double, r);
}

// lane row kg: result column c holds the input's column (c - KA kg) mod 16
template <typename R>
__device__ inline R row_skew(R e) {
  constexpr int A = SweepK<R>::KA;
  const R a = dpp_mov<kDppRowRor + A, 0xA>(e, e);      // rows 1 and 3
  return dpp_mov<kDppRowRor + 2 * A, 0xC>(a, a);       // rows 2 and 3
}

// clamp(rint(x), lo, hi) as in quant_unit (lo <= hi): one median-of-three
// for float
__device__ inline float round_clamp(float x, float lo, float hi) {
  return __builtin_amdgcn_fmed3f(__builtin_rintf(x), lo, hi);
}
__device__ inline double round_clamp(double x, double lo, double hi) {
  return quant_unit(x, lo, hi);
}

// Lanes whose accumulator entry r lies on in-tile anti-diagonal t (lane l
// holds row(l, r) of column l % 16), as a wave mask.
template <typename R>
constexpr uint64_t entry_lanes(int t, int r) {
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l) {
    const int row = std::is_same<R, float>::value ? 4 * (l >> 4) + r : (l >> 4) + 4 * r;
    if (row + (l & 15) == t) m |= uint64_t(1) << l;
  }
  return m;
}

template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Waves of a leaf workgroup: wave w of the prologue takes the block's earlier
// tiles of columns J = Jlo + w, Jlo + w + kLeafWaves, ...
constexpr int kLeafWaves = 4;

template <typename R>
__global__ __launch_bounds__(64 * kLeafWaves) void leaf_kernel(int K, int K0, int Mt, int Nt, int64_t m,
                                                   int64_t n, R* __restrict__ Wk,
                                                   const R* __restrict__ LBp,
                                                   const R* __restrict__ LAp,
                                                   R* __restrict__ Mc, LeafParams<R> lp,
                                                   BatchStrides bs) {
  constexpr int T = 16;
  {  // problem blockIdx.y of a batch: its workspace and outputs
    const int64_t b = blockIdx.y;
    Wk += b * bs.ws;
    LBp += b * bs.ws;
    LAp += b * bs.ws;
    Mc += b * bs.ws;
    lp.V += b * bs.v;
    if (lp.Wt) lp.Wt += b * bs.wt;
    if (lp.scales) lp.scales += b * bs.s;
  }
  typedef Mfma<R> MF;
  typedef typename MF::acc_t acc_t;
  __shared__ R red[kLeafWaves - 1][T][T + 1];
  __shared__ __attribute__((aligned(16))) R fm[kLeafWaves][T * T];  // fresh-column shares
  __shared__ R lat[T][T + 1];
  // sweep: value at rounding, one copy per lane row kg; lane (kg, c) writes
  // step t to row t - c + (T - 1) of its copy (a real entry's slot when row
  // t - c is one of its own rows, an unread one otherwise)
  constexpr int kOwRows = 3 * T - 2, kOwLd = T + 1 + (int)(sizeof(float) / sizeof(R));
  __shared__ R owv[4][kOwRows][kOwLd];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, kg = lane >> 4;
  const int P = (K - (Nt - 1) > 0 ? K - (Nt - 1) : 0) + (int)blockIdx.x;
  const int Q = K - P;
  R* tW = Wk + ((int64_t)P * Nt + Q) * T * T;

  // sweep inputs, requested before the prologue so that their latency
  // overlaps it: this thread's element of L^A[Q,Q] and, on wave 0, the tile
  // and its lbK operands (lbK[s] = L^B[P,P][c][KA kg + KB s])
  constexpr int KA = SweepK<R>::KA, KB = SweepK<R>::KB;
  const R lat_v = tid < T * T ? LAp[tri_index(Q, Q) * T * T + tid] : R(0);
  R w0[4], lbK[4];
  if (wave == 0) {
    const R* lb = LBp + tri_index(P, P) * T * T + c * T + KA * kg;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      w0[r] = tW[MF::row(lane, r) * T + c];
      lbK[r] = lb[KB * r];
    }
  }

  // ---- 1. prologue: acc = sum over J of M[P][J] L^A[Q,J]^T, with
  // M[P][J] = sum_I L^B[P,I] E[I,J] over the block's earlier tiles (I, J).
  // Row P's partial sums are kept between the leaves of a block in Mc (slot
  // J of row P, MFMA lane layout: lane l holds M[c][row(l, r)] at l * 4 + r):
  // from leaf K - 1 to K only column J = Q - 1 gains a term (I = P) and
  // column J = Q is new (I < P), so a leaf adds d + 1 tile products instead
  // of recomputing all (d + 1)(d + 2) / 2 - 1 of them (d = K - K0).
  constexpr int NJ = (kLeafBlock - 1 + kLeafWaves - 1) / kLeafWaves;  // cached columns per wave
  constexpr int NI = (kLeafBlock - 1 + kLeafWaves - 1) / kLeafWaves;  // fresh-column terms per wave
  const int d = K - K0;
  const bool keep = d + 1 < kLeafBlock;  // a later leaf of this block reads the cache
  acc_t acc = MF::zero();
  acc_t fresh = MF::zero();  // this wave's share of M[P][Q]
  R* McP = Mc + (int64_t)P * Nt * T * T;
  if (d > 0) {
    const int Jlo = K0 - P > 0 ? K0 - P : 0;
    const int Ilo = K0 - Q > 0 ? K0 - Q : 0;  // fresh column: Ilo <= I <= P - 1
    // every load first: cached columns J = Jlo + wave + kLeafWaves t < Q,
    // their L^A tiles, the update term of J = Q - 1, this wave's terms of
    // the fresh column, and L^A[Q,Q]
    R la[NJ][4], mc[NJ][4], laq[4], eu[4], lu[4], ef[NI][4], lf[NI][4];
    // Float: no branch around these loads (a load under a branch made the
    // compiler wait there for every load in flight, the sweep operands
    // included; columns J >= Q read slot Q instead and are never used, and
    // the cache is selected away before the block's third leaf): 1.8 %
    // faster solve. Double: 3.6 % slower that way, so it keeps the guards.
    constexpr bool kFlatLoads = std::is_same<R, float>::value;
#pragma unroll
    for (int t = 0; t < NJ; ++t) {
      const int J = Jlo + wave + kLeafWaves * t;
      if constexpr (kFlatLoads) {
        const int Jc = J < Q ? J : Q;
        const R* La = LAp + tri_index(Q, Jc) * T * T;
#pragma unroll
        for (int s = 0; s < 4; ++s) la[t][s] = La[c * T + MF::row(lane, s)];
        EVec<R>::load4(McP + (int64_t)Jc * T * T + lane * 4, mc[t]);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) { la[t][s] = R(0); mc[t][s] = R(0); }
        if (J < Q) {
          const R* La = LAp + tri_index(Q, J) * T * T;
#pragma unroll
          for (int s = 0; s < 4; ++s) la[t][s] = La[c * T + MF::row(lane, s)];
          if (d >= 2) EVec<R>::load4(McP + (int64_t)J * T * T + lane * 4, mc[t]);
        }
      }
    }
    {
      const R* La = LAp + tri_index(Q, Q) * T * T;
#pragma unroll
      for (int s = 0; s < 4; ++s) laq[s] = La[c * T + MF::row(lane, s)];
    }
    const bool upd = Q >= 1 && Q - 1 >= Jlo && (Q - 1 - Jlo) % kLeafWaves == wave;
    if (upd) {
      const R* E = Wk + ((int64_t)P * Nt + Q - 1) * T * T;
      EVec<R>::load4(LBp + tri_index(P, P) * T * T + c * T + 4 * kg, lu);
#pragma unroll
      for (int s = 0; s < 4; ++s) eu[s] = E[(4 * kg + s) * T + c];
    }
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int I = Ilo + wave + kLeafWaves * u;
      if (I <= P - 1) {
        const R* E = Wk + ((int64_t)I * Nt + Q) * T * T;
        EVec<R>::load4(LBp + tri_index(P, I) * T * T + c * T + 4 * kg, lf[u]);
#pragma unroll
        for (int s = 0; s < 4; ++s) ef[u][s] = E[(4 * kg + s) * T + c];
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) { ef[u][s] = R(0); lf[u][s] = R(0); }
      }
    }
    // fresh column: this wave's terms, and its part of the outer product
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      if (Ilo + wave + kLeafWaves * u > P - 1) break;
#pragma unroll
      for (int s = 0; s < 4; ++s) fresh = MF::mma(ef[u][s], lf[u][s], fresh);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = MF::mma(fresh[s], laq[s], acc);
    // cached columns (J = Q - 1 gains its term and is stored back)
#pragma unroll
    for (int t = 0; t < NJ; ++t) {
      const int J = Jlo + wave + kLeafWaves * t;
      if (J >= Q) break;
      acc_t mt;
#pragma unroll
      for (int r = 0; r < 4; ++r) mt[r] = (!kFlatLoads || d >= 2) ? mc[t][r] : R(0);
      if (J == Q - 1) {
#pragma unroll
        for (int s = 0; s < 4; ++s) mt = MF::mma(eu[s], lu[s], mt);
        if (keep) {
          R o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = mt[r];
          EVec<R>::store4(McP + (int64_t)J * T * T + lane * 4, o);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = MF::mma(mt[s], la[t][s], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) fm[wave][lane * 4 + r] = fresh[r];
  }
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave - 1][MF::row(lane, r)][c] = acc[r];
  }
  if (tid < T * T) lat[tid >> 4][tid & 15] = lat_v;
  __syncthreads();
  if (wave == 1 && d > 0 && keep) {
    // the fresh column M[P][Q] for the next leaf of the block, summed over
    // the waves in a fixed order
    R o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      R v = fm[0][lane * 4 + r];
#pragma unroll
      for (int w = 1; w < kLeafWaves; ++w) v += fm[w][lane * 4 + r];
      o[r] = v;
    }
    EVec<R>::store4(McP + (int64_t)Q * T * T + lane * 4, o);
  }
  if (wave > 0) return;

  // ---- 2. sweep on wave 0
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = MF::row(lane, r);
    R pro = w0[r];
#pragma unroll
    for (int w = 0; w < kLeafWaves - 1; ++w) pro += red[w][row][c];
    acc[r] += pro;
  }
  R laK[2 * T - 1];  // laK[j] = L^A[Q,Q][c][j - KA kg]
#pragma unroll
  for (int j = 0; j < 2 * T - 1; ++j) {
    const int jj = j - KA * kg;
    laK[j] = (jj >= 0 && jj < T) ? lat[c][jj] : R(0);
  }
  const R lo = lp.lo, hi = lp.hi;  // +-infinity for the unbounded alphabet

  // One wave's vector instructions do not overlap its own MFMA chain on
  // gfx950 (measured: each independent fma adds its ~6 cycles to a chain of
  // four dependent 16x16x4 MFMAs), so the step is kept to the fewest vector
  // instructions. Which lanes hold their entry r on step t is fixed by the
  // lane layout, so the select masks are compile-time wave masks (scalar
  // moves, no compares). A lane with no entry on the step keeps acc[0], any
  // finite value: the broadcasts read only lanes at columns t - k inside the
  // tile, which do have an entry, and the other broadcast values meet exact
  // zeros of laK. Padding entries may be selected: they start at exact zero,
  // and an error reaches an entry only through factors that are exact zeros
  // between padding and real rows or columns, so neither side changes the
  // other. The value at rounding goes to the lane row's own LDS copy at a
  // constant offset per step.
  R* owl = &owv[kg][T - 1 - c][c];
  static_for<0, 2 * T - 1>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    R x = acc[0];
    static_for<1, 4>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      constexpr uint64_t msk = entry_lanes<R>(t, r);
      if constexpr (msk != 0) x = __builtin_amdgcn_inverse_ballot_w64(msk) ? acc[r] : x;
    });
    owl[t * kOwLd] = x;
    if constexpr (t < 2 * T - 2) {
      const R es = row_skew(round_clamp(x, lo, hi) - x);
      static_for<0, 4>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        // MFMA s takes the rows k = KA kg + KB s: it contributes only if some
        // such k has its column t - k inside the tile (k >= t - (T - 1)) and
        // k <= t; the last step's update reaches no later anti-diagonal. The
        // skipped products add exact zeros or are never read.
        if constexpr (t - KB * s >= 0 && KA * 3 + KB * s >= t - (T - 1)) {
          const R ev = row_bcast<(t - KB * s) & 15>(es);
          acc = MF::mma(lbK[s] * ev, laK[t - KB * s], acc);
        }
      });
    }
  });
  wave_sync_lds();
  // write back: errors (code units) into the workspace, codes and the values
  // at rounding (back in the units of W) to the outputs
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = lane + 64 * u;
    const int p = idx >> 4, q = idx & 15;
    const int64_t gi = (int64_t)P * T + p, gjj = (int64_t)Q * T + q;
    const bool valid = gi < m && gjj < n;
    const R x = owv[std::is_same<R, float>::value ? p >> 2 : p & 3][p + T - 1][q];
    const R cq = quant_unit(x, lo, hi);
    tW[idx] = valid ? cq - x : R(0);
    if (valid) {
      lp.V[gi * lp.ldv + gjj] = (int32_t)cq;
      if (lp.Wt) {
        R sv = R(1);
        if (lp.scale_mode == 1) sv = lp.scales[gi];
        else if (lp.scale_mode == 2) sv = lp.scales[gjj];
        lp.Wt[gi * lp.ldwt + gjj] = lp.scale_mode ? sv * x : x;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host wrappers
// ---------------------------------------------------------------------------
template <typename R>
hipError_t launch_pack_w(const SolveGeom& g, const R* W, int64_t ldw, const R* scales,
                         int scale_mode, R* Wk, hipStream_t s) {
  const int64_t nt = (int64_t)g.Mt * g.Nt;
  if (nt == 0 || g.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL((pack_w_kernel<R, kTile>), dim3((unsigned)nt, (unsigned)g.batch), dim3(256),
                     0, s, g.m, g.n, g.Nt, W, ldw, scales, scale_mode, Wk, g.bs);
  return hipGetLastError();
}

template <typename R>
hipError_t launch_pack_l(const SolveGeom& g, bool lb, const R* L, int64_t ld, const R* scales,
                         R* Lp, hipStream_t s) {
  const int64_t dim = lb ? g.m : g.n;
  const int Dt = lb ? g.Mt : g.Nt;
  const int64_t nt = (int64_t)Dt * (Dt + 1) / 2;
  if (nt == 0 || g.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL((pack_l_kernel<R, kTile>), dim3((unsigned)nt, (unsigned)g.batch), dim3(256),
                     0, s, dim, L, ld, lb ? g.bs.lb : g.bs.la, scales, g.bs.s, Lp, g.bs.ws);
  return hipGetLastError();
}

static inline void diag_range(const SolveGeom& g, int K, int* lo, int* hi) {
  *lo = K - (g.Nt - 1) > 0 ? K - (g.Nt - 1) : 0;
  *hi = K < g.Mt - 1 ? K : g.Mt - 1;
}

template <typename R>
hipError_t launch_leaf(const SolveGeom& g, int K, int K0, R* Wk, const R* LBp, const R* LAp,
                       R* Mc, const LeafParams<R>& lp, hipStream_t s, hipEvent_t ev0,
                       hipEvent_t ev1) {
  static_assert(kTile == 16, "the leaf kernel works on 16 x 16 tiles");
  int lo, hi;
  diag_range(g, K, &lo, &hi);
  if (hi < lo || g.batch <= 0) {
    // nothing to do; keep the timing events valid (zero duration)
    if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return hipErrorUnknown;
    if (ev1 && hipEventRecord(ev1, s) != hipSuccess) return hipErrorUnknown;
    return hipSuccess;
  }
  const dim3 grid(hi - lo + 1, g.batch), block(64 * kLeafWaves);
  if (ev0 || ev1)  // the events are stamped by the dispatch packet itself
    hipExtLaunchKernelGGL((leaf_kernel<R>), grid, block, 0, s, ev0, ev1, 0, K, K0, g.Mt, g.Nt,
                          g.m, g.n, Wk, LBp, LAp, Mc, lp, g.bs);
  else
    hipLaunchKernelGGL((leaf_kernel<R>), grid, block, 0, s, K, K0, g.Mt, g.Nt, g.m, g.n, Wk, LBp,
                       LAp, Mc, lp, g.bs);
  return hipGetLastError();
}

#define BK_INST(R)                                                                              \
  template hipError_t launch_pack_w<R>(const SolveGeom&, const R*, int64_t, const R*, int, R*,  \
                                       hipStream_t);                                            \
  template hipError_t launch_pack_l<R>(const SolveGeom&, bool, const R*, int64_t, const R*, R*, \
                                       hipStream_t);                                            \
  template hipError_t launch_leaf<R>(const SolveGeom&, int, int, R*, const R*, const R*, R*,    \
                                     const LeafParams<R>&, hipStream_t, hipEvent_t, hipEvent_t);
BK_INST(float)
BK_INST(double)
#undef BK_INST

}  // namespace bk
