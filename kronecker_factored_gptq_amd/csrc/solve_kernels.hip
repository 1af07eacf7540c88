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

// Sentinel of the leaf rows' error copy: a NaN bit pattern that no error
// takes (an error that is NaN is stored as the default quiet NaN).
template <typename R> struct Sentinel;
template <> struct Sentinel<float> {
  typedef uint32_t U;
  static constexpr U bits = 0xFFFFFFFFu;
  __device__ static inline float qnan() { return __builtin_nanf(""); }
};
template <> struct Sentinel<double> {
  typedef uint64_t U;
  static constexpr U bits = ~(uint64_t)0;
  __device__ static inline double qnan() { return __builtin_nan(""); }
};
template <typename R>
__device__ inline bool is_sentinel(R v) {
  return __builtin_bit_cast(typename Sentinel<R>::U, v) == Sentinel<R>::bits;
}
template <typename R>
__device__ inline R sentinel_value() {
  return __builtin_bit_cast(R, Sentinel<R>::bits);
}


// ---------------------------------------------------------------------------
// Pack kernels. A workgroup moves a strip of kPackTiles consecutive tiles of
// one tile row (16 rows x 64 columns): every row of the strip is one
// contiguous run of the source, read in 16-byte vectors when the source rows
// are 16-byte aligned, and each tile row of the destination is a contiguous
// 16-byte-aligned run too.
// ---------------------------------------------------------------------------
constexpr int kPackTiles = 4;
// 16-byte vector of R
template <typename R> struct PackVec;
template <> struct PackVec<float> {
  typedef float4 T;
  static constexpr int N = 4;
};
template <> struct PackVec<double> {
  typedef double2 T;
  static constexpr int N = 2;
};

// Pack U = W / s (row-major W, ldw) into tiles; padding is zero. mode: 0 no
// scales, 1 per-row, 2 per-column. Also sets the leaf blocks' error copy to
// the sentinel and their ticket counters and status word to zero. Grid:
// (Mt * ceil(Nt / kPackTiles), batch); vec: W and ldw allow 16-byte loads.
template <typename R, int T>
__global__ __launch_bounds__(256) void pack_w_kernel(int64_t m, int64_t n, int Nt,
                                                     const R* __restrict__ W, int64_t ldw,
                                                     const R* __restrict__ sc, int mode, int vec,
                                                     R* __restrict__ Wk, BatchStrides bs,
                                                     int* __restrict__ sync, int64_t sync_stride,
                                                     int sync_words, R* __restrict__ Eb) {
  typedef PackVec<R> V;
  typedef typename V::T vt;
  constexpr int VN = V::N, SW = kPackTiles * T, NV = T * SW / VN;
  const int64_t b = blockIdx.y;  // problem of a batch
  W += b * bs.w;
  if (sc) sc += b * bs.s;
  Wk += b * bs.ws;
  const int ns = (Nt + kPackTiles - 1) / kPackTiles;
  const int64_t P = blockIdx.x / ns;
  const int Q0 = (int)(blockIdx.x % ns) * kPackTiles;
  if (sync && blockIdx.x == 0) {
    sync += b * sync_stride;
    for (int i = threadIdx.x; i < sync_words; i += blockDim.x) sync[i] = 0;
  }
  for (int f = threadIdx.x; f < NV; f += blockDim.x) {
    const int r = f / (SW / VN), c = (f % (SW / VN)) * VN;  // strip row, first column
    const int Q = Q0 + c / T;
    if (Q >= Nt) continue;
    const int64_t i = P * T + r, j0 = (int64_t)Q0 * T + c;
    R v[VN];
    if (i < m && vec && j0 + VN <= n) {
      const vt x = *reinterpret_cast<const vt*>(W + i * ldw + j0);
      __builtin_memcpy(v, &x, sizeof x);
    } else {
#pragma unroll
      for (int e = 0; e < VN; ++e) v[e] = (i < m && j0 + e < n) ? W[i * ldw + j0 + e] : R(0);
    }
#pragma unroll
    for (int e = 0; e < VN; ++e) {
      if (i < m && j0 + e < n) {
        if (mode == 1) v[e] = v[e] / sc[i];
        else if (mode == 2) v[e] = v[e] / sc[j0 + e];
      }
    }
    const int64_t o = ((P * Nt + Q) * T + r) * T + c % T;
    vt y;
    __builtin_memcpy(&y, v, sizeof y);
    *reinterpret_cast<vt*>(Wk + o) = y;
    if (Eb) {
      // the leaf blocks' error copy starts as the sentinel
      R z[VN];
#pragma unroll
      for (int e = 0; e < VN; ++e) z[e] = sentinel_value<R>();
      __builtin_memcpy(&y, z, sizeof y);
      *reinterpret_cast<vt*>(Eb + b * bs.ws + o) = y;
    }
  }
}

// Pack the strict lower triangle of a normalised factor into lower tiles,
// scaled to code units when sc is given (entry (i, j) times s_j / s_i); the
// diagonal is 1, everything above it and on padding 0. Grid: (ceil(Dt /
// kPackTiles), min(Dt, 65535), batch): strip x of tile rows y, y + gridDim.y,
// ... (strips past a row's diagonal tile are skipped); vec: L and ld allow
// 16-byte loads.
template <typename R, int T>
__global__ __launch_bounds__(256) void pack_l_kernel(int64_t dim, int64_t Dt, const R* __restrict__ L,
                                                     int64_t ld, int64_t sL, int vec,
                                                     const R* __restrict__ sc, int64_t sS,
                                                     R* __restrict__ Lp, int64_t sLp) {
  typedef PackVec<R> V;
  typedef typename V::T vt;
  constexpr int VN = V::N, SW = kPackTiles * T, NV = T * SW / VN;
  const int64_t b = blockIdx.z;  // problem of a batch
  L += b * sL;
  if (sc) sc += b * sS;
  Lp += b * sLp;
  const int I0 = (int)blockIdx.x * kPackTiles;
  for (int64_t P = blockIdx.y; P < Dt; P += gridDim.y) {
  if (I0 > P) continue;
  for (int f = threadIdx.x; f < NV; f += blockDim.x) {
    const int r = f / (SW / VN), c = (f % (SW / VN)) * VN;
    const int I = I0 + c / T;
    if (I > P) continue;
    const int64_t i = P * T + r, j0 = (int64_t)I0 * T + c;
    R v[VN];
    if (i < dim && vec && j0 + VN <= i) {
      const vt x = *reinterpret_cast<const vt*>(L + i * ld + j0);
      __builtin_memcpy(v, &x, sizeof x);
    } else {
#pragma unroll
      for (int e = 0; e < VN; ++e) v[e] = (j0 + e < i && i < dim) ? L[i * ld + j0 + e] : R(0);
    }
#pragma unroll
    for (int e = 0; e < VN; ++e) {
      const int64_t j = j0 + e;
      if (i == j) v[e] = R(1);
      else if (j < i && i < dim) {
        if (sc) v[e] = v[e] * sc[j] / sc[i];
      } else {
        v[e] = R(0);
      }
    }
    const int64_t o = ((P * (P + 1) / 2 + I) * T + r) * T + c % T;
    vt y;
    __builtin_memcpy(&y, v, sizeof y);
    *reinterpret_cast<vt*>(Lp + o) = y;
  }
  }
}

// ---------------------------------------------------------------------------
// Leaf block [K0, K1) of G = kLeafBlock tile anti-diagonals, in one launch:
// one workgroup per tile row P of the block, walking its tiles (P, Q) from
// left to right, one per tile anti-diagonal K = P + Q; T = 16.
//
// 1. Prologue: add the errors of the tiles (I, J) of the same block on
//    earlier tile anti-diagonals, I <= P, J <= Q, as
//    sum_J (sum_I L^B[P,I] E[I,J]) L^A[Q,J]^T — the updates between tile
//    anti-diagonals of one block are done here, left-looking, instead of by
//    internal nodes (any grouping of the updates gives the same codes,
//    Appendix B). The inner sums M[P][J] of the row are carried from tile to
//    tile in registers: per tile, column Q - 1 gains its I = P term and
//    column Q is new (its terms I < P come from the rows above). The inner
//    sum is computed transposed, M^T = E^T L^B^T, because the MFMA result
//    layout of M^T is exactly the A-operand layout of the outer product with
//    k = its row index: no data movement between the two products.
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

// Waves of a leaf workgroup: wave 0 sweeps, the others prepare the prologue.
constexpr int kLeafWaves = 4;

// Errors handed from one row workgroup to the rows below inside a launch.
// The L2s of the eight XCDs are not coherent with each other, and an
// agent-scope release / acquire writes back / invalidates the whole L2 at
// every hand-off (measured: 18-21 us per tile anti-diagonal). So they move as
// relaxed device-scope accesses instead: loads that bypass the XCD's L2 and
// write-through stores.
template <typename R>
__device__ inline R ld_dev(const R* p) {
  return __hip_atomic_load(const_cast<R*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename R>
__device__ inline void st_dev(R* p, R v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// The leaf block kernel. The row's carried sums M[P][J] stay in registers,
// its own previous tile's errors in LDS; the only data from other
// workgroups are the
// errors E[I][Q] (I < P) of the rows above in the tile's column, read from a
// copy Eb that starts filled with a sentinel NaN pattern no error takes: a
// reader polls the values themselves until none is the sentinel (no flags,
// and no writer waits for its stores to complete). Wave 0 sweeps tile k while
// waves 1-3 prepare tile k + 1: the products over the row's finished columns,
// and the new column's terms from the rows above (which finish their tile on
// the same tile anti-diagonal at about the same time); after the sweep only
// the finished tile's own column remains (its I = P term and its product).
// Rows only wait for rows above them, which take their tickets first, so
// every wait is for a running workgroup.
// ---------------------------------------------------------------------------
// worker waves of a row workgroup, and columns / new-column terms per worker
constexpr int kRowWorkers = kLeafWaves - 1;
constexpr int kRowCols = (kLeafBlock + kRowWorkers - 1) / kRowWorkers;
constexpr int kRowTerms = (kLeafBlock - 1 + kRowWorkers - 1) / kRowWorkers;

template <typename R>
struct RowLds {
  static constexpr int T = 16;
  static constexpr int kOwRows = 3 * T - 2, kOwLd = T + 1 + (int)(sizeof(float) / sizeof(R));
  // by tile parity: the workers' prologue sums, the new column's shares,
  // L^A[Q,Q] of the tile, and a finished column's M[P][Q] for its owner
  R red[2][kRowWorkers][T][T + 1];
  __attribute__((aligned(16))) R fm[2][kRowWorkers][T * T];
  // rows of L^A[Q,Q] stored at kLatPad .. kLatPad + T - 1 of a zero row, so
  // that the sweep's lane-shifted window (columns j - KA kg, j = 0 .. 2T - 2)
  // is one contiguous, unmasked read per lane (16-byte aligned for float)
  static constexpr int kVn = 16 / (int)sizeof(R);
  static constexpr int kLatPad = 3 * SweepK<R>::KA;
  static constexpr int kLatLd = (kLatPad + 2 * T - 1 + kVn - 1) / kVn * kVn;
  __attribute__((aligned(16))) R lat[2][T][kLatLd];
  __attribute__((aligned(16))) R ms[2][T * T];
  R owv[4][kOwRows][kOwLd];
  int ticket;
};

template <typename R>
__global__ __launch_bounds__(64 * kLeafWaves) void leaf_rows_kernel(
    int K0, int K1, int blk, int nblocks, int Mt, int Nt, int64_t m, int64_t n,
    R* __restrict__ Wk, R* __restrict__ Eb, const R* __restrict__ LBp, const R* __restrict__ LAp,
    LeafParams<R> lp, BatchStrides bs, int* __restrict__ sync, int64_t sync_stride, int polls) {
  constexpr int T = 16;
  typedef Mfma<R> MF;
  typedef typename MF::acc_t acc_t;
  typedef RowLds<R> LT;
  constexpr int kOwLd = LT::kOwLd;
  constexpr int KA = SweepK<R>::KA, KB = SweepK<R>::KB;
  {  // problem blockIdx.y of a batch: its workspace and outputs
    const int64_t b = blockIdx.y;
    Wk += b * bs.ws;
    Eb += b * bs.ws;
    LBp += b * bs.ws;
    LAp += b * bs.ws;
    lp.V += b * bs.v;
    if (lp.Wt) lp.Wt += b * bs.wt;
    if (lp.scales) lp.scales += b * bs.s;
    sync += b * sync_stride;
  }
  __shared__ LT L;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, kg = lane >> 4;
  // the zero padding of the L^A[Q,Q] rows (the rows themselves are written
  // per tile)
  for (int e = tid; e < 2 * T * LT::kLatLd; e += 64 * kLeafWaves) (&L.lat[0][0][0])[e] = R(0);
  if (tid == 0)
    L.ticket = __hip_atomic_fetch_add(sync + blk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int Plo = K0 - (Nt - 1) > 0 ? K0 - (Nt - 1) : 0;
  const int P = Plo + L.ticket;
  // the row's tiles in the block: Q = Qa .. Qb (tile anti-diagonals P + Q)
  const int Qa = K0 - P > 0 ? K0 - P : 0;
  const int Qb = K1 - 1 - P < Nt - 1 ? K1 - 1 - P : Nt - 1;
  const int nt = Qb - Qa + 1;
  const int Jlo = Qa;
  const R lo = lp.lo, hi = lp.hi;  // +-infinity for the unbounded alphabet
  int* status = sync + nblocks;

  if (wave == 0) {
    // ---- sweeper: tile k - 1 in iteration k, then the finished column's
    // I = P term and its product for the next tile
    R lbK[4], lu[4], w0[4];
    {
      const R* lb = LBp + tri_index(P, P) * T * T + c * T + KA * kg;
#pragma unroll
      for (int r = 0; r < 4; ++r) lbK[r] = lb[KB * r];
      EVec<R>::load4(LBp + tri_index(P, P) * T * T + c * T + 4 * kg, lu);
      const R* tW = Wk + ((int64_t)P * Nt + Qa) * T * T;
#pragma unroll
      for (int r = 0; r < 4; ++r) w0[r] = tW[MF::row(lane, r) * T + c];
    }
    // the scales the pre-rounding outputs need: this row's four rows (row
    // scales, the same for every tile of the row), or the tile's column
    // (column scales, loaded for the next tile after each write-back)
    R srow[4], scol = R(1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t gi = (int64_t)P * T + 4 * kg + s;
      srow[s] = (lp.Wt && lp.scale_mode == 1 && gi < m) ? lp.scales[gi] : R(1);
    }
    if (lp.Wt && lp.scale_mode == 2) {
      const int64_t gj = (int64_t)Qa * T + c;
      scol = gj < n ? lp.scales[gj] : R(1);
    }
    acc_t contrib = MF::zero();  // M[P][Q-1] L^A[Q,Q-1]^T for the tile about to be swept
    for (int k = 1; k <= nt; ++k) {
      __syncthreads();  // the tile's prologue sums and L^A[Q,Q] are in LDS
      const int Q = Qa + k - 1;
      const int pb = (k - 1) & 1;
      acc_t acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = MF::row(lane, r);
        R pro = w0[r];
#pragma unroll
        for (int w = 0; w < kRowWorkers; ++w) pro += L.red[pb][w][row][c];
        acc[r] = pro + contrib[r];
      }
      R laK[2 * T - 1];  // laK[j] = L^A[Q,Q][c][j - KA kg] (zero outside the tile)
      {
        const R* lr = &L.lat[pb][c][LT::kLatPad - KA * kg];
        if constexpr (sizeof(R) == 4) {
#pragma unroll
          for (int i = 0; i < (2 * T - 1 + 3) / 4; ++i) {
            const float4 v = reinterpret_cast<const float4*>(lr)[i];
            const R vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * i + e < 2 * T - 1) laK[4 * i + e] = vv[e];
          }
        } else {
#pragma unroll
          for (int j = 0; j < 2 * T - 1; ++j) laK[j] = lr[j];
        }
      }
      // the next tile's W and L^A[Q+1,Q], requested before the sweep
      R la1[4];
      if (k < nt) {
        const R* tW = Wk + ((int64_t)P * Nt + Q + 1) * T * T;
#pragma unroll
        for (int r = 0; r < 4; ++r) w0[r] = tW[MF::row(lane, r) * T + c];
        const R* La = LAp + tri_index(Q + 1, Q) * T * T;
#pragma unroll
        for (int s = 0; s < 4; ++s) la1[s] = La[c * T + MF::row(lane, s)];
      }
      // the sweep
      R* owl = &L.owv[kg][T - 1 - c][c];
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
            if constexpr (t - KB * s >= 0 && KA * 3 + KB * s >= t - (T - 1)) {
              const R ev = row_bcast<(t - KB * s) & 15>(es);
              acc = MF::mma(lbK[s] * ev, laK[t - KB * s], acc);
            }
          });
        }
      });
      wave_sync_lds();
      // write back, each lane the tile rows 4 kg + s of column c (the
      // operand layout of the finished column's I = P term). In the order
      // the next steps need them: the four values read together, the errors
      // into the copy the rows below poll, the finished column's sum and its
      // product for the next tile (the next sweep waits for these), and only
      // then the workspace and the outputs
      R* tW = Wk + ((int64_t)P * Nt + Q) * T * T;
      R* tE = Eb + ((int64_t)P * Nt + Q) * T * T;
      R xv[4], cqv[4], ev[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) xv[s] = L.owv[std::is_same<R, float>::value ? kg : s][4 * kg + s + T - 1][c];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int p = 4 * kg + s;
        const bool valid = (int64_t)P * T + p < m && (int64_t)Q * T + c < n;
        cqv[s] = quant_unit(xv[s], lo, hi);
        ev[s] = valid ? cqv[s] - xv[s] : R(0);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
        st_dev(tE + (4 * kg + s) * T + c, ev[s] != ev[s] ? Sentinel<R>::qnan() : ev[s]);
      if (k < nt) {
        // column Q is finished: M[P][Q] = its new-column sum (the workers'
        // shares, in a fixed order) plus L^B[P,P] E[P][Q], kept by the
        // column's owner for the row's later tiles, and its product with
        // L^A[Q+1,Q] for the next tile
        acc_t mt;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          R v = L.fm[pb][0][lane * 4 + r];
#pragma unroll
          for (int w = 1; w < kRowWorkers; ++w) v += L.fm[pb][w][lane * 4 + r];
          mt[r] = v;
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) mt = MF::mma(ev[s], lu[s], mt);
#pragma unroll
        for (int r = 0; r < 4; ++r) L.ms[pb][lane * 4 + r] = mt[r];
        contrib = MF::zero();
#pragma unroll
        for (int s = 0; s < 4; ++s) contrib = MF::mma(mt[s], la1[s], contrib);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int p = 4 * kg + s;
        const int64_t gi = (int64_t)P * T + p, gjj = (int64_t)Q * T + c;
        tW[p * T + c] = ev[s];
        if (gi < m && gjj < n) {
          lp.V[gi * lp.ldv + gjj] = (int32_t)cqv[s];
          if (lp.Wt) {
            const R sv = lp.scale_mode == 1 ? srow[s] : scol;
            lp.Wt[gi * lp.ldwt + gjj] = lp.scale_mode ? sv * xv[s] : xv[s];
          }
        }
      }
      if (lp.Wt && lp.scale_mode == 2 && k < nt) {
        const int64_t gj1 = (int64_t)(Q + 1) * T + c;
        scol = gj1 < n ? lp.scales[gj1] : R(1);
      }
    }
    return;
  }

  // ---- workers: wave 1 + wid owns columns J = Jlo + wid + kRowWorkers t and
  // the new column's terms I = Ilo + wid + kRowWorkers u; in iteration k they
  // prepare tile k while wave 0 sweeps tile k - 1
  const int wid = wave - 1;
  acc_t mreg[kRowCols];  // M[P][J] (MFMA result layout of M^T), owned columns
#pragma unroll
  for (int t = 0; t < kRowCols; ++t) mreg[t] = MF::zero();
  for (int k = 0; k < nt; ++k) {
    const int Q = Qa + k;
    // column Q - 2, finished by wave 0 one iteration ago, to its owner
    if (k >= 2 && (Q - 2 - Jlo) % kRowWorkers == wid) {
      const int t = (Q - 2 - Jlo) / kRowWorkers;
      acc_t mt;
#pragma unroll
      for (int r = 0; r < 4; ++r) mt[r] = L.ms[k & 1][lane * 4 + r];
#pragma unroll
      for (int u = 0; u < kRowCols; ++u)
        if (u == t) mreg[u] = mt;
    }
    acc_t acc = MF::zero();
    acc_t fresh = MF::zero();
    R latv[4], la[kRowCols][4], laq[4], lf[kRowTerms][4], ef[kRowTerms][4];
    {
      const R* Lq = LAp + tri_index(Q, Q) * T * T;
#pragma unroll
      for (int u = 0; u < 4; ++u) latv[u] = Lq[lane + 64 * u];
#pragma unroll
      for (int s = 0; s < 4; ++s) laq[s] = Lq[c * T + MF::row(lane, s)];
    }
#pragma unroll
    for (int t = 0; t < kRowCols; ++t) {
      const int J = Jlo + wid + kRowWorkers * t;
      const int Jc = J <= Q - 2 ? J : Q;
      const R* La = LAp + tri_index(Q, Jc) * T * T;
#pragma unroll
      for (int s = 0; s < 4; ++s) la[t][s] = La[c * T + MF::row(lane, s)];
    }
    const int Ilo = K0 - Q > 0 ? K0 - Q : 0;
#pragma unroll
    for (int u = 0; u < kRowTerms; ++u) {
      const int I = Ilo + wid + kRowWorkers * u;
      if (I <= P - 1) {
        EVec<R>::load4(LBp + tri_index(P, I) * T * T + c * T + 4 * kg, lf[u]);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) lf[u][s] = R(0);
      }
    }
    // the products over the row's finished columns J <= Q - 2 (local data)
#pragma unroll
    for (int t = 0; t < kRowCols; ++t) {
      const int J = Jlo + wid + kRowWorkers * t;
      if (J > Q - 2) break;
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = MF::mma(mreg[t][s], la[t][s], acc);
    }
    // then the new column's terms from the rows above, the values polled
    // until none is the sentinel: rows I <= P - 2 (finished a tile
    // anti-diagonal earlier, as a rule already written) together, then
    // the row right above (I = P - 1, which sweeps its tile on the same
    // tile anti-diagonal as this row's current one), whose term is this
    // wave's last in the order of I
    bool ok = true;
    {
      bool done = false;
      for (int it = 0; it <= polls && !done; ++it) {
        bool mine = true;
#pragma unroll
        for (int u = 0; u < kRowTerms; ++u) {
          const int I = Ilo + wid + kRowWorkers * u;
          const R* E = Eb + ((int64_t)I * Nt + Q) * T * T;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            ef[u][s] = I <= P - 2 ? ld_dev(E + (4 * kg + s) * T + c) : R(0);
            mine = mine && !is_sentinel(ef[u][s]);
          }
        }
        done = __builtin_amdgcn_ballot_w64(!mine) == 0;
        if (!done && it < polls) __builtin_amdgcn_s_sleep(1);
      }
      ok = done;
    }
#pragma unroll
    for (int u = 0; u < kRowTerms; ++u) {
      if (Ilo + wid + kRowWorkers * u > P - 2) break;
#pragma unroll
      for (int s = 0; s < 4; ++s) fresh = MF::mma(ef[u][s], lf[u][s], fresh);
    }
    if (P - 1 >= Ilo && (P - 1 - Ilo) % kRowWorkers == wid) {
      const int uc = (P - 1 - Ilo) / kRowWorkers;
      const R* E = Eb + ((int64_t)(P - 1) * Nt + Q) * T * T + (4 * kg) * T + c;
      R e4[4];
      bool done = false;
      for (int it = 0; it <= polls && !done; ++it) {
        bool mine = true;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          e4[s] = ld_dev(E + s * T);
          mine = mine && !is_sentinel(e4[s]);
        }
        done = __builtin_amdgcn_ballot_w64(!mine) == 0;
        if (!done && it < polls) __builtin_amdgcn_s_sleep(1);
      }
#pragma unroll
      for (int u = 0; u < kRowTerms; ++u)
        if (u == uc) {
#pragma unroll
          for (int s = 0; s < 4; ++s) fresh = MF::mma(e4[s], lf[u][s], fresh);
        }
      ok = ok && done;
    }
    if (!ok && lane == 0)
      __hip_atomic_fetch_or(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = MF::mma(fresh[s], laq[s], acc);
    const int pb = k & 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      L.fm[pb][wid][lane * 4 + r] = fresh[r];
      L.red[pb][wid][MF::row(lane, r)][c] = acc[r];
    }
    if (wid == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = lane + 64 * u;
        L.lat[pb][idx >> 4][LT::kLatPad + (idx & 15)] = latv[u];
      }
    }
    __syncthreads();  // tile k's prologue sums and L^A[Q,Q] are in LDS
  }
}

// ---------------------------------------------------------------------------
// Host wrappers
// ---------------------------------------------------------------------------
template <typename R>
hipError_t launch_pack_w(const SolveGeom& g, const R* W, int64_t ldw, const R* scales,
                         int scale_mode, R* Wk, hipStream_t s, const LeafSync& ls) {
  const int64_t nt = (int64_t)g.Mt * ((g.Nt + kPackTiles - 1) / kPackTiles);
  if (nt == 0 || g.batch <= 0) return hipSuccess;
  // 16-byte loads need every row start of every problem 16-byte aligned
  constexpr int VN = 16 / sizeof(R);
  const int vec = reinterpret_cast<uintptr_t>(W) % 16 == 0 && ldw % VN == 0 &&
                  (g.batch == 1 || g.bs.w % VN == 0);
  hipLaunchKernelGGL((pack_w_kernel<R, kTile>), dim3((unsigned)nt, (unsigned)g.batch), dim3(256),
                     0, s, g.m, g.n, g.Nt, W, ldw, scales, scale_mode, vec, Wk, g.bs, ls.sync,
                     ls.stride, ls.nblocks + 1, static_cast<R*>(ls.eb));
  return hipGetLastError();
}

template <typename R>
hipError_t launch_pack_l(const SolveGeom& g, bool lb, const R* L, int64_t ld, const R* scales,
                         R* Lp, hipStream_t s) {
  const int64_t dim = lb ? g.m : g.n;
  const int Dt = lb ? g.Mt : g.Nt;
  if (Dt == 0 || g.batch <= 0) return hipSuccess;
  constexpr int VN = 16 / sizeof(R);
  const int64_t sL = lb ? g.bs.lb : g.bs.la;
  const int vec = reinterpret_cast<uintptr_t>(L) % 16 == 0 && ld % VN == 0 &&
                  (g.batch == 1 || sL % VN == 0);
  const dim3 grid((unsigned)((Dt + kPackTiles - 1) / kPackTiles),
                  (unsigned)(Dt < 65535 ? Dt : 65535), (unsigned)g.batch);
  hipLaunchKernelGGL((pack_l_kernel<R, kTile>), grid, dim3(256), 0, s, dim, (int64_t)Dt, L, ld,
                     sL, vec, scales, g.bs.s, Lp, g.bs.ws);
  return hipGetLastError();
}

template <typename R>
hipError_t launch_leaf_rows(const SolveGeom& g, int K0, int K1, int blk, R* Wk, const R* LBp,
                            const R* LAp, const LeafParams<R>& lp, const LeafSync& ls,
                            hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  static_assert(kTile == 16, "the leaf kernel works on 16 x 16 tiles");
  const int Plo = K0 - (g.Nt - 1) > 0 ? K0 - (g.Nt - 1) : 0;
  const int Phi = K1 - 1 < g.Mt - 1 ? K1 - 1 : g.Mt - 1;
  if (Phi < Plo || K1 <= K0 || g.batch <= 0) {
    if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return hipErrorUnknown;
    if (ev1 && hipEventRecord(ev1, s) != hipSuccess) return hipErrorUnknown;
    return hipSuccess;
  }
  if (!ls.sync || !ls.eb || blk < 0 || blk >= ls.nblocks || K1 - K0 > kLeafBlock)
    return hipErrorInvalidValue;
  int* counters = ls.sync;
  R* Eb = static_cast<R*>(ls.eb);
  const dim3 grid((unsigned)(Phi - Plo + 1), g.batch), block(64 * kLeafWaves);
  if (ev0 || ev1)
    hipExtLaunchKernelGGL((leaf_rows_kernel<R>), grid, block, 0, s, ev0, ev1, 0, K0, K1, blk,
                          ls.nblocks, g.Mt, g.Nt, g.m, g.n, Wk, Eb, LBp, LAp, lp, g.bs, counters,
                          ls.stride, ls.polls);
  else
    hipLaunchKernelGGL((leaf_rows_kernel<R>), grid, block, 0, s, K0, K1, blk, ls.nblocks, g.Mt,
                       g.Nt, g.m, g.n, Wk, Eb, LBp, LAp, lp, g.bs, counters, ls.stride,
                       ls.polls);
  return hipGetLastError();
}

#define BK_INST(R)                                                                              \
  template hipError_t launch_pack_w<R>(const SolveGeom&, const R*, int64_t, const R*, int, R*,  \
                                       hipStream_t, const LeafSync&);                           \
  template hipError_t launch_pack_l<R>(const SolveGeom&, bool, const R*, int64_t, const R*, R*, \
                                       hipStream_t);                                            \
  template hipError_t launch_leaf_rows<R>(const SolveGeom&, int, int, int, R*, const R*,         \
                                          const R*, const LeafParams<R>&, const LeafSync&,       \
                                          hipStream_t, hipEvent_t, hipEvent_t);
BK_INST(float)
BK_INST(double)
#undef BK_INST

}  // namespace bk
