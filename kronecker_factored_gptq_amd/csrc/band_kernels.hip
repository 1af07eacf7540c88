// Band products of a large internal node, on MFMA (gfx950).
//
// An internal node over tile anti-diagonals [k, l), split at mid, applies the
// errors E recorded on [k, mid) to the tiles on [mid, l) as the two
// "restricted band products" of "BaKron: Efficient Quantization with
// Kronecker-Factored Hessians" (arXiv 2608.06291), Appendix C:
//   stage 1: M[P,J]  = sum_I L^B[P,I] E[I,J],   I <= P, k <= I+J < mid
//   stage 2: W[P,Q] += sum_J M[P,J] L^A[Q,J]^T, J <= Q, J < mid,
//            k <= P+J <= l-1, written only where mid <= P+Q <= l-1.
// (Subscripts are 16 x 16 solver tiles.)
//
// Each workgroup owns an MB x MB block of solver tiles (a BM = 16*MB square
// macro tile) and walks K two solver tiles (32 elements) at a time. Four
// waves in a 2 x 2 arrangement each hold a (BM/2)^2 accumulator of 16 x 16
// MFMA blocks. Solver tiles are contiguous in HBM, so a 16-byte load by
// every lane of a wave moves exactly one tile (float) or half a tile
// (double): tile masks are wave-uniform and every load is fully coalesced.
// Operands are double-buffered in LDS with k contiguous (one 128-bit read
// per lane per four MFMAs); stage 1's E tiles keep their natural row-major
// order (k = row) and are read one element per MFMA.
#include <hip/hip_ext.h>

#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace bk {

template <typename R> struct Vec16;
template <> struct Vec16<float> {
  typedef float4 T;
  static constexpr int N = 4;
  __device__ static inline T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ static inline float get(const T& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }
};
template <> struct Vec16<double> {
  typedef double2 T;
  static constexpr int N = 2;
  __device__ static inline T zero() { return make_double2(0.0, 0.0); }
  __device__ static inline double get(const T& v, int e) { return e == 0 ? v.x : v.y; }
};

template <typename R, int MB>
struct BandShape {
  static constexpr int T = kTile;
  static constexpr int BKT = 2;                  // K step in solver tiles
  static constexpr int BK = BKT * T;             // K step in elements
  static constexpr int BM = MB * T;              // macro tile edge
  static constexpr int WT = BM / 2;              // wave tile edge
  static constexpr int NBW = WT / 16;            // MFMA blocks per wave edge
  static constexpr int VN = Vec16<R>::N;         // elements per 16-byte vector
  static constexpr int LDK = BK + VN;            // k-contiguous rows, 16-byte aligned
  static constexpr int LDC = BM + VN;            // column-contiguous rows (stage-1 B)
  static constexpr int TV = T * T / VN;          // vectors per solver tile
  static constexpr int NV = MB * BKT * TV / 256; // vectors per thread per operand per K step
  static constexpr int KL = BK / 4;              // k values per lane per K step
  // global loads run PD K steps ahead (register ring): the small float tiles
  // do little MFMA work per step, so one step does not cover the latency
  static constexpr int PD = (sizeof(R) == 4 && MB <= 4) ? 2 : 1;
  static_assert(NV >= 1 && (MB * BKT * TV) % 256 == 0, "macro tile too small for 256 threads");
};

// Geometry of the output macro tile (row block pb, column block number bx of
// that row) of one stage: first column tile C0 and the K range [Klo, Khi] in
// solver tiles. Shared by the kernels and the host-side launch planning.
struct BandTile {
  int P0, C0, Klo, Khi;
};
// Column tiles [Clo, Chi] that row block pb of a stage writes; false if none.
__host__ __device__ inline bool band_cols(int stage, int k, int mid, int l, int Nt, int MB, int pb,
                                          int* Clo, int* Chi) {
  const int P0 = pb * MB;
  int lo, hi;
  if (stage == 1) {  // M[P, J] is needed where stage 2 reads it: J < mid, P + J <= l - 1
    lo = k - (P0 + MB - 1); if (lo < 0) lo = 0;
    hi = Nt - 1; if (mid - 1 < hi) hi = mid - 1; if (l - 1 - P0 < hi) hi = l - 1 - P0;
  } else {           // W[P, Q] on mid <= P + Q <= l - 1
    lo = mid - (P0 + MB - 1); if (lo < 0) lo = 0;
    hi = Nt - 1; if (l - 1 - P0 < hi) hi = l - 1 - P0;
  }
  *Clo = lo;
  *Chi = hi;
  return lo <= hi;
}
__host__ __device__ inline bool band_tile(int stage, int k, int mid, int l, int Mt, int Nt, int MB,
                                          int pb, int bx, BandTile* t) {
  const int P0 = pb * MB;
  int Clo, Chi;
  if (!band_cols(stage, k, mid, l, Nt, MB, pb, &Clo, &Chi)) return false;
  const int cb = Clo / MB + bx;
  if (cb > Chi / MB) return false;
  const int C0 = cb * MB;
  int Klo, Khi;
  if (stage == 1) {  // I <= P, k <= I + J < mid
    Klo = k - (C0 + MB - 1); if (Klo < 0) Klo = 0;
    Khi = P0 + MB - 1; if (mid - 1 - C0 < Khi) Khi = mid - 1 - C0; if (Mt - 1 < Khi) Khi = Mt - 1;
  } else {           // J <= Q, J < mid, k <= P + J <= l - 1
    Klo = k - (P0 + MB - 1); if (Klo < 0) Klo = 0;
    Khi = C0 + MB - 1; if (mid - 1 < Khi) Khi = mid - 1; if (Nt - 1 < Khi) Khi = Nt - 1;
    if (l - 1 - P0 < Khi) Khi = l - 1 - P0;
  }
  t->P0 = P0;
  t->C0 = C0;
  t->Klo = Klo;
  t->Khi = Khi;
  return Klo <= Khi;
}

template <typename R>
struct BandArgs {
  int k, mid, l, Mt, Nt;
  int maxw;  // column blocks per row block (workgroups per row block)
  R* Wk;
  const R* LBp;
  const R* LAp;
  R* Mb;
  int64_t sws;  // workspace stride between the problems of a batch (elements)
};

// One-dimensional grid (per problem of a batch: blockIdx.y) of nPb8 * maxw workgroups, nPb8 = row blocks rounded up
// to a multiple of the 8 XCDs. Workgroup w runs on XCD w % 8 (round-robin
// dispatch), and all workgroups of one row block go to the same XCD, so a row
// panel of the left operand is fetched into one L2 only. Within an XCD the
// row blocks are taken so that the macro tiles with the longest K ranges
// start first (stage 1: the last row blocks; stage 2: the last column blocks
// of a row).
constexpr int kXcds = 8;
template <typename R, int STAGE, int MB>
__global__ __launch_bounds__(256) void band_kernel(BandArgs<R> a) {
  typedef BandShape<R, MB> S;
  typedef Vec16<R> VV;
  typedef typename VV::T vec_t;
  typedef Mfma<R> MF;
  typedef typename MF::acc_t acc_t;
  constexpr int T = S::T;
  constexpr int B_ROWS = STAGE == 1 ? S::BK : S::BM;
  constexpr int B_LD = STAGE == 1 ? S::LDC : S::LDK;

  // one LDS block: the double-buffered operands, reused by the epilogue
  typedef R AsT[2][S::BM][S::LDK];
  typedef R BsT[2][B_ROWS][B_LD];
  constexpr size_t kOps = sizeof(AsT) + sizeof(BsT);
  constexpr size_t kOut = sizeof(R) * S::BM * S::BM;
  __shared__ __attribute__((aligned(16))) char smem[kOps > kOut ? kOps : kOut];
  AsT& As = *reinterpret_cast<AsT*>(smem);
  BsT& Bs = *reinterpret_cast<BsT*>(smem + sizeof(AsT));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int r16 = lane & 15, kg = lane >> 4;
  const int k = a.k, mid = a.mid, l = a.l, Mt = a.Mt, Nt = a.Nt;

  const int w = blockIdx.x;
  const int xcd = w % kXcds, idx = w / kXcds;
  const int rowj = idx / a.maxw;
  int bx = idx % a.maxw;
  const int nPb8 = (int)gridDim.x / a.maxw;
  const int pl = xcd + kXcds * rowj;  // row block in dispatch order
  const int pb = STAGE == 1 ? nPb8 - 1 - pl : pl;
  if (pb >= (Mt + MB - 1) / MB) return;
  if (STAGE == 2) {
    int Clo, Chi;
    if (!band_cols(STAGE, k, mid, l, Nt, MB, pb, &Clo, &Chi)) return;
    bx = Chi / MB - Clo / MB - bx;
    if (bx < 0) return;
  }
  BandTile bt;
  if (!band_tile(STAGE, k, mid, l, Mt, Nt, MB, pb, bx, &bt)) return;
  const int P0 = bt.P0, C0 = bt.C0;
  const int Klo = bt.Klo, Khi = bt.Khi;

  const int64_t bo = (int64_t)blockIdx.y * a.sws;
  R* __restrict__ Wk = a.Wk + bo;
  const R* __restrict__ LBp = a.LBp + bo;
  const R* __restrict__ LAp = a.LAp + bo;
  R* __restrict__ Mb = a.Mb + bo;

  acc_t acc[S::NBW][S::NBW];
#pragma unroll
  for (int i = 0; i < S::NBW; ++i)
#pragma unroll
    for (int j = 0; j < S::NBW; ++j) acc[i][j] = MF::zero();

  vec_t ra[S::PD][S::NV], rb[S::PD][S::NV];

  // global -> register set SET for the K step starting at solver tile kk0
  auto gload = [&](int kk0, auto SETC) {
    constexpr int set = decltype(SETC)::value;
#pragma unroll
    for (int u = 0; u < S::NV; ++u) {
      const int f = u * 256 + tid;
      const int ti = f / S::TV;               // tile index within the operand block
      const int at = ti / S::BKT, kt = ti % S::BKT;
      const int v = f % S::TV;
      const int vo = (v % T) * (T / S::VN) + v / T;  // 16-byte vector of row v % 16
      const int kk = kk0 + kt;
      const int P = P0 + at, C = C0 + at;
      vec_t va = VV::zero(), vb = VV::zero();
      if (STAGE == 1) {
        if (kk <= Khi && P < Mt && kk <= P)
          va = reinterpret_cast<const vec_t*>(LBp + tri_index(P, kk) * T * T)[vo];
        const int sd = kk + C;
        if (kk <= Khi && C < Nt && sd >= k && sd < mid)
          vb = reinterpret_cast<const vec_t*>(Wk + ((int64_t)kk * Nt + C) * T * T)[vo];
      } else {
        const int sd = P + kk;
        if (kk <= Khi && P < Mt && kk <= mid - 1 && sd >= k && sd <= l - 1)
          va = reinterpret_cast<const vec_t*>(Mb + ((int64_t)P * Nt + kk) * T * T)[vo];
        if (kk <= Khi && C < Nt && kk <= C)
          vb = reinterpret_cast<const vec_t*>(LAp + tri_index(C, kk) * T * T)[vo];
      }
      ra[set][u] = va;
      rb[set][u] = vb;
    }
  };
  // registers -> LDS buffer. Vector v of a tile holds row v % 16, columns
  // VN * (v / 16) ..: eight consecutive lanes then write eight different rows,
  // which the padded row strides place on eight different bank groups.
  auto sstore = [&](int buf, auto SETC) {
    constexpr int set = decltype(SETC)::value;
#pragma unroll
    for (int u = 0; u < S::NV; ++u) {
      const int f = u * 256 + tid;
      const int ti = f / S::TV;
      const int at = ti / S::BKT, kt = ti % S::BKT;
      const int v = f % S::TV;
      const int r = v % T, c = (v / T) * S::VN;
      *reinterpret_cast<vec_t*>(&As[buf][at * T + r][kt * T + c]) = ra[set][u];
      if (STAGE == 1)  // E[k = r][col = c]: keep rows of k
        *reinterpret_cast<vec_t*>(&Bs[buf][kt * T + r][at * T + c]) = rb[set][u];
      else             // L^A[col = r][k = c]: k contiguous per column
        *reinterpret_cast<vec_t*>(&Bs[buf][at * T + r][kt * T + c]) = rb[set][u];
    }
  };
  // MFMAs over one K step. Lane group kg takes k = (sc * 4 + kg) * VN + e:
  // the four groups of one sub-step sit VN apart, which keeps stage 1's
  // row-wise B reads of lane groups 0 and 1 (and 2 and 3) on disjoint banks.
  auto compute = [&](int buf) {
#pragma unroll
    for (int sc = 0; sc < S::KL / S::VN; ++sc) {
      const int k0 = (sc * 4 + kg) * S::VN;
      vec_t af[S::NBW], bf[S::NBW];
#pragma unroll
      for (int i = 0; i < S::NBW; ++i)
        af[i] = *reinterpret_cast<const vec_t*>(&As[buf][wr * S::WT + i * 16 + r16][k0]);
      R b1[S::NBW][S::VN];
#pragma unroll
      for (int j = 0; j < S::NBW; ++j) {
        if (STAGE == 1) {
#pragma unroll
          for (int e = 0; e < S::VN; ++e) b1[j][e] = Bs[buf][k0 + e][wc * S::WT + j * 16 + r16];
        } else {
          bf[j] = *reinterpret_cast<const vec_t*>(&Bs[buf][wc * S::WT + j * 16 + r16][k0]);
        }
      }
#pragma unroll
      for (int e = 0; e < S::VN; ++e)
#pragma unroll
        for (int i = 0; i < S::NBW; ++i)
#pragma unroll
          for (int j = 0; j < S::NBW; ++j) {
            const R bv = STAGE == 1 ? b1[j][e] : VV::get(bf[j], e);
            acc[i][j] = MF::mma(VV::get(af[i], e), bv, acc[i][j]);
          }
    }
  };

  {
    // register set it % PD holds K step it; LDS buffer it % 2 is computed
    typedef std::integral_constant<int, 0> I0;
    typedef std::integral_constant<int, (S::PD > 1 ? 1 : 0)> I1;
    typedef std::integral_constant<int, (S::PD > 2 ? 2 : 0)> I2;
    const int nsteps = (Khi - Klo) / S::BKT + 1;
    gload(Klo, I0());
    if (S::PD > 1 && 1 < nsteps) gload(Klo + S::BKT, I1());
    if (S::PD > 2 && 2 < nsteps) gload(Klo + 2 * S::BKT, I2());
    sstore(0, I0());
    __syncthreads();
    auto step = [&](auto PH, int it) {
      constexpr int ph = decltype(PH)::value;
      if (it + S::PD < nsteps) gload(Klo + (it + S::PD) * S::BKT, PH);
      compute(it & 1);
      if (it + 1 < nsteps) sstore((it + 1) & 1, std::integral_constant<int, (ph + 1) % S::PD>());
      __syncthreads();
    };
    for (int it0 = 0; it0 < nsteps; it0 += S::PD) {
      step(I0(), it0);
      if (S::PD > 1 && it0 + 1 < nsteps) step(I1(), it0 + 1);
      if (S::PD > 2 && it0 + 2 < nsteps) step(I2(), it0 + 2);
    }
  }

  // Epilogue through LDS: the macro tile is laid out as its MB x MB solver
  // tiles (each 16 x 16 contiguous, as in HBM), then every wave moves whole
  // tiles with one 16-byte access per lane.
  R* Cs = reinterpret_cast<R*>(smem);
#pragma unroll
  for (int i = 0; i < S::NBW; ++i)
#pragma unroll
    for (int j = 0; j < S::NBW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wr * S::WT + i * 16 + MF::row(lane, r);
        const int col = wc * S::WT + j * 16 + r16;
        Cs[((row / T) * MB + col / T) * T * T + (row % T) * T + (col % T)] = acc[i][j][r];
      }
  __syncthreads();
  R* out = STAGE == 1 ? Mb : Wk;
  constexpr int VPT = S::TV / 64;  // 16-byte vectors per lane per tile
  for (int t = wave; t < MB * MB; t += 4) {
    const int P = P0 + t / MB, C = C0 + t % MB;
    if (P >= Mt || C >= Nt) continue;
    if (STAGE == 2 && (P + C < mid || P + C > l - 1)) continue;
    vec_t* dst = reinterpret_cast<vec_t*>(out + ((int64_t)P * Nt + C) * T * T);
    const vec_t* src = reinterpret_cast<const vec_t*>(Cs + t * T * T);
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      const int v = q * 64 + lane;
      vec_t x = src[v];
      if (STAGE == 2) {
        const vec_t w = dst[v];
        x = x + w;
      }
      dst[v] = x;
    }
  }
}

// Macro-tile size by node width l - k (tile anti-diagonals): 2 x 2 solver
// tiles (32 x 32) below QMIN_BIG, 4 x 4 (64 x 64) from it on. Measured on
// the 4096 x 4096 float32 solve (leaf blocks of 12): 32 x 32 for every node
// but the top one (widths up to 259) gives 8.05 ms for the solve against
// 8.63 with 64 x 64 everywhere and 8.18 with 32 x 32 everywhere (more
// workgroups and less padding on the narrow bands); 128 x 128 tiles were
// slower still.
template <typename R> struct BandChoice;
template <> struct BandChoice<float> { static constexpr int BIG = 4, SMALL = 2, QMIN_BIG = 300; };
// Float64 (measured on the 4096 x 4096 solve in float64): 64 x 64 from width 100 gives
// 12.45 ms against 12.74 from width 32, 12.77 from 300 and 13.40 from 1000.
template <> struct BandChoice<double> { static constexpr int BIG = 4, SMALL = 2, QMIN_BIG = 100; };

template <typename R, int MB>
static hipError_t launch_band_mb(const SolveGeom& g, int k, int mid, int l, int stage,
                                 const BandBuffers<R>& bb, hipStream_t s, hipEvent_t ev0,
                                 hipEvent_t ev1) {
  const int nPb = (g.Mt + MB - 1) / MB;
  int maxw = 0;
  for (int pb = 0; pb < nPb; ++pb) {
    int Clo, Chi;
    if (!band_cols(stage, k, mid, l, g.Nt, MB, pb, &Clo, &Chi)) continue;
    const int w = Chi / MB - Clo / MB + 1;
    if (w > maxw) maxw = w;
  }
  if (maxw == 0) {
    // nothing to do; keep the timing events valid (zero duration)
    if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return hipErrorUnknown;
    if (ev1 && hipEventRecord(ev1, s) != hipSuccess) return hipErrorUnknown;
    return hipSuccess;
  }
  BandArgs<R> a;
  a.k = k; a.mid = mid; a.l = l; a.Mt = g.Mt; a.Nt = g.Nt;
  a.maxw = maxw;
  a.Wk = bb.Wk; a.LBp = bb.LBp; a.LAp = bb.LAp; a.Mb = bb.Mb;
  a.sws = g.bs.ws;
  const int nPb8 = (nPb + kXcds - 1) / kXcds * kXcds;
  // nPb8 * maxw is a multiple of the XCD count, so in the 2-D grid workgroup
  // (x, y) still lands on XCD x % 8
  const dim3 grid((unsigned)(nPb8 * maxw), (unsigned)(g.batch > 0 ? g.batch : 1)), block(256);
  if (ev0 || ev1) {
    // the events are stamped by the dispatch packet itself: exact kernel time
    if (stage == 1)
      hipExtLaunchKernelGGL((band_kernel<R, 1, MB>), grid, block, 0, s, ev0, ev1, 0, a);
    else
      hipExtLaunchKernelGGL((band_kernel<R, 2, MB>), grid, block, 0, s, ev0, ev1, 0, a);
  } else if (stage == 1) {
    hipLaunchKernelGGL((band_kernel<R, 1, MB>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((band_kernel<R, 2, MB>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <typename R>
hipError_t launch_node_band(const SolveGeom& g, int k, int mid, int l, int stage,
                            const BandBuffers<R>& bb, hipStream_t s, hipEvent_t ev0,
                            hipEvent_t ev1) {
  if (l - k >= BandChoice<R>::QMIN_BIG)
    return launch_band_mb<R, BandChoice<R>::BIG>(g, k, mid, l, stage, bb, s, ev0, ev1);
  return launch_band_mb<R, BandChoice<R>::SMALL>(g, k, mid, l, stage, bb, s, ev0, ev1);
}

template hipError_t launch_node_band<float>(const SolveGeom&, int, int, int, int,
                                            const BandBuffers<float>&, hipStream_t, hipEvent_t,
                                            hipEvent_t);
template hipError_t launch_node_band<double>(const SolveGeom&, int, int, int, int,
                                             const BandBuffers<double>&, hipStream_t, hipEvent_t,
                                             hipEvent_t);

}  // namespace bk
