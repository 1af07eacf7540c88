// Float64 MFMA GEMM for the factorisation and the loss (gfx950).
//
// C = alpha * A * op(B) + beta * C with v_mfma_f64_16x16x4 blocks; K advances
// 16 at a time through double-buffered LDS. Two kernels: 64 x 64 output
// blocks on four waves (2 x 2), and 128 x 128 blocks on eight waves (2 x 4,
// twice the MFMA work per loaded byte) for the products that still give at
// least 256 such blocks. Options: only lower output blocks (symmetric rank-k
// update), A lower triangular (K ends with the row block), B lower
// triangular (K ends with the column block when op(B) = B^T, starts with it
// when op(B) = B), a batch of independent problems of one shape (grid z), and a dot epilogue that reduces sum(C_block .* D_block) per block
// instead of storing C (loss). With a triangular operand the blocks with the
// longest K ranges are dispatched first.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace bk {

namespace {
constexpr int GTRI = 64;  // granularity of the triangular options
constexpr int GK = 16;    // K step
constexpr int GLD = GK + 2;
}  // namespace

// Output block and problem of this workgroup. With a triangular operand the
// K range of a block grows with its row (A lower) or column (B lower, op(B)
// = B^T) or shrinks with its column (B lower, op(B) = B): the linear
// workgroup number is mapped so that blocks are dispatched longest K range
// first across both problems of a batch, which keeps the greedy placement
// of blocks on compute units balanced.
struct BlockMap {
  int64_t bm, bn;
  int z;
};
// block of linear workgroup number lin in a grid of X column blocks, Y row
// blocks and Z problems
__device__ inline BlockMap map_block_lin(const Gemm64Args& a, int64_t lin, int64_t X, int64_t Y,
                                         int64_t Z) {
  BlockMap m;
  if (a.a_lower) {
    const int64_t q = lin / (X * Z), r = lin % (X * Z);
    m.bm = Y - 1 - q;
    m.bn = r % X;
    m.z = (int)(r / X);
  } else if (a.b_lower) {
    const int64_t q = lin / (Y * Z), r = lin % (Y * Z);
    m.bn = a.transB ? X - 1 - q : q;
    m.bm = r % Y;
    m.z = (int)(r / Y);
  } else {
    m.bn = lin % X;
    m.bm = (lin / X) % Y;
    m.z = (int)(lin / (X * Y));
  }
  return m;
}
template <bool TRI>
__device__ inline BlockMap map_block(const Gemm64Args& a) {
  if constexpr (!TRI) return BlockMap{(int64_t)blockIdx.y, (int64_t)blockIdx.x, (int)blockIdx.z};
  const int64_t X = gridDim.x, Y = gridDim.y, Z = gridDim.z;
  return map_block_lin(a, blockIdx.x + X * (blockIdx.y + Y * (int64_t)blockIdx.z), X, Y, Z);
}

// One output block (bmap) of one problem; nbx = column blocks of the grid
// (indexes the dot epilogue's per-block partials).
template <int GB, bool VEC, bool TRI>
__device__ __forceinline__ void gemm64_block(const Gemm64Args& a, const BlockMap bmap,
                                             int64_t nbx) {
  typedef Mfma<double> MF;
  typedef MF::acc_t acc_t;
  constexpr int WT = GB / 2, NBW = WT / 16;
  constexpr int PER = GB * GK / 256;  // elements per thread per operand per K step
  __shared__ double As[2][GB][GLD];
  __shared__ double Bs[2][GB][GLD];
  __shared__ double red[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int r16 = lane & 15, kg = lane >> 4;
  const int64_t bm = bmap.bm, bn = bmap.bn;
  const int z = bmap.z;
  const double* __restrict__ Ap = a.A + z * a.sA;
  const double* __restrict__ Bp = a.B + z * a.sB;
  double* Cp = a.C + z * a.sC;
  const int64_t row0 = bm * GB, col0 = bn * GB;
  // lower_out is decided on the 64-granular triangle: a block is computed if
  // any of its 64 x 64 sub-blocks is on or below the diagonal
  const bool skip = a.lower_out && col0 / GTRI > (row0 + GB - 1) / GTRI;

  acc_t acc[NBW][NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = MF::zero();

  int64_t kend = a.K, kbeg = 0;
  if (a.a_lower && row0 + GB < kend) kend = row0 + GB;
  if (a.b_lower) {
    if (a.transB) {
      if (col0 + GB < kend) kend = col0 + GB;
    } else {
      kbeg = col0;
    }
  }

  // global loads run PD K steps ahead in a register ring: the small
  // products of the factor's lower levels have few K steps, each too short to
  // cover a load's latency
  constexpr int PD = 4;
  double ra[PD][PER], rb[PD][PER];
  auto kin = [&](int64_t gk) { return gk < kend && gk >= kbeg; };
  // exact 64-granular triangular structure of A (row gr) and B (column gn)
  auto ain = [&](int64_t gr, int64_t gk) {
    return gr < a.M && kin(gk) && (!TRI || !a.a_lower || gk < (gr / GTRI + 1) * GTRI);
  };
  auto bin = [&](int64_t gn, int64_t gk) {
    if (gn >= a.N || !kin(gk)) return false;
    if (!TRI || !a.b_lower) return true;
    return a.transB ? gk < (gn / GTRI + 1) * GTRI : gk >= (gn / GTRI) * GTRI;
  };
  auto gload = [&](int64_t k0, auto SETC) {
    constexpr int set = decltype(SETC)::value;
    if (VEC) {
#pragma unroll
      for (int u = 0; u < PER / 2; ++u) {
        const int e = 2 * (u * 256 + tid);
        {
          const int r = e / GK, c = e % GK;
          const int64_t gr = row0 + r, gk = k0 + c;
          double2 v = make_double2(0.0, 0.0);
          const bool i0 = ain(gr, gk), i1 = ain(gr, gk + 1);
          if (i0 && i1) v = *reinterpret_cast<const double2*>(Ap + gr * a.lda + gk);
          else {
            if (i0) v.x = Ap[gr * a.lda + gk];
            if (i1) v.y = Ap[gr * a.lda + gk + 1];
          }
          ra[set][2 * u] = v.x; ra[set][2 * u + 1] = v.y;
        }
        if (a.transB) {
          const int r = e / GK, c = e % GK;
          const int64_t gn = col0 + r, gk = k0 + c;
          double2 v = make_double2(0.0, 0.0);
          const bool i0 = bin(gn, gk), i1 = bin(gn, gk + 1);
          if (i0 && i1) v = *reinterpret_cast<const double2*>(Bp + gn * a.ldb + gk);
          else {
            if (i0) v.x = Bp[gn * a.ldb + gk];
            if (i1) v.y = Bp[gn * a.ldb + gk + 1];
          }
          rb[set][2 * u] = v.x; rb[set][2 * u + 1] = v.y;
        } else {
          const int kr = e / GB, cc = e % GB;
          const int64_t gk = k0 + kr, gn = col0 + cc;
          double2 v = make_double2(0.0, 0.0);
          const bool i0 = bin(gn, gk), i1 = bin(gn + 1, gk);
          if (i0 && i1) v = *reinterpret_cast<const double2*>(Bp + gk * a.ldb + gn);
          else {
            if (i0) v.x = Bp[gk * a.ldb + gn];
            if (i1) v.y = Bp[gk * a.ldb + gn + 1];
          }
          rb[set][2 * u] = v.x; rb[set][2 * u + 1] = v.y;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = u * 256 + tid;
        {
          const int r = e / GK, c = e % GK;
          const int64_t gr = row0 + r, gk = k0 + c;
          ra[set][u] = ain(gr, gk) ? Ap[gr * a.lda + gk] : 0.0;
        }
        if (a.transB) {
          const int r = e / GK, c = e % GK;
          const int64_t gn = col0 + r, gk = k0 + c;
          rb[set][u] = bin(gn, gk) ? Bp[gn * a.ldb + gk] : 0.0;
        } else {
          const int kr = e / GB, cc = e % GB;
          const int64_t gk = k0 + kr, gn = col0 + cc;
          rb[set][u] = bin(gn, gk) ? Bp[gk * a.ldb + gn] : 0.0;
        }
      }
    }
  };
  auto sstore = [&](int buf, auto SETC) {
    constexpr int set = decltype(SETC)::value;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = VEC ? 2 * ((u >> 1) * 256 + tid) + (u & 1) : u * 256 + tid;
      As[buf][e / GK][e % GK] = ra[set][u];
      if (a.transB) Bs[buf][e / GK][e % GK] = rb[set][u];
      else Bs[buf][e % GB][e / GB] = rb[set][u];
    }
  };

  if (!skip && kend > kbeg) {
    typedef std::integral_constant<int, 0> I0;
    typedef std::integral_constant<int, 1> I1;
    typedef std::integral_constant<int, 2> I2;
    typedef std::integral_constant<int, 3> I3;
    static_assert(PD == 4, "ring of four register sets");
    const int64_t k00 = kbeg / GK * GK;
    const int64_t nk = (kend - k00 + GK - 1) / GK;
    // register set it % PD holds K step it; LDS buffer it % 2 is computed
    gload(k00, I0());
    if (1 < nk) gload(k00 + GK, I1());
    if (2 < nk) gload(k00 + 2 * GK, I2());
    if (3 < nk) gload(k00 + 3 * GK, I3());
    sstore(0, I0());
    __syncthreads();
    auto step = [&](auto PH, int64_t it) {
      constexpr int ph = decltype(PH)::value;
      const int buf = (int)(it & 1);
#pragma unroll
      for (int st = 0; st < GK / 4; ++st) {
        double af[NBW], bf[NBW];
#pragma unroll
        for (int i = 0; i < NBW; ++i) af[i] = As[buf][wr * WT + i * 16 + r16][4 * kg + st];
#pragma unroll
        for (int j = 0; j < NBW; ++j) bf[j] = Bs[buf][wc * WT + j * 16 + r16][4 * kg + st];
#pragma unroll
        for (int i = 0; i < NBW; ++i)
#pragma unroll
          for (int j = 0; j < NBW; ++j) acc[i][j] = MF::mma(af[i], bf[j], acc[i][j]);
      }
      if (it + 1 < nk) sstore(buf ^ 1, std::integral_constant<int, (ph + 1) % PD>());
      // set ph is free once step it is in LDS: refill it with step it + PD
      if (it + PD < nk) gload(k00 + (it + PD) * GK, PH);
      __syncthreads();
    };
    for (int64_t it0 = 0; it0 < nk; it0 += PD) {
      step(I0(), it0);
      if (it0 + 1 < nk) step(I1(), it0 + 1);
      if (it0 + 2 < nk) step(I2(), it0 + 2);
      if (it0 + 3 < nk) step(I3(), it0 + 3);
    }
  }

  if (a.dot) {
    double part = 0.0;
    if (!skip) {
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t gr = row0 + wr * WT + i * 16 + MF::row(lane, r);
            const int64_t gc = col0 + wc * WT + j * 16 + r16;
            if (gr < a.M && gc < a.N) {
              double wgt = 1.0;
              if (a.sym_dot) wgt = gr > gc ? 2.0 : (gr == gc ? 1.0 : 0.0);
              part += wgt * a.alpha * acc[i][j][r] * a.dot[z * a.sDot + gr * a.lddot + gc];
            }
          }
    }
    // fixed-order reduction: wave butterfly, then the four waves in order
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (lane == 0) red[wave] = part;
    __syncthreads();
    if (tid == 0)
      a.partial[z * a.sPart + bm * nbx + bn] = ((red[0] + red[1]) + red[2]) + red[3];
    return;
  }
  if (skip) return;
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t gr = row0 + wr * WT + i * 16 + MF::row(lane, r);
        const int64_t gc = col0 + wc * WT + j * 16 + r16;
        // lower_out: leave 64 x 64 sub-blocks strictly above the diagonal untouched
        if (a.lower_out && gc / GTRI > gr / GTRI) continue;
        if (gr < a.M && gc < a.N) {
          double v = a.alpha * acc[i][j][r];
          if (a.beta != 0.0) v += a.beta * Cp[gr * a.ldc + gc];
          Cp[gr * a.ldc + gc] = v;
        }
      }
}

template <int GB, bool VEC, bool TRI>
__global__ __launch_bounds__(256) void gemm64_kernel(Gemm64Args a) {
  gemm64_block<GB, VEC, TRI>(a, map_block<TRI>(a), gridDim.x);
}

// Two independent products of one launch (one-dimensional grid: the blocks
// of a0, then those of a1, each mapped as in gemm64_kernel).
template <int GB, bool TRI>
__global__ __launch_bounds__(256) void gemm64_pair_kernel(Gemm64Args a0, Gemm64Args a1,
                                                          int64_t X0, int64_t Y0, int64_t X1,
                                                          int64_t Y1) {
  const int64_t w = blockIdx.x, n0 = X0 * Y0 * a0.batch;
  if (w < n0) gemm64_block<GB, false, TRI>(a0, map_block_lin(a0, w, X0, Y0, a0.batch), X0);
  else gemm64_block<GB, false, TRI>(a1, map_block_lin(a1, w - n0, X1, Y1, a1.batch), X1);
}

// Large-tile variant: BM x BN output blocks, WM x WN waves (64 * WM * WN
// threads), each wave a (BM / WM) x (BN / WN) sub-block of 16 x 16 MFMA
// blocks; otherwise the same options and the same K loop as gemm64_kernel.
// Twice the MFMA work per loaded byte of the 64 x 64 kernel. The main loop
// and the dot epilogue are shared with the stream-K kernel below.
template <int BM, int BN, int WM, int WN>
struct BigCfg {
  static constexpr int NT = 64 * WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN, NBM = TM / 16, NBN = TN / 16;
  static constexpr int PA = BM * GK / NT, PB = BN * GK / NT;
  static_assert(PA >= 1 && PB >= 1 && BM % GTRI == 0 && BN % GTRI == 0, "tile shape");
  typedef Mfma<double>::acc_t acc_t;
};

// acc += A[row0.., kbeg..kend) op(B)[kbeg..kend), col0..) for the block at
// (row0, col0); ends with a barrier (the LDS buffers are free again).
template <int BM, int BN, int WM, int WN, bool TRI>
__device__ __forceinline__ void big_mainloop(const Gemm64Args& a, int z, int64_t row0,
                                             int64_t col0, int64_t kbeg, int64_t kend,
                                             typename BigCfg<BM, BN, WM, WN>::acc_t (
                                                 &acc)[BigCfg<BM, BN, WM, WN>::NBM]
                                                      [BigCfg<BM, BN, WM, WN>::NBN],
                                             double (*As)[BM][GLD], double (*Bs)[BN][GLD]) {
  typedef BigCfg<BM, BN, WM, WN> C;
  typedef Mfma<double> MF;
  constexpr int NT = C::NT, TM = C::TM, TN = C::TN, NBM = C::NBM, NBN = C::NBN;
  constexpr int PA = C::PA, PB = C::PB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane & 15, kg = lane >> 4;
  const double* __restrict__ Ap = a.A + z * a.sA;
  const double* __restrict__ Bp = a.B + z * a.sB;
  auto kin = [&](int64_t gk) { return gk < kend && gk >= kbeg; };
  auto ain = [&](int64_t gr, int64_t gk) {
    return gr < a.M && kin(gk) && (!TRI || !a.a_lower || gk < (gr / GTRI + 1) * GTRI);
  };
  auto bin = [&](int64_t gn, int64_t gk) {
    if (gn >= a.N || !kin(gk)) return false;
    if (!TRI || !a.b_lower) return true;
    return a.transB ? gk < (gn / GTRI + 1) * GTRI : gk >= (gn / GTRI) * GTRI;
  };
  double ra[PA], rb[PB];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < PA; ++u) {
      const int e = u * NT + tid;
      const int r = e / GK, c = e % GK;
      const int64_t gr = row0 + r, gk = k0 + c;
      ra[u] = ain(gr, gk) ? Ap[gr * a.lda + gk] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int e = u * NT + tid;
      if (a.transB) {
        const int r = e / GK, c = e % GK;
        const int64_t gn = col0 + r, gk = k0 + c;
        rb[u] = bin(gn, gk) ? Bp[gn * a.ldb + gk] : 0.0;
      } else {
        const int kr = e / BN, cc = e % BN;
        const int64_t gk = k0 + kr, gn = col0 + cc;
        rb[u] = bin(gn, gk) ? Bp[gk * a.ldb + gn] : 0.0;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PA; ++u) {
      const int e = u * NT + tid;
      As[buf][e / GK][e % GK] = ra[u];
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int e = u * NT + tid;
      if (a.transB) Bs[buf][e / GK][e % GK] = rb[u];
      else Bs[buf][e % BN][e / BN] = rb[u];
    }
  };
  if (kend <= kbeg) return;
  const int64_t k00 = kbeg / GK * GK;
  gload(k00);
  sstore(0);
  __syncthreads();
  const int64_t nk = (kend - k00 + GK - 1) / GK;
  for (int64_t it = 0; it < nk; ++it) {
    const int buf = (int)(it & 1);
    if (it + 1 < nk) gload(k00 + (it + 1) * GK);
#pragma unroll
    for (int st = 0; st < GK / 4; ++st) {
      double af[NBM], bf[NBN];
#pragma unroll
      for (int i = 0; i < NBM; ++i) af[i] = As[buf][wm * TM + i * 16 + r16][4 * kg + st];
#pragma unroll
      for (int j = 0; j < NBN; ++j) bf[j] = Bs[buf][wn * TN + j * 16 + r16][4 * kg + st];
#pragma unroll
      for (int i = 0; i < NBM; ++i)
#pragma unroll
        for (int j = 0; j < NBN; ++j) acc[i][j] = MF::mma(af[i], bf[j], acc[i][j]);
    }
    if (it + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }
}

// This thread's share of sum(alpha C_block .* dot_block) (sym_dot weights).
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ double big_dot(const Gemm64Args& a, int z, int64_t row0, int64_t col0,
                                          const typename BigCfg<BM, BN, WM, WN>::acc_t (
                                              &acc)[BigCfg<BM, BN, WM, WN>::NBM]
                                                   [BigCfg<BM, BN, WM, WN>::NBN]) {
  typedef BigCfg<BM, BN, WM, WN> C;
  typedef Mfma<double> MF;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN, r16 = lane & 15;
  double part = 0.0;
#pragma unroll
  for (int i = 0; i < C::NBM; ++i)
#pragma unroll
    for (int j = 0; j < C::NBN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t gr = row0 + wm * C::TM + i * 16 + MF::row(lane, r);
        const int64_t gc = col0 + wn * C::TN + j * 16 + r16;
        if (gr < a.M && gc < a.N) {
          double wgt = 1.0;
          if (a.sym_dot) wgt = gr > gc ? 2.0 : (gr == gc ? 1.0 : 0.0);
          part += wgt * a.alpha * acc[i][j][r] * a.dot[z * a.sDot + gr * a.lddot + gc];
        }
      }
  return part;
}

// Fixed-order workgroup sum of one value per thread (result on thread 0).
template <int NW>
__device__ __forceinline__ double wg_sum(double part, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if (lane == 0) red[wave] = part;
  __syncthreads();
  double t = red[0];
  for (int q = 1; q < NW; ++q) t += red[q];
  return t;
}

// One BM x BN output block (bmap) of one problem; nbx = column blocks of the
// grid (indexes the dot epilogue's per-block partials).
template <int BM, int BN, int WM, int WN, bool TRI>
__device__ __forceinline__ void big_block(const Gemm64Args& a, const BlockMap bmap, int64_t nbx) {
  typedef BigCfg<BM, BN, WM, WN> C;
  typedef Mfma<double> MF;
  __shared__ double As[2][BM][GLD];
  __shared__ double Bs[2][BN][GLD];
  __shared__ double red[WM * WN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane & 15;
  const int64_t bm = bmap.bm, bn = bmap.bn;
  const int z = bmap.z;
  double* Cp = a.C + z * a.sC;
  const int64_t row0 = bm * BM, col0 = bn * BN;
  const bool skip = a.lower_out && col0 >= row0 + BM;

  typename C::acc_t acc[C::NBM][C::NBN];
#pragma unroll
  for (int i = 0; i < C::NBM; ++i)
#pragma unroll
    for (int j = 0; j < C::NBN; ++j) acc[i][j] = MF::zero();

  int64_t kend = a.K, kbeg = 0;
  if (a.a_lower && row0 + BM < kend) kend = row0 + BM;
  if (a.b_lower) {
    if (a.transB) {
      if (col0 + BN < kend) kend = col0 + BN;
    } else {
      kbeg = col0;
    }
  }
  if (!skip) big_mainloop<BM, BN, WM, WN, TRI>(a, z, row0, col0, kbeg, kend, acc, As, Bs);

  if (a.dot) {
    const double part = skip ? 0.0 : big_dot<BM, BN, WM, WN>(a, z, row0, col0, acc);
    const double t = wg_sum<WM * WN>(part, red);
    if (tid == 0) a.partial[z * a.sPart + bm * nbx + bn] = t;
    return;
  }
  if (skip) return;
#pragma unroll
  for (int i = 0; i < C::NBM; ++i)
#pragma unroll
    for (int j = 0; j < C::NBN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t gr = row0 + wm * C::TM + i * 16 + MF::row(lane, r);
        const int64_t gc = col0 + wn * C::TN + j * 16 + r16;
        if (a.lower_out && gc / GTRI > gr / GTRI) continue;
        if (gr < a.M && gc < a.N) {
          double v = a.alpha * acc[i][j][r];
          if (a.beta != 0.0) v += a.beta * Cp[gr * a.ldc + gc];
          Cp[gr * a.ldc + gc] = v;
        }
      }
}

template <int BM, int BN, int WM, int WN, bool TRI>
__global__ __launch_bounds__(64 * WM * WN) void gemm_big_kernel(Gemm64Args a) {
  big_block<BM, BN, WM, WN, TRI>(a, map_block<TRI>(a), gridDim.x);
}

// Two independent products of one launch on BS x BS blocks: first the blocks
// on or below the diagonal of a0 (a square lower-block product without a
// triangular operand: n0 = nb (nb + 1) / 2 blocks per problem, all with the
// same K range), then the blocks of a1 (X1 x Y1 per problem) mapped longest
// K range first as in gemm_big_kernel. The two products share the machine,
// so the half of the grid that a lower-block product alone leaves idle runs
// the other product.
template <int BS, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_big_pair_kernel(Gemm64Args a0,
                                                                    Gemm64Args a1, int64_t n0,
                                                                    int64_t X1, int64_t Y1) {
  const int64_t w = blockIdx.x;
  if (w < n0) {
    // a0's lower blocks, problem fastest: block b of the lower triangle in
    // row-major order is (bm, b - bm (bm + 1) / 2)
    const int64_t b = w / a0.batch;
    int64_t bm = (int64_t)((__builtin_sqrt(8.0 * (double)b + 1.0) - 1.0) * 0.5);
    while (bm * (bm + 1) / 2 > b) --bm;
    while ((bm + 1) * (bm + 2) / 2 <= b) ++bm;
    const BlockMap m{bm, b - bm * (bm + 1) / 2, (int)(w % a0.batch)};
    big_block<BS, BS, WM, WN, true>(a0, m, 0);
  } else {
    big_block<BS, BS, WM, WN, true>(a1, map_block_lin(a1, w - n0, X1, Y1, a1.batch), X1);
  }
}

// Stream-K dot product over the lower blocks of a square product (the
// loss). Blocks are BM x BN with BM = RB BN (RB = 1 or 2); row block bm
// holds the column blocks bn < RB (bm + 1), which cover its part of the
// lower triangle. The nblk blocks times nk K steps form one list of
// block-steps, cut into gridDim.x equal contiguous ranges, one per
// workgroup. The dot epilogue is linear in the block's product, so a
// workgroup adds the epilogue of each partial K range it holds and writes
// one partial; every workgroup has the same amount of MFMA work whatever
// the number of blocks.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_sk_lower_dot_kernel(Gemm64Args a,
                                                                         int64_t nk,
                                                                         int64_t total) {
  typedef BigCfg<BM, BN, WM, WN> C;
  typedef Mfma<double> MF;
  constexpr int RB = BM / BN;
  static_assert(RB * BN == BM && (RB == 1 || RB == 2), "block shape");
  __shared__ double As[2][BM][GLD];
  __shared__ double Bs[2][BN][GLD];
  __shared__ double red[WM * WN];
  const int64_t g = blockIdx.x, G = gridDim.x;
  const int64_t it1 = total * (g + 1) / G;
  double part = 0.0;
  for (int64_t it = total * g / G; it < it1;) {
    const int64_t b = it / nk, kb = it % nk;
    const int64_t cnt = (nk - kb) < (it1 - it) ? (nk - kb) : (it1 - it);
    // blocks before row bm: RB bm (bm + 1) / 2
    int64_t bm = (int64_t)((__builtin_sqrt(8.0 * (double)b / RB + 1.0) - 1.0) * 0.5);
    while (RB * bm * (bm + 1) / 2 > b) --bm;
    while (RB * (bm + 1) * (bm + 2) / 2 <= b) ++bm;
    const int64_t bn = b - RB * bm * (bm + 1) / 2;
    typename C::acc_t acc[C::NBM][C::NBN];
#pragma unroll
    for (int i = 0; i < C::NBM; ++i)
#pragma unroll
      for (int j = 0; j < C::NBN; ++j) acc[i][j] = MF::zero();
    const int64_t kbeg = kb * GK, kend = (kb + cnt) * GK < a.K ? (kb + cnt) * GK : a.K;
    big_mainloop<BM, BN, WM, WN, false>(a, 0, bm * BM, bn * BN, kbeg, kend, acc, As, Bs);
    part += big_dot<BM, BN, WM, WN>(a, 0, bm * BM, bn * BN, acc);
    it += cnt;
  }
  const double t = wg_sum<WM * WN>(part, red);
  if (threadIdx.x == 0) a.partial[g] = t;
}

// Kernel choice: the 128 x 128 eight-wave kernel when it still gives at
// least 256 workgroups, else the 64 x 64 kernel (more workgroups for the
// smaller products and the lower-block ones).
// Stream-K: the dot product of a square lower-block product (one problem,
// no triangular operand), on one workgroup per compute unit.
constexpr int kSkGrid = 256;
static bool use_sk(const Gemm64Args& a) {
  return a.lower_out && a.dot && a.sym_dot && a.batch == 1 && !a.a_lower && !a.b_lower &&
         a.M == a.N;
}
// blocks of 128 x 128 (256 x 128 blocks measured slower here: the stream-K
// loop state makes that kernel spill)
static int64_t sk_total(const Gemm64Args& a, int64_t* nk) {
  const int64_t nb = (a.M + 127) / 128;
  *nk = (a.K + GK - 1) / GK;
  return nb * (nb + 1) / 2 * *nk;
}

static bool use_big(const Gemm64Args& a) {
  // lower-block products (half of the blocks idle) balance better on the
  // finer 64 x 64 grid
  if (a.lower_out) return false;
  const int64_t t = ((a.M + 127) / 128) * ((a.N + 127) / 128) * a.batch;
  return t >= 256;
}

int64_t gemm64_num_blocks(int64_t M, int64_t N) {
  const int64_t b = ((M + 63) / 64) * ((N + 63) / 64);
  return b > kSkGrid ? b : kSkGrid;
}

int64_t gemm64_partials(const Gemm64Args& a) {
  if (use_sk(a)) {
    int64_t nk;
    const int64_t t = sk_total(a, &nk);
    return t < kSkGrid ? t : kSkGrid;
  }
  if (use_big(a)) return ((a.M + 127) / 128) * ((a.N + 127) / 128);
  return ((a.M + 63) / 64) * ((a.N + 63) / 64);
}

template <int GB>
static hipError_t launch_gb(const Gemm64Args& a, bool vec, hipStream_t s) {
  dim3 grid((unsigned)((a.N + GB - 1) / GB), (unsigned)((a.M + GB - 1) / GB), (unsigned)a.batch);
  const bool tri = a.a_lower || a.b_lower;
  if (vec) {
    if (tri) hipLaunchKernelGGL((gemm64_kernel<GB, true, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gemm64_kernel<GB, true, false>), grid, dim3(256), 0, s, a);
  } else {
    if (tri) hipLaunchKernelGGL((gemm64_kernel<GB, false, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gemm64_kernel<GB, false, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// Block size of the 64 x 64 kernel family for a, or 0 when a goes to
// another kernel (stream-K, 256 x 128, 128 x 128).
static int small_block(const Gemm64Args& a) {
  if (use_sk(a)) return 0;
  if (!a.a_lower && !a.b_lower && !a.dot &&
      ((a.M + 255) / 256) * ((a.N + 127) / 128) * a.batch >= 256)
    return 0;
  if (use_big(a)) return 0;
  const int64_t b64 = ((a.M + 63) / 64) * ((a.N + 63) / 64) * a.batch;
  return (!a.dot && b64 <= 512) ? 32 : 64;
}

// The pair of a square lower-block product a0 (no triangular operand) and
// a1 on 128 x 128 blocks, when together they give at least this many blocks
// (the factor's top node at 4096: Schur update on its lower blocks and
// C21 Y11, 1.02 -> 0.79 ms against two launches; the order-2048 nodes' 200
// blocks stay on the 32 x 32 pair kernel, which measured as fast)
constexpr int64_t kBigPairMinBlocks = 256;

hipError_t launch_gemm64_pair(const Gemm64Args& a0, const Gemm64Args& a1, hipStream_t s) {
  if (a0.lower_out && !a0.a_lower && !a0.b_lower && a0.M == a0.N && !a0.dot && !a1.dot &&
      a0.M > 0 && a1.M > 0 && a1.N > 0 && a0.batch == a1.batch && a0.batch >= 1 &&
      a0.batch <= kMaxGemmBatch) {
    const int64_t nb = (a0.M + 127) / 128;
    const int64_t n0 = nb * (nb + 1) / 2 * a0.batch;
    const int64_t X1 = (a1.N + 127) / 128, Y1 = (a1.M + 127) / 128;
    const int64_t n1 = X1 * Y1 * a1.batch;
    if (n0 + n1 >= kBigPairMinBlocks) {
      hipLaunchKernelGGL((gemm_big_pair_kernel<128, 2, 4>), dim3((unsigned)(n0 + n1)), dim3(512),
                         0, s, a0, a1, n0, X1, Y1);
      return hipGetLastError();
    }
  }
  const int g0 = small_block(a0), g1 = small_block(a1);
  const bool empty0 = a0.M <= 0 || a0.N <= 0, empty1 = a1.M <= 0 || a1.N <= 0;
  if (empty0 || empty1 || g0 == 0 || g0 != g1 || a0.dot || a1.dot || a0.batch != a1.batch ||
      a0.batch < 1 || a0.batch > kMaxGemmBatch) {
    const hipError_t e = launch_gemm64(a0, s);
    return e != hipSuccess ? e : launch_gemm64(a1, s);
  }
  const int GB = g0;
  const int64_t X0 = (a0.N + GB - 1) / GB, Y0 = (a0.M + GB - 1) / GB;
  const int64_t X1 = (a1.N + GB - 1) / GB, Y1 = (a1.M + GB - 1) / GB;
  const int64_t nwg = (X0 * Y0 + X1 * Y1) * a0.batch;
  if (GB == 32)
    hipLaunchKernelGGL((gemm64_pair_kernel<32, true>), dim3((unsigned)nwg), dim3(256), 0, s, a0,
                       a1, X0, Y0, X1, Y1);
  else
    hipLaunchKernelGGL((gemm64_pair_kernel<64, true>), dim3((unsigned)nwg), dim3(256), 0, s, a0,
                       a1, X0, Y0, X1, Y1);
  return hipGetLastError();
}

hipError_t launch_gemm64(const Gemm64Args& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.batch < 1 || a.batch > kMaxGemmBatch) return hipErrorInvalidValue;
  // 16-byte vectors need every row start of A and B 16-byte aligned; they
  // measured slower than element loads here (more registers, lower
  // occupancy), so they are off
  const bool vec = false && (a.lda % 2 == 0) && (a.ldb % 2 == 0) && (a.sA % 2 == 0) &&
                   (a.sB % 2 == 0) && (reinterpret_cast<uintptr_t>(a.A) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(a.B) % 16 == 0);
  if (use_sk(a)) {
    int64_t nk;
    const int64_t t = sk_total(a, &nk);
    if (t == 0) return hipSuccess;
    const int64_t G = t < kSkGrid ? t : kSkGrid;
    hipLaunchKernelGGL((gemm_sk_lower_dot_kernel<128, 128, 2, 4>), dim3((unsigned)G), dim3(512),
                       0, s, a, nk, t);
    return hipGetLastError();
  }
  // products with at least 256 blocks of 256 x 128 (the loss's D A, the
  // factor's top Schur complement on its lower blocks): 4 x 2 waves of
  // 64 x 64, a third more MFMA work per loaded byte again
  if (!a.a_lower && !a.b_lower && !a.dot &&
      ((a.M + 255) / 256) * ((a.N + 127) / 128) * a.batch >= 256) {
    dim3 grid((unsigned)((a.N + 127) / 128), (unsigned)((a.M + 255) / 256), (unsigned)a.batch);
    hipLaunchKernelGGL((gemm_big_kernel<256, 128, 4, 2, false>), grid, dim3(512), 0, s, a);
    return hipGetLastError();
  }
  if (use_big(a)) {
    dim3 grid((unsigned)((a.N + 127) / 128), (unsigned)((a.M + 127) / 128), (unsigned)a.batch);
    if (a.a_lower || a.b_lower)
      hipLaunchKernelGGL((gemm_big_kernel<128, 128, 2, 4, true>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_big_kernel<128, 128, 2, 4, false>), grid, dim3(512), 0, s, a);
    return hipGetLastError();
  }
  // small products (the factor's lower levels, up to the order-2048 nodes at
  // n = 4096): 32 x 32 blocks give four times the workgroups, each with a
  // quarter of the dependent MFMA chain (up to 512 blocks of 64 x 64 measured
  // best: factor 6.30 -> 6.21 ms at 4096, 26.4 -> 25.9 ms at 8192)
  const int64_t b64 = ((a.M + 63) / 64) * ((a.N + 63) / 64) * a.batch;
  if (!a.dot && b64 <= 512) return launch_gb<32>(a, vec, s);
  return launch_gb<64>(a, vec, s);
}

}  // namespace bk
