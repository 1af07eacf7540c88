// BaKron-antidiagonal on gfx950: "BaKron: Efficient Quantization with
// Kronecker-Factored Hessians" (arXiv 2608.06291), §3.3 Algorithm 3 on the
// whole matrix, the solver the paper measures BaKron against (Table 3).
//
// For each anti-diagonal k = 0 .. m+n-2 (0-based, k = i + j) every entry on
// it is rounded at once, then the errors Delta (supported on anti-diagonal k)
// are applied to every later entry as one rank-d product (Appendix C's cost
// analysis of Algorithm 3):
//   W += [L^B_{i_1} .. L^B_{i_d}] D_delta [L^A_{j_1} .. L^A_{j_d}]^T,
// i_t = i0 + t, j_t = k - i_t. Term t reaches only rows p >= i_t and columns
// q >= j_t (the factors are lower triangular), so an output tile needs only
// the t with i_t <= its last row and j_t <= its last column.
//
// One launch per anti-diagonal: launch k applies the errors of anti-diagonal
// k to the tiles that hold later entries and, in the same epilogue, rounds
// the entries of anti-diagonal k + 1 (which are final once the update of k
// is added) and records their errors for launch k + 1.
//
// The solve runs in code units like the BaKron path: U = S^-1 W and the
// scaled side's factor conjugated by the scales, so a rounding is a plain
// clamp(rint(u)) with error c - u.
//
// Workspace (HBM): U as Mp x Np row-major (m, n rounded up to 64, zero
// padding), the factors TRANSPOSED so that the columns L^B_{i_t}, L^A_{j_t}
// the product gathers are contiguous rows (LBt: m rows of Mp, LAt: n rows
// of Np, zero padding), and two error vectors of min(m, n) entries.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace bk {

constexpr int kAdTile = 64;  // output tile edge
constexpr int kAdK = 16;     // anti-diagonal entries per K step

// Transposed, scaled copy of a normalised factor: Lt[i][p] = L[p][i] (times
// s_i / s_p when scales are given, the code-unit conjugation), 1 on the
// diagonal, 0 above it and on the padding columns p in [dim, ldt).
template <typename R>
__global__ __launch_bounds__(256) void ad_pack_lt_kernel(int64_t dim, const R* __restrict__ L,
                                                         int64_t ld, const R* __restrict__ sc,
                                                         R* __restrict__ Lt, int64_t ldt) {
  __shared__ R tile[32][33];
  const int64_t i0 = (int64_t)blockIdx.y * 32, p0 = (int64_t)blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  // read L[p][i] for p in [p0, p0+32), i in [i0, i0+32): row p, column i
  for (int r = ty; r < 32; r += 8) {
    const int64_t p = p0 + r, i = i0 + tx;
    R v = R(0);
    if (p < dim && i < dim) {
      if (p == i) v = R(1);
      else if (i < p) {
        v = L[p * ld + i];
        if (sc) v = v * sc[i] / sc[p];
      }
    }
    tile[r][tx] = v;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int64_t i = i0 + r, p = p0 + tx;
    if (i < dim && p < ldt) Lt[i * ldt + p] = tile[tx][r];
  }
}

// U = W / s into the padded Mp x Np copy.
template <typename R>
__global__ __launch_bounds__(256) void ad_pack_u_kernel(int64_t m, int64_t n, const R* __restrict__ W,
                                                        int64_t ldw, const R* __restrict__ sc,
                                                        int mode, R* __restrict__ U, int64_t Mp,
                                                        int64_t Np) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= Mp * Np) return;
  const int64_t i = idx / Np, j = idx % Np;
  R v = R(0);
  if (i < m && j < n) {
    v = W[i * ldw + j];
    if (mode == 1) v = v / sc[i];
    else if (mode == 2) v = v / sc[j];
  }
  U[idx] = v;
}

template <typename R>
struct AdArgs {
  int64_t m, n, Mp, Np;
  int k;           // anti-diagonal whose errors are applied; -1: none (first launch)
  int tiles_n;     // output tiles per row of tiles
  R* U;
  const R* LBt;
  const R* LAt;
  const R* dcur;   // errors of anti-diagonal k, entry t at dcur[t] (i = i0(k) + t)
  R* dnext;        // errors of anti-diagonal k + 1
  int32_t* V;
  int64_t ldv;
  R* Wt;           // nullable
  int64_t ldwt;
  const R* scales;
  int scale_mode;
  R lo, hi;
};

template <typename R> struct AdVec;
template <> struct AdVec<float> {
  typedef float4 T;
  static constexpr int N = 4;
};
template <> struct AdVec<double> {
  typedef double2 T;
  static constexpr int N = 2;
};

template <typename R>
__global__ __launch_bounds__(256) void ad_step_kernel(AdArgs<R> a) {
  typedef Mfma<R> MF;
  typedef typename MF::acc_t acc_t;
  typedef typename AdVec<R>::T vec_t;
  constexpr int VN = AdVec<R>::N;
  constexpr int BM = kAdTile, BK = kAdK;
  constexpr int VPR = BM / VN;            // vectors per operand row
  constexpr int NV = BK * VPR / 256;      // vectors per thread per operand per K step
  constexpr int LDS_LD = BM + VN;         // padded row length
  __shared__ __attribute__((aligned(16))) R As[2][BK][LDS_LD];
  __shared__ __attribute__((aligned(16))) R Bs[2][BK][LDS_LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t P = blockIdx.x / a.tiles_n, Q = blockIdx.x % a.tiles_n;
  const int64_t p0 = P * BM, q0 = Q * BM;
  const int64_t pmax = p0 + BM - 1 < a.m - 1 ? p0 + BM - 1 : a.m - 1;
  const int64_t qmax = q0 + BM - 1 < a.n - 1 ? q0 + BM - 1 : a.n - 1;
  const int k = a.k;
  // nothing of this tile lies after anti-diagonal k
  if (pmax + qmax < (int64_t)k + 1) return;

  // terms t of anti-diagonal k that reach this tile: i_t <= pmax, j_t <= qmax
  int64_t tlo = 1, thi = 0, i0 = 0;
  if (k >= 0) {
    i0 = k - (a.n - 1) > 0 ? k - (a.n - 1) : 0;
    const int64_t ilast = k < a.m - 1 ? k : a.m - 1;
    tlo = k - i0 - qmax > 0 ? k - i0 - qmax : 0;
    thi = (ilast < pmax ? ilast : pmax) - i0;
  }

  acc_t acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = MF::zero();

  if (tlo <= thi) {
    vec_t ra[NV], rb[NV];
    // K step starting at entry t0 -> registers: row tt of the step is term
    // t = t0 + tt: L^B column i_t (row i_t of LBt) scaled by its error, and
    // L^A column j_t (row j_t of LAt), each at this tile's 64 positions
    auto gload = [&](int64_t t0) {
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int f = u * 256 + tid;
        const int tt = f / VPR, c = (f % VPR) * VN;
        const int64_t t = t0 + tt;
        vec_t va, vb;
#pragma unroll
        for (int e = 0; e < VN; ++e) { reinterpret_cast<R*>(&va)[e] = R(0); reinterpret_cast<R*>(&vb)[e] = R(0); }
        if (t <= thi) {
          const int64_t it = i0 + t, jt = k - it;
          const R dt = a.dcur[t];
          va = *reinterpret_cast<const vec_t*>(a.LBt + it * a.Mp + p0 + c);
          vb = *reinterpret_cast<const vec_t*>(a.LAt + jt * a.Np + q0 + c);
#pragma unroll
          for (int e = 0; e < VN; ++e) reinterpret_cast<R*>(&va)[e] *= dt;
        }
        ra[u] = va;
        rb[u] = vb;
      }
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int f = u * 256 + tid;
        const int tt = f / VPR, c = (f % VPR) * VN;
        *reinterpret_cast<vec_t*>(&As[buf][tt][c]) = ra[u];
        *reinterpret_cast<vec_t*>(&Bs[buf][tt][c]) = rb[u];
      }
    };
    auto compute = [&](int buf) {
#pragma unroll
      for (int kk = 0; kk < BK / 4; ++kk) {
        const int kr = kk * 4 + (lane >> 4);
        R av[2], bv[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) av[x] = As[buf][kr][wr * 32 + x * 16 + (lane & 15)];
#pragma unroll
        for (int y = 0; y < 2; ++y) bv[y] = Bs[buf][kr][wc * 32 + y * 16 + (lane & 15)];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int y = 0; y < 2; ++y) acc[x][y] = MF::mma(av[x], bv[y], acc[x][y]);
      }
    };
    const int64_t nsteps = (thi - tlo) / BK + 1;
    gload(tlo);
    sstore(0);
    __syncthreads();
    for (int64_t it = 0; it < nsteps; ++it) {
      if (it + 1 < nsteps) gload(tlo + (it + 1) * BK);
      compute((int)(it & 1));
      if (it + 1 < nsteps) sstore((int)((it + 1) & 1));
      __syncthreads();
    }
  }

  // epilogue: add the update to every entry after anti-diagonal k; round the
  // entries of anti-diagonal k + 1, now final
  const int64_t kn = (int64_t)k + 1;
  const int64_t i0n = kn - (a.n - 1) > 0 ? kn - (a.n - 1) : 0;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t p = p0 + wr * 32 + x * 16 + MF::row(lane, r);
        const int64_t q = q0 + wc * 32 + y * 16 + (lane & 15);
        if (p >= a.m || q >= a.n || p + q < kn) continue;
        R* up = a.U + p * a.Np + q;
        const R u = *up + acc[x][y][r];
        if (p + q == kn) {
          const R c = quant_unit(u, a.lo, a.hi);
          a.V[p * a.ldv + q] = (int32_t)c;
          if (a.Wt) {
            R sv = R(1);
            if (a.scale_mode == 1) sv = a.scales[p];
            else if (a.scale_mode == 2) sv = a.scales[q];
            a.Wt[p * a.ldwt + q] = a.scale_mode ? sv * u : u;
          }
          a.dnext[p - i0n] = c - u;
        } else {
          *up = u;
        }
      }
}

template <typename R>
hipError_t launch_antidiag_solve(int64_t m, int64_t n, const R* W, int64_t ldw, const R* LA,
                                 int64_t ldla, const R* LB, int64_t ldlb, R lo, R hi,
                                 int scale_mode, const R* scales, int32_t* V, int64_t ldv, R* Wt,
                                 int64_t ldwt, void* ws, hipStream_t s) {
  if (m <= 0 || n <= 0) return hipSuccess;
  const AntidiagLayout L = antidiag_layout(sizeof(R), m, n);
  char* base = static_cast<char*>(ws);
  R* U = reinterpret_cast<R*>(base + L.u);
  R* LBt = reinterpret_cast<R*>(base + L.lbt);
  R* LAt = reinterpret_cast<R*>(base + L.lat);
  R* d0 = reinterpret_cast<R*>(base + L.d0);
  R* d1 = reinterpret_cast<R*>(base + L.d1);
  const R* scB = scale_mode == 1 ? scales : nullptr;
  const R* scA = scale_mode == 2 ? scales : nullptr;
  {
    const int64_t tot = L.Mp * L.Np;
    hipLaunchKernelGGL((ad_pack_u_kernel<R>), dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s,
                       m, n, W, ldw, scales, scale_mode, U, L.Mp, L.Np);
    if (hipGetLastError() != hipSuccess) return hipErrorUnknown;
    hipLaunchKernelGGL((ad_pack_lt_kernel<R>), dim3((unsigned)(L.Mp / 32), (unsigned)((m + 31) / 32)),
                       dim3(256), 0, s, m, LB, ldlb, scB, LBt, L.Mp);
    if (hipGetLastError() != hipSuccess) return hipErrorUnknown;
    hipLaunchKernelGGL((ad_pack_lt_kernel<R>), dim3((unsigned)(L.Np / 32), (unsigned)((n + 31) / 32)),
                       dim3(256), 0, s, n, LA, ldla, scA, LAt, L.Np);
    if (hipGetLastError() != hipSuccess) return hipErrorUnknown;
  }
  AdArgs<R> a;
  a.m = m; a.n = n; a.Mp = L.Mp; a.Np = L.Np;
  a.tiles_n = (int)(L.Np / kAdTile);
  a.U = U; a.LBt = LBt; a.LAt = LAt;
  a.V = V; a.ldv = ldv; a.Wt = Wt; a.ldwt = ldwt;
  a.scales = scales; a.scale_mode = scale_mode;
  a.lo = lo; a.hi = hi;
  const int64_t tiles_m = L.Mp / kAdTile;
  // launch k applies anti-diagonal k and rounds k + 1: k = -1 .. m + n - 3
  const int64_t last = m + n - 3;
  for (int64_t k = -1; k <= last; ++k) {
    a.k = (int)k;
    a.dcur = (k & 1) ? d1 : d0;
    a.dnext = (k & 1) ? d0 : d1;
    // every tile whose last entry lies on anti-diagonal <= k exits at once
    hipLaunchKernelGGL((ad_step_kernel<R>), dim3((unsigned)(tiles_m * a.tiles_n)), dim3(256), 0, s,
                       a);
    if (hipGetLastError() != hipSuccess) return hipErrorUnknown;
  }
  return hipSuccess;
}

#define BK_INST(R)                                                                              \
  template hipError_t launch_antidiag_solve<R>(int64_t, int64_t, const R*, int64_t, const R*,    \
                                               int64_t, const R*, int64_t, R, R, int, const R*, \
                                               int32_t*, int64_t, R*, int64_t, void*, hipStream_t);
BK_INST(float)
BK_INST(double)
#undef BK_INST

}  // namespace bk
