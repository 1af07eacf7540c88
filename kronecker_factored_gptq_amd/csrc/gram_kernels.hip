// Kronecker factors from samples, on MFMA (gfx950): the weighted Gram
//   G = (1/N) sum_k w_k x_k x_k^T  (+ damp_rel * mean(diag G) * I)
// of the N rows x_k of X (N x d, row-major). With w = 1 this is the K-FAC
// factor E[a a^T] (or E[b b^T]); with w_k = |b_k|^2 (or |a_k|^2) it is the
// one-step Shampoo factor E[(b^T b) a a^T] of "BaKron: Efficient Quantization
// with Kronecker-Factored Hessians" (arXiv 2608.06291), §4.2 and Appendix A.2;
// the damping is the mean-diagonal regularisation of its experiments.
//
// gram_kernel: G = X^T diag(w) X on the lower BM x BM blocks only (the
// product is symmetric), four waves in a 2 x 2 arrangement, K (the sample
// index) in steps of 16 through double-buffered LDS. Both MFMA operands come
// from rows of X, which is exactly the operand layout the MFMA wants when k
// is the sample index (lane l reads X[k][c0 + l % 16] for k = l / 16):
// global loads are contiguous row segments, LDS rows are k. The weights
// scale the B operand as it is stored to LDS. gram_mirror_kernel copies the
// lower triangle to the upper one; gram_damp_kernel (one workgroup) adds the
// damping after reading the whole diagonal, so no workgroup reads a diagonal
// entry another has already damped.
#include "device.hpp"
#include "launch.hpp"

namespace bk {

namespace {
constexpr int kGramBK = 16;   // samples per K step
constexpr int kGramPad = 16;  // LDS row padding (elements)
}  // namespace

template <typename R, int BM>
__global__ __launch_bounds__(256) void gram_kernel(int64_t N, int64_t d, const R* __restrict__ X,
                                                   int64_t ldx, const R* __restrict__ w, R alpha,
                                                   R* __restrict__ G, int64_t ldg) {
  typedef Mfma<R> MF;
  typedef typename MF::acc_t acc_t;
  constexpr int WT = BM / 2, NBW = WT / 16;
  constexpr int LD = BM + kGramPad;
  constexpr int PER = kGramBK * BM / 256;  // elements per thread per operand per K step
  __shared__ R As[2][kGramBK][LD];
  __shared__ R Bs[2][kGramBK][LD];

  // lower block (bm >= bn) of linear number blockIdx.x, row-wise
  const int64_t t = blockIdx.x;
  int64_t bm = (int64_t)((__builtin_sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while (bm * (bm + 1) / 2 > t) --bm;
  while ((bm + 1) * (bm + 2) / 2 <= t) ++bm;
  const int64_t bn = t - bm * (bm + 1) / 2;
  const int64_t r0 = bm * BM, c0 = bn * BM;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int r16 = lane & 15, kg = lane >> 4;

  acc_t acc[NBW][NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = MF::zero();

  R ra[PER], rb[PER];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = u * 256 + tid;
      const int kr = e / BM, c = e % BM;
      const int64_t k = k0 + kr;
      R a = R(0), b = R(0);
      if (k < N) {
        if (r0 + c < d) a = X[k * ldx + r0 + c];
        if (c0 + c < d) {
          b = X[k * ldx + c0 + c];
          if (w) b *= w[k];
        }
      }
      ra[u] = a;
      rb[u] = b;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = u * 256 + tid;
      As[buf][e / BM][e % BM] = ra[u];
      Bs[buf][e / BM][e % BM] = rb[u];
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < kGramBK / 4; ++s) {
      const int k = 4 * s + kg;
      R af[NBW], bf[NBW];
#pragma unroll
      for (int i = 0; i < NBW; ++i) af[i] = As[buf][k][wr * WT + i * 16 + r16];
#pragma unroll
      for (int j = 0; j < NBW; ++j) bf[j] = Bs[buf][k][wc * WT + j * 16 + r16];
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = MF::mma(af[i], bf[j], acc[i][j]);
    }
  };

  const int64_t nsteps = (N + kGramBK - 1) / kGramBK;
  if (nsteps > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
    for (int64_t it = 0; it < nsteps; ++it) {
      if (it + 1 < nsteps) gload((it + 1) * kGramBK);
      compute((int)(it & 1));
      if (it + 1 < nsteps) sstore((int)((it + 1) & 1));
      __syncthreads();
    }
  }

  // lower triangle of the block (all of it below the diagonal blocks)
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = r0 + wr * WT + i * 16 + MF::row(lane, r);
        const int64_t col = c0 + wc * WT + j * 16 + r16;
        if (row < d && col <= row) G[row * ldg + col] = alpha * acc[i][j][r];
      }
}

// G[i][j] = G[j][i] for i < j, by 32 x 32 tiles through LDS (upper tiles only).
template <typename R>
__global__ __launch_bounds__(256) void gram_mirror_kernel(int64_t d, R* __restrict__ G,
                                                          int64_t ldg) {
  __shared__ R tile[32][33];
  const int64_t ti = blockIdx.y, tj = blockIdx.x;  // destination tile (ti <= tj)
  if (ti > tj) return;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  // source: lower tile (tj, ti), read row-wise
  for (int r = ty; r < 32; r += 8) {
    const int64_t i = tj * 32 + r, j = ti * 32 + tx;
    tile[r][tx] = (i < d && j < d && j <= i) ? G[i * ldg + j] : R(0);
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int64_t i = ti * 32 + r, j = tj * 32 + tx;  // upper element (i, j) = (j, i)
    if (i < d && j < d && i < j) G[i * ldg + j] = tile[tx][r];
  }
}

// One workgroup: mean of the diagonal (float64, fixed order), then add
// damp_rel times it to every diagonal entry.
template <typename R>
__global__ __launch_bounds__(256) void gram_damp_kernel(int64_t d, R* __restrict__ G, int64_t ldg,
                                                        double damp_rel) {
  __shared__ double red[256];
  double sum = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 256) sum += (double)G[i * ldg + i];
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const R add = (R)(damp_rel * (red[0] / (double)d));
  for (int64_t i = threadIdx.x; i < d; i += 256) G[i * ldg + i] += add;
}

// out[k] = sum_j X[k][j]^2, float64 sums in a fixed order, one row per workgroup.
template <typename R>
__global__ __launch_bounds__(256) void sample_sqnorms_kernel(int64_t d, const R* __restrict__ X,
                                                             int64_t ldx, R* __restrict__ out) {
  __shared__ double red[256];
  const R* row = X + (int64_t)blockIdx.x * ldx;
  double s = 0.0;
  for (int64_t j = threadIdx.x; j < d; j += 256) {
    const double v = (double)row[j];
    s += v * v;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = (R)red[0];
}

// Block edge: 128 when that still gives at least four lower blocks per
// compute unit (1024), else 64 (more, smaller workgroups balance better).
template <typename R> struct GramBig;
template <> struct GramBig<float> { static constexpr int BM = 128; };
template <> struct GramBig<double> { static constexpr int BM = 64; };

template <typename R>
hipError_t launch_gram(int64_t N, int64_t d, const R* X, int64_t ldx, const R* w, double damp_rel,
                       R* G, int64_t ldg, hipStream_t s) {
  if (d <= 0) return hipSuccess;
  const R alpha = N > 0 ? (R)(1.0 / (double)N) : R(0);
  constexpr int BIG = GramBig<R>::BM;
  const int64_t nb_big = (d + BIG - 1) / BIG, nb64 = (d + 63) / 64;
  if (BIG != 64 && nb_big * (nb_big + 1) / 2 >= 1024) {
    hipLaunchKernelGGL((gram_kernel<R, BIG>), dim3((unsigned)(nb_big * (nb_big + 1) / 2)),
                       dim3(256), 0, s, N, d, X, ldx, w, alpha, G, ldg);
  } else {
    hipLaunchKernelGGL((gram_kernel<R, 64>), dim3((unsigned)(nb64 * (nb64 + 1) / 2)), dim3(256),
                       0, s, N, d, X, ldx, w, alpha, G, ldg);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nt = (unsigned)((d + 31) / 32);
  hipLaunchKernelGGL((gram_mirror_kernel<R>), dim3(nt, nt), dim3(256), 0, s, d, G, ldg);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (damp_rel != 0.0) {
    hipLaunchKernelGGL((gram_damp_kernel<R>), dim3(1), dim3(256), 0, s, d, G, ldg, damp_rel);
    e = hipGetLastError();
  }
  return e;
}

template <typename R>
hipError_t launch_sample_sqnorms(int64_t N, int64_t d, const R* X, int64_t ldx, R* out,
                                 hipStream_t s) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL((sample_sqnorms_kernel<R>), dim3((unsigned)N), dim3(256), 0, s, d, X, ldx,
                     out);
  return hipGetLastError();
}

#define BK_INST(R)                                                                          \
  template hipError_t launch_gram<R>(int64_t, int64_t, const R*, int64_t, const R*, double, \
                                     R*, int64_t, hipStream_t);                             \
  template hipError_t launch_sample_sqnorms<R>(int64_t, int64_t, const R*, int64_t, R*,     \
                                               hipStream_t);
BK_INST(float)
BK_INST(double)
#undef BK_INST

}  // namespace bk
