// Per-row scale search for gfx950: the optional MSE shrink of the per-row
// absmax scales in the experimental setup of "BaKron: Efficient Quantization
// with Kronecker-Factored Hessians" (arXiv 2608.06291), Appendix D: start
// from s_max = absmax / hi and shrink it by up to a factor 1 / (1 - max_shrink)
// (the pages: up to 2), keeping the candidate whose round-to-nearest squared
// error over the row is smallest.
//
// Candidates: s_k = (R)(s_max * f_k), f_k = 1 - (max_shrink * k) / grid in
// float64, k = 0..grid. Error of s_k: sum_j (w_j - s_k c_j)^2 with
// c_j = clamp(rint(w_j / s_k), lo, hi) (true division in R, the quantizer of
// §3.1), each term and the sum in float64. Smallest error wins, ties go to
// the smaller k (the larger scale); an all-zero row gets scale 1.
//
// One workgroup per row. Every thread walks its elements once per chunk of
// kChunk candidates, keeping one float64 partial per candidate; partials are
// reduced across the wave with XOR shuffles, then across the four waves in a
// fixed order, so the result is deterministic. The row is re-read once per
// chunk and stays in the L1/L2 caches after the first pass; the kernel is
// bound by the vector ALU (a division and a float64 square per element and
// candidate), not by HBM.
#include "device.hpp"
#include "launch.hpp"

namespace bk {

constexpr int kScaleChunk = 16;

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
template <typename R>
__device__ inline R wave_max(R v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const R u = __shfl_xor(v, o, 64);
    v = u > v ? u : v;
  }
  return v;
}

__device__ inline double shrink_factor(int k, int grid, double max_shrink) {
  return grid == 0 ? 1.0 : 1.0 - (max_shrink * (double)k) / (double)grid;
}

template <typename R>
__global__ __launch_bounds__(256) void row_scales_mse_kernel(int64_t n, const R* __restrict__ W,
                                                             int64_t ldw, R lo, R hi, R hi_code,
                                                             int grid, double max_shrink,
                                                             R* __restrict__ s_out) {
  __shared__ R wmax[4];
  __shared__ double part[4][kScaleChunk];
  __shared__ double errs[kScaleMaxGrid + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const R* __restrict__ row = W + (int64_t)blockIdx.x * ldw;

  R mx = R(0);
  for (int64_t j = tid; j < n; j += 256) {
    const R v = row[j];
    const R a = v < R(0) ? -v : v;
    mx = a > mx ? a : mx;
  }
  mx = wave_max(mx);
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  mx = wmax[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) mx = wmax[w] > mx ? wmax[w] : mx;
  if (mx == R(0)) {
    if (tid == 0) s_out[blockIdx.x] = R(1);
    return;
  }
  const R smax = mx / hi_code;

  for (int k0 = 0; k0 <= grid; k0 += kScaleChunk) {
    R sk[kScaleChunk];
    double acc[kScaleChunk];
#pragma unroll
    for (int c = 0; c < kScaleChunk; ++c) {
      sk[c] = (R)((double)smax * shrink_factor(k0 + c, grid, max_shrink));
      acc[c] = 0.0;
    }
    for (int64_t j = tid; j < n; j += 256) {
      const R w = row[j];
      const double wd = (double)w;
#pragma unroll
      for (int c = 0; c < kScaleChunk; ++c) {
        const R code = quant_unit(w / sk[c], lo, hi);
        const double e = wd - (double)sk[c] * (double)code;
        acc[c] += e * e;
      }
    }
#pragma unroll
    for (int c = 0; c < kScaleChunk; ++c) {
      const double v = wave_sum(acc[c]);
      if (lane == 0) part[wave][c] = v;
    }
    __syncthreads();
    if (tid < kScaleChunk && k0 + tid <= grid)
      errs[k0 + tid] = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
    __syncthreads();
  }
  if (tid == 0) {
    int best = 0;
    for (int k = 1; k <= grid; ++k)
      if (errs[k] < errs[best]) best = k;
    s_out[blockIdx.x] = (R)((double)smax * shrink_factor(best, grid, max_shrink));
  }
}

template <typename R>
hipError_t launch_row_scales_mse(int64_t m, int64_t n, const R* W, int64_t ldw, int32_t lo,
                                 int32_t hi, int32_t hi_code, int32_t grid, double max_shrink,
                                 R* s_out, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL((row_scales_mse_kernel<R>), dim3((unsigned)m), dim3(256), 0, s, n, W, ldw,
                     (R)lo, (R)hi, (R)hi_code, grid, max_shrink, s_out);
  return hipGetLastError();
}

template hipError_t launch_row_scales_mse<float>(int64_t, int64_t, const float*, int64_t, int32_t,
                                                 int32_t, int32_t, int32_t, double, float*,
                                                 hipStream_t);
template hipError_t launch_row_scales_mse<double>(int64_t, int64_t, const double*, int64_t,
                                                  int32_t, int32_t, int32_t, int32_t, double,
                                                  double*, hipStream_t);

}  // namespace bk
