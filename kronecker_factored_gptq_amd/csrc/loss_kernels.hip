// Loss and scale kernels for gfx950.
//
// Loss: tr(B D A D^T) with D = W - s (.) V ("BaKron: Efficient Quantization
// with Kronecker-Factored Hessians", arXiv 2608.06291, Proposition 3.1: it is
// the quadratic form of vec(D) under A (x) B). Evaluated in float64 as
// sum_ij (B D)_ij (D A)_ij, which equals the trace because A is symmetric.
// Row scales: s_i = max_j |W_ij| / hi (Appendix D: per-row absmax scales).
#include "device.hpp"
#include "launch.hpp"

namespace bk {

// X = symmetric float64 copy of A built from its lower triangle.
template <typename R>
__global__ __launch_bounds__(256) void sym_to_f64_kernel(int64_t n, const R* __restrict__ A,
                                                         int64_t lda, double* __restrict__ X,
                                                         int64_t sA, int64_t sX) {
  __shared__ double t[32][33];
  A += (int64_t)blockIdx.z * sA;  // problem blockIdx.z of a batch
  X += (int64_t)blockIdx.z * sX;
  const int bi = blockIdx.y, bj = blockIdx.x;
  const int sbr = bi > bj ? bi : bj, sbc = bi > bj ? bj : bi;  // source tile (lower)
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) {
    const int64_t gr = (int64_t)sbr * 32 + r, gc = (int64_t)sbc * 32 + tx;
    double v = 0.0;
    if (gr < n && gc < n && gc <= gr) v = (double)A[gr * lda + gc];
    t[r][tx] = v;
  }
  __syncthreads();
  for (int ii = ty; ii < 32; ii += 8) {
    const int64_t i = (int64_t)bi * 32 + ii, j = (int64_t)bj * 32 + tx;
    if (i >= n || j >= n) continue;
    double v;
    if (bi > bj) v = t[ii][tx];
    else if (bi < bj) v = t[tx][ii];
    else v = ii >= tx ? t[ii][tx] : t[tx][ii];
    X[i * n + j] = v;
  }
}

// D = W - s (.) V in float64.
template <typename R>
__global__ __launch_bounds__(256) void residual_kernel(int64_t m, int64_t n, const R* __restrict__ W,
                                                       int64_t ldw, const int32_t* __restrict__ V,
                                                       int64_t ldv, int scale_mode,
                                                       const R* __restrict__ scales,
                                                       double* __restrict__ D,
                                                       ResidualStrides st) {
  {  // problem blockIdx.z of a batch
    const int64_t b = blockIdx.z;
    W += b * st.w;
    V += b * st.v;
    if (scales) scales += b * st.s;
    D += b * st.d;
  }
  const int64_t i = blockIdx.y;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < n; j += (int64_t)gridDim.x * 256) {
    double s = 1.0;
    if (scale_mode == 1) s = (double)scales[i];
    else if (scale_mode == 2) s = (double)scales[j];
    D[i * n + j] = (double)W[i * ldw + j] - s * (double)V[i * ldv + j];
  }
}

// out = sum of partial[0..count), in a fixed order (deterministic).
__global__ __launch_bounds__(256) void sum_partials_kernel(const double* __restrict__ partial,
                                                           int64_t count, double* __restrict__ out,
                                                           int64_t sPart) {
  __shared__ double red[256];
  partial += (int64_t)blockIdx.x * sPart;  // problem blockIdx.x of a batch
  out += blockIdx.x;
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < count; i += 256) s += partial[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

template <typename R>
__global__ __launch_bounds__(256) void row_scales_kernel(int64_t n, const R* __restrict__ W,
                                                         int64_t ldw, R hi, R* __restrict__ s) {
  __shared__ R red[256];
  const int64_t i = blockIdx.x;
  R mx = R(0);
  for (int64_t j = threadIdx.x; j < n; j += 256) {
    const R v = W[i * ldw + j];
    const R a = v < R(0) ? -v : v;
    mx = a > mx ? a : mx;
  }
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = red[threadIdx.x] > red[threadIdx.x + w] ? red[threadIdx.x] : red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) s[i] = red[0] == R(0) ? R(1) : red[0] / hi;
}

// ---------------------------------------------------------------------------
template <typename R>
hipError_t launch_sym_to_f64(int64_t n, const R* A, int64_t lda, double* X, hipStream_t s,
                             int batch, int64_t sA, int64_t sX) {
  if (n <= 0 || batch <= 0) return hipSuccess;
  const unsigned nb = (unsigned)((n + 31) / 32);
  hipLaunchKernelGGL((sym_to_f64_kernel<R>), dim3(nb, nb, (unsigned)batch), dim3(256), 0, s, n, A,
                     lda, X, sA, sX);
  return hipGetLastError();
}

template <typename R>
hipError_t launch_residual_f64(int64_t m, int64_t n, const R* W, int64_t ldw, const int32_t* V,
                               int64_t ldv, int scale_mode, const R* scales, double* D,
                               hipStream_t s, int batch, ResidualStrides st) {
  if (m <= 0 || n <= 0 || batch <= 0) return hipSuccess;
  unsigned gx = (unsigned)((n + 255) / 256);
  if (gx > 64) gx = 64;
  hipLaunchKernelGGL((residual_kernel<R>), dim3(gx, (unsigned)m, (unsigned)batch), dim3(256), 0, s,
                     m, n, W, ldw, V, ldv, scale_mode, scales, D, st);
  return hipGetLastError();
}

hipError_t launch_sum_partials(const double* partial, int64_t count, double* out, hipStream_t s,
                               int batch, int64_t sPart) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(sum_partials_kernel, dim3((unsigned)batch), dim3(256), 0, s, partial, count,
                     out, sPart);
  return hipGetLastError();
}

template <typename R>
hipError_t launch_row_scales(int64_t m, int64_t n, const R* W, int64_t ldw, int32_t hi, R* s_out,
                             hipStream_t s) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL((row_scales_kernel<R>), dim3((unsigned)m), dim3(256), 0, s, n, W, ldw, (R)hi,
                     s_out);
  return hipGetLastError();
}

#define BK_INST(R)                                                                               \
  template hipError_t launch_sym_to_f64<R>(int64_t, const R*, int64_t, double*, hipStream_t,    \
                                           int, int64_t, int64_t);                               \
  template hipError_t launch_residual_f64<R>(int64_t, int64_t, const R*, int64_t, const int32_t*, \
                                             int64_t, int, const R*, double*, hipStream_t, int,  \
                                             ResidualStrides);                                   \
  template hipError_t launch_row_scales<R>(int64_t, int64_t, const R*, int64_t, int32_t, R*,     \
                                           hipStream_t);
BK_INST(float)
BK_INST(double)
#undef BK_INST

}  // namespace bk
