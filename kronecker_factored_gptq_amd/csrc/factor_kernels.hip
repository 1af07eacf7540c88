// Factor kernels (float64) for gfx950.
//
// The solver needs L = Cholesky(A^-1) with columns divided by their
// diagonal ("BaKron: Efficient Quantization with Kronecker-Factored
// Hessians", arXiv 2608.06291, §3.2 Algorithm 2, first two steps; Cholesky
// and RevCholesky as defined in §3.1). We never form A^-1: with J the
// reversal permutation and C = Cholesky(J A J), A = (J C J)(J C J)^T, so
// A^-1 = (J C^-T J)(J C^-T J)^T and J C^-T J is lower triangular with a
// positive diagonal, i.e. it IS Cholesky(A^-1). Steps:
//   X = J A J (lower triangle)      load_reversed_kernel
//   X = Cholesky(X) in place        blocked, right-looking, 64-wide panels:
//                                   diag block in LDS (+ its inverse),
//                                   panel = A21 * inv(L11)^T, trailing
//                                   rank-64 update on MFMA (gemm64)
//   X = X^-1 in place               blocked from the bottom block up:
//                                   X21 = -X22^-1 X21 inv(X11) (gemm64)
//   L[i][j] = Y[n-1-j][n-1-i], normalised by its diagonal  store_normalized
#include <climits>

#include "device.hpp"
#include "launch.hpp"

namespace bk {

namespace {
constexpr int NB = 64;  // Cholesky panel width
}

// X[i][j] = A[n-1-j][n-1-i] for i >= j (the lower triangle of J A J read from
// the lower triangle of A), 0 above the diagonal. 32 x 32 tiles through LDS.
template <typename R>
__global__ __launch_bounds__(256) void load_reversed_kernel(int64_t n, const R* __restrict__ A,
                                                            int64_t lda, double* __restrict__ X) {
  __shared__ double tile[32][33];
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

// Cholesky of the bs x bs diagonal block at (kb, kb) in LDS, plus its
// lower-triangular inverse. A pivot that is not positive and finite records
// kb + j in *info (smallest wins) and the factorisation continues with NaN.
__global__ __launch_bounds__(256) void potrf_diag_kernel(int64_t n, int64_t kb, int bs,
                                                         double* __restrict__ X,
                                                         double* __restrict__ Dinv,
                                                         int32_t* __restrict__ info) {
  __shared__ double L[NB][NB + 1];
  __shared__ double Y[NB][NB + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e < NB * NB; e += 256) {
    const int r = e / NB, c = e % NB;
    double v = 0.0;
    if (r < bs && c <= r) v = X[(kb + r) * n + kb + c];
    L[r][c] = v;
    Y[r][c] = 0.0;
  }
  __syncthreads();
  for (int j = 0; j < bs; ++j) {
    if (tid == 0) {
      const double piv = L[j][j];
      if (!(piv > 0.0) || !(piv < INFINITY)) {
        atomicMin(info, (int32_t)(kb + j));
        L[j][j] = __builtin_nan("");
      } else {
        L[j][j] = __builtin_sqrt(piv);
      }
    }
    __syncthreads();
    const double djj = L[j][j];
    for (int i = j + 1 + tid; i < bs; i += 256) L[i][j] /= djj;
    __syncthreads();
    // trailing update of the block: L[i][c] -= L[i][j] L[c][j], j < c <= i
    const int rem = bs - j - 1;
    for (int e = tid; e < rem * rem; e += 256) {
      const int i = j + 1 + e / rem, c = j + 1 + e % rem;
      if (c <= i) L[i][c] -= L[i][j] * L[c][j];
    }
    __syncthreads();
  }
  // inverse of the lower-triangular L: column c by thread c
  if (tid < bs) {
    const int c = tid;
    Y[c][c] = 1.0 / L[c][c];
    for (int r = c + 1; r < bs; ++r) {
      double sum = 0.0;
      for (int k = c; k < r; ++k) sum += L[r][k] * Y[k][c];
      Y[r][c] = -sum / L[r][r];
    }
  }
  __syncthreads();
  for (int e = tid; e < NB * NB; e += 256) {
    const int r = e / NB, c = e % NB;
    if (r < bs && c < bs) {
      if (c <= r) X[(kb + r) * n + kb + c] = L[r][c];
      Dinv[kb * NB + r * NB + c] = c <= r ? Y[r][c] : 0.0;
    }
  }
}

// Copy the stored inverse of diagonal block (kb, kb) into X (upper part 0).
__global__ __launch_bounds__(256) void put_diag_inverse_kernel(int64_t n, int64_t kb, int bs,
                                                               double* __restrict__ X,
                                                               const double* __restrict__ Dinv) {
  for (int e = threadIdx.x; e < bs * bs; e += 256) {
    const int r = e / bs, c = e % bs;
    X[(kb + r) * n + kb + c] = c <= r ? Dinv[kb * NB + r * NB + c] : 0.0;
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
                                                               R* __restrict__ L, int64_t ldl,
                                                               R* __restrict__ d) {
  __shared__ double tile[32][33];
  __shared__ double diag[32];
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
hipError_t launch_load_reversed(int64_t n, const R* A, int64_t lda, double* X, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned nb = (unsigned)((n + 31) / 32);
  hipLaunchKernelGGL((load_reversed_kernel<R>), dim3(nb, nb), dim3(256), 0, s, n, A, lda, X);
  return hipGetLastError();
}

template <typename R>
hipError_t launch_store_normalized(int64_t n, const double* Y, R* L, int64_t ldl, R* d,
                                   hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned nb = (unsigned)((n + 31) / 32);
  hipLaunchKernelGGL((store_normalized_kernel<R>), dim3(nb, nb), dim3(256), 0, s, n, Y, L, ldl,
                     d);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t count, int32_t v, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, p,
                     count, v);
  return hipGetLastError();
}

// Cholesky then triangular inverse of the n x n lower triangle of X, in place.
// Dinv: (ceil(n/64) * 64) x 64 scratch for the diagonal-block inverses;
// Tmp: n x 64 scratch. info must hold INT_MAX on entry.
hipError_t factor_cholesky_inverse(int64_t n, double* X, double* Dinv, double* Tmp,
                                   int32_t* info, hipStream_t s) {
  hipError_t err;
  for (int64_t kb = 0; kb < n; kb += NB) {
    const int bs = (int)((n - kb) < NB ? (n - kb) : NB);
    hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(256), 0, s, n, kb, bs, X, Dinv, info);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t r0 = kb + bs, nr = n - r0;
    if (nr <= 0) break;
    // panel: X[r0:, kb:kb+bs] = X[r0:, kb:kb+bs] * inv(L11)^T. In place is
    // safe: one 64-wide output column block, and each block reads its rows of
    // A completely (K = bs <= 64) before it writes them.
    Gemm64Args p{};
    p.M = nr; p.N = bs; p.K = bs;
    p.A = X + r0 * n + kb; p.lda = n;
    p.B = Dinv + kb * NB; p.ldb = NB; p.transB = 1;
    p.C = X + r0 * n + kb; p.ldc = n;
    p.alpha = 1.0; p.beta = 0.0;
    if ((err = launch_gemm64(p, s)) != hipSuccess) return err;
    // trailing: X[r0:, r0:] -= P P^T, lower 64-blocks only
    Gemm64Args t{};
    t.M = nr; t.N = nr; t.K = bs;
    t.A = X + r0 * n + kb; t.lda = n;
    t.B = X + r0 * n + kb; t.ldb = n; t.transB = 1;
    t.C = X + r0 * n + r0; t.ldc = n;
    t.alpha = -1.0; t.beta = 1.0; t.lower_out = 1;
    if ((err = launch_gemm64(t, s)) != hipSuccess) return err;
  }
  // triangular inverse, bottom block first
  const int64_t nblk = (n + NB - 1) / NB;
  for (int64_t jb = nblk - 1; jb >= 0; --jb) {
    const int64_t kb = jb * NB;
    const int bs = (int)((n - kb) < NB ? (n - kb) : NB);
    const int64_t r0 = kb + bs, nr = n - r0;
    if (nr > 0) {
      // Tmp = X22^-1 (already in place, lower) * X21
      Gemm64Args g1{};
      g1.M = nr; g1.N = bs; g1.K = nr;
      g1.A = X + r0 * n + r0; g1.lda = n; g1.a_lower = 1;
      g1.B = X + r0 * n + kb; g1.ldb = n; g1.transB = 0;
      g1.C = Tmp; g1.ldc = NB;
      g1.alpha = 1.0; g1.beta = 0.0;
      if ((err = launch_gemm64(g1, s)) != hipSuccess) return err;
      // X21 = -Tmp * inv(X11)
      Gemm64Args g2{};
      g2.M = nr; g2.N = bs; g2.K = bs;
      g2.A = Tmp; g2.lda = NB;
      g2.B = Dinv + kb * NB; g2.ldb = NB; g2.transB = 0;
      g2.C = X + r0 * n + kb; g2.ldc = n;
      g2.alpha = -1.0; g2.beta = 0.0;
      if ((err = launch_gemm64(g2, s)) != hipSuccess) return err;
    }
    hipLaunchKernelGGL(put_diag_inverse_kernel, dim3(1), dim3(256), 0, s, n, kb, bs, X, Dinv);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

template hipError_t launch_load_reversed<float>(int64_t, const float*, int64_t, double*, hipStream_t);
template hipError_t launch_load_reversed<double>(int64_t, const double*, int64_t, double*, hipStream_t);
template hipError_t launch_store_normalized<float>(int64_t, const double*, float*, int64_t, float*, hipStream_t);
template hipError_t launch_store_normalized<double>(int64_t, const double*, double*, int64_t, double*, hipStream_t);

}  // namespace bk
