// Float64 MFMA GEMM for the factorisation and the loss (gfx950).
//
// C = alpha * A * op(B) + beta * C over 64 x 64 output blocks, 256 threads in
// four waves (2 x 2), each wave a 32 x 32 sub-block of 2 x 2
// v_mfma_f64_16x16x4 blocks; K advances 16 at a time through double-buffered
// LDS. Options: only lower output blocks (symmetric rank-k update), A lower
// triangular (K ends with the row block), B lower triangular (K ends with the
// column block when op(B) = B^T, starts with it when op(B) = B), a batch of
// two independent problems of one shape (grid z), and a dot epilogue that
// reduces sum(C_block .* D_block) per block instead of storing C (loss).
#include "device.hpp"
#include "launch.hpp"

namespace bk {

namespace {
constexpr int GB = 64;  // block edge
constexpr int GK = 16;  // K step
constexpr int GLD = GK + 2;
}  // namespace

__global__ __launch_bounds__(256) void gemm64_kernel(Gemm64Args a) {
  typedef Mfma<double> MF;
  typedef MF::acc_t acc_t;
  __shared__ double As[2][GB][GLD];
  __shared__ double Bs[2][GB][GLD];
  __shared__ double red[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int r16 = lane & 15, kg = lane >> 4;
  const int64_t bm = blockIdx.y, bn = blockIdx.x;
  const int z = blockIdx.z;
  const double* __restrict__ Ap = a.A[z];
  const double* __restrict__ Bp = a.B[z];
  double* Cp = a.C[z];
  const int64_t row0 = bm * GB, col0 = bn * GB;
  const bool skip = a.lower_out && bn > bm;

  acc_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = MF::zero();

  int64_t kend = a.K, kbeg = 0;
  if (a.a_lower && row0 + GB < kend) kend = row0 + GB;
  if (a.b_lower) {
    if (a.transB) {
      if (col0 + GB < kend) kend = col0 + GB;
    } else {
      kbeg = col0;
    }
  }

  double ra[4], rb[4];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = u * 256 + tid;
      {  // A tile: 64 rows x 16 k
        const int r = e / GK, c = e % GK;
        const int64_t gr = row0 + r, gk = k0 + c;
        ra[u] = (gr < a.M && gk < kend && gk >= kbeg) ? Ap[gr * a.lda + gk] : 0.0;
      }
      if (a.transB) {  // B is N x K
        const int r = e / GK, c = e % GK;
        const int64_t gn = col0 + r, gk = k0 + c;
        rb[u] = (gn < a.N && gk < kend && gk >= kbeg) ? Bp[gn * a.ldb + gk] : 0.0;
      } else {  // B is K x N
        const int kr = e / GB, cc = e % GB;
        const int64_t gk = k0 + kr, gn = col0 + cc;
        rb[u] = (gn < a.N && gk < kend && gk >= kbeg) ? Bp[gk * a.ldb + gn] : 0.0;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = u * 256 + tid;
      As[buf][e / GK][e % GK] = ra[u];
      if (a.transB) Bs[buf][e / GK][e % GK] = rb[u];
      else Bs[buf][e % GB][e / GB] = rb[u];
    }
  };

  if (!skip && kend > kbeg) {
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
        double af[2], bf[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = As[buf][wr * 32 + i * 16 + r16][4 * kg + st];
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = Bs[buf][wc * 32 + j * 16 + r16][4 * kg + st];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = MF::mma(af[i], bf[j], acc[i][j]);
      }
      if (it + 1 < nk) sstore(buf ^ 1);
      __syncthreads();
    }
  }

  if (a.dot[0]) {
    double part = 0.0;
    if (!skip) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t gr = row0 + wr * 32 + i * 16 + MF::row(lane, r);
            const int64_t gc = col0 + wc * 32 + j * 16 + r16;
            if (gr < a.M && gc < a.N) part += a.alpha * acc[i][j][r] * a.dot[z][gr * a.lddot + gc];
          }
    }
    // fixed-order reduction: wave butterfly, then the four waves in order
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (lane == 0) red[wave] = part;
    __syncthreads();
    if (tid == 0) a.partial[z][bm * gridDim.x + bn] = ((red[0] + red[1]) + red[2]) + red[3];
    return;
  }
  if (skip) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t gr = row0 + wr * 32 + i * 16 + MF::row(lane, r);
        const int64_t gc = col0 + wc * 32 + j * 16 + r16;
        if (gr < a.M && gc < a.N) {
          double v = a.alpha * acc[i][j][r];
          if (a.beta != 0.0) v += a.beta * Cp[gr * a.ldc + gc];
          Cp[gr * a.ldc + gc] = v;
        }
      }
}

int64_t gemm64_num_blocks(int64_t M, int64_t N) {
  return ((M + GB - 1) / GB) * ((N + GB - 1) / GB);
}

hipError_t launch_gemm64(const Gemm64Args& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.batch < 1 || a.batch > 2) return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.N + GB - 1) / GB), (unsigned)((a.M + GB - 1) / GB), (unsigned)a.batch);
  hipLaunchKernelGGL(gemm64_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bk
