// Device helpers for the gfx950 BaKron kernels: MFMA wrappers, the
// quantizer, and the tiled workspace addressing shared by the solve kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bk {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v4d __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// 16x16x4 MFMA, float and double. Operand layout (both types): lane l holds
// A[l % 16][l / 16] and B[l / 16][l % 16]. Result: lane l, register r holds
// D[row][l % 16] with row = 4*(l/16) + r for float and row = l/16 + 4*r for
// double (measured on gfx950).
// ---------------------------------------------------------------------------
template <typename R> struct Mfma;

template <> struct Mfma<float> {
  typedef v4f acc_t;
  __device__ static inline acc_t zero() { return acc_t{0.f, 0.f, 0.f, 0.f}; }
  __device__ static inline acc_t mma(float a, float b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline int row(int lane, int r) { return 4 * (lane >> 4) + r; }
};

template <> struct Mfma<double> {
  typedef v4d acc_t;
  __device__ static inline acc_t zero() { return acc_t{0.0, 0.0, 0.0, 0.0}; }
  __device__ static inline acc_t mma(double a, double b, acc_t c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  __device__ static inline int row(int lane, int r) { return (lane >> 4) + 4 * r; }
};

// ---------------------------------------------------------------------------
// Quantizer (§3.1 of the BaKron paper: closest alphabet element after scaling).
// c = clamp(rint(x / s), lo, hi); rint rounds half to even. True division.
// ---------------------------------------------------------------------------
__device__ inline float quant_code(float x, float s, float lo, float hi, bool unbounded) {
  float c = __builtin_rintf(x / s);
  if (!unbounded) c = fminf(fmaxf(c, lo), hi);
  return c;
}
__device__ inline double quant_code(double x, double s, double lo, double hi, bool unbounded) {
  double c = __builtin_rint(x / s);
  if (!unbounded) c = fmin(fmax(c, lo), hi);
  return c;
}

// ---------------------------------------------------------------------------
// Tiled workspace addressing. W is held as Mt x Nt tiles of T x T elements,
// tile (P, Q) contiguous and row-major inside. Normalised factors are held as
// packed lower-triangular tile arrays: tile (P, I), I <= P, at P(P+1)/2 + I.
// ---------------------------------------------------------------------------
__host__ __device__ inline int64_t tri_index(int64_t P, int64_t I) { return P * (P + 1) / 2 + I; }

}  // namespace bk
