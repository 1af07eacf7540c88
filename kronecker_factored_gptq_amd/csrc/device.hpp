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
// Quantizer (§3.1 of the BaKron paper: closest alphabet element after
// scaling), applied in code units, i.e. to u = x / s, which the solve keeps
// directly: c = clamp(rint(u), lo, hi), rint rounding half to even, with
// lo = -inf, hi = +inf for the unbounded alphabet.
// ---------------------------------------------------------------------------
__device__ inline float fmin_(float a, float b) { return fminf(a, b); }
__device__ inline float fmax_(float a, float b) { return fmaxf(a, b); }
__device__ inline double fmin_(double a, double b) { return fmin(a, b); }
__device__ inline double fmax_(double a, double b) { return fmax(a, b); }
__device__ inline float quant_unit(float u, float lo, float hi) {
  return fminf(fmaxf(__builtin_rintf(u), lo), hi);
}
__device__ inline double quant_unit(double u, double lo, double hi) {
  return fmin(fmax(__builtin_rint(u), lo), hi);
}

// ---------------------------------------------------------------------------
// Tiled workspace addressing. W is held as Mt x Nt tiles of T x T elements,
// tile (P, Q) contiguous and row-major inside. Normalised factors are held as
// packed lower-triangular tile arrays: tile (P, I), I <= P, at P(P+1)/2 + I.
// ---------------------------------------------------------------------------
__host__ __device__ inline int64_t tri_index(int64_t P, int64_t I) { return P * (P + 1) / 2 + I; }

}  // namespace bk
