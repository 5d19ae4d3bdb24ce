// Shared device/host definitions of the gptmi kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define GPT_WAVE 64

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// Butterfly reductions across the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// The RoPE (cos, sin) table [T][D / 2], written by a kernel that runs anyway
// before its readers (cs == nullptr: none).  Entry (t, i) is the angle
// t * theta_i, theta_i = base^(-2i/D) (given in double), formed and reduced
// to [-pi, pi] in double, then the float sincos of the residue: a few ulp
// at any position.
constexpr int ROPE_MAX_HALF = 64;
struct RopeJob {
  float2* cs;
  int T, half;
  double theta[ROPE_MAX_HALF];
};
__device__ __forceinline__ float2 rope_entry(const RopeJob& rj, int e) {
  constexpr double TWO_PI = 6.283185307179586476925286766559;
  const int t = e / rj.half, i = e - t * rj.half;
  const double a = (double)t * rj.theta[i];
  const float r = (float)(a - TWO_PI * rint(a * (1.0 / TWO_PI)));
  float sn, c;
  sincosf(r, &sn, &c);
  return make_float2(c, sn);
}

// Vector of 8 storage elements converted to/from fp32.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float* f) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16* p, const float* f) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)f[i];
    *reinterpret_cast<bf16x8*>(p) = v;
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* f) {
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* f) {
    reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
};

// erf(x) by Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26:
// erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
// t = 1 / (1 + p x) for x >= 0 (odd extension), |error| <= 1.5e-7.
// Inline arithmetic (one exp, one reciprocal) so GEMM epilogues make no
// calls; e receives exp(-x^2).
__device__ __forceinline__ float erf_as(float x, float& e) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  e = __expf(-ax * ax);
  return copysignf(fmaf(-poly, e, 1.0f), x);
}

// GELU with the exact (erf) form, g = u Phi(u), and its derivative
// dg = Phi(u) + u phi(u), from one erf evaluation: with x = u / sqrt 2 the
// exponential of the erf formula is exp(-u^2 / 2) = sqrt(2 pi) phi(u).
__device__ __forceinline__ void gelu_and_grad(float u, float& g, float& dg) {
  float e;
  const float cdf = 0.5f * (1.0f + erf_as(u * 0.70710678118654752f, e));
  g = u * cdf;
  dg = fmaf(u, e * 0.39894228040143268f, cdf);
}

static inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
