// Shared device helpers for the gfx950 kernels: element types, 16-byte
// fragments, MFMA wrappers, hardware exp2/log2, wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define WAVE 64

// Elements of T in one 16-byte fragment, and the K span one fragment covers
// in the 16x16 MFMA family: bf16 -> 8 elements, one 16x16x32 op (k = 32);
// fp32 -> 4 elements, four 16x16x4 ops (k = 16).
template <typename T> struct Tr;
template <> struct Tr<float> {
  static constexpr int E = 4;
  static constexpr int KFRAG = 16;
};
template <> struct Tr<bf16> {
  static constexpr int E = 8;
  static constexpr int KFRAG = 32;
};

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& v) {
  static_assert(sizeof(To) == sizeof(From), "size");
  return __builtin_bit_cast(To, v);
}

// acc[16x16] += A_frag . B_frag over the fragment's k span.  Lane l holds row
// (l % 16) of A and column (l % 16) of B, k elements (l / 16) * E .. + E - 1;
// acc lane layout: rows (l / 16) * 4 + r, column l % 16.
__device__ __forceinline__ void mfma_frag(f32x4& acc, const uint4& a, const uint4& b, bf16) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_frag(f32x4& acc, const uint4& a, const uint4& b, float) {
  // The 4 k elements a lane holds feed four 16x16x4 ops; in op j the lane's
  // k slot (l / 16) carries element j.  A and B use the same assignment.
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// Hardware transcendental units (v_exp_f32 = 2^x, v_log_f32 = log2 x).
#define LOG2E 1.4426950408889634f
#define LN2 0.6931471805599453f
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_exp(float x) { return hw_exp2(x * LOG2E); }

// tanh from its definition through e^(2x): tanh x = 1 - 2 / (e^(2x) + 1), with
// the hardware reciprocal (v_rcp_f32, 1 ulp); e = inf gives rcp = 0, tanh = 1.
__device__ __forceinline__ float tanh_exp(float x) {
  float e = hw_exp2(x * (2.0f * LOG2E));
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

// tanh-approximate GELU and its derivative (Hendrycks & Gimpel 2016).
#define GELU_K 0.7978845608028654f  // sqrt(2/pi)
#define GELU_A 0.044715f
__device__ __forceinline__ float gelu_f(float u) {
  float t = tanh_exp(GELU_K * (u + GELU_A * u * u * u));
  return 0.5f * u * (1.0f + t);
}
__device__ __forceinline__ float gelu_grad_f(float u) {
  float t = tanh_exp(GELU_K * (u + GELU_A * u * u * u));
  float dt = GELU_K * (1.0f + 3.0f * GELU_A * u * u);
  return 0.5f * (1.0f + t) + 0.5f * u * (1.0f - t * t) * dt;
}
// both from one exponential: with x = K (u + A u^3), 0.5 (1 + tanh x) is the
// logistic h = 1 / (1 + e^(-2x)), so g = u h and, since 1 - tanh^2 = 4 h (1 - h),
// dg = h + u h (1 - h) 2 x'(u) = h (1 + u (1 - h) 2K (1 + 3 A u^2)).
// e = inf (u very negative) gives h = 0, g = -0, dg = 0; e = 0 gives h = 1.
__device__ __forceinline__ void gelu_both(float u, float& g, float& dg) {
  constexpr float C1 = -2.0f * LOG2E * GELU_K, C2 = C1 * GELU_A;
  const float u2 = u * u;
  const float e = hw_exp2(u * __builtin_fmaf(C2, u2, C1));
  const float h = __builtin_amdgcn_rcpf(1.0f + e);
  g = u * h;
  const float dx = __builtin_fmaf(6.0f * GELU_A * GELU_K, u2, 2.0f * GELU_K);
  dg = __builtin_fmaf(h, u * (1.0f - h) * dx, h);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// Load / store 4 consecutive elements as fp32.
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const bf16* p) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}
__device__ __forceinline__ void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ void store4(bf16* p, float4 v) {
  bf16x4 o;
  o[0] = (bf16)v.x; o[1] = (bf16)v.y; o[2] = (bf16)v.z; o[3] = (bf16)v.w;
  *reinterpret_cast<bf16x4*>(p) = o;
}

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
