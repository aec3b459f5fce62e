// Elementwise steps of the second block variant (CS336 pretraining page,
// sections 4 and 6: RoPE on Q and K, a SwiGLU feed-forward), HBM-bound: each
// thread takes four consecutive channels of one row (one 8- or 16-byte load
// and store per operand), arithmetic in fp32.
//
// RoPE rotates channel pairs (2i, 2i+1) of each head by t * theta^(-2i/D) at
// position t: (a, b) -> (a cos - b sin, a sin + b cos); the backward applies
// the transpose (the rotation by minus the angle) to the gradient.
// SwiGLU: h = silu(g) * u with silu(g) = g / (1 + e^-g); its backward is
// dg = dh * u * silu'(g), du = dh * silu(g), silu'(g) = s (1 + g (1 - s)) with
// s the logistic of g.
#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(T* __restrict__ qkv, int rows, int C, int Tn, int D,
                                                   const float2* __restrict__ tab, int inverse) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // group of 4 channels of q | k
  const int per_row = (2 * C) >> 2;
  if (i >= (int64_t)rows * per_row) return;
  const int row = (int)(i / per_row), c = (int)(i % per_row) * 4;  // c in [0, 2C): q then k
  const int d = c % D, t = row % Tn;
  T* p = qkv + (int64_t)row * 3 * C + c;
  const float4 v = load4(p);
  const float2 r0 = tab[(int64_t)t * (D >> 1) + (d >> 1)], r1 = tab[(int64_t)t * (D >> 1) + (d >> 1) + 1];
  const float s0 = inverse ? -r0.y : r0.y, s1 = inverse ? -r1.y : r1.y;
  store4(p, make_float4(v.x * r0.x - v.y * s0, v.x * s0 + v.y * r0.x, v.z * r1.x - v.w * s1, v.z * s1 + v.w * r1.x));
}

__device__ __forceinline__ float logistic(float g) { return __builtin_amdgcn_rcpf(1.f + hw_exp2(-g * LOG2E)); }

template <typename T>
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const T* __restrict__ u, T* __restrict__ h, int rows, int F) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = F >> 2;
  if (i >= (int64_t)rows * per_row) return;
  const int row = (int)(i / per_row), c = (int)(i % per_row) * 4;
  const T* ur = u + (int64_t)row * 2 * F;
  const float4 g = load4(ur + c), up = load4(ur + F + c);
  store4(h + (int64_t)row * F + c, make_float4(g.x * logistic(g.x) * up.x, g.y * logistic(g.y) * up.y,
                                               g.z * logistic(g.z) * up.z, g.w * logistic(g.w) * up.w));
}

template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const T* __restrict__ u, const T* __restrict__ dh,
                                                         T* __restrict__ du, int rows, int F) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = F >> 2;
  if (i >= (int64_t)rows * per_row) return;
  const int row = (int)(i / per_row), c = (int)(i % per_row) * 4;
  const T* ur = u + (int64_t)row * 2 * F;
  const float4 g = load4(ur + c), up = load4(ur + F + c), d = load4(dh + (int64_t)row * F + c);
  float gs[4] = {g.x, g.y, g.z, g.w}, us[4] = {up.x, up.y, up.z, up.w}, ds[4] = {d.x, d.y, d.z, d.w};
  float dg[4], dup[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float sg = logistic(gs[k]);
    dg[k] = ds[k] * us[k] * sg * (1.f + gs[k] * (1.f - sg));
    dup[k] = ds[k] * gs[k] * sg;
  }
  T* o = du + (int64_t)row * 2 * F;
  store4(o + c, make_float4(dg[0], dg[1], dg[2], dg[3]));
  store4(o + F + c, make_float4(dup[0], dup[1], dup[2], dup[3]));
}

}  // namespace

hipError_t rope_qk(int dtype, void* qkv, int rows, int C, int Tn, int D, const float2* tab, int inverse,
                   hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (C % 4 || D % 4 || C % D || Tn <= 0) return hipErrorInvalidValue;
  const int64_t n = (int64_t)rows * (2 * C / 4);
  const dim3 grid((unsigned)cdiv(n, 256));
  if (dtype == BF16)
    hipLaunchKernelGGL(rope_kernel<bf16>, grid, dim3(256), 0, s, (bf16*)qkv, rows, C, Tn, D, tab, inverse);
  else
    hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(256), 0, s, (float*)qkv, rows, C, Tn, D, tab, inverse);
  return hipGetLastError();
}

hipError_t swiglu_fwd(int dtype, const void* u, void* h, int rows, int F, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (F % 4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)cdiv((int64_t)rows * (F / 4), 256));
  if (dtype == BF16)
    hipLaunchKernelGGL(swiglu_fwd_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)u, (bf16*)h, rows, F);
  else
    hipLaunchKernelGGL(swiglu_fwd_kernel<float>, grid, dim3(256), 0, s, (const float*)u, (float*)h, rows, F);
  return hipGetLastError();
}

hipError_t swiglu_bwd(int dtype, const void* u, const void* dh, void* du, int rows, int F, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (F % 4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)cdiv((int64_t)rows * (F / 4), 256));
  if (dtype == BF16)
    hipLaunchKernelGGL(swiglu_bwd_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)u, (const bf16*)dh, (bf16*)du,
                       rows, F);
  else
    hipLaunchKernelGGL(swiglu_bwd_kernel<float>, grid, dim3(256), 0, s, (const float*)u, (const float*)dh,
                       (float*)du, rows, F);
  return hipGetLastError();
}

}  // namespace gk
