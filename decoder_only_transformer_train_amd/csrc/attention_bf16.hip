// Causal flash attention for bf16, head size 64, on gfx950 32x32x16 MFMAs.
//
// Same method as the fp32 kernels in attention.hip (online softmax over
// 64-key blocks, log-sum-exp saved for a recomputing backward, dK/dV and dQ
// in separate atomic-free kernels), laid out for the 32x32 MFMA:
//  * The forward and dQ kernels give a workgroup a 256-query block; wave w
//    owns the 32-row tiles w and 7 - w of it, so every wave has one early and
//    one late tile and the causal work is balanced.  The dK/dV kernel gives
//    a workgroup 128 keys, one 32-key tile per wave.
//  * Scores are computed in the orientation whose C tile feeds the next
//    product as its B operand: lane l of a 32x32 C tile holds column l % 32
//    and rows (e / 4) * 8 + (l / 32) * 4 + e % 4, e = 0..15; the 8 values of
//    one 16-row half are exactly a 32x32x16 B fragment when the A operand
//    reads the matching rows of a transposed LDS tile (two 8-byte reads).
//  * Transposed LDS tiles are written from registers after a 4x8 transpose,
//    so every LDS store is 8 bytes wide.
#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int HD = 64;                 // head size
constexpr int PR = HD * 2 + 16;        // pitch (bytes) of a row tile [64][64]
constexpr int PT = 64 * 2 + 16;        // pitch (bytes) of a transposed tile [64 d][64 rows]
constexpr float NEG_INF = -__builtin_huge_valf();

__device__ __forceinline__ void mma32(f32x16& c, const uint4& a, const uint4& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0, 0, 0);
}
__device__ __forceinline__ void zero16(f32x16& c) {
#pragma unroll
  for (int e = 0; e < 16; ++e) c[e] = 0.f;
}
// row offset (within a 32-row C tile) of accumulator e for lane group g
__device__ __forceinline__ int crow(int e, int g) { return (e >> 2) * 8 + g * 4 + (e & 3); }

// rows [row0, row0 + 64) x 64 of a [T][ld] operand into a row tile (pitch PR)
__device__ __forceinline__ void load_rows(const bf16* __restrict__ gsrc, int64_t ld, int row0, int nvalid, char* s,
                                          int t) {
  for (int i = t; i < 512; i += 256) {
    const int r = i >> 3, c = i & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row0 + r < nvalid) v = *reinterpret_cast<const uint4*>(gsrc + (int64_t)(row0 + r) * ld + c * 8);
    *reinterpret_cast<uint4*>(s + r * PR + c * 16) = v;
  }
}
// the same rows into a transposed tile [64 d][64 rows] (pitch PT): a unit is
// 4 rows x 8 columns, transposed in registers into 8 rows of 4 (8 bytes)
__device__ __forceinline__ void load_trans(const bf16* __restrict__ gsrc, int64_t ld, int row0, int nvalid, char* s,
                                           int t) {
  if (t >= 128) return;
  const int rg = t >> 3, dc = t & 7;
  uint4 r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + rg * 4 + i;
    r[i] = (row < nvalid) ? *reinterpret_cast<const uint4*>(gsrc + (int64_t)row * ld + dc * 8) : make_uint4(0, 0, 0, 0);
  }
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int wi = e >> 1;
    uint32_t lo, hi;
    if (e & 1) {
      lo = (w0[wi] >> 16) | (w1[wi] & 0xFFFF0000u);
      hi = (w2[wi] >> 16) | (w3[wi] & 0xFFFF0000u);
    } else {
      lo = (w0[wi] & 0xFFFFu) | (w1[wi] << 16);
      hi = (w2[wi] & 0xFFFFu) | (w3[wi] << 16);
    }
    *reinterpret_cast<uint2*>(s + (dc * 8 + e) * PT + rg * 8) = make_uint2(lo, hi);
  }
}
// 32x32x16 operand fragment of row `row` of a row tile, k step kk (d = kk*16 ..)
__device__ __forceinline__ uint4 frag_row(const char* s, int row, int kk, int g) {
  return *reinterpret_cast<const uint4*>(s + row * PR + kk * 32 + g * 16);
}
// fragment of row `row` of a transposed tile over the 16-row run hh:
// slots 0-3 = rows 16 hh + 4 g + j, slots 4-7 = rows 16 hh + 8 + 4 g + j
__device__ __forceinline__ uint4 frag_tr(const char* s, int row, int hh, int g) {
  const char* p = s + row * PT;
  const uint2 lo = *reinterpret_cast<const uint2*>(p + (16 * hh + 4 * g) * 2);
  const uint2 hi = *reinterpret_cast<const uint2*>(p + (16 * hh + 8 + 4 * g) * 2);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}
// B fragment from half hh of a 32x32 C tile (accumulators 8 hh .. 8 hh + 7),
// whose slot order matches frag_tr
__device__ __forceinline__ uint4 pack_half(const f32x16& c, int hh) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (bf16)c[8 * hh + j];
  return bitcast<uint4>(v);
}

__global__ __launch_bounds__(256, 2) void fa_fwd_kernel(const bf16* __restrict__ qkv, bf16* __restrict__ o,
                                                        float* __restrict__ lse2, int Tn, int H) {
  __shared__ __attribute__((aligned(16))) char sK[64 * PR];
  __shared__ __attribute__((aligned(16))) char sVt[64 * PT];
  const int nqb = (Tn + 255) / 256;
  const int qb = nqb - 1 - blockIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int Cc = H * HD;
  const int64_t ld = 3 * (int64_t)Cc;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 5, c32 = lane & 31;
  const int q0 = qb * 256;
  const int qt[2] = {w, 7 - w};
  int q[2];
  uint4 qf[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    q[i] = q0 + qt[i] * 32 + c32;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[i][kk] = (q[i] < Tn) ? *reinterpret_cast<const uint4*>(base + (int64_t)q[i] * ld + h * HD + kk * 16 + g * 8)
                              : make_uint4(0, 0, 0, 0);
  }
  f32x16 oacc[2][2];
  float m[2] = {NEG_INF, NEG_INF}, l[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) { zero16(oacc[i][0]); zero16(oacc[i][1]); }
  const float cs = LOG2E / 8.0f;  // log2(e) / sqrt(64)
  const int nkb = (min(Tn, q0 + 256) + 63) / 64;
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    load_rows(base + Cc + h * HD, ld, kb * 64, Tn, sK, t);
    load_trans(base + 2 * Cc + h * HD, ld, kb * 64, Tn, sVt, t);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int qlo = q0 + qt[i] * 32;
      if (kb * 64 > qlo + 31) continue;  // every key of the block is after every query of the tile
      const int qc = min(q[i], Tn - 1);
      f32x16 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        zero16(s[kt]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) mma32(s[kt], frag_row(sK, kt * 32 + c32, kk, g), qf[i][kk]);
      }
      float mx = NEG_INF;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb * 64 + kt * 32 + crow(e, g);
          const float v = (key <= qc) ? s[kt][e] * cs : NEG_INF;
          s[kt][e] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
      const float mnew = fmaxf(m[i], mx);
      const float alpha = hw_exp2(m[i] - mnew);
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = hw_exp2(s[kt][e] - mnew);
          s[kt][e] = p;
          ls += p;
        }
      ls += __shfl_xor(ls, 32, WAVE);
      l[i] = l[i] * alpha + ls;
      m[i] = mnew;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) oacc[i][dt] *= alpha;
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const uint4 bp = pack_half(s[hh >> 1], hh & 1);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) mma32(oacc[i][dt], frag_tr(sVt, dt * 32 + c32, hh, g), bp);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (q[i] >= Tn) continue;
    const float inv = 1.f / l[i];
    bf16* orow = o + (int64_t)(b * Tn + q[i]) * Cc + h * HD;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        store4(orow + dt * 32 + r4 * 8 + g * 4,
               make_float4(oacc[i][dt][4 * r4] * inv, oacc[i][dt][4 * r4 + 1] * inv, oacc[i][dt][4 * r4 + 2] * inv,
                           oacc[i][dt][4 * r4 + 3] * inv));
    if (g == 0) lse2[(int64_t)bh * Tn + q[i]] = m[i] + hw_log2(l[i]);
  }
}

// dK, dV for a 128-key block (one 32-key tile per wave): loops over 64-query
// blocks from the block's diagonal to the end.
__global__ __launch_bounds__(256, 2) void fa_bwd_dkdv_kernel(const bf16* __restrict__ qkv, const bf16* __restrict__ dO,
                                                             const float* __restrict__ lse2,
                                                             const float* __restrict__ Dv, bf16* __restrict__ dqkv,
                                                             int Tn, int H) {
  __shared__ __attribute__((aligned(16))) char sQ[64 * PR];
  __shared__ __attribute__((aligned(16))) char sQt[64 * PT];
  __shared__ __attribute__((aligned(16))) char sdO[64 * PR];
  __shared__ __attribute__((aligned(16))) char sdOt[64 * PT];
  __shared__ float slse[64], sDv[64];
  const int nqb = (Tn + 63) / 64;
  const int kb = blockIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int Cc = H * HD;
  const int64_t ld = 3 * (int64_t)Cc;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const bf16* dob = dO + (int64_t)b * Tn * Cc;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 5, c32 = lane & 31;
  const int k0 = kb * 128;
  const int klo = k0 + w * 32;
  const int key = klo + c32;
  uint4 kf[4], vf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const bool ok = key < Tn;
    const int64_t off = (int64_t)key * ld + h * HD + kk * 16 + g * 8;
    kf[kk] = ok ? *reinterpret_cast<const uint4*>(base + Cc + off) : make_uint4(0, 0, 0, 0);
    vf[kk] = ok ? *reinterpret_cast<const uint4*>(base + 2 * Cc + off) : make_uint4(0, 0, 0, 0);
  }
  f32x16 dk[2], dv[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) { zero16(dk[dt]); zero16(dv[dt]); }
  const float cs = LOG2E / 8.0f;
  for (int qb = k0 / 64; qb < nqb; ++qb) {
    __syncthreads();
    load_rows(base + h * HD, ld, qb * 64, Tn, sQ, t);
    load_trans(base + h * HD, ld, qb * 64, Tn, sQt, t);
    load_rows(dob + h * HD, Cc, qb * 64, Tn, sdO, t);
    load_trans(dob + h * HD, Cc, qb * 64, Tn, sdOt, t);
    if (t < 64) {
      const int qq = qb * 64 + t;
      slse[t] = qq < Tn ? lse2[(int64_t)bh * Tn + qq] : 0.f;
      sDv[t] = qq < Tn ? Dv[(int64_t)bh * Tn + qq] : 0.f;
    }
    __syncthreads();
    if (qb * 64 + 63 < klo) continue;  // every query of the block is before every key of the tile
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      f32x16 s, dp;
      zero16(s);
      zero16(dp);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        mma32(s, frag_row(sQ, qt * 32 + c32, kk, g), kf[kk]);
        mma32(dp, frag_row(sdO, qt * 32 + c32, kk, g), vf[kk]);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int qi = qt * 32 + crow(e, g);
        const int qrow = qb * 64 + qi;
        const bool ok = (key <= qrow) && (qrow < Tn) && (key < Tn);
        const float p = ok ? hw_exp2(s[e] * cs - slse[qi]) : 0.f;
        s[e] = p;
        dp[e] = p * (dp[e] - sDv[qi]);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint4 bp = pack_half(s, hh);
        const uint4 bds = pack_half(dp, hh);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          mma32(dv[dt], frag_tr(sdOt, dt * 32 + c32, qt * 2 + hh, g), bp);
          mma32(dk[dt], frag_tr(sQt, dt * 32 + c32, qt * 2 + hh, g), bds);
        }
      }
    }
  }
  if (key < Tn) {
    bf16* krow = dqkv + (int64_t)(b * Tn + key) * ld + Cc + h * HD;
    bf16* vrow = krow + Cc;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = dt * 32 + r4 * 8 + g * 4;
        store4(krow + d, make_float4(dk[dt][4 * r4] * 0.125f, dk[dt][4 * r4 + 1] * 0.125f,
                                     dk[dt][4 * r4 + 2] * 0.125f, dk[dt][4 * r4 + 3] * 0.125f));
        store4(vrow + d, make_float4(dv[dt][4 * r4], dv[dt][4 * r4 + 1], dv[dt][4 * r4 + 2], dv[dt][4 * r4 + 3]));
      }
  }
}

// dQ for a 256-query block: loops over 64-key blocks up to the block's diagonal.
__global__ __launch_bounds__(256, 2) void fa_bwd_dq_kernel(const bf16* __restrict__ qkv, const bf16* __restrict__ dO,
                                                           const float* __restrict__ lse2,
                                                           const float* __restrict__ Dv, bf16* __restrict__ dqkv,
                                                           int Tn, int H) {
  __shared__ __attribute__((aligned(16))) char sK[64 * PR];
  __shared__ __attribute__((aligned(16))) char sKt[64 * PT];
  __shared__ __attribute__((aligned(16))) char sV[64 * PR];
  const int nqb = (Tn + 255) / 256;
  const int qb = nqb - 1 - blockIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int Cc = H * HD;
  const int64_t ld = 3 * (int64_t)Cc;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 5, c32 = lane & 31;
  const int q0 = qb * 256;
  const int qt[2] = {w, 7 - w};
  int q[2];
  uint4 qf[2][4], dof[2][4];
  float lq[2], dq_[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    q[i] = q0 + qt[i] * 32 + c32;
    const bool ok = q[i] < Tn;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qf[i][kk] = ok ? *reinterpret_cast<const uint4*>(base + (int64_t)q[i] * ld + h * HD + kk * 16 + g * 8)
                     : make_uint4(0, 0, 0, 0);
      dof[i][kk] = ok ? *reinterpret_cast<const uint4*>(dO + (int64_t)(b * Tn + q[i]) * Cc + h * HD + kk * 16 + g * 8)
                      : make_uint4(0, 0, 0, 0);
    }
    lq[i] = ok ? lse2[(int64_t)bh * Tn + q[i]] : 0.f;
    dq_[i] = ok ? Dv[(int64_t)bh * Tn + q[i]] : 0.f;
  }
  f32x16 dq[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) { zero16(dq[i][0]); zero16(dq[i][1]); }
  const float cs = LOG2E / 8.0f;
  const int nkb = (min(Tn, q0 + 256) + 63) / 64;
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    load_rows(base + Cc + h * HD, ld, kb * 64, Tn, sK, t);
    load_trans(base + Cc + h * HD, ld, kb * 64, Tn, sKt, t);
    load_rows(base + 2 * Cc + h * HD, ld, kb * 64, Tn, sV, t);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int qlo = q0 + qt[i] * 32;
      if (kb * 64 > qlo + 31) continue;
      const bool qok = q[i] < Tn;
      f32x16 s[2], dp[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        zero16(s[kt]);
        zero16(dp[kt]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          mma32(s[kt], frag_row(sK, kt * 32 + c32, kk, g), qf[i][kk]);
          mma32(dp[kt], frag_row(sV, kt * 32 + c32, kk, g), dof[i][kk]);
        }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kkey = kb * 64 + kt * 32 + crow(e, g);
          const bool ok = qok && kkey <= q[i];
          const float p = ok ? hw_exp2(s[kt][e] * cs - lq[i]) : 0.f;
          s[kt][e] = p * (dp[kt][e] - dq_[i]);
        }
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const uint4 bds = pack_half(s[hh >> 1], hh & 1);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) mma32(dq[i][dt], frag_tr(sKt, dt * 32 + c32, hh, g), bds);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (q[i] >= Tn) continue;
    bf16* qrow = dqkv + (int64_t)(b * Tn + q[i]) * ld + h * HD;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        store4(qrow + dt * 32 + r4 * 8 + g * 4,
               make_float4(dq[i][dt][4 * r4] * 0.125f, dq[i][dt][4 * r4 + 1] * 0.125f,
                           dq[i][dt][4 * r4 + 2] * 0.125f, dq[i][dt][4 * r4 + 3] * 0.125f));
  }
}

}  // namespace

hipError_t attn_fwd_bf16_d64(const void* qkv, void* o, float* lse, int B, int Tn, int H, hipStream_t s) {
  dim3 grid((Tn + 255) / 256, B * H);
  hipLaunchKernelGGL(fa_fwd_kernel, grid, dim3(256), 0, s, (const bf16*)qkv, (bf16*)o, lse, Tn, H);
  return hipGetLastError();
}

hipError_t attn_bwd_bf16_d64(const void* qkv, const void* dO, const float* lse, const float* Dv, void* dqkv, int B,
                             int Tn, int H, hipStream_t s) {
  dim3 grid((Tn + 255) / 256, B * H);
  hipLaunchKernelGGL(fa_bwd_dkdv_kernel, dim3((Tn + 127) / 128, B * H), dim3(256), 0, s, (const bf16*)qkv,
                     (const bf16*)dO, lse, Dv, (bf16*)dqkv, Tn, H);
  hipLaunchKernelGGL(fa_bwd_dq_kernel, grid, dim3(256), 0, s, (const bf16*)qkv, (const bf16*)dO, lse, Dv,
                     (bf16*)dqkv, Tn, H);
  return hipGetLastError();
}

}  // namespace gk
