// Causal flash attention for gfx950: forward, and backward as two kernels.
//
// Method (lecture, flash-attention section; Zero page, Attention): scores
// S = Q K^T / sqrt(D) with j > i excluded, row softmax, O = P V, computed
// one 64-key block at a time with an online (running max / running sum)
// softmax kept in registers, so no [T, T] matrix is ever stored; the backward
// recomputes S and P from the saved log-sum-exp.
//
// Register orientation is chosen so that no score tile needs a transpose:
//   forward and dQ compute S^T = K Q^T; an MFMA C tile then holds, per lane,
//   4 consecutive keys of one query column, which is exactly the lane
//   layout of the B operand of the next product O^T += V^T P^T
//   (dQ^T += K^T dS^T); the A operands V^T / K^T come from a transposed
//   LDS copy.  The dK/dV kernel computes S = Q K^T, whose C tiles feed
//   dV^T += dO^T P and dK^T += Q^T dS the same way.  Softmax statistics are
//   kept in the log2 domain (scores pre-multiplied by log2 e / sqrt(D)) and
//   exponentials use the hardware exp2.
// Workgroup: 4 waves; a wave owns 16 query (or key) columns of a 64-block.
#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr float NEG_INF = -__builtin_huge_valf();

template <typename T, int D>
struct Cfg {
  static constexpr int E = Tr<T>::E;
  static constexpr int KFRAG = Tr<T>::KFRAG;
  static constexpr int KF = D / KFRAG;          // fragments along D
  static constexpr int PR = D * (int)sizeof(T) + 16;   // pitch of a [64][D] tile
  static constexpr int PT = 64 * (int)sizeof(T) + 16;  // pitch of a [D][64] tile
  static constexpr int NF64 = 64 / KFRAG;       // fragments along a 64-long axis
  static constexpr int DT = D / 16;             // 16-row tiles along D
};

// Load rows [row0, row0 + 64) x D of a [T][ld] operand into LDS, row-major
// and/or transposed ([D][64]); rows >= nvalid read as zero.
template <typename T, int D, bool ROW, bool TRANS>
__device__ __forceinline__ void load_tile(const T* __restrict__ g, int64_t ld, int row0, int nvalid,
                                          char* s_row, char* s_tr, int t) {
  using C = Cfg<T, D>;
  constexpr int CPR = D * (int)sizeof(T) / 16;
  for (int i = t; i < 64 * CPR; i += 256) {
    const int r = i / CPR, c = i % CPR;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row0 + r < nvalid) v = *reinterpret_cast<const uint4*>(g + (int64_t)(row0 + r) * ld + c * C::E);
    if constexpr (ROW) *reinterpret_cast<uint4*>(s_row + r * C::PR + c * 16) = v;
    if constexpr (TRANS) {
      const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int j = 0; j < C::E; ++j)
        *reinterpret_cast<T*>(s_tr + (c * C::E + j) * C::PT + r * (int)sizeof(T)) = e[j];
    }
  }
}

// A/B fragment f (k = f * KFRAG ..) of row `row` of a row-major [64][D] tile.
template <typename T, int D>
__device__ __forceinline__ uint4 row_frag(const char* s, int row, int f, int g) {
  return *reinterpret_cast<const uint4*>(s + row * Cfg<T, D>::PR + f * 64 + g * 16);
}

// Fragment f along the 64-long axis of row `row` of a transposed [D][64]
// tile, in the slot order of pack_cfrag: bf16 slots 0-3 = axis f*32 + g*4 + j,
// slots 4-7 = axis f*32 + 16 + g*4 + j; fp32 slots = axis f*16 + g*4 + j.
template <typename T, int D>
__device__ __forceinline__ uint4 tr_frag(const char* s, int row, int f, int g) {
  const char* p = s + row * Cfg<T, D>::PT;
  if constexpr (sizeof(T) == 2) {
    const uint2 lo = *reinterpret_cast<const uint2*>(p + (f * 32 + g * 4) * 2);
    const uint2 hi = *reinterpret_cast<const uint2*>(p + (f * 32 + 16 + g * 4) * 2);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  } else {
    return *reinterpret_cast<const uint4*>(p + (f * 16 + g * 4) * 4);
  }
}

// Pack C-tile values (tiles of 16 along the 64-long axis, lane rows g*4 + r)
// into B-operand fragment f with the slot order of tr_frag.
template <typename T>
__device__ __forceinline__ uint4 pack_cfrag(const f32x4* s, int f) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 v;
    const f32x4 a = s[2 * f], b = s[2 * f + 1];
    v[0] = (bf16)a[0]; v[1] = (bf16)a[1]; v[2] = (bf16)a[2]; v[3] = (bf16)a[3];
    v[4] = (bf16)b[0]; v[5] = (bf16)b[1]; v[6] = (bf16)b[2]; v[7] = (bf16)b[3];
    return bitcast<uint4>(v);
  } else {
    return bitcast<uint4>(s[f]);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const T* __restrict__ qkv, T* __restrict__ o,
                                                       float* __restrict__ lse2, int Tn, int H) {
  using C = Cfg<T, D>;
  __shared__ __attribute__((aligned(16))) char sK[64 * C::PR];
  __shared__ __attribute__((aligned(16))) char sVt[D * C::PT];
  const int nqb = (Tn + 63) / 64;
  const int qb = nqb - 1 - blockIdx.x;  // longest rows first
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int Cc = H * D;
  const int64_t ld = 3 * (int64_t)Cc;
  const T* base = qkv + (int64_t)b * Tn * ld;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4, c16 = lane & 15;
  const int q = qb * 64 + w * 16 + c16;
  const int qc = min(q, Tn - 1);
  uint4 qf[C::KF];
#pragma unroll
  for (int f = 0; f < C::KF; ++f)
    qf[f] = (q < Tn) ? *reinterpret_cast<const uint4*>(base + (int64_t)q * ld + h * D + f * C::KFRAG + g * C::E)
                     : make_uint4(0, 0, 0, 0);
  f32x4 oacc[C::DT];
#pragma unroll
  for (int i = 0; i < C::DT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = NEG_INF, l = 0.f;
  const float cs = LOG2E / sqrtf((float)D);
  for (int kb = 0; kb <= qb; ++kb) {
    __syncthreads();
    load_tile<T, D, true, false>(base + Cc + h * D, ld, kb * 64, Tn, sK, nullptr, t);
    load_tile<T, D, false, true>(base + 2 * Cc + h * D, ld, kb * 64, Tn, nullptr, sVt, t);
    __syncthreads();
    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < C::KF; ++f) mfma_frag(s[kt], row_frag<T, D>(sK, kt * 16 + c16, f, g), qf[f], T());
    }
    float mx = NEG_INF;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb * 64 + kt * 16 + g * 4 + r;
        const float v = (key <= qc) ? s[kt][r] * cs : NEG_INF;
        s[kt][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
    const float mnew = fmaxf(m, mx);
    const float alpha = hw_exp2(m - mnew);
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = hw_exp2(s[kt][r] - mnew);
        s[kt][r] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 16, WAVE);
    ls += __shfl_xor(ls, 32, WAVE);
    l = l * alpha + ls;
    m = mnew;
#pragma unroll
    for (int i = 0; i < C::DT; ++i) oacc[i] *= alpha;
#pragma unroll
    for (int f = 0; f < C::NF64; ++f) {
      const uint4 bp = pack_cfrag<T>(s, f);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
        mfma_frag(oacc[dt], tr_frag<T, D>(sVt, dt * 16 + c16, f, g), bp, T());
    }
  }
  if (q < Tn) {
    const float inv = 1.f / l;
    T* orow = o + (int64_t)(b * Tn + q) * Cc + h * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      store4(orow + dt * 16 + g * 4, make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv));
    if (g == 0) lse2[(int64_t)bh * Tn + q] = m + hw_log2(l);
  }
}

// Dv[b,h,t] = sum_d dO[t, h*D + d] * O[t, h*D + d].  A thread reads one 16-byte
// chunk of both rows; the D/E lanes of one head reduce with shuffles.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ dO,
                                                           float* __restrict__ Dv, int N, int Tn, int H) {
  constexpr int E = Tr<T>::E, LPH = D / E;  // lanes per head
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // chunk index over N * H * D / E
  const int64_t total = (int64_t)N * H * LPH;
  float s = 0.f;
  if (i < total) {
    const float4 a0 = load4(o + i * E), c0 = load4(dO + i * E);
    s = a0.x * c0.x + a0.y * c0.y + a0.z * c0.z + a0.w * c0.w;
    if constexpr (E == 8) {
      const float4 a1 = load4(o + i * E + 4), c1 = load4(dO + i * E + 4);
      s += a1.x * c1.x + a1.y * c1.y + a1.z * c1.z + a1.w * c1.w;
    }
  }
#pragma unroll
  for (int off = LPH / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, WAVE);
  if (i < total && (i % LPH) == 0) {
    const int64_t nh = i / LPH;
    const int n = (int)(nh / H), h = (int)(nh % H);
    const int b = n / Tn, tt = n % Tn;
    Dv[((int64_t)b * H + h) * Tn + tt] = s;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(const T* __restrict__ qkv, const T* __restrict__ dO,
                                                            const float* __restrict__ lse2,
                                                            const float* __restrict__ Dv, T* __restrict__ dqkv,
                                                            int Tn, int H) {
  using C = Cfg<T, D>;
  __shared__ __attribute__((aligned(16))) char sQ[64 * C::PR];
  __shared__ __attribute__((aligned(16))) char sQt[D * C::PT];
  __shared__ __attribute__((aligned(16))) char sdO[64 * C::PR];
  __shared__ __attribute__((aligned(16))) char sdOt[D * C::PT];
  __shared__ float slse[64], sDv[64];
  const int nqb = (Tn + 63) / 64;
  const int kb = blockIdx.x;  // key block 0 has the most query blocks: first
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int Cc = H * D;
  const int64_t ld = 3 * (int64_t)Cc;
  const T* base = qkv + (int64_t)b * Tn * ld;
  const T* dob = dO + (int64_t)b * Tn * Cc;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4, c16 = lane & 15;
  const int key = kb * 64 + w * 16 + c16;
  uint4 kf[C::KF], vf[C::KF];
#pragma unroll
  for (int f = 0; f < C::KF; ++f) {
    const bool ok = key < Tn;
    const int64_t off = (int64_t)key * ld + h * D + f * C::KFRAG + g * C::E;
    kf[f] = ok ? *reinterpret_cast<const uint4*>(base + Cc + off) : make_uint4(0, 0, 0, 0);
    vf[f] = ok ? *reinterpret_cast<const uint4*>(base + 2 * Cc + off) : make_uint4(0, 0, 0, 0);
  }
  f32x4 dk[C::DT], dv[C::DT];
#pragma unroll
  for (int i = 0; i < C::DT; ++i) dk[i] = dv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float cs = LOG2E / sqrtf((float)D);
  for (int qb = kb; qb < nqb; ++qb) {
    __syncthreads();
    load_tile<T, D, true, true>(base + h * D, ld, qb * 64, Tn, sQ, sQt, t);
    load_tile<T, D, true, true>(dob + h * D, Cc, qb * 64, Tn, sdO, sdOt, t);
    if (t < 64) {
      const int qq = qb * 64 + t;
      slse[t] = qq < Tn ? lse2[(int64_t)bh * Tn + qq] : 0.f;
      sDv[t] = qq < Tn ? Dv[(int64_t)bh * Tn + qq] : 0.f;
    }
    __syncthreads();
    f32x4 s[4], dp[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      s[qt] = dp[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < C::KF; ++f) {
        mfma_frag(s[qt], row_frag<T, D>(sQ, qt * 16 + c16, f, g), kf[f], T());
        mfma_frag(dp[qt], row_frag<T, D>(sdO, qt * 16 + c16, f, g), vf[f], T());
      }
    }
#pragma unroll
    for (int qt = 0; qt < 4; ++qt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = qt * 16 + g * 4 + r;
        const int qrow = qb * 64 + qi;
        const bool ok = (key <= qrow) && (qrow < Tn) && (key < Tn);
        const float p = ok ? hw_exp2(s[qt][r] * cs - slse[qi]) : 0.f;
        s[qt][r] = p;
        dp[qt][r] = p * (dp[qt][r] - sDv[qi]);
      }
#pragma unroll
    for (int f = 0; f < C::NF64; ++f) {
      const uint4 bp = pack_cfrag<T>(s, f);
      const uint4 bds = pack_cfrag<T>(dp, f);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        mfma_frag(dv[dt], tr_frag<T, D>(sdOt, dt * 16 + c16, f, g), bp, T());
        mfma_frag(dk[dt], tr_frag<T, D>(sQt, dt * 16 + c16, f, g), bds, T());
      }
    }
  }
  if (key < Tn) {
    const float sc = 1.f / sqrtf((float)D);
    T* krow = dqkv + (int64_t)(b * Tn + key) * ld + Cc + h * D;
    T* vrow = krow + Cc;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      store4(krow + dt * 16 + g * 4, make_float4(dk[dt][0] * sc, dk[dt][1] * sc, dk[dt][2] * sc, dk[dt][3] * sc));
      store4(vrow + dt * 16 + g * 4, make_float4(dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]));
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(const T* __restrict__ qkv, const T* __restrict__ dO,
                                                          const float* __restrict__ lse2,
                                                          const float* __restrict__ Dv, T* __restrict__ dqkv,
                                                          int Tn, int H) {
  using C = Cfg<T, D>;
  __shared__ __attribute__((aligned(16))) char sK[64 * C::PR];
  __shared__ __attribute__((aligned(16))) char sKt[D * C::PT];
  __shared__ __attribute__((aligned(16))) char sV[64 * C::PR];
  const int nqb = (Tn + 63) / 64;
  const int qb = nqb - 1 - blockIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int Cc = H * D;
  const int64_t ld = 3 * (int64_t)Cc;
  const T* base = qkv + (int64_t)b * Tn * ld;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4, c16 = lane & 15;
  const int q = qb * 64 + w * 16 + c16;
  const bool qok = q < Tn;
  uint4 qf[C::KF], dof[C::KF];
#pragma unroll
  for (int f = 0; f < C::KF; ++f) {
    qf[f] = qok ? *reinterpret_cast<const uint4*>(base + (int64_t)q * ld + h * D + f * C::KFRAG + g * C::E)
                : make_uint4(0, 0, 0, 0);
    dof[f] = qok ? *reinterpret_cast<const uint4*>(dO + (int64_t)(b * Tn + q) * Cc + h * D + f * C::KFRAG + g * C::E)
                 : make_uint4(0, 0, 0, 0);
  }
  const float lq = qok ? lse2[(int64_t)bh * Tn + q] : 0.f;
  const float dq_ = qok ? Dv[(int64_t)bh * Tn + q] : 0.f;
  f32x4 dq[C::DT];
#pragma unroll
  for (int i = 0; i < C::DT; ++i) dq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float cs = LOG2E / sqrtf((float)D);
  for (int kb = 0; kb <= qb; ++kb) {
    __syncthreads();
    load_tile<T, D, true, true>(base + Cc + h * D, ld, kb * 64, Tn, sK, sKt, t);
    load_tile<T, D, true, false>(base + 2 * Cc + h * D, ld, kb * 64, Tn, sV, nullptr, t);
    __syncthreads();
    f32x4 s[4], dp[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = dp[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < C::KF; ++f) {
        mfma_frag(s[kt], row_frag<T, D>(sK, kt * 16 + c16, f, g), qf[f], T());
        mfma_frag(dp[kt], row_frag<T, D>(sV, kt * 16 + c16, f, g), dof[f], T());
      }
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb * 64 + kt * 16 + g * 4 + r;
        const bool ok = qok && key <= q;
        const float p = ok ? hw_exp2(s[kt][r] * cs - lq) : 0.f;
        s[kt][r] = p * (dp[kt][r] - dq_);
      }
#pragma unroll
    for (int f = 0; f < C::NF64; ++f) {
      const uint4 bds = pack_cfrag<T>(s, f);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) mfma_frag(dq[dt], tr_frag<T, D>(sKt, dt * 16 + c16, f, g), bds, T());
    }
  }
  if (qok) {
    const float sc = 1.f / sqrtf((float)D);
    T* qrow = dqkv + (int64_t)(b * Tn + q) * ld + h * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      store4(qrow + dt * 16 + g * 4, make_float4(dq[dt][0] * sc, dq[dt][1] * sc, dq[dt][2] * sc, dq[dt][3] * sc));
  }
}

template <typename T, int D>
hipError_t fwd_t(const void* qkv, void* o, float* lse, int B, int Tn, int H, hipStream_t s) {
  dim3 grid((Tn + 63) / 64, B * H);
  hipLaunchKernelGGL((attn_fwd_kernel<T, D>), grid, dim3(256), 0, s, (const T*)qkv, (T*)o, lse, Tn, H);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_t(const void* qkv, const void* o, const void* dO, const float* lse, float* Dv, void* dqkv,
                 int B, int Tn, int H, hipStream_t s) {
  const int N = B * Tn;
  hipLaunchKernelGGL((attn_bwd_pre_kernel<T, D>), dim3(cdiv((int64_t)N * H * (D / Tr<T>::E), 256)), dim3(256), 0,
                     s, (const T*)o, (const T*)dO, Dv, N, Tn, H);
  if constexpr (sizeof(T) == 2 && D == 64) return attn_bwd_bf16_d64(qkv, dO, lse, Dv, dqkv, B, Tn, H, s);
  dim3 grid((Tn + 63) / 64, B * H);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D>), grid, dim3(256), 0, s, (const T*)qkv, (const T*)dO, lse, Dv,
                     (T*)dqkv, Tn, H);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D>), grid, dim3(256), 0, s, (const T*)qkv, (const T*)dO, lse, Dv,
                     (T*)dqkv, Tn, H);
  return hipGetLastError();
}

}  // namespace

hipError_t attn_fwd(int dtype, const void* qkv, void* o, float* lse, int B, int Tn, int H, int D, hipStream_t s) {
  if (dtype == BF16 && D == 64) return attn_fwd_bf16_d64(qkv, o, lse, B, Tn, H, s);
  if (dtype == F32 && D == 64) return fwd_t<float, 64>(qkv, o, lse, B, Tn, H, s);
  if (dtype == F32 && D == 32) return fwd_t<float, 32>(qkv, o, lse, B, Tn, H, s);
  if (dtype == F32 && D == 16) return fwd_t<float, 16>(qkv, o, lse, B, Tn, H, s);
  return hipErrorInvalidValue;
}

hipError_t attn_bwd(int dtype, const void* qkv, const void* o, const void* dO, const float* lse, float* Dv,
                    void* dqkv, int B, int Tn, int H, int D, hipStream_t s) {
  if (dtype == BF16 && D == 64) return bwd_t<bf16, 64>(qkv, o, dO, lse, Dv, dqkv, B, Tn, H, s);
  if (dtype == F32 && D == 64) return bwd_t<float, 64>(qkv, o, dO, lse, Dv, dqkv, B, Tn, H, s);
  if (dtype == F32 && D == 32) return bwd_t<float, 32>(qkv, o, dO, lse, Dv, dqkv, B, Tn, H, s);
  if (dtype == F32 && D == 16) return bwd_t<float, 16>(qkv, o, dO, lse, Dv, dqkv, B, Tn, H, s);
  return hipErrorInvalidValue;
}

}  // namespace gk
