// Optimiser, initialisation and embedding-gradient kernels for gfx950.
//
// AdamW (CS336 page, section 2 AdamW; lecture, AdamW and fused optimiser):
// one flat, float4-vectorised pass over every parameter (the arena keeps all
// decayed matrices in one contiguous range, so the decay group is a single
// index bound), reading p, g, m, v and writing p, m, v and the bf16 shadow.
// The global gradient norm (lecture and CS336 page, gradient clipping) is a
// fixed-grid two-stage reduction, so it is bit-reproducible.
// The token-embedding gradient is a deterministic segmented sum: token ids
// are sorted with their positions (bitonic sort in LDS), runs of equal ids
// are summed inside 64-row chunks, then chunk partials are added in order.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace gk {
namespace {

constexpr int NORM_BLOCKS = 1024;

__global__ __launch_bounds__(256) void sumsq_kernel(const float* __restrict__ g, int64_t n4,
                                                    float* __restrict__ part) {
  __shared__ float red[4];
  float s = 0.f;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const float4 v = g4[i];
    s += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// scal: [0] norm, [1] clip scale, [2] finite flag (1/0), [3] AdamW step size a,
//       [4] sticky non-finite flag; step_dev: applied update count t.
__global__ void norm_finish_kernel(const float* __restrict__ part, int nblk, float clip, float* scal) {
  __shared__ float red[4];
  float s = 0.f;
  for (int i = threadIdx.x; i < nblk; i += 256) s += part[i];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float norm = sqrtf(red[0] + red[1] + red[2] + red[3]);
    scal[0] = norm;
    scal[1] = (clip > 0.f) ? fminf(1.f, clip / (norm + 1e-6f)) : 1.f;
    const bool fin = isfinite(norm);
    scal[2] = fin ? 1.f : 0.f;
    if (!fin) scal[4] = 1.f;
  }
}

__global__ void adamw_prep_kernel(float* scal, int* step_dev, float lr, float b1, float b2) {
  if (scal[2] == 0.f) return;
  const int t = step_dev[0] + 1;
  step_dev[0] = t;
  // bias corrections in double: 1 - b^t loses digits in float for small t
  const double c1 = 1.0 - pow((double)b1, (double)t);
  const double c2 = 1.0 - pow((double)b2, (double)t);
  scal[3] = (float)((double)lr * sqrt(c2) / c1);
}

// Streaming loads and stores (non-temporal: p, g, m, v are touched once per
// step) of two float4 groups per thread, whose eight loads are issued before
// any arithmetic; one thread per pair of groups, no grid-stride loop.
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream(const float* p, int64_t i) {
  const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p) + i);
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(float* p, int64_t i, float4 a) {
  const f32x4v v = {a.x, a.y, a.z, a.w};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4v*>(p) + i);
}
constexpr int ADAMW_U = 2;  // float4 groups per thread

__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    bf16* __restrict__ shadow, int64_t n4, int64_t n4_decay,
                                                    const float* __restrict__ scal, float lr, float b1, float b2,
                                                    float eps, float wd) {
  if (scal[2] == 0.f) return;  // non-finite gradient norm: no update
  const float cs = scal[1], a = scal[3];
  const float dec = 1.f - lr * wd;
  const int64_t i0 = (int64_t)blockIdx.x * 256 * ADAMW_U + threadIdx.x;
  float4 p4[ADAMW_U], g4[ADAMW_U], m4[ADAMW_U], v4[ADAMW_U];
#pragma unroll
  for (int u = 0; u < ADAMW_U; ++u) {
    const int64_t i = i0 + u * 256;
    if (i < n4) {
      p4[u] = ld_stream(p, i);
      g4[u] = ld_stream(g, i);
      m4[u] = ld_stream(m, i);
      v4[u] = ld_stream(v, i);
    }
  }
#pragma unroll
  for (int u = 0; u < ADAMW_U; ++u) {
    const int64_t i = i0 + u * 256;
    if (i >= n4) continue;
    const float d = (i < n4_decay) ? dec : 1.f;
    float pa[4] = {p4[u].x, p4[u].y, p4[u].z, p4[u].w}, ga[4] = {g4[u].x, g4[u].y, g4[u].z, g4[u].w};
    float ma[4] = {m4[u].x, m4[u].y, m4[u].z, m4[u].w}, va[4] = {v4[u].x, v4[u].y, v4[u].z, v4[u].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float gk_ = ga[k] * cs;
      ma[k] = b1 * ma[k] + (1.f - b1) * gk_;
      va[k] = b2 * va[k] + (1.f - b2) * gk_ * gk_;
      pa[k] = pa[k] * d - a * ma[k] / (sqrtf(va[k]) + eps);
    }
    const float4 pp = make_float4(pa[0], pa[1], pa[2], pa[3]);
    st_stream(p, i, pp);
    st_stream(m, i, make_float4(ma[0], ma[1], ma[2], ma[3]));
    st_stream(v, i, make_float4(va[0], va[1], va[2], va[3]));
    if (shadow) store4(shadow + 4 * i, pp);
  }
}

__global__ void to_bf16_kernel(const float* __restrict__ x, bf16* __restrict__ y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    y[i] = (bf16)x[i];
}

__global__ void fill_kernel(float* __restrict__ x, int64_t n, float value) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = value;
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): counter-based generator.
__device__ __forceinline__ uint4 philox(uint4 c, uint2 k) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(M0, c.x), lo0 = M0 * c.x;
    const uint32_t hi1 = __umulhi(M1, c.z), lo1 = M1 * c.z;
    c = make_uint4(hi1 ^ c.y ^ k.x, lo1, hi0 ^ c.w ^ k.y, lo0);
    k.x += W0;
    k.y += W1;
  }
  return c;
}

// x[i] = std * z, z ~ N(0,1) by Box-Muller on the first two words of
// philox(counter = offset + i, key = seed).
__global__ void init_normal_kernel(float* __restrict__ x, int64_t n, float std, uint64_t seed, uint64_t offset) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const uint64_t ctr = offset + (uint64_t)i;
    const uint4 r = philox(make_uint4((uint32_t)ctr, (uint32_t)(ctr >> 32), 0u, 0u),
                           make_uint2((uint32_t)seed, (uint32_t)(seed >> 32)));
    const float u1 = ((float)r.x + 1.0f) * 2.3283064365386963e-10f;  // (0, 1]
    const float u2 = (float)r.y * 2.3283064365386963e-10f;
    const float rad = sqrtf(-2.0f * hw_log2(u1) * LN2);
    x[i] = std * rad * cosf(6.283185307179586f * u2);
  }
}

// keys (tok << shift) | position of positions [base, base + n), sorted ascending
// into keys[base ..] (bitonic over P >= n slots in LDS, one workgroup per chunk:
// chunk c = blockIdx.x starts at base = c * SORT_MAX)
constexpr int SORT_MAX = 16384;
__global__ __launch_bounds__(1024) void sort_kernel(const int32_t* __restrict__ tok, int n_total, int shift, int P,
                                                    uint32_t* __restrict__ keys) {
  __shared__ uint32_t sk[SORT_MAX];
  const int t = threadIdx.x;
  const int base = blockIdx.x * SORT_MAX;
  const int n = min(SORT_MAX, n_total - base);
  for (int i = t; i < P; i += 1024)
    sk[i] = (i < n) ? (((uint32_t)tok[base + i] << shift) | (uint32_t)(base + i)) : 0xFFFFFFFFu;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = t; i < P; i += 1024) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint32_t a = sk[i], b = sk[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            sk[i] = b;
            sk[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = t; i < n; i += 1024) keys[base + i] = sk[i];
}

// Merge of nch sorted chunks (chunk c: chunk[c * SORT_MAX ..], its length
// min(SORT_MAX, n - c * SORT_MAX)) by rank: keys are distinct (they hold the
// position), so a key's place in the merged order is its index in its own
// chunk plus the number of smaller keys in each other chunk (a lower bound).
__global__ __launch_bounds__(256) void merge_rank_kernel(const uint32_t* __restrict__ chunk, int n, int nch,
                                                         uint32_t* __restrict__ keys) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int c = i / SORT_MAX;
  const uint32_t k = chunk[i];
  int rank = i - c * SORT_MAX;
  for (int d = 0; d < nch; ++d) {
    if (d == c) continue;
    const uint32_t* a = chunk + (int64_t)d * SORT_MAX;
    int lo = 0, hi = min(SORT_MAX, n - d * SORT_MAX);  // first index with a[idx] >= k
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (a[mid] < k) lo = mid + 1;
      else hi = mid;
    }
    rank += lo;
  }
  keys[rank] = k;
}

// pass 1: per 64-row chunk of sorted positions, sum each run of equal ids into part[run start]
__global__ __launch_bounds__(256) void embed_bwd_chunk_kernel(const uint32_t* __restrict__ keys, int n,
                                                              int shift, const float* __restrict__ dres, int C,
                                                              float* __restrict__ part) {
  const int i0 = blockIdx.x * 64, i1 = min(n, i0 + 64);
  const uint32_t pmask = (1u << shift) - 1u;
  const int nc = C >> 2;
  for (int j = threadIdx.x; j < nc; j += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int run = i0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = keys[i];
      const float4 v = load4(dres + (int64_t)(k & pmask) * C + 4 * j);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      if (i == i1 - 1 || (keys[i + 1] >> shift) != (k >> shift)) {
        store4(part + (int64_t)run * C + 4 * j, acc);
        acc = make_float4(0.f, 0.f, 0.f, 0.f);
        run = i + 1;
      }
    }
  }
}

// pass 2: a workgroup per sorted position; segment starts add their chunk partials in order
__global__ __launch_bounds__(256) void embed_bwd_seg_kernel(const uint32_t* __restrict__ keys, int n, int shift,
                                                            const float* __restrict__ part, int C,
                                                            float* __restrict__ dwte) {
  const int i = blockIdx.x;
  const uint32_t id = keys[i] >> shift;
  if (i > 0 && (keys[i - 1] >> shift) == id) return;
  const int nc = C >> 2;
  for (int j = threadIdx.x; j < nc; j += 256) {
    float4 s = load4(part + (int64_t)i * C + 4 * j);
    for (int c = i / 64 + 1; c * 64 < n && (keys[c * 64] >> shift) == id; ++c) {
      const float4 v = load4(part + (int64_t)c * 64 * C + 4 * j);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    float* row = dwte + (int64_t)id * C + 4 * j;
    const float4 o = load4(row);
    store4(row, make_float4(o.x + s.x, o.y + s.y, o.z + s.z, o.w + s.w));
  }
}

__global__ void wpe_bwd_kernel(const float* __restrict__ dres, int B, int Tn, int C, float* __restrict__ dwpe,
                               int accumulate) {
  const int tt = blockIdx.x;
  for (int c = threadIdx.x; c < C; c += 256) {
    float s = 0.f;
    for (int b = 0; b < B; ++b) s += dres[((int64_t)b * Tn + tt) * C + c];
    float* o = dwpe + (int64_t)tt * C + c;
    *o = accumulate ? *o + s : s;
  }
}

}  // namespace

int sumsq_blocks(int64_t) { return NORM_BLOCKS; }

hipError_t sumsq_partial(const float* g, int64_t n, float* part, int* nblk, hipStream_t s) {
  if (nblk) *nblk = NORM_BLOCKS;
  hipLaunchKernelGGL(sumsq_kernel, dim3(NORM_BLOCKS), dim3(256), 0, s, g, n / 4, part);
  return hipGetLastError();
}

hipError_t norm_finish(const float* part, int nblk, float clip, float* scal, hipStream_t s) {
  hipLaunchKernelGGL(norm_finish_kernel, dim3(1), dim3(256), 0, s, part, nblk, clip, scal);
  return hipGetLastError();
}

hipError_t adamw_prep(float* scal, float lr, float b1, float b2, int* step_dev, hipStream_t s) {
  hipLaunchKernelGGL(adamw_prep_kernel, dim3(1), dim3(1), 0, s, scal, step_dev, lr, b1, b2);
  return hipGetLastError();
}

hipError_t adamw_range(float* p, const float* g, float* m, float* v, void* shadow, int64_t lo, int64_t hi,
                       int64_t n_decay, const float* scal, float lr, float b1, float b2, float eps, float wd,
                       hipStream_t s) {
  if ((lo | hi) & 3 || hi < lo) return hipErrorInvalidValue;
  const int64_t n4 = (hi - lo) / 4;
  const int64_t blocks = cdiv(n4, 256 * ADAMW_U);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t d4 = std::min(std::max<int64_t>(n_decay - lo, 0), hi - lo) / 4;  // decayed prefix of the range
  bf16* sh = shadow ? (bf16*)shadow + lo : nullptr;
  hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p + lo, g + lo, m + lo, v + lo, sh, n4, d4,
                     scal, lr, b1, b2, eps, wd);
  return hipGetLastError();
}

hipError_t adamw(float* p, const float* g, float* m, float* v, void* shadow, int64_t n, int64_t n_decay,
                 float* scal, float lr, float b1, float b2, float eps, float wd, int* step_dev, hipStream_t s) {
  if (hipError_t e = adamw_prep(scal, lr, b1, b2, step_dev, s)) return e;
  return adamw_range(p, g, m, v, shadow, 0, n, n_decay, scal, lr, b1, b2, eps, wd, s);
}

hipError_t to_bf16(const float* x, void* y, int64_t n, hipStream_t s) {
  const int blocks = (int)std::min<int64_t>(cdiv(n, 256), 8192);
  hipLaunchKernelGGL(to_bf16_kernel, dim3(blocks), dim3(256), 0, s, x, (bf16*)y, n);
  return hipGetLastError();
}

hipError_t fill_f32(float* x, int64_t n, float value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>(cdiv(n, 256), 8192);
  hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(256), 0, s, x, n, value);
  return hipGetLastError();
}

hipError_t init_normal(float* x, int64_t n, float std, uint64_t seed, uint64_t offset, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>(cdiv(n, 256), 8192);
  hipLaunchKernelGGL(init_normal_kernel, dim3(blocks), dim3(256), 0, s, x, n, std, seed, offset);
  return hipGetLastError();
}

hipError_t sort_tokens(const int32_t* tok, int n, uint32_t* keys, uint32_t* tmp, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n > SORT_MAX_TOKENS) return hipErrorInvalidValue;
  int shift = 0;
  while ((1 << shift) < n) ++shift;
  if (n <= SORT_MAX) {
    int P = 1;
    while (P < n) P <<= 1;
    hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(1024), 0, s, tok, n, shift, P, keys);
    return hipGetLastError();
  }
  if (!tmp) return hipErrorInvalidValue;
  // chunks of SORT_MAX sorted side by side into tmp, then merged by rank into keys
  const int nch = (n + SORT_MAX - 1) / SORT_MAX;
  hipLaunchKernelGGL(sort_kernel, dim3(nch), dim3(1024), 0, s, tok, n, shift, SORT_MAX, tmp);
  hipLaunchKernelGGL(merge_rank_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, tmp, n, nch, keys);
  return hipGetLastError();
}

hipError_t wpe_bwd(const float* dres, int B, int Tn, int C, float* dwpe, int accumulate, hipStream_t s) {
  hipLaunchKernelGGL(wpe_bwd_kernel, dim3(Tn), dim3(256), 0, s, dres, B, Tn, C, dwpe, accumulate);
  return hipGetLastError();
}

hipError_t embed_bwd_ws(const uint32_t* keys, int n, const float* dres, int C, float* part, float* dwte,
                        hipStream_t s) {
  int shift = 0;
  while ((1 << shift) < n) ++shift;
  hipLaunchKernelGGL(embed_bwd_chunk_kernel, dim3(cdiv(n, 64)), dim3(256), 0, s, keys, n, shift, dres, C, part);
  hipLaunchKernelGGL(embed_bwd_seg_kernel, dim3(n), dim3(256), 0, s, keys, n, shift, part, C, dwte);
  return hipGetLastError();
}

}  // namespace gk
