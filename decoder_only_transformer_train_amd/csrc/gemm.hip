// MFMA GEMM for gfx950: C[m][n] = sum_k A(m,k) B(n,k) with fused epilogues.
//
// bf16 products run on 32x32x16 MFMAs (the shape that reaches the chip's
// dense peak from one wave per SIMD) in a direct-load kernel: operand tiles go
// from global memory straight into LDS with buffer_load_dwordx4 ... lds, one
// wave instruction filling 1 KB, so no registers are spent staging them and
// several k-tiles stay in flight.  k-contiguous operands sit in LDS as rows of
// k with XOR-permuted 16-byte chunks and are read with ds_read_b128;
// row-contiguous operands (the weight- and data-gradient products) sit as rows
// of k-rows and are read with the LDS transpose read ds_read_b64_tr_b16, so no
// operand is ever transposed in registers.  Every bf16 product runs a 256x256
// tile of 8 waves (2 x 4 sub-tiles of 128 x 64, two waves per SIMD, so one
// issues its loads while the other keeps the MFMA pipe busy) with 2 stages of
// 64 k and one workgroup per CU, or its 256x192 variant (4 x 2 sub-tiles of
// 64 x 96) where that fills the CUs better; 4-wave 256x128 and 256x256 tiles
// stay selectable for tuning.  fp32 products (16x16x4 f32 MFMA) use a
// register-staged 128x128 kernel with padded LDS rows.
// Operands are read through buffer descriptors whose range ends at the
// operand, so loads past M, N or K return zeros without a branch.  Epilogues
// stage the accumulators through LDS so bias, residual and GELU work uses
// coalesced 16/8-byte accesses.  Workgroup ids are remapped so each XCD (ids
// are dealt round-robin to the 8 XCDs) works on a contiguous, grouped run of
// tiles that share operand rows in its L2.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <cstdlib>

namespace gk {
namespace {

// MFMA geometry: bf16 uses 32x32x16 (one 16-byte fragment per lane: row lane % 32,
// k-group lane / 32 of 8 elements; 16 accumulators per lane), fp32 uses four
// 16x16x4 ops per fragment (row lane % 16, k-group lane / 16 of 4 elements).
template <typename T> struct Mf;
template <> struct Mf<bf16> {
  static constexpr int R = 32, KG = 2, NA = 16;
  typedef f32x16 acc_t;
  static __device__ __forceinline__ void mma(acc_t& c, const uint4& a, const uint4& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ int row(int i, int lane) { return (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3); }
  static __device__ __forceinline__ int col(int lane) { return lane & 31; }
};
template <> struct Mf<float> {
  static constexpr int R = 16, KG = 4, NA = 4;
  typedef f32x4 acc_t;
  static __device__ __forceinline__ void mma(acc_t& c, const uint4& a, const uint4& b) { mfma_frag(c, a, b, 0.f); }
  static __device__ __forceinline__ int row(int i, int lane) { return (lane >> 4) * 4 + i; }
  static __device__ __forceinline__ int col(int lane) { return lane & 15; }
};

constexpr int TKB = 128;          // k bytes per tile (bf16: 64, fp32: 32 elements)
constexpr int PITCH = TKB + 16;   // LDS row pitch (bytes)
constexpr int GROUP_M = 8;

struct Params {
  const void* A;
  const void* B;
  int64_t lda, ldb;
  int M, N, K;
  int k_per_split;
  void* C;
  int64_t ldc;
  const float* bias;
  const float* R;
  void* C2;
  const void* aux;
  int accumulate;
  int tiles_m, tiles_n;
  float* ws;
  float* dv;
  int tn, heads;
  const float* lse;     // EPI_CE_GRAD: per-row log-sum-exp (natural log)
  const int32_t* rowi;  // EPI_CE_GRAD: per-row target class
  int col0;             // EPI_CE_GRAD: class of output column 0
  float scale;          // EPI_CE_GRAD
};

// EPI_CE_GRAD: the cross-entropy gradient at logit x of class `cls` in a row
// with log-sum-exp lse and target y: scale (exp(x - lse) - [cls == y]).
__device__ __forceinline__ float ce_grad(float x, float lse, int y, int cls, float scale) {
  return (hw_exp2((x - lse) * LOG2E) - (cls == y ? 1.f : 0.f)) * scale;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Buffer resource over [p, p + bytes): loads past the end return zero, which
// is how every tile edge (rows past M/N, k-rows past K) is handled.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint4 bload(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <typename T, int TRANS, int ROWS>
struct Loader {
  static constexpr int NR = ROWS / 32;  // 16-byte registers per thread
  uint4 r[NR];
  // TRANS == 0: operand stored [rows][ld], k contiguous.
  // TRANS == 1: operand stored [K][ld], rows contiguous; a unit is 4 k-rows x E elements.
  __device__ __forceinline__ void load(rsrc_t rs, int64_t ld, int row0, int k0, int t) {
    constexpr int E = Tr<T>::E;
    if constexpr (TRANS == 0) {
      const int cc = t & 7;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int64_t row = row0 + (t >> 3) + 32 * i;
        r[i] = bload(rs, (uint32_t)((row * ld + k0 + cc * E) * (int64_t)sizeof(T)));
      }
    } else {
      constexpr int MCH = ROWS / E;
#pragma unroll
      for (int u = 0; u < NR / 4; ++u) {
        const int unit = t + 256 * u;
        const int mc = unit % MCH, kg = unit / MCH;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t k = k0 + kg * 4 + i;
          r[4 * u + i] = bload(rs, (uint32_t)((k * ld + row0 + mc * E) * (int64_t)sizeof(T)));
        }
      }
    }
  }
  __device__ __forceinline__ void store(char* s, int t) const {
    if constexpr (TRANS == 0) {
      const int cc = t & 7;
#pragma unroll
      for (int i = 0; i < NR; ++i)
        *reinterpret_cast<uint4*>(s + ((t >> 3) + 32 * i) * PITCH + cc * 16) = r[i];
    } else {
      constexpr int E = Tr<T>::E;
      constexpr int MCH = ROWS / E;
#pragma unroll
      for (int u = 0; u < NR / 4; ++u) {
        const int unit = t + 256 * u;
        const int mc = unit % MCH, kg = unit / MCH;
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[4 * u + 0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[4 * u + 1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[4 * u + 2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[4 * u + 3]);
        if constexpr (sizeof(T) == 2) {
          // 4 k-rows x 8 elements -> 8 rows x 4 k-elements (8 bytes each).  Lanes
          // that store together hold different m-chunks whose rows are 8 apart; each
          // lane starts its 8 stores at row (mc % 8) so one store instruction spreads
          // over the banks instead of stacking on 8 of them.
          uint2 out[8];
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
            out[e] = make_uint2(lo, hi);
          }
          const int rot = mc & 7;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int e = (j + rot) & 7;
            uint2 v = out[0];
#pragma unroll
            for (int q = 1; q < 8; ++q)
              if (e == q) v = out[q];
            *reinterpret_cast<uint2*>(s + (mc * 8 + e) * PITCH + kg * 8) = v;
          }
        } else {
          // fp32: 4 k-rows x 4 elements -> 4 rows x 4 k-elements (16 bytes each)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *reinterpret_cast<uint4*>(s + (mc * 4 + e) * PITCH + kg * 16) =
                make_uint4(w0[e], w1[e], w2[e], w3[e]);
        }
      }
    }
  }
};

// Work item of this workgroup: output tile (tm, tn) and k-split kz.  The
// hardware places workgroup i on XCD i % 8; each XCD is given a contiguous
// range of the (split-major, then grouped-tile) work list, so the workgroups
// sharing an XCD's L2 share k-slabs of the operands (a split-K product reads
// each split's slabs once per XCD instead of once per tile column) and, within
// a split, form GROUP_M-row blocks of tiles.
__device__ __forceinline__ void tile_coords(const Params& p, int& tm, int& tn, int& kz) {
  const int total = gridDim.x, lin = blockIdx.x;
  const int tiles = p.tiles_m * p.tiles_n;
  const int x = lin & 7, base = total >> 3, rem = total & 7;
  // XCD x holds base + (x < rem) work items.  A single-split grid whose tile
  // count is not a multiple of 8 keeps the hardware order (measured: the LM
  // head's 50304-row weight gradient fetched 28% more with the remap)
  const int w = (total == tiles && rem) ? lin : x * base + min(x, rem) + (lin >> 3);
  kz = w / tiles;
  const int id = w - kz * tiles;
  const int per_group = GROUP_M * p.tiles_n;
  const int group = id / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(GROUP_M, p.tiles_m - first_m);
  const int in = id - group * per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}


// Epilogue through LDS: the accumulator tile is written to LDS as fp32 rows
// (PASS_ROWS rows per pass), then every thread handles groups of 4 adjacent
// columns with 16-byte (fp32) / 8-byte (bf16) coalesced global accesses.
// One group of 4 adjacent columns of row m, loading its own inputs (tiles too
// large to prefetch a whole pass of inputs in registers).
template <typename T, int EPI, int SPLIT>
__device__ __forceinline__ void epi_group_inline(const Params& p, int m, int n, float4 a) {
  float v[4] = {a.x, a.y, a.z, a.w};
  const bool full = n + 3 < p.N;
  if constexpr (SPLIT) {
    float* o = p.ws + (int64_t)m * p.N + n;  // ws: this split's slice
    if (full && (p.N & 3) == 0) {
      *reinterpret_cast<float4*>(o) = a;
    } else {
      for (int k = 0; k < 4; ++k)
        if (n + k < p.N) o[k] = v[k];
    }
    return;
  }
  const int64_t o = (int64_t)m * p.ldc + n;
  if constexpr (EPI == EPI_CE_GRAD) {
    const float l = p.lse[m];
    const int y = p.rowi[m];
    for (int k = 0; k < 4; ++k)
      if (n + k < p.N) reinterpret_cast<T*>(p.C)[o + k] = from_f<T>(ce_grad(v[k], l, y, p.col0 + n + k, p.scale));
    return;
  }
  if (!full || (p.ldc & 3)) {  // ragged edge: element by element
    for (int k = 0; k < 4; ++k) {
      if (n + k >= p.N) break;
      const float bn = p.bias ? p.bias[n + k] : 0.f;
      const float x = v[k];
      if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_ODOT) reinterpret_cast<T*>(p.C)[o + k] = from_f<T>(x + bn);
      else if constexpr (EPI == EPI_RESID) reinterpret_cast<float*>(p.C)[o + k] = p.R[o + k] + (x + bn);
      else if constexpr (EPI == EPI_GELU) {
        float gg, dg;
        gelu_both(x + bn, gg, dg);
        reinterpret_cast<T*>(p.C)[o + k] = from_f<T>(dg);
        reinterpret_cast<T*>(p.C2)[o + k] = from_f<T>(gg);
      } else if constexpr (EPI == EPI_GELU_BWD) {
        reinterpret_cast<T*>(p.C)[o + k] = from_f<T>(x * to_f(reinterpret_cast<const T*>(p.aux)[o + k]));
      } else {
        float* c = reinterpret_cast<float*>(p.C);
        c[o + k] = p.accumulate ? c[o + k] + x : x;
      }
    }
    return;
  }
  float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (p.bias) b4 = *reinterpret_cast<const float4*>(p.bias + n);
  if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_ODOT) {
    store4(reinterpret_cast<T*>(p.C) + o, make_float4(a.x + b4.x, a.y + b4.y, a.z + b4.z, a.w + b4.w));
  } else if constexpr (EPI == EPI_RESID) {
    const float4 r = *reinterpret_cast<const float4*>(p.R + o);
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + o) =
        make_float4(r.x + (a.x + b4.x), r.y + (a.y + b4.y), r.z + (a.z + b4.z), r.w + (a.w + b4.w));
  } else if constexpr (EPI == EPI_GELU) {
    float g0, g1, g2, g3, d0, d1, d2, d3;
    gelu_both(a.x + b4.x, g0, d0);
    gelu_both(a.y + b4.y, g1, d1);
    gelu_both(a.z + b4.z, g2, d2);
    gelu_both(a.w + b4.w, g3, d3);
    store4(reinterpret_cast<T*>(p.C) + o, make_float4(d0, d1, d2, d3));
    store4(reinterpret_cast<T*>(p.C2) + o, make_float4(g0, g1, g2, g3));
  } else if constexpr (EPI == EPI_GELU_BWD) {
    const float4 u = load4(reinterpret_cast<const T*>(p.aux) + o);
    store4(reinterpret_cast<T*>(p.C) + o, make_float4(a.x * u.x, a.y * u.y, a.z * u.z, a.w * u.w));
  } else {
    float* c = reinterpret_cast<float*>(p.C) + o;
    if (p.accumulate) {
      const float4 c0 = *reinterpret_cast<const float4*>(c);
      a = make_float4(c0.x + a.x, c0.y + a.y, c0.z + a.z, c0.w + a.w);
    }
    *reinterpret_cast<float4*>(c) = a;
  }
}

// Epilogue inputs other than the accumulators: the residual (EPI_RESID), the
// pre-activation (EPI_GELU_BWD) or the previous output (EPI_F32 accumulating).
template <int EPI, int SPLIT>
__device__ __forceinline__ constexpr bool epi_reads() {
  return !SPLIT && (EPI == EPI_RESID || EPI == EPI_GELU_BWD || EPI == EPI_F32 || EPI == EPI_STORE_ODOT ||
                    EPI == EPI_CE_GRAD);
}
// (EPI_CE_GRAD: the row's log-sum-exp and target, as (lse, bits of y, 0, 0))
template <typename T, int EPI, int SPLIT>
__device__ __forceinline__ float4 epi_load(const Params& p, int m, int64_t o) {
  if constexpr (EPI == EPI_CE_GRAD) return make_float4(p.lse[m], __int_as_float(p.rowi[m]), 0.f, 0.f);
  else if constexpr (EPI == EPI_RESID) return *reinterpret_cast<const float4*>(p.R + o);
  else if constexpr (EPI == EPI_GELU_BWD || EPI == EPI_STORE_ODOT) return load4(reinterpret_cast<const T*>(p.aux) + o);
  else if constexpr (EPI == EPI_F32) {
    if (p.accumulate) return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.C) + o);
  }
  return make_float4(0.f, 0.f, 0.f, 0.f);
}

// One group of 4 adjacent columns of row m inside the output (16-byte aligned),
// with in = epi_load of it and b4 = its bias, both loaded ahead: no loads here.
template <typename T, int EPI, int SPLIT>
__device__ __forceinline__ void epi_group_full(const Params& p, int m, int n, float4 a, float4 in, float4 b4) {
  if constexpr (SPLIT) {
    *reinterpret_cast<float4*>(p.ws + (int64_t)m * p.N + n) = a;  // ws: this split's slice
    return;
  }
  const int64_t o = (int64_t)m * p.ldc + n;
  if constexpr (EPI == EPI_CE_GRAD) {
    const int y = __float_as_int(in.y), c = p.col0 + n;
    store4(reinterpret_cast<T*>(p.C) + o, make_float4(ce_grad(a.x, in.x, y, c, p.scale), ce_grad(a.y, in.x, y, c + 1, p.scale),
                                                      ce_grad(a.z, in.x, y, c + 2, p.scale),
                                                      ce_grad(a.w, in.x, y, c + 3, p.scale)));
  } else if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_ODOT) {
    store4(reinterpret_cast<T*>(p.C) + o, make_float4(a.x + b4.x, a.y + b4.y, a.z + b4.z, a.w + b4.w));
  } else if constexpr (EPI == EPI_RESID) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + o) =
        make_float4(in.x + (a.x + b4.x), in.y + (a.y + b4.y), in.z + (a.z + b4.z), in.w + (a.w + b4.w));
  } else if constexpr (EPI == EPI_GELU) {
    float g0, g1, g2, g3, d0, d1, d2, d3;
    gelu_both(a.x + b4.x, g0, d0);
    gelu_both(a.y + b4.y, g1, d1);
    gelu_both(a.z + b4.z, g2, d2);
    gelu_both(a.w + b4.w, g3, d3);
    store4(reinterpret_cast<T*>(p.C) + o, make_float4(d0, d1, d2, d3));
    store4(reinterpret_cast<T*>(p.C2) + o, make_float4(g0, g1, g2, g3));
  } else if constexpr (EPI == EPI_GELU_BWD) {
    store4(reinterpret_cast<T*>(p.C) + o, make_float4(a.x * in.x, a.y * in.y, a.z * in.z, a.w * in.w));
  } else {
    if (p.accumulate) a = make_float4(in.x + a.x, in.y + a.y, in.z + a.z, in.w + a.w);
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + o) = a;
  }
}

// One group of 4 adjacent columns of row m.  full: the group is inside N and
// 16-byte aligned, in = epi_load of it and b4 = its bias, both loaded ahead.
template <typename T, int EPI, int SPLIT>
__device__ __forceinline__ void epi_group(const Params& p, int m, int n, float4 a, bool full, float4 in, float4 b4) {
  float v[4] = {a.x, a.y, a.z, a.w};
  if constexpr (SPLIT) {
    float* o = p.ws + (int64_t)m * p.N + n;  // ws: this split's slice
    if (full && (p.N & 3) == 0) {
      *reinterpret_cast<float4*>(o) = a;
    } else {
      for (int k = 0; k < 4; ++k)
        if (n + k < p.N) o[k] = v[k];
    }
    return;
  }
  const int64_t o = (int64_t)m * p.ldc + n;
  if constexpr (EPI == EPI_CE_GRAD) {
    if (!full) {  // ragged edge: element by element, the row's values loaded here
      const float l = p.lse[m];
      const int y = p.rowi[m];
      for (int k = 0; k < 4; ++k)
        if (n + k < p.N) reinterpret_cast<T*>(p.C)[o + k] = from_f<T>(ce_grad(v[k], l, y, p.col0 + n + k, p.scale));
    } else {
      epi_group_full<T, EPI, SPLIT>(p, m, n, a, in, b4);
    }
    return;
  }
  if (!full) {  // ragged edge: element by element
    for (int k = 0; k < 4; ++k) {
      if (n + k >= p.N) break;
      const float bn = p.bias ? p.bias[n + k] : 0.f;
      const float x = v[k];
      if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_ODOT) reinterpret_cast<T*>(p.C)[o + k] = from_f<T>(x + bn);
      else if constexpr (EPI == EPI_RESID) reinterpret_cast<float*>(p.C)[o + k] = p.R[o + k] + (x + bn);
      else if constexpr (EPI == EPI_GELU) {
        float gg, dg;
        gelu_both(x + bn, gg, dg);
        reinterpret_cast<T*>(p.C)[o + k] = from_f<T>(dg);
        reinterpret_cast<T*>(p.C2)[o + k] = from_f<T>(gg);
      } else if constexpr (EPI == EPI_GELU_BWD) {
        reinterpret_cast<T*>(p.C)[o + k] = from_f<T>(x * to_f(reinterpret_cast<const T*>(p.aux)[o + k]));
      } else {
        float* c = reinterpret_cast<float*>(p.C);
        c[o + k] = p.accumulate ? c[o + k] + x : x;
      }
    }
    return;
  }
  if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_ODOT) {
    store4(reinterpret_cast<T*>(p.C) + o, make_float4(a.x + b4.x, a.y + b4.y, a.z + b4.z, a.w + b4.w));
  } else if constexpr (EPI == EPI_RESID) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + o) =
        make_float4(in.x + (a.x + b4.x), in.y + (a.y + b4.y), in.z + (a.z + b4.z), in.w + (a.w + b4.w));
  } else if constexpr (EPI == EPI_GELU) {
    float g0, g1, g2, g3, d0, d1, d2, d3;
    gelu_both(a.x + b4.x, g0, d0);
    gelu_both(a.y + b4.y, g1, d1);
    gelu_both(a.z + b4.z, g2, d2);
    gelu_both(a.w + b4.w, g3, d3);
    store4(reinterpret_cast<T*>(p.C) + o, make_float4(d0, d1, d2, d3));
    store4(reinterpret_cast<T*>(p.C2) + o, make_float4(g0, g1, g2, g3));
  } else if constexpr (EPI == EPI_GELU_BWD) {
    store4(reinterpret_cast<T*>(p.C) + o, make_float4(a.x * in.x, a.y * in.y, a.z * in.z, a.w * in.w));
  } else {
    if (p.accumulate) a = make_float4(in.x + a.x, in.y + a.y, in.z + a.z, in.w + a.w);
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + o) = a;
  }
}

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// EPI_STORE_ODOT: one lane's share of a row sum over a head's 64 columns: the
// group as stored (T-rounded acc + bias) times its aux values; the 16 lanes
// of the quarter wave (one row, one head) add theirs and the first writes it.
// valid (row and columns inside the output) is the same for the 16 lanes.
template <typename T>
__device__ __forceinline__ void odot_rowsum(const Params& p, int m, int n, float4 a, float4 b4, float4 o, bool valid,
                                            int lane) {
  float d = 0.f;
  if (valid)
    d = to_f(from_f<T>(a.x + b4.x)) * o.x + to_f(from_f<T>(a.y + b4.y)) * o.y + to_f(from_f<T>(a.z + b4.z)) * o.z +
        to_f(from_f<T>(a.w + b4.w)) * o.w;
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) d += __shfl_xor(d, off, WAVE);
  if (valid && (lane & 15) == 0) {
    const int b = m / p.tn, tt = m - b * p.tn;
    p.dv[((int64_t)b * p.heads + n / 64) * p.tn + tt] = d;
  }
}

// Stage acc through LDS (smem, at least PASS_ROWS * (BN + 4) floats) and run
// the epilogue.  Waves whose sub-tile rows fall in the current pass write.
// Thread t handles the column groups g = t + i * NT of a pass (row g / CG,
// 4 columns at 4 * (g % CG)).  Its groups cycle through NCOL column positions
// (one when NT is a multiple of CG), whose bias is loaded once; the pass's
// other inputs are loaded before the accumulators are staged, so their latency
// overlaps the staging.
template <typename T, int EPI, int SPLIT, int BM, int BN, int PASS_ROWS, typename ACC, int FM, int FN, int NT = 256,
          int WCOLS = 2>
__device__ __forceinline__ void epilogue_lds(const Params& p, ACC (&acc)[FM][FN], char* smem, int m0, int n0,
                                             int wm, int wn, int lane, int t) {
  using M_ = Mf<T>;
  constexpr int WROWS = NT / 64 / WCOLS;  // waves: WROWS rows x WCOLS columns of sub-tiles
  constexpr int WM = BM / WROWS, WN = BN / WCOLS;
  constexpr int LDW = BN + 4;
  constexpr int CG = BN / 4;                     // column groups per row
  constexpr int NG = PASS_ROWS * CG / NT;        // a thread's groups per pass
  constexpr int NCOL = CG / gcd_c(NT % CG, CG);  // distinct column positions of a thread
  // a thread's NG groups of a pass are unrolled and every group uses the bias
  // loaded once above: a load inside the group loop would be waited for after
  // the previous groups' stores, and vmcnt counts stores too, so each group
  // would wait for the last one's stores to complete.  Epilogues that read an
  // input keep a pass of it in registers, which bounds them to NG <= 16.
  constexpr bool IN = epi_reads<EPI, SPLIT>() && NG <= 16;
  constexpr bool UNR = IN || !epi_reads<EPI, SPLIT>();
  static_assert((PASS_ROWS * CG) % NT == 0 && WROWS * WCOLS * 64 == NT, "epilogue thread mapping");
  float* st = reinterpret_cast<float*>(smem);
  // group i's row in the pass and its column position (index i % NCOL)
  auto row_of = [&](int i) { return NCOL == 1 ? t / CG + i * (NT / CG) : (t + i * NT) / CG; };
  int c4[NCOL], n[NCOL];
  bool full[NCOL];
  float4 b4[NCOL];
#pragma unroll
  for (int j = 0; j < NCOL; ++j) {
    c4[j] = (t + j * NT) % CG;
    n[j] = n0 + c4[j] * 4;
    full[j] = n[j] + 3 < p.N && (SPLIT || (p.ldc & 3) == 0);
    b4[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!SPLIT && EPI != EPI_STORE_ODOT && full[j] && p.bias) b4[j] = *reinterpret_cast<const float4*>(p.bias + n[j]);
  }
  // the whole tile inside the output, every group 16-byte aligned
  const bool tile_full = m0 + BM <= p.M && n0 + BN <= p.N && (SPLIT ? (p.N & 3) == 0 : (p.ldc & 3) == 0);
  // A 16-bit input (the GELU derivative) is loaded for every pass before the
  // first store, kept as raw bf16 pairs (as many registers as one pass of
  // floats): a later pass's loads would otherwise wait for the earlier passes'
  // stores.  Wider inputs are loaded pass by pass (register budget).
  constexpr int NP = BM / PASS_ROWS;
  constexpr bool PRE = IN && (EPI == EPI_GELU_BWD || EPI == EPI_STORE_ODOT) && sizeof(T) == 2;
  // EPI_STORE_ODOT: the 16 lanes of a thread quarter-wave hold one row's 64
  // columns of one head, which their row sum reduces over
  constexpr bool ODOT = EPI == EPI_STORE_ODOT && IN && NCOL == 1 && CG % 16 == 0;
  uint2 raw[PRE ? NP : 1][PRE ? NG : 1];
  if constexpr (PRE) {
#pragma unroll
    for (int ps = 0; ps < NP; ++ps)
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int m = m0 + ps * PASS_ROWS + row_of(i), j = i % NCOL;
        raw[ps][i] = (full[j] && m < p.M) ? *reinterpret_cast<const uint2*>(reinterpret_cast<const T*>(p.aux) +
                                                                            (int64_t)m * p.ldc + n[j])
                                          : make_uint2(0u, 0u);
      }
  }
#pragma unroll
  for (int pass = 0; pass < NP; ++pass) {
    float4 in[IN ? NG : 1];
    if constexpr (PRE) {
#pragma unroll
      for (int i = 0; i < NG; ++i) {  // bf16 element k sits in the high half of its 32-bit slot
        const uint2 v = raw[pass][i];
        in[i] = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                            __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
      }
    } else if constexpr (IN) {
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int m = m0 + pass * PASS_ROWS + row_of(i), j = i % NCOL;
        in[i] = (full[j] && m < p.M) ? epi_load<T, EPI, SPLIT>(p, m, (int64_t)m * p.ldc + n[j])
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    __syncthreads();
    if (wm * WM >= pass * PASS_ROWS && wm * WM < (pass + 1) * PASS_ROWS) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < M_::NA; ++e) {
            const int r = wm * WM - pass * PASS_ROWS + i * M_::R + M_::row(e, lane);
            const int c = wn * WN + j * M_::R + M_::col(lane);
            st[r * LDW + c] = acc[i][j][e];
          }
    }
    __syncthreads();
    if constexpr (UNR) {
      if (tile_full) {  // no loads among the stores: nothing makes a group wait for earlier stores
#pragma unroll
        for (int i = 0; i < NG; ++i) {
          const int r = row_of(i), j = i % NCOL;
          float4 x_in = make_float4(0.f, 0.f, 0.f, 0.f);
          if constexpr (IN) x_in = in[i];
          const float4 a = *reinterpret_cast<const float4*>(st + r * LDW + c4[j] * 4);
          epi_group_full<T, EPI, SPLIT>(p, m0 + pass * PASS_ROWS + r, n[j], a, x_in, b4[j]);
          if constexpr (ODOT) odot_rowsum<T>(p, m0 + pass * PASS_ROWS + r, n[j], a, b4[j], x_in, true, lane);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
          const int r = row_of(i), j = i % NCOL;
          const int m = m0 + pass * PASS_ROWS + r;
          const bool ok = m < p.M && n[j] < p.N;
          float4 x_in = make_float4(0.f, 0.f, 0.f, 0.f);
          if constexpr (IN) x_in = in[i];
          const float4 a = *reinterpret_cast<const float4*>(st + r * LDW + c4[j] * 4);
          if (ok) epi_group<T, EPI, SPLIT>(p, m, n[j], a, full[j], x_in, b4[j]);
          if constexpr (ODOT) odot_rowsum<T>(p, m, n[j], a, b4[j], x_in, ok, lane);  // every lane shuffles
        }
      }
    } else {
      for (int g = t; g < PASS_ROWS * CG; g += NT) {
        const int r = g / CG, c = g % CG;
        const int m = m0 + pass * PASS_ROWS + r, nn = n0 + c * 4;
        if (m >= p.M || nn >= p.N) continue;
        epi_group_inline<T, EPI, SPLIT>(p, m, nn, *reinterpret_cast<const float4*>(st + r * LDW + c * 4));
      }
    }
  }
}

template <typename T, int TA, int TB, int EPI, int SPLIT, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_kernel(Params p) {
  using M_ = Mf<T>;
  constexpr int WM = BM / 2, WN = BN / 2;          // wave sub-tile
  constexpr int FM = WM / M_::R, FN = WN / M_::R;  // MFMA tiles per wave
  constexpr int KSTEPS = TKB / (M_::KG * 16);
  constexpr int STAGE = (BM + BN) * PITCH;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  int tm, tn, kz;
  tile_coords(p, tm, tn, kz);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb0 = kz * p.k_per_split;
  Params pe = p;  // the epilogue's view: a split writes its own slice of the workspace
  if (SPLIT) pe.ws = p.ws + (int64_t)kz * p.M * p.N;
  const int kend = min(p.K, kb0 + p.k_per_split);
  constexpr int BK = TKB / sizeof(T);
  const int nk = (kend - kb0 + BK - 1) / BK;

  const rsrc_t ra = make_rsrc(p.A, (TA ? (int64_t)p.K : (int64_t)p.M) * p.lda * (int64_t)sizeof(T));
  const rsrc_t rb = make_rsrc(p.B, (TB ? (int64_t)p.K : (int64_t)p.N) * p.ldb * (int64_t)sizeof(T));
  typename M_::acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < M_::NA; ++e) acc[i][j][e] = 0.f;

  const int frow = lane % M_::R, fk = (lane / M_::R) * 16;
  auto compute = [&](const char* sa) {
    const char* sb = sa + BM * PITCH;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uint4 af[FM], bfr[FN];
      const int koff = ks * (M_::KG * 16) + fk;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const uint4*>(sa + (wm * WM + i * M_::R + frow) * PITCH + koff);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(sb + (wn * WN + j * M_::R + frow) * PITCH + koff);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) M_::mma(acc[i][j], af[i], bfr[j]);
    }
  };

  char* buf0 = smem;
  char* buf1 = smem + STAGE;
  Loader<T, TA, BM> la;
  Loader<T, TB, BN> lb;
  if (nk > 0) {
    la.load(ra, p.lda, m0, kb0, t);
    lb.load(rb, p.ldb, n0, kb0, t);
    la.store(buf0, t);
    lb.store(buf0 + BM * PITCH, t);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(ra, p.lda, m0, kb0 + (kt + 1) * BK, t);
      lb.load(rb, p.ldb, n0, kb0 + (kt + 1) * BK, t);
    }
    compute((kt & 1) ? buf1 : buf0);
    if (more) {
      char* sn = (kt & 1) ? buf0 : buf1;
      la.store(sn, t);
      lb.store(sn + BM * PITCH, t);
    }
    __syncthreads();
  }

  // epilogue through LDS (the main loop's stages are free now)
  static_assert(2 * STAGE >= (BM <= 128 ? BM : 128) * (BN + 4) * 4, "LDS too small for the epilogue");
  epilogue_lds<T, EPI, SPLIT, BM, BN, (BM <= 128 ? BM : 128)>(pe, acc, smem, m0, n0, wm, wn, lane, t);
}

// 256x256 bf16 tile, 4 waves of 128x128, 32x32x16 MFMAs, explicitly interleaved:
// every k-step issues its 16 MFMAs interleaved with the LDS reads of the next
// k-step; the next tile's LDS stores and the tile after that's global loads are
// spread over the middle k-steps; one barrier per k-tile, placed so the last
// k-step's MFMAs overlap it.  The loop is branch-free: loads past the operands
// read zeros through the buffer descriptors and land in the unused LDS stage.
#define SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
}  // namespace
namespace dl {
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

// Tile configuration: BM = 256 rows x BN columns, BK k per stage, ST stages,
// OCC workgroups per CU (the register and LDS budget follow from it).
template <int BN_, int BK_, int ST_, int OCC_, int WAVES_ = 4, int WROWS_ = 2>
struct DlCfg {
  static constexpr int BM = 256, BN = BN_, BK = BK_, ST = ST_, OCC = OCC_, WAVES = WAVES_, WROWS = WROWS_;
  static constexpr int THREADS = 64 * WAVES, WCOLS = WAVES / WROWS;
  static constexpr int WM = BM / WROWS, WN = BN / WCOLS, FM = WM / 32, FN = WN / 32, KSTEPS = BK / 16;
  static_assert(FM * 32 * WROWS == BM && FN * 32 * WCOLS == BN, "whole 32x32 MFMA tiles per wave");
  static constexpr int WAVES_PER_SIMD = OCC * WAVES / 4;  // for the launch bounds
};

// k-contiguous operand rows hold BK * 2 bytes = CPR 16-byte chunks; the chunk
// order is XOR-permuted by row so that the 16 rows one ds_read_b128 pass
// touches land on distinct banks
template <int CPR>
__device__ __forceinline__ int swz_nt(int row) {
  if constexpr (CPR == 4) return (row >> 2) & 3;
  else return (row >> 1) & 7;
}
// row-contiguous operands: k-row kr's chunks are XOR-permuted so the 4 k-rows
// a transpose read pass touches do not stack on the same banks.  Rows of 24
// chunks (192 columns) already alternate between the two 128-byte halves of
// the banks from one k-row to the next; k-rows two apart are moved by 64
// bytes, an XOR below 8 so every chunk stays inside the row.
template <int CPR>
__device__ __forceinline__ int swz_t(int kr) {
  if constexpr (CPR == 24) return ((kr >> 1) & 1) << 2;
  else return ((kr & 3) << 1) | ((kr & 1) << 3);
}

// one wave instruction: lane i's 16 bytes at voff land at lds + 16 i (kept out of
// templates: host-side template instantiation drops kernels that call it directly)
__device__ __forceinline__ void load_lds16(rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

template <int TRANS, int ROWS, int BK, int WAVES = 4>
struct DlOperand {
  static constexpr int BYTES = ROWS * BK * 2;      // per stage
  static constexpr int NI = BYTES / 1024 / WAVES;  // load instructions per wave per stage
  static_assert(NI * 1024 * WAVES == BYTES, "whole load instructions per wave");
  static constexpr int CPR = TRANS ? ROWS / 8 : BK / 8;  // 16-byte chunks per LDS row
  static_assert(TRANS ? (CPR == 24 || (CPR >= 16 && (CPR & (CPR - 1)) == 0)) : (CPR == 4 || CPR == 8),
                "chunk permutations stay inside the row");
  uint32_t off[NI];
  uint32_t kstep;  // bytes per BK of k
  __device__ __forceinline__ void init(int64_t ld, int row0, int kb0, int w, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      // the instruction's lane writes LDS chunk q: row q / CPR, position q % CPR
      const int q = (w * NI + i) * 64 + lane;
      const int r = q / CPR, cq = q % CPR;
      int64_t e;
      if constexpr (TRANS == 0) {
        const int c = cq ^ swz_nt<CPR>(r);
        e = (int64_t)(row0 + r) * ld + kb0 + c * 8;
      } else {
        const int c = cq ^ swz_t<CPR>(r);
        e = (int64_t)(kb0 + r) * ld + row0 + c * 8;
      }
      off[i] = (uint32_t)(e * 2);
    }
    kstep = TRANS ? (uint32_t)(BK * ld * 2) : (uint32_t)(BK * 2);
  }
  __device__ __forceinline__ void issue(rsrc_t r, char* lds, int kt, int w) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) load_lds16(r, lds + (w * NI + i) * 1024, off[i] + (uint32_t)kt * kstep);
  }
  // 32x32x16 fragment: rows rb..rb+31 of the tile, k-step ks (16 k)
  __device__ __forceinline__ uint4 frag(const char* lds, int rb, int ks, int lane) const {
    if constexpr (TRANS == 0) {
      const int row = rb + (lane & 31);
      const int c = (ks * 2 + (lane >> 5)) ^ swz_nt<CPR>(row);
      return *reinterpret_cast<const uint4*>(lds + row * (BK * 2) + c * 16);
    } else {
      const int g = lane >> 4, s = lane & 15;
      const int mm = rb + 16 * (g & 1) + 4 * (s & 3);
      const int kr0 = ks * 16 + 8 * (g >> 1) + (s >> 2);
      const int c = mm >> 3, sub = (mm & 7) * 2;
      const char* p0 = lds + kr0 * (ROWS * 2) + ((c ^ swz_t<CPR>(kr0)) * 16) + sub;
      const char* p1 = lds + (kr0 + 4) * (ROWS * 2) + ((c ^ swz_t<CPR>(kr0 + 4)) * 16) + sub;
      v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p0);
      v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p1);
      uint2 a = bitcast<uint2>(lo), b = bitcast<uint2>(hi);
      return make_uint4(a.x, a.y, b.x, b.y);
    }
  }
};

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt simm16 on gfx9: vmcnt bits [3:0] and [15:14]; expcnt [6:4] and
  // lgkmcnt [11:8] left at their maxima (no wait)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// wait until at most n tiles' loads (NL instructions each per wave) are outstanding, n in 0..3
template <int NL>
__device__ __forceinline__ void wait_tiles(int n) {
  if constexpr (3 * NL < 64) {
    if (n >= 3) { wait_vm<3 * NL>(); return; }
  }
  if constexpr (2 * NL < 64) {
    if (n == 2) { wait_vm<2 * NL>(); return; }
  }
  if (n >= 1) wait_vm<NL>();
  else wait_vm<0>();
}

// Iteration j: once tile j has landed (explicit vmcnt wait) and every wave is
// past the barrier - so every read of tile j-1 is complete - tile j+ST-1 is
// loaded into tile j-1's stage (wr); then tile j's k-steps are read from its
// stage (rd), each interleaved with the MFMAs of the previous k-step (for
// k-step 0, the last k-step of tile j-1).  rd and wr are distinct stages:
// declaring them __restrict__ lets the compiler drop its blanket wait on
// outstanding direct-to-LDS loads before each LDS read; the real dependencies
// are the explicit wait and the barrier.
template <int TA, int TB, typename C, int NL>
__device__ __forceinline__ void dl_iter(const char* __restrict__ rd, char* __restrict__ wr, int kt, int nk,
                                        const DlOperand<TA, 256, C::BK, C::WAVES>& oa,
                                        const DlOperand<TB, C::BN, C::BK, C::WAVES>& ob,
                                        rsrc_t ra, rsrc_t rb, f32x16 (&acc)[C::FM][C::FN], uint4 (&fa)[2][C::FM],
                                        uint4 (&fb)[2][C::FN], int wm, int wn, int w, int lane) {
  constexpr int FM = C::FM, FN = C::FN, ST = C::ST;
  constexpr int ABYTES = DlOperand<TA, 256, C::BK, C::WAVES>::BYTES;
  constexpr int NR = (TA ? 2 : 1) * FM + (TB ? 2 : 1) * FN;  // LDS read instructions per k-step
  wait_tiles<NL>(min(ST - 2, nk - 1 - kt));
  __syncthreads();
  if (kt + ST - 1 < nk) {
    oa.issue(ra, wr, kt + ST - 1, w);
    ob.issue(rb, wr + ABYTES, kt + ST - 1, w);
  }
#pragma unroll
  for (int h = 0; h < C::KSTEPS; ++h) {
    const int sl = h & 1;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[sl][i] = oa.frag(rd, wm * C::WM + i * 32, h, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[sl][j] = ob.frag(rd + ABYTES, wn * C::WN + j * 32, h, lane);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) Mf<bf16>::mma(acc[i][j], fa[sl ^ 1][i], fb[sl ^ 1][j]);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      SGB(0x008, 1);
      SGB(0x100, 1);
    }
    SGB(0x008, FM * FN - NR > 0 ? FM * FN - NR : 0);
  }
}

template <int TA, int TB, int EPI, int SPLIT, typename C>
__global__ __launch_bounds__(C::THREADS, C::WAVES_PER_SIMD) void gemm_dl_kernel(Params p) {
  typedef bf16 T;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, FM = C::FM, FN = C::FN, ST = C::ST;
  using OA = DlOperand<TA, BM, BK, C::WAVES>;
  using OB = DlOperand<TB, BN, BK, C::WAVES>;
  constexpr int STAGE = OA::BYTES + OB::BYTES;
  constexpr int NL = OA::NI + OB::NI;
  constexpr int EPI_BYTES = 128 * (BN + 4) * 4;
  constexpr int SMEM = (ST * STAGE > EPI_BYTES) ? ST * STAGE : EPI_BYTES;
  static_assert(C::KSTEPS % 2 == 0, "k-steps alternate between two fragment slots");
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w / C::WCOLS, wn = w % C::WCOLS;
  int tm, tn, kz;
  tile_coords(p, tm, tn, kz);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb0 = kz * p.k_per_split;
  Params pe = p;  // the epilogue's view: a split writes its own slice of the workspace
  if (SPLIT) pe.ws = p.ws + (int64_t)kz * p.M * p.N;
  const int kend = min(p.K, kb0 + p.k_per_split);
  const int nk = (kend - kb0 + BK - 1) / BK;
  const rsrc_t ra = make_rsrc(p.A, (TA ? (int64_t)p.K : (int64_t)p.M) * p.lda * 2);
  const rsrc_t rb = make_rsrc(p.B, (TB ? (int64_t)p.K : (int64_t)p.N) * p.ldb * 2);
  OA oa;
  OB ob;
  oa.init(p.lda, m0, kb0, w, lane);
  ob.init(p.ldb, n0, kb0, w, lane);
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // slot 1 holds "the last k-step of tile -1": zeros, so the first MFMAs on it add nothing
  uint4 fa[2][FM], fb[2][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) fa[1][i] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < FN; ++j) fb[1][j] = make_uint4(0, 0, 0, 0);
  // prologue: tiles 0..ST-2 in flight (stage ST-1 is filled by the first iteration)
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nk) {
      oa.issue(ra, smem + s * STAGE, s, w);
      ob.issue(rb, smem + s * STAGE + OA::BYTES, s, w);
    }
  int sc = 0;  // stage of tile kt
  for (int kt = 0; kt < nk; ++kt) {
    const int sw = sc == 0 ? ST - 1 : sc - 1;
    dl_iter<TA, TB, C, NL>(smem + sc * STAGE, smem + sw * STAGE, kt, nk, oa, ob, ra, rb, acc, fa, fb, wm, wn, w,
                           lane);
    sc = sc + 1 == ST ? 0 : sc + 1;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) Mf<bf16>::mma(acc[i][j], fa[1][i], fb[1][j]);
  __syncthreads();
  epilogue_lds<T, EPI, SPLIT, BM, BN, 128, f32x16, FM, FN, C::THREADS, C::WCOLS>(pe, acc, smem, m0, n0, wm, wn,
                                                                                lane, t);
}

}  // namespace dl
namespace {
using dl::gemm_dl_kernel;
// out[m][n] = (acc ? out : 0) + sum_z ws[z][m][n], z in increasing order
__global__ void splitk_reduce(const float* __restrict__ ws, int splits, int M, int N, float* out,
                              int64_t ldc, int accumulate) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)M * N;
  if (i >= total) return;
  float s = 0.f;
  for (int z = 0; z < splits; ++z) s += ws[(int64_t)z * total + i];
  const int64_t m = i / N, n = i % N;
  float* c = out + m * ldc + n;
  *c = accumulate ? *c + s : s;
}
// the same four columns at a time (N and ldc multiples of 4, 16-byte aligned rows)
__global__ void splitk_reduce4(const float* __restrict__ ws, int splits, int M, int N, float* out, int64_t ldc,
                               int accumulate) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
  const int64_t total = (int64_t)M * N;
  if (4 * i >= total) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int z = 0; z < splits; ++z) {
    const float4 v = *reinterpret_cast<const float4*>(ws + (int64_t)z * total + 4 * i);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  const int64_t m = 4 * i / N, n = 4 * i % N;
  float4* c = reinterpret_cast<float4*>(out + m * ldc + n);
  if (accumulate) {
    const float4 o = *c;
    s = make_float4(o.x + s.x, o.y + s.y, o.z + s.z, o.w + s.w);
  }
  *c = s;
}

// Timing events of the main kernel: when both are set they are attached to
// its dispatch (hipExtLaunchKernel), so timing adds no packets to the stream.
struct Ev {
  hipEvent_t start = nullptr, stop = nullptr;
};

template <typename T, int TA, int TB, int EPI, int SPLIT, int BM, int BN>
hipError_t launch(const Params& p, int splits, hipStream_t s, Ev ev) {
  dim3 grid(p.tiles_m * p.tiles_n * splits);
  if (ev.start)
    hipExtLaunchKernelGGL((gemm_kernel<T, TA, TB, EPI, SPLIT, BM, BN>), grid, dim3(256), 0, s, ev.start, ev.stop, 0,
                          p);
  else
    hipLaunchKernelGGL((gemm_kernel<T, TA, TB, EPI, SPLIT, BM, BN>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int TA, int TB, int EPI, int SPLIT, typename C>
hipError_t launch_dl(const Params& p, int splits, hipStream_t s, Ev ev) {
  dim3 grid(p.tiles_m * p.tiles_n * splits);
  if (ev.start)
    hipExtLaunchKernelGGL((gemm_dl_kernel<TA, TB, EPI, SPLIT, C>), grid, dim3(C::THREADS), 0, s, ev.start, ev.stop, 0,
                          p);
  else
    hipLaunchKernelGGL((gemm_dl_kernel<TA, TB, EPI, SPLIT, C>), grid, dim3(C::THREADS), 0, s, p);
  return hipGetLastError();
}

template <typename T, int TA, int TB, int EPI, int SPLIT>
hipError_t launch_tile(const Params& p, int tile, int splits, hipStream_t s, Ev ev) {
  if constexpr (sizeof(T) == 2) {
    if (tile == 0) return launch_dl<TA, TB, EPI, SPLIT, dl::DlCfg<128, 32, 3, 2>>(p, splits, s, ev);
    if (tile == 1) return launch_dl<TA, TB, EPI, SPLIT, dl::DlCfg<256, 64, 2, 1>>(p, splits, s, ev);
    if (tile == 3) return launch_dl<TA, TB, EPI, SPLIT, dl::DlCfg<256, 64, 2, 1, 8>>(p, splits, s, ev);
    if (tile == 5) return launch_dl<TA, TB, EPI, SPLIT, dl::DlCfg<256, 32, 4, 1, 8>>(p, splits, s, ev);
    if (tile == 6) return launch_dl<TA, TB, EPI, SPLIT, dl::DlCfg<256, 32, 3, 1, 8>>(p, splits, s, ev);
    if constexpr (!SPLIT) {
      if (tile == 4) return launch_dl<TA, TB, EPI, SPLIT, dl::DlCfg<192, 64, 2, 1, 8, 4>>(p, splits, s, ev);
    }
  }
  return launch<T, TA, TB, EPI, SPLIT, 128, 128>(p, splits, s, ev);
}

template <typename T>
hipError_t dispatch(const Gemm& g, const Params& p, int tile, int splits, hipStream_t s, Ev ev) {
  const int key = g.a_trans * 100 + g.b_trans * 10 + g.epi;
  if (splits > 1) {
    if (g.a_trans == 1 && g.b_trans == 1) return launch_tile<T, 1, 1, EPI_F32, 1>(p, tile, splits, s, ev);
    if (g.a_trans == 0 && g.b_trans == 1) return launch_tile<T, 0, 1, EPI_F32, 1>(p, tile, splits, s, ev);
    return hipErrorInvalidValue;
  }
  switch (key) {
    case 0 + EPI_STORE: return launch_tile<T, 0, 0, EPI_STORE, 0>(p, tile, 1, s, ev);
    case 0 + EPI_RESID: return launch_tile<T, 0, 0, EPI_RESID, 0>(p, tile, 1, s, ev);
    case 0 + EPI_GELU: return launch_tile<T, 0, 0, EPI_GELU, 0>(p, tile, 1, s, ev);
    case 0 + EPI_F32: return launch_tile<T, 0, 0, EPI_F32, 0>(p, tile, 1, s, ev);
    case 0 + EPI_CE_GRAD: return launch_tile<T, 0, 0, EPI_CE_GRAD, 0>(p, tile, 1, s, ev);
    case 10 + EPI_F32: return launch_tile<T, 0, 1, EPI_F32, 0>(p, tile, 1, s, ev);
    case 10 + EPI_STORE: return launch_tile<T, 0, 1, EPI_STORE, 0>(p, tile, 1, s, ev);
    case 10 + EPI_GELU_BWD: return launch_tile<T, 0, 1, EPI_GELU_BWD, 0>(p, tile, 1, s, ev);
    case 10 + EPI_STORE_ODOT:
      if constexpr (sizeof(T) == 2) return launch_tile<T, 0, 1, EPI_STORE_ODOT, 0>(p, tile, 1, s, ev);
      return hipErrorInvalidValue;
    case 110 + EPI_F32: return launch_tile<T, 1, 1, EPI_F32, 0>(p, tile, 1, s, ev);
    default: return hipErrorInvalidValue;
  }
}

// tiles: 0 = bf16 256x128 direct-load (2 per CU), 1 = bf16 256x256 direct-load
// (BK 64, 1 per CU), 2 = 128x128 register-staged (fp32 and the fallback),
// 3 = bf16 256x256 direct-load with 8 waves (two per SIMD, so one issues its
// loads while the other keeps the MFMA pipe busy; BK 64, 1 per CU), 4 = the
// same with 192 columns (waves 4 x 2): N = 768 products
// of 16384 rows make 256 tiles, one per CU, instead of 192
constexpr int TILE_BM[7] = {256, 256, 128, 256, 256, 256, 256};
constexpr int TILE_BN[7] = {128, 256, 128, 256, 192, 256, 256};

// Tile and K-split choice from measurements of the step's shapes on MI355X:
// the 8-wave 256x256 kernel for every bf16 product, or its 192-column variant
// where that fills the CUs better (forward products with N = 768: -10 to -12%
// alone; QKV, N = 2304: -4 to -12%).  Same-box step A/B against
// the 256x128 kernel (two workgroups per CU) and the 4-wave 256x256 kernel:
// forward products -0.28 ms, data gradients -0.2, weight gradients -0.3, the
// LM-head data gradient and the attention projection -0.1 each.  Tiles 0 and 1
// stay selectable for tuning runs.  Split-K (fp32 outputs only) takes the
// largest split count whose workgroups fill at most 192 of the 256 CUs (512
// slots for the two-per-CU tile 0) with at least 512 k per split: the weight
// gradients run beside the data-gradient chain, and leaving it a quarter of the
// CUs (and a quarter less split-K workspace traffic) was 0.14 ms faster per
// step than a full round (same box, 3 x 20 steps; 160 and 224 CUs: +0.07, +0.02).
void choose(int M, int N, int K, bool can_split, int dtype, int a_trans, int b_trans, int* tile_out,
            int* splits_out) {
  (void)a_trans;
  int tile = dtype == BF16 ? 3 : 2;
  // the 192-column tile where it needs at least 10% fewer tile-columns x rounds
  // of one workgroup per CU (N = 768: 256 tiles in one round instead of 192;
  // N = 2304: 768 tiles in three rounds instead of 576 in three).  Forward
  // (k-contiguous B) products only: the N = 768 data gradients are 10-17%
  // faster alone with it, but the step was not (same box, 3 x 20 steps: layer
  // data gradients +0.02 ms, LM-head data gradient +0.2 ms), since the 192
  // tiles of the 256-column kernel leave 64 CUs to the weight gradients that
  // run beside them on the second stream.
  static const bool dgrad192 = [] {
    const char* e = getenv("GPT_GEMM_DGRAD192");
    return e && e[0] == '1';
  }();
  if (tile == 3 && !can_split && (!b_trans || dgrad192)) {
    const int64_t r3 = cdiv(cdiv(M, 256) * cdiv(N, 256), 256), r4 = cdiv(cdiv(M, 256) * cdiv(N, 192), 256);
    if (r4 * 192 * 10 < r3 * 256 * 9) tile = 4;
  }
  int splits = 1;
  if (can_split) {
    const int64_t tiles = (int64_t)cdiv(M, TILE_BM[tile]) * cdiv(N, TILE_BN[tile]);
    const int64_t round = tile == 0 ? 512 : 192;  // workgroup slots split-K may fill
    const int64_t by_round = round / tiles, by_k = K / 512;
    splits = (int)std::max<int64_t>(1, std::min(by_round, by_k));
  }
  *tile_out = tile;
  *splits_out = splits;
}

}  // namespace

hipError_t splits_reduce(const float* ws, int splits, int M, int N, float* out, int64_t ldc, int accumulate,
                         hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int64_t total = (int64_t)M * N;
  if ((N & 3) == 0 && (ldc & 3) == 0 && ((uintptr_t)out & 15) == 0 && ((uintptr_t)ws & 15) == 0)
    hipLaunchKernelGGL(splitk_reduce4, dim3(cdiv(total / 4, 256)), dim3(256), 0, s, ws, splits, M, N, out, ldc,
                       accumulate);
  else
    hipLaunchKernelGGL(splitk_reduce, dim3(cdiv(total, 256)), dim3(256), 0, s, ws, splits, M, N, out, ldc,
                       accumulate);
  return hipGetLastError();
}

int gemm_pick_splits(int M, int N, int K, int a_trans, int b_trans) {
  int tile = 2, splits = 1;
  choose(M, N, K, true, BF16, a_trans, b_trans, &tile, &splits);
  return splits;
}

// GPT_GEMM_TILE=0..6 pins the tile (TILE_BM x TILE_BN) for tuning runs.
static int forced_tile() {
  static const int v = [] {
    const char* e = getenv("GPT_GEMM_TILE");
    return (e && e[0] >= '0' && e[0] <= '6') ? e[0] - '0' : -1;
  }();
  return v;
}

hipError_t gemm(const Gemm& g, hipStream_t s, hipEvent_t after_main, hipEvent_t before_main) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const bool can_split = g.ws != nullptr && g.splits > 1 && g.epi == EPI_F32;
  int tile = 2, splits = 1;
  choose(g.M, g.N, g.K, can_split, g.dtype, g.a_trans, g.b_trans, &tile, &splits);
  if (forced_tile() >= 0 && g.dtype == BF16) tile = forced_tile();
  if (tile == 4 && can_split) tile = 3;  // split-K products keep the 256-column tile
  // direct-to-LDS loads move 16-byte chunks: rows of other strides take the register-staged kernel
  if (tile != 2 && ((g.lda & 7) || (g.ldb & 7) || ((uintptr_t)g.A & 15) || ((uintptr_t)g.B & 15))) tile = 2;
  if (g.epi == EPI_STORE_ODOT) {  // row sums need 16 lanes per head-row: tiles 0, 2, 3 (one column slot per thread)
    if (g.dtype != BF16 || !g.dv || !g.aux || g.bias || g.tn <= 0 || g.heads <= 0 || g.N != 64 * g.heads ||
        g.M % g.tn || (g.ldc & 3))
      return hipErrorInvalidValue;
    if (tile == 1 || tile == 4) tile = 3;
  }
  if (g.epi == EPI_CE_GRAD && (!g.lse || !g.rowi || g.bias)) return hipErrorInvalidValue;
  if (can_split) splits = std::min(splits, g.splits);
  Params p{};
  p.A = g.A;
  p.B = g.B;
  p.lda = g.lda;
  p.ldb = g.ldb;
  p.M = g.M;
  p.N = g.N;
  p.K = g.K;
  p.C = g.C;
  p.ldc = g.ldc;
  p.bias = g.bias;
  p.R = g.R;
  p.C2 = g.C2;
  p.aux = g.aux;
  p.accumulate = g.accumulate;
  p.dv = g.dv;
  p.tn = g.tn;
  p.heads = g.heads;
  p.lse = g.lse;
  p.rowi = g.rowi;
  p.col0 = g.col0;
  p.scale = g.scale;
  p.tiles_m = cdiv(g.M, TILE_BM[tile]);
  p.tiles_n = cdiv(g.N, TILE_BN[tile]);
  p.ws = g.ws;
  const int bk = TKB / (g.dtype == BF16 ? 2 : 4);
  // a k-contiguous operand is read in whole k-tiles: its rows must be padded
  // (with zeros) up to the next tile when K is not a multiple of it
  const int64_t kpad = (int64_t)cdiv(g.K, bk) * bk;
  if ((!g.a_trans && g.lda < kpad) || (!g.b_trans && g.ldb < kpad)) return hipErrorInvalidValue;

  if (splits > 1) {
    // never more partial slices than the workspace holds
    const int64_t fit = g.ws_floats / ((int64_t)g.M * g.N);
    if (fit < splits) splits = (int)std::max<int64_t>(1, fit);
  }
  if (splits > 1) {
    const int kps = cdiv(cdiv(g.K, splits), bk) * bk;
    p.k_per_split = kps;
    splits = cdiv(g.K, kps);
    if ((int64_t)splits * g.M * g.N > g.ws_floats) return hipErrorInvalidValue;
  } else {
    p.k_per_split = g.K;
  }
  Ev ev;
  if (before_main && after_main) ev = Ev{before_main, after_main};
  hipError_t e =
      (g.dtype == BF16) ? dispatch<bf16>(g, p, tile, splits, s, ev) : dispatch<float>(g, p, tile, splits, s, ev);
  if (e == hipSuccess && after_main && !ev.start) e = hipEventRecord(after_main, s);
  if (e != hipSuccess || splits <= 1) return e;
  const int64_t total = (int64_t)g.M * g.N;
  if ((g.N & 3) == 0 && (g.ldc & 3) == 0 && ((uintptr_t)g.C & 15) == 0 && ((uintptr_t)g.ws & 15) == 0)
    hipLaunchKernelGGL(splitk_reduce4, dim3(cdiv(total / 4, 256)), dim3(256), 0, s, g.ws, splits, g.M, g.N,
                       reinterpret_cast<float*>(g.C), g.ldc, g.accumulate);
  else
    hipLaunchKernelGGL(splitk_reduce, dim3(cdiv(total, 256)), dim3(256), 0, s, g.ws, splits, g.M,
                       g.N, reinterpret_cast<float*>(g.C), g.ldc, g.accumulate);
  return hipGetLastError();
}

}  // namespace gk
