// MFMA GEMM for gfx950: C[m][n] = sum_k A(m,k) B(n,k) with fused epilogues.
//
// One template serves fp32 (16x16x4 f32 MFMA) and bf16 (32x32x16 bf16 MFMA,
// the shape that reaches the chip's dense peak from a single wave per SIMD):
// operand tiles are staged in LDS as [rows][128 bytes of k] with a 16-byte
// row pad, so every lane reads one conflict-free 16-byte fragment per MFMA
// step regardless of the element type.  Operands are read through buffer
// descriptors whose range ends at the operand, so loads past M, N or K
// return zeros without a branch.  Operands whose k dimension
// is not contiguous in memory (the weight-gradient and data-gradient
// products) are transposed in registers on their way into LDS, so global
// loads stay 16-byte and coalesced.  Workgroup: 4 waves in 2x2; the tile is
// BM x BN (256x256, 256x128 or 128x128, chosen per shape), each wave owns a
// (BM/2) x (BN/2) sub-tile.  LDS is double-buffered with the next tile's
// global loads in flight during the current tile's MFMAs; the 256x256 bf16
// kernel additionally interleaves its LDS reads, stores and global loads
// with the MFMAs by explicit scheduling groups.  Workgroup ids are
// remapped so each XCD (ids are dealt round-robin to the 8 XCDs) works on a
// contiguous, grouped run of tiles that share operand rows in its L2.
#include "common.h"
#include "kernels.h"

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
};

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

__device__ __forceinline__ void tile_coords(const Params& p, int& tm, int& tn) {
  const int nwg = gridDim.x;
  int id = blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
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
template <typename T, int EPI, int SPLIT>
__device__ __forceinline__ void epi_group(const Params& p, int m, int n, float4 a) {
  float v[4] = {a.x, a.y, a.z, a.w};
  const bool full = n + 3 < p.N;
  if constexpr (SPLIT) {
    float* o = p.ws + ((int64_t)blockIdx.z * p.M + m) * p.N + n;
    if (full && (p.N & 3) == 0) {
      *reinterpret_cast<float4*>(o) = a;
    } else {
      for (int k = 0; k < 4; ++k)
        if (n + k < p.N) o[k] = v[k];
    }
    return;
  }
  const int64_t o = (int64_t)m * p.ldc + n;
  if (!full || (p.ldc & 3)) {  // ragged edge: element by element
    for (int k = 0; k < 4; ++k) {
      if (n + k >= p.N) break;
      const float bn = p.bias ? p.bias[n + k] : 0.f;
      const float x = v[k];
      if constexpr (EPI == EPI_STORE) reinterpret_cast<T*>(p.C)[o + k] = from_f<T>(x + bn);
      else if constexpr (EPI == EPI_RESID) reinterpret_cast<float*>(p.C)[o + k] = p.R[o + k] + (x + bn);
      else if constexpr (EPI == EPI_GELU) {
        reinterpret_cast<T*>(p.C)[o + k] = from_f<T>(x + bn);
        reinterpret_cast<T*>(p.C2)[o + k] = from_f<T>(gelu_f(x + bn));
      } else if constexpr (EPI == EPI_GELU_BWD) {
        reinterpret_cast<T*>(p.C)[o + k] = from_f<T>(x * gelu_grad_f(to_f(reinterpret_cast<const T*>(p.aux)[o + k])));
      } else {
        float* c = reinterpret_cast<float*>(p.C);
        c[o + k] = p.accumulate ? c[o + k] + x : x;
      }
    }
    return;
  }
  float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (p.bias) b4 = *reinterpret_cast<const float4*>(p.bias + n);
  if constexpr (EPI == EPI_STORE) {
    store4(reinterpret_cast<T*>(p.C) + o, make_float4(a.x + b4.x, a.y + b4.y, a.z + b4.z, a.w + b4.w));
  } else if constexpr (EPI == EPI_RESID) {
    const float4 r = *reinterpret_cast<const float4*>(p.R + o);
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + o) =
        make_float4(r.x + (a.x + b4.x), r.y + (a.y + b4.y), r.z + (a.z + b4.z), r.w + (a.w + b4.w));
  } else if constexpr (EPI == EPI_GELU) {
    const float4 u = make_float4(a.x + b4.x, a.y + b4.y, a.z + b4.z, a.w + b4.w);
    store4(reinterpret_cast<T*>(p.C) + o, u);
    store4(reinterpret_cast<T*>(p.C2) + o, make_float4(gelu_f(u.x), gelu_f(u.y), gelu_f(u.z), gelu_f(u.w)));
  } else if constexpr (EPI == EPI_GELU_BWD) {
    const float4 u = load4(reinterpret_cast<const T*>(p.aux) + o);
    store4(reinterpret_cast<T*>(p.C) + o, make_float4(a.x * gelu_grad_f(u.x), a.y * gelu_grad_f(u.y),
                                                      a.z * gelu_grad_f(u.z), a.w * gelu_grad_f(u.w)));
  } else {
    float* c = reinterpret_cast<float*>(p.C) + o;
    if (p.accumulate) {
      const float4 c0 = *reinterpret_cast<const float4*>(c);
      a = make_float4(c0.x + a.x, c0.y + a.y, c0.z + a.z, c0.w + a.w);
    }
    *reinterpret_cast<float4*>(c) = a;
  }
}

// Stage acc through LDS (smem, at least PASS_ROWS * (BN + 4) floats) and run
// the epilogue.  Waves whose sub-tile rows fall in the current pass write.
template <typename T, int EPI, int SPLIT, int BM, int BN, int PASS_ROWS, typename ACC, int FM, int FN>
__device__ __forceinline__ void epilogue_lds(const Params& p, ACC (&acc)[FM][FN], char* smem, int m0, int n0,
                                             int wm, int wn, int lane, int t) {
  using M_ = Mf<T>;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int LDW = BN + 4;
  float* st = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int pass = 0; pass < BM / PASS_ROWS; ++pass) {
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
    for (int g = t; g < PASS_ROWS * (BN / 4); g += 256) {
      const int r = g / (BN / 4), c4 = g % (BN / 4);
      const int m = m0 + pass * PASS_ROWS + r, n = n0 + c4 * 4;
      if (m >= p.M || n >= p.N) continue;
      epi_group<T, EPI, SPLIT>(p, m, n, *reinterpret_cast<const float4*>(st + r * LDW + c4 * 4));
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
  int tm, tn;
  tile_coords(p, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb0 = blockIdx.z * p.k_per_split;
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
  epilogue_lds<T, EPI, SPLIT, BM, BN, (BM <= 128 ? BM : 128)>(p, acc, smem, m0, n0, wm, wn, lane, t);
}

// 256x256 bf16 tile, 4 waves of 128x128, 32x32x16 MFMAs, explicitly interleaved:
// every k-step issues its 16 MFMAs interleaved with the LDS reads of the next
// k-step; the next tile's LDS stores and the tile after that's global loads are
// spread over the middle k-steps; one barrier per k-tile, placed so the last
// k-step's MFMAs overlap it.  The loop is branch-free: loads past the operands
// read zeros through the buffer descriptors and land in the unused LDS stage.
#define SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
template <int TA, int TB, int EPI, int SPLIT>
__global__ __launch_bounds__(256, 1) void gemm256_kernel(Params p) {
  typedef bf16 T;
  using M_ = Mf<T>;
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128;
  constexpr int FM = 4, FN = 4;
  constexpr int STAGE = (BM + BN) * PITCH;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  tile_coords(p, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb0 = blockIdx.z * p.k_per_split;
  const int kend = min(p.K, kb0 + p.k_per_split);
  constexpr int BK = 64;
  const int nk = (kend - kb0 + BK - 1) / BK;
  const rsrc_t ra = make_rsrc(p.A, (TA ? (int64_t)p.K : (int64_t)p.M) * p.lda * 2);
  const rsrc_t rb = make_rsrc(p.B, (TB ? (int64_t)p.K : (int64_t)p.N) * p.ldb * 2);
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int frow = lane & 31, fk = (lane >> 5) * 16;
  const int arow = (wm * WM + frow) * PITCH + fk, brow = (wn * WN + frow) * PITCH + fk;
  Loader<T, TA, BM> la;
  Loader<T, TB, BN> lb;
  uint4 fa[2][FM], fb[2][FN];
  auto read_frags = [&](const char* st, int ks, int slot) {
    const char* sa = st + arow + ks * 32;
    const char* sb = st + BM * PITCH + brow + ks * 32;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[slot][i] = *reinterpret_cast<const uint4*>(sa + i * 32 * PITCH);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[slot][j] = *reinterpret_cast<const uint4*>(sb + j * 32 * PITCH);
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) M_::mma(acc[i][j], fa[slot][i], fb[slot][j]);
  };
  constexpr int NLOAD = Loader<T, TA, BM>::NR + Loader<T, TB, BN>::NR;          // buffer loads per tile
  constexpr int NSTORE = (TA ? (BM / 32) / 4 * 16 : BM / 32) + (TB ? (BN / 32) / 4 * 16 : BN / 32);
  // prologue: tile 0 into LDS stage 0, tile 1 in flight, k-step 0 fragments read
  la.load(ra, p.lda, m0, kb0, t);
  lb.load(rb, p.ldb, n0, kb0, t);
  la.store(smem, t);
  lb.store(smem + BM * PITCH, t);
  la.load(ra, p.lda, m0, kb0 + BK, t);
  lb.load(rb, p.ldb, n0, kb0 + BK, t);
  __syncthreads();
  read_frags(smem, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STAGE;
    char* nxt = smem + ((kt & 1) ^ 1) * STAGE;
    // k-step 0: MFMAs on slot 0, read k-step 1 into slot 1
    read_frags(cur, 1, 1);
    mfmas(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) { SGB(0x008, 1); SGB(0x100, 1); }
    SGB(0x008, 8);
    // k-step 1: store the next tile into the other stage while computing
    read_frags(cur, 2, 0);
    la.store(nxt, t);
    lb.store(nxt + BM * PITCH, t);
    mfmas(1);
#pragma unroll
    for (int i = 0; i < 8; ++i) { SGB(0x008, 1); SGB(0x100, 1); }
#pragma unroll
    for (int i = 0; i < 8; ++i) { SGB(0x008, 1); SGB(0x200, NSTORE / 8); }
    // k-step 2: global loads of the tile after next
    read_frags(cur, 3, 1);
    la.load(ra, p.lda, m0, kb0 + (kt + 2) * BK, t);
    lb.load(rb, p.ldb, n0, kb0 + (kt + 2) * BK, t);
    mfmas(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) { SGB(0x008, 1); SGB(0x100, 1); }
#pragma unroll
    for (int i = 0; i < 8; ++i) { SGB(0x008, 1); SGB(0x020, NLOAD / 8); }
    __syncthreads();
    // k-step 3: MFMAs on slot 1, read k-step 0 of the next tile into slot 0
    read_frags(nxt, 0, 0);
    mfmas(1);
#pragma unroll
    for (int i = 0; i < 8; ++i) { SGB(0x008, 1); SGB(0x100, 1); }
    SGB(0x008, 8);
  }

  epilogue_lds<T, EPI, SPLIT, BM, BN, 128>(p, acc, smem, m0, n0, wm, wn, lane, t);
}

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

template <typename T, int TA, int TB, int EPI, int SPLIT, int BM, int BN>
hipError_t launch(const Params& p, int splits, hipStream_t s) {
  dim3 grid(p.tiles_m * p.tiles_n, 1, splits);
  hipLaunchKernelGGL((gemm_kernel<T, TA, TB, EPI, SPLIT, BM, BN>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T, int TA, int TB, int EPI, int SPLIT>
hipError_t launch_tile(const Params& p, int tile, int splits, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (tile == 0) {
      dim3 grid(p.tiles_m * p.tiles_n, 1, splits);
      hipLaunchKernelGGL((gemm256_kernel<TA, TB, EPI, SPLIT>), grid, dim3(256), 0, s, p);
      return hipGetLastError();
    }
  }
  switch (tile) {
    case 0: return launch<T, TA, TB, EPI, SPLIT, 256, 256>(p, splits, s);
    case 1: return launch<T, TA, TB, EPI, SPLIT, 256, 128>(p, splits, s);
    default: return launch<T, TA, TB, EPI, SPLIT, 128, 128>(p, splits, s);
  }
}

template <typename T>
hipError_t dispatch(const Gemm& g, const Params& p, int tile, int splits, hipStream_t s) {
  const int key = g.a_trans * 100 + g.b_trans * 10 + g.epi;
  if (splits > 1) {
    if (g.a_trans == 1 && g.b_trans == 1) return launch_tile<T, 1, 1, EPI_F32, 1>(p, tile, splits, s);
    if (g.a_trans == 0 && g.b_trans == 1) return launch_tile<T, 0, 1, EPI_F32, 1>(p, tile, splits, s);
    return hipErrorInvalidValue;
  }
  switch (key) {
    case 0 + EPI_STORE: return launch_tile<T, 0, 0, EPI_STORE, 0>(p, tile, 1, s);
    case 0 + EPI_RESID: return launch_tile<T, 0, 0, EPI_RESID, 0>(p, tile, 1, s);
    case 0 + EPI_GELU: return launch_tile<T, 0, 0, EPI_GELU, 0>(p, tile, 1, s);
    case 0 + EPI_F32: return launch_tile<T, 0, 0, EPI_F32, 0>(p, tile, 1, s);
    case 10 + EPI_F32: return launch_tile<T, 0, 1, EPI_F32, 0>(p, tile, 1, s);
    case 10 + EPI_STORE: return launch_tile<T, 0, 1, EPI_STORE, 0>(p, tile, 1, s);
    case 10 + EPI_GELU_BWD: return launch_tile<T, 0, 1, EPI_GELU_BWD, 0>(p, tile, 1, s);
    case 110 + EPI_F32: return launch_tile<T, 1, 1, EPI_F32, 0>(p, tile, 1, s);
    default: return hipErrorInvalidValue;
  }
}

constexpr int TILE_BM[3] = {256, 256, 128};
constexpr int TILE_BN[3] = {256, 128, 128};

// Tile and K-split choice from measurements of the step's shapes on MI355X:
// 128x128 (two workgroups per CU) wins for K up to ~3K with most epilogues;
// the interleaved 256x256 kernel wins for long-K products with enough tiles.
// Split-K (weight gradients only) is sized so that tiles x splits fills about
// two workgroups per CU with at least 512 k per split.
void choose(int M, int N, int K, bool can_split, int dtype, int a_trans, int b_trans, int* tile_out,
            int* splits_out) {
  int tile = 2;
  const int64_t t256 = (int64_t)cdiv(M, 256) * cdiv(N, 256);
  if (dtype == BF16 && !a_trans && ((b_trans && K >= 3072) || K >= 8192) && t256 >= 160) tile = 0;
  int splits = 1;
  if (can_split) {
    const int64_t tiles = (int64_t)cdiv(M, TILE_BM[tile]) * cdiv(N, TILE_BN[tile]);
    while (tiles * splits < 512 && K / (splits * 2) >= 512) splits *= 2;
  }
  *tile_out = tile;
  *splits_out = splits;
}

}  // namespace

int gemm_pick_splits(int M, int N, int K) {
  int tile = 2, splits = 1;
  choose(M, N, K, true, BF16, 1, 1, &tile, &splits);
  return splits;
}

// GPT_GEMM_TILE=0|1|2 pins the tile (256x256, 256x128, 128x128) for tuning runs.
static int forced_tile() {
  static const int v = [] {
    const char* e = getenv("GPT_GEMM_TILE");
    return (e && e[0] >= '0' && e[0] <= '2') ? e[0] - '0' : -1;
  }();
  return v;
}

hipError_t gemm(const Gemm& g, hipStream_t s, hipEvent_t after_main) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const bool can_split = g.ws != nullptr && g.splits > 1 && g.epi == EPI_F32;
  int tile = 2, splits = 1;
  choose(g.M, g.N, g.K, can_split, g.dtype, g.a_trans, g.b_trans, &tile, &splits);
  if (forced_tile() >= 0) tile = forced_tile();
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
  p.tiles_m = cdiv(g.M, TILE_BM[tile]);
  p.tiles_n = cdiv(g.N, TILE_BN[tile]);
  p.ws = g.ws;
  const int bk = TKB / (g.dtype == BF16 ? 2 : 4);
  // a k-contiguous operand is read in whole k-tiles: its rows must be padded
  // (with zeros) up to the next tile when K is not a multiple of it
  const int64_t kpad = (int64_t)cdiv(g.K, bk) * bk;
  if ((!g.a_trans && g.lda < kpad) || (!g.b_trans && g.ldb < kpad)) return hipErrorInvalidValue;
  if (splits > 1) {
    const int kps = cdiv(cdiv(g.K, splits), bk) * bk;
    p.k_per_split = kps;
    splits = cdiv(g.K, kps);
  } else {
    p.k_per_split = g.K;
  }
  hipError_t e = (g.dtype == BF16) ? dispatch<bf16>(g, p, tile, splits, s) : dispatch<float>(g, p, tile, splits, s);
  if (e == hipSuccess && after_main) e = hipEventRecord(after_main, s);
  if (e != hipSuccess || splits <= 1) return e;
  const int64_t total = (int64_t)g.M * g.N;
  hipLaunchKernelGGL(splitk_reduce, dim3(cdiv(total, 256)), dim3(256), 0, s, g.ws, splits, g.M,
                     g.N, reinterpret_cast<float*>(g.C), g.ldc, g.accumulate);
  return hipGetLastError();
}

}  // namespace gk
