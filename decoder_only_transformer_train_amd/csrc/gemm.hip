// MFMA GEMM for gfx950: C[m][n] = sum_k A(m,k) B(n,k) with fused epilogues.
//
// One template serves fp32 (16x16x4 f32 MFMA) and bf16 (16x16x32 bf16 MFMA):
// operand tiles are staged in LDS as [128 rows][128 bytes of k] with a
// 16-byte row pad, so every lane reads one conflict-free 16-byte fragment
// per MFMA step regardless of the element type.  Operands whose k dimension
// is not contiguous in memory (the weight-gradient and data-gradient
// products) are transposed in registers on their way into LDS, so global
// loads stay 16-byte and coalesced.  Workgroup: 4 waves in 2x2; the tile is
// BM x BN (256x256, 256x128 or 128x128, chosen per shape), each wave owns a
// (BM/2) x (BN/2) sub-tile, so a 256x256 tile reads half the LDS bytes per
// MFMA of a 128x128 one.  LDS is double-buffered with the next tile's global
// loads in flight during the current tile's MFMAs.  Workgroup ids are
// remapped so each XCD (ids are dealt round-robin to the 8 XCDs) works on a
// contiguous, grouped run of tiles that share operand rows in its L2.
#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

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

template <typename T, int TRANS, int ROWS>
struct Loader {
  static constexpr int NR = ROWS / 32;  // 16-byte registers per thread
  uint4 r[NR];
  // TRANS == 0: operand stored [rows][ld], k contiguous.
  // TRANS == 1: operand stored [K][ld], rows contiguous; a unit is 4 k-rows x E elements.
  __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, int row0, int rows,
                                       int k0, int kend, int t) {
    constexpr int E = Tr<T>::E;
    if constexpr (TRANS == 0) {
      const int cc = t & 7;
      const int k = k0 + cc * E;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int row = row0 + (t >> 3) + 32 * i;
        if (row < rows && k < kend)
          r[i] = *reinterpret_cast<const uint4*>(base + (int64_t)row * ld + k);
        else
          r[i] = make_uint4(0, 0, 0, 0);
      }
    } else {
      constexpr int MCH = ROWS / E;
#pragma unroll
      for (int u = 0; u < NR / 4; ++u) {
        const int unit = t + 256 * u;
        const int mc = unit % MCH, kg = unit / MCH;
        const int row = row0 + mc * E;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = k0 + kg * 4 + i;
          if (k < kend && row < rows)
            r[4 * u + i] = *reinterpret_cast<const uint4*>(base + (int64_t)k * ld + row);
          else
            r[4 * u + i] = make_uint4(0, 0, 0, 0);
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
          // 4 k-rows x 8 elements -> 8 rows x 4 k-elements (8 bytes each)
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
            *reinterpret_cast<uint2*>(s + (mc * 8 + e) * PITCH + kg * 8) = make_uint2(lo, hi);
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

template <typename T, int TA, int TB, int EPI, int SPLIT, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_kernel(Params p) {
  constexpr int WM = BM / 2, WN = BN / 2;    // wave sub-tile
  constexpr int FM = WM / 16, FN = WN / 16;  // 16x16 MFMA tiles per wave
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

  const T* A = reinterpret_cast<const T*>(p.A);
  const T* B = reinterpret_cast<const T*>(p.B);
  Loader<T, TA, BM> la;
  Loader<T, TB, BN> lb;
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    la.load(A, p.lda, m0, p.M, kb0, kend, t);
    lb.load(B, p.ldb, n0, p.N, kb0, kend, t);
    la.store(smem, t);
    lb.store(smem + BM * PITCH, t);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(A, p.lda, m0, p.M, kb0 + (kt + 1) * BK, kend, t);
      lb.load(B, p.ldb, n0, p.N, kb0 + (kt + 1) * BK, kend, t);
    }
    const char* sa = smem + cur * STAGE;
    const char* sb = sa + BM * PITCH;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 af[FM], bfr[FN];
      const int koff = ks * 64 + (lane >> 4) * 16;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const uint4*>(sa + (wm * WM + i * 16 + (lane & 15)) * PITCH + koff);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(sb + (wn * WN + j * 16 + (lane & 15)) * PITCH + koff);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mfma_frag(acc[i][j], af[i], bfr[j], T());
    }
    if (more) {
      char* sn = smem + (cur ^ 1) * STAGE;
      la.store(sn, t);
      lb.store(sn + BM * PITCH, t);
    }
    __syncthreads();
  }

  // epilogue: lane holds rows (lane / 16) * 4 + r, column lane % 16 of each 16x16 tile
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * WN + j * 16 + (lane & 15);
      if (n >= p.N) continue;
      const float bn = (p.bias != nullptr) ? p.bias[n] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * WM + i * 16 + (lane >> 4) * 4 + r;
        if (m >= p.M) continue;
        const float a = acc[i][j][r];
        if constexpr (SPLIT) {
          p.ws[((int64_t)blockIdx.z * p.M + m) * p.N + n] = a;
        } else {
          const int64_t o = (int64_t)m * p.ldc + n;
          if constexpr (EPI == EPI_STORE) {
            reinterpret_cast<T*>(p.C)[o] = from_f<T>(a + bn);
          } else if constexpr (EPI == EPI_RESID) {
            reinterpret_cast<float*>(p.C)[o] = p.R[o] + (a + bn);
          } else if constexpr (EPI == EPI_GELU) {
            const float u = a + bn;
            reinterpret_cast<T*>(p.C)[o] = from_f<T>(u);
            reinterpret_cast<T*>(p.C2)[o] = from_f<T>(gelu_f(u));
          } else if constexpr (EPI == EPI_GELU_BWD) {
            const float u = to_f(reinterpret_cast<const T*>(p.aux)[o]);
            reinterpret_cast<T*>(p.C)[o] = from_f<T>(a * gelu_grad_f(u));
          } else {  // EPI_F32
            float* c = reinterpret_cast<float*>(p.C);
            c[o] = p.accumulate ? c[o] + a : a;
          }
        }
      }
    }
  }
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
constexpr int TILE_SLOTS[3] = {256, 256, 512};          // resident workgroups on 256 CUs
constexpr double TILE_RATE[3] = {1.0, 0.8, 0.55};       // relative MFMA efficiency per tile

// Pick the tile (and, for split-capable products, the K split) with the
// smallest modelled time: waves of resident workgroups x per-tile work / rate.
void choose(int M, int N, int K, bool can_split, int* tile_out, int* splits_out) {
  double best = 1e300;
  for (int t = 0; t < 3; ++t) {
    const int64_t tiles = (int64_t)cdiv(M, TILE_BM[t]) * cdiv(N, TILE_BN[t]);
    for (int sp = 1; sp <= (can_split ? 32 : 1); ++sp) {
      const int kps = cdiv(cdiv(K, sp), 64) * 64;
      if (sp > 1 && kps < 256) break;
      const int64_t wgs = tiles * sp;
      const double waves = (double)((wgs + TILE_SLOTS[t] - 1) / TILE_SLOTS[t]);
      double cost = waves * (double)TILE_BM[t] * TILE_BN[t] * kps / TILE_RATE[t];
      if (sp > 1) cost += 3.0 * (double)sp * M * N;  // partial sums written, read, reduced
      if (cost < best * 0.999) {
        best = cost;
        *tile_out = t;
        *splits_out = sp;
      }
    }
  }
}

}  // namespace

int gemm_pick_splits(int M, int N, int K) {
  int tile = 2, splits = 1;
  choose(M, N, K, true, &tile, &splits);
  return splits;
}

hipError_t gemm(const Gemm& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const bool can_split = g.ws != nullptr && g.splits > 1 && g.epi == EPI_F32;
  int tile = 2, splits = 1;
  choose(g.M, g.N, g.K, can_split, &tile, &splits);
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
  if (splits > 1) {
    const int kps = cdiv(cdiv(g.K, splits), bk) * bk;
    p.k_per_split = kps;
    splits = cdiv(g.K, kps);
  } else {
    p.k_per_split = g.K;
  }
  hipError_t e = (g.dtype == BF16) ? dispatch<bf16>(g, p, tile, splits, s) : dispatch<float>(g, p, tile, splits, s);
  if (e != hipSuccess || splits <= 1) return e;
  const int64_t total = (int64_t)g.M * g.N;
  hipLaunchKernelGGL(splitk_reduce, dim3(cdiv(total, 256)), dim3(256), 0, s, g.ws, splits, g.M,
                     g.N, reinterpret_cast<float*>(g.C), g.ldc, g.accumulate);
  return hipGetLastError();
}

}  // namespace gk
