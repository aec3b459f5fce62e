// HBM-bound row kernels for gfx950: LayerNorm forward / backward (fused with
// the embedding gather and the residual-gradient add), column reductions and
// the fixed-order mean of the per-row losses.
//
// LayerNorm (lecture, pre-LN blocks and final LayerNorm; Zero page,
// Transformer Block): y = (x - mu) / sqrt(var + 1e-5) * g + b over the C
// channels of a row, biased variance, statistics in fp32.  With rms set the
// same kernels compute RMSNorm (CS336 pretraining page, the second block
// variant): mu = 0, no shift, y = x / sqrt(mean(x^2) + 1e-5) * g.  One wavefront owns
// one row; each lane keeps its float4 slices of the row in registers, so the
// row is read once.
#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr float LN_EPS = 1e-5f;
constexpr int MAXV = 8;  // float4 slices per lane: C <= 2048

// NV float4 slices per lane (C <= 256 NV): the registers, and so the
// occupancy, follow the row width (with a fixed 8 slots: 132 VGPRs, 3 waves
// per SIMD at C = 768)
template <typename T, bool EMBED, int NV, bool RMS>
__global__ __launch_bounds__(256) void ln_fwd_kernel(const float* __restrict__ x, const int32_t* __restrict__ tok,
                                                     const float* __restrict__ wte, const float* __restrict__ wpe,
                                                     int Tn, float* __restrict__ res0, const float* __restrict__ g,
                                                     const float* __restrict__ bb, T* __restrict__ y,
                                                     float* __restrict__ mu, float* __restrict__ rs, int rows, int C) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int nc = C >> 2;
  // every load (row, gain, shift) is issued before the first store: a load
  // issued after a store would wait for it (the vector memory counter counts both)
  float4 v[NV], gv[NV], bv[NV];
  int64_t wrow = 0;
  if constexpr (EMBED) wrow = (int64_t)tok[row] * C;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = lane + 64 * i;
    if (j < nc) {
      if constexpr (EMBED) {
        const float4 a = load4(wte + wrow + 4 * j);
        const float4 p = wpe ? load4(wpe + (int64_t)(row % Tn) * C + 4 * j) : make_float4(0.f, 0.f, 0.f, 0.f);
        v[i] = make_float4(a.x + p.x, a.y + p.y, a.z + p.z, a.w + p.w);
      } else {
        v[i] = load4(x + (int64_t)row * C + 4 * j);
      }
      gv[i] = load4(g + 4 * j);
      if constexpr (RMS) bv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      else bv[i] = load4(bb + 4 * j);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = lane + 64 * i;
    if (j < nc) {
      if constexpr (EMBED) store4(res0 + (int64_t)row * C + 4 * j, v[i]);
      s += v[i].x + v[i].y + v[i].z + v[i].w;
    }
  }
  const float mean = RMS ? 0.f : wave_sum(s) / C;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = lane + 64 * i;
    if (j < nc) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      ss += a * a + b * b + c * c + d * d;
    }
  }
  const float r = rsqrtf(wave_sum(ss) / C + LN_EPS);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = lane + 64 * i;
    if (j < nc) {
      const float4 gg = gv[i], b4 = bv[i];
      store4(y + (int64_t)row * C + 4 * j,
             make_float4((v[i].x - mean) * r * gg.x + b4.x, (v[i].y - mean) * r * gg.y + b4.y,
                         (v[i].z - mean) * r * gg.z + b4.z, (v[i].w - mean) * r * gg.w + b4.w));
    }
  }
  if (lane == 0) {
    mu[row] = mean;
    rs[row] = r;
  }
}

// LayerNorm backward.  dx = rstd (dxh - mean(dxh) - xh mean(dxh xh)) with
// dxh = dy g, xh = (x - mu) rstd; dres_out = dres_in + dx and its T copy.
// A workgroup handles LNB_ROWS rows and writes one partial row of
// [sum dy*xh | sum dy | sum dres_out] (3C floats): the gain and shift
// gradients, and the column sums of the residual gradient it produces (the
// bias gradient of the linear layer that feeds this residual stream).
constexpr int LNB_ROWS = 32;

// One wave takes one row at a time with no prefetch of the next, and x-hat and
// dy*g are recomputed for the output instead of kept: at C <= 768 (NV <= 3) the
// kernel stays within 120 VGPRs, so one of its workgroups fits on a CU beside an
// 8-wave GEMM workgroup (2 x 196 VGPRs per SIMD) of the other stream; with the
// prefetch (182 VGPRs) it waited for whole GEMM workgroups to finish.  Wider rows
// keep 24 NV floats per lane live (row data and column partials), so they take
// two workgroups per CU and up to 256 VGPRs (one and 512 above C = 1792)
// instead of spilling to scratch (C = 1024: 28-84 bytes per lane, C = 1600:
// 520-592 at four per CU; C = 1600 takes NV = 7).  A lane
// past the row (C not a multiple of 256) loads the last column slice and drops it.
template <typename TY, typename T, int NV, bool DRES, bool RMS>
__global__ __launch_bounds__(256, NV <= 3 ? 4 : (NV <= 7 ? 2 : 1)) void ln_bwd_kernel(const TY* __restrict__ dy, const float* __restrict__ x,
                                                         const float* __restrict__ mu, const float* __restrict__ rs,
                                                         const float* __restrict__ g, const float* __restrict__ dres_in,
                                                         float* __restrict__ dres_out, T* __restrict__ dres_T,
                                                         float* __restrict__ part, int rows, int C) {
  __shared__ float red[4][NV * 256];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nc = C >> 2;
  int jj[NV];
  bool ok[NV];
  float4 pg[NV], pb[NV], pc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = lane + 64 * i;
    ok[i] = j < nc;
    jj[i] = ok[i] ? j : nc - 1;
    pg[i] = pb[i] = pc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int r0 = blockIdx.x * LNB_ROWS;
  for (int k = 0; k < LNB_ROWS / 4; ++k) {
    const int row = r0 + w + 4 * k;
    if (row >= rows) break;
    float4 xv[NV], dv[NV], gv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t o = (int64_t)row * C + 4 * jj[i];
      xv[i] = load4(x + o);
      dv[i] = load4(dy + o);
      gv[i] = load4(g + 4 * jj[i]);
    }
    const float m = mu[row], r = rs[row];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (!ok[i]) { dv[i] = make_float4(0.f, 0.f, 0.f, 0.f); }
      const float4 xq = xv[i], d = dv[i], gg = gv[i];
      const float4 xh = make_float4((xq.x - m) * r, (xq.y - m) * r, (xq.z - m) * r, (xq.w - m) * r);
      const float4 dxh = make_float4(d.x * gg.x, d.y * gg.y, d.z * gg.z, d.w * gg.w);
      s1 += dxh.x + dxh.y + dxh.z + dxh.w;
      s2 += dxh.x * xh.x + dxh.y * xh.y + dxh.z * xh.z + dxh.w * xh.w;
      pg[i].x += d.x * xh.x; pg[i].y += d.y * xh.y; pg[i].z += d.z * xh.z; pg[i].w += d.w * xh.w;
      pb[i].x += d.x; pb[i].y += d.y; pb[i].z += d.z; pb[i].w += d.w;
    }
    const float m1 = RMS ? 0.f : wave_sum(s1) / C, m2 = wave_sum(s2) / C;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t o = (int64_t)row * C + 4 * jj[i];
      const float4 xq = xv[i], d = dv[i], gg = gv[i];
      const float4 prev = DRES ? load4(dres_in + o) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 xh = make_float4((xq.x - m) * r, (xq.y - m) * r, (xq.z - m) * r, (xq.w - m) * r);
      const float4 dxh = make_float4(d.x * gg.x, d.y * gg.y, d.z * gg.z, d.w * gg.w);
      const float4 out = make_float4(prev.x + r * (dxh.x - m1 - xh.x * m2), prev.y + r * (dxh.y - m1 - xh.y * m2),
                                     prev.z + r * (dxh.z - m1 - xh.z * m2), prev.w + r * (dxh.w - m1 - xh.w * m2));
      if (ok[i]) {
        store4(dres_out + o, out);
        store4(dres_T + o, out);
        pc[i].x += out.x; pc[i].y += out.y; pc[i].z += out.z; pc[i].w += out.w;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    if (q) __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (ok[i]) *reinterpret_cast<float4*>(&red[w][4 * (lane + 64 * i)]) = q == 0 ? pg[i] : (q == 1 ? pb[i] : pc[i]);
    __syncthreads();
    for (int c = threadIdx.x; c < C; c += 256)
      part[(int64_t)blockIdx.x * 3 * C + q * C + c] = red[0][c] + red[1][c] + red[2][c] + red[3][c];
  }
}

// Split-row form for C = 256 * WPR (the 124M width takes WPR = 3): a workgroup
// of WPR waves takes one row at a time, each lane owning 4 columns, so a lane
// keeps 12 column partials instead of 12 * NV and the kernel fits in 64 VGPRs:
// two of its waves fit on a SIMD beside an 8-wave GEMM workgroup of the other
// stream (the one-wave-per-row kernel above gets one).  The row's two sums
// cross the waves through LDS, one barrier per row (two slots, alternating by
// row, so a wave that runs ahead never overwrites sums still being read).  The
// next row's loads are issued before this row's barrier.  Column partials need
// no LDS reduction: no two threads of a workgroup own the same column.
template <typename TY, typename T, int WPR, bool DRES, bool RMS>
__global__ __launch_bounds__(64 * WPR, 8) void ln_bwd_rows_kernel(
    const TY* __restrict__ dy, const float* __restrict__ x, const float* __restrict__ mu,
    const float* __restrict__ rs, const float* __restrict__ g, const float* __restrict__ dres_in,
    float* __restrict__ dres_out, T* __restrict__ dres_T, float* __restrict__ part, int rows) {
  constexpr int C = 256 * WPR;
  __shared__ float2 sums[2][WPR];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = w * 256 + 4 * lane;
  const float4 gg = load4(g + col);
  float4 pg = make_float4(0.f, 0.f, 0.f, 0.f), pb = pg, pc = pg;
  const int r0 = blockIdx.x * LNB_ROWS;
  const int nr = min(LNB_ROWS, rows - r0);
  float4 xv = make_float4(0.f, 0.f, 0.f, 0.f), dv = xv, pv = xv;
  if (nr > 0) {
    const int64_t o = (int64_t)r0 * C + col;
    xv = load4(x + o);
    dv = load4(dy + o);
    if (DRES) pv = load4(dres_in + o);
  }
  for (int k = 0; k < nr; ++k) {
    const int row = r0 + k;
    const float m = mu[row], r = rs[row];
    const float4 xq = xv, d = dv, prev = pv;
    if (k + 1 < nr) {  // next row's loads ahead of this row's barrier
      const int64_t o = (int64_t)(row + 1) * C + col;
      xv = load4(x + o);
      dv = load4(dy + o);
      if (DRES) pv = load4(dres_in + o);
    }
    const float4 xh = make_float4((xq.x - m) * r, (xq.y - m) * r, (xq.z - m) * r, (xq.w - m) * r);
    const float4 dxh = make_float4(d.x * gg.x, d.y * gg.y, d.z * gg.z, d.w * gg.w);
    float s1 = dxh.x + dxh.y + dxh.z + dxh.w;
    float s2 = dxh.x * xh.x + dxh.y * xh.y + dxh.z * xh.z + dxh.w * xh.w;
    pg.x += d.x * xh.x; pg.y += d.y * xh.y; pg.z += d.z * xh.z; pg.w += d.w * xh.w;
    pb.x += d.x; pb.y += d.y; pb.z += d.z; pb.w += d.w;
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    if (lane == 0) sums[k & 1][w] = make_float2(s1, s2);
    __syncthreads();
    float t1 = 0.f, t2 = 0.f;
#pragma unroll
    for (int i = 0; i < WPR; ++i) {
      const float2 v = sums[k & 1][i];
      t1 += v.x;
      t2 += v.y;
    }
    const float m1 = RMS ? 0.f : t1 / C, m2 = t2 / C;
    const float4 out = make_float4(prev.x + r * (dxh.x - m1 - xh.x * m2), prev.y + r * (dxh.y - m1 - xh.y * m2),
                                   prev.z + r * (dxh.z - m1 - xh.z * m2), prev.w + r * (dxh.w - m1 - xh.w * m2));
    const int64_t o = (int64_t)row * C + col;
    store4(dres_out + o, out);
    store4(dres_T + o, out);
    pc.x += out.x; pc.y += out.y; pc.z += out.z; pc.w += out.w;
  }
  float* pp = part + (int64_t)blockIdx.x * 3 * C + col;
  store4(pp, pg);
  store4(pp + C, pb);
  store4(pp + 2 * C, pc);
}

// Batched fixed-order column reductions: job j adds sum_r part[r][c] (rows in
// order, in 16 interleaved row groups added in order) into out[c], or stores it.
// Block b belongs to the job with first_block <= b < next job's first_block and
// covers 16 of its columns.
__global__ __launch_bounds__(256) void reduce_jobs_kernel(const RedJob* __restrict__ jobs, int njobs, int accumulate) {
  __shared__ float red[16][17];
  int lo = 0, hi = njobs - 1;
  while (lo < hi) {  // last job whose first_block <= blockIdx.x
    const int mid = (lo + hi + 1) >> 1;
    if (jobs[mid].first_block <= (int)blockIdx.x) lo = mid;
    else hi = mid - 1;
  }
  const RedJob J = jobs[lo];
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int c = ((int)blockIdx.x - J.first_block) * 16 + cl;
  float s = 0.f;
  if (c < J.cols)
    for (int r = rg; r < J.nrows; r += 16) s += J.part[(int64_t)r * J.ld + c];
  red[rg][cl] = s;
  __syncthreads();
  if (rg == 0 && c < J.cols) {
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) tot += red[i][cl];
    J.out[c] = accumulate ? J.out[c] + tot : tot;
  }
}

// out[c] (+)= sum_r part[r][c]: a block covers 16 columns with 16 row groups;
// each thread sums its rows in order, then the 16 group sums are added in order.
__global__ __launch_bounds__(256) void reduce_rows_kernel(const float* __restrict__ part, int nrows, int cols,
                                                          int64_t ld, float* out, int accumulate) {
  __shared__ float red[16][17];
  const int cl = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int c = blockIdx.x * 16 + cl;
  float s = 0.f;
  if (c < cols)
    for (int r = rg; r < nrows; r += 16) s += part[(int64_t)r * ld + c];
  red[rg][cl] = s;
  __syncthreads();
  if (rg == 0 && c < cols) {
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) tot += red[i][cl];
    out[c] = accumulate ? out[c] + tot : tot;
  }
}

// part[y][c] = sum of rows [256 y, 256 y + 256) of column c.  A thread owns 8
// consecutive columns (16-byte loads for bf16, two for fp32) and a quarter of
// the block's rows; the four quarters are added in order through LDS.
template <typename T>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const T* __restrict__ x, int rows, int cols,
                                                             float* __restrict__ part) {
  __shared__ float red[4][64 * 8];
  const int ch = threadIdx.x & 63, sub = threadIdx.x >> 6;
  const int chunk = blockIdx.x * 64 + ch;
  const int c0 = chunk * 8;
  const int r0 = blockIdx.y * 256;
  const int r1 = min(rows, r0 + 256);
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  if (c0 < cols) {
#pragma unroll 4
    for (int r = r0 + sub; r < r1; r += 4) {
      const T* p = x + (int64_t)r * cols + c0;
      const float4 a = load4(p), b = load4(p + 4);
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) red[sub][ch * 8 + k] = acc[k];
  __syncthreads();
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int c = blockIdx.x * 512 + i;
    if (c < cols) part[(int64_t)blockIdx.y * cols + c] = red[0][i] + red[1][i] + red[2][i] + red[3][i];
  }
}

// out[0] = mean of x[0..n) summed in a fixed order; also ring[slot].  1024
// threads; thread t adds x[t], x[t + 1024], ... in order, then the waves' sums
// are added in wave order.
__global__ __launch_bounds__(1024) void mean_kernel(const float* __restrict__ x, int n, float* out, float* ring,
                                                    int slot) {
  __shared__ float red[16];
  const int t = threadIdx.x;
  float s = 0.f;
#pragma unroll 8
  for (int i = t; i < n; i += 1024) s += x[i];
  s = wave_sum(s);
  if ((t & 63) == 0) red[t >> 6] = s;
  __syncthreads();
  if (t == 0) {
    float m = red[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) m += red[k];
    m /= n;
    out[0] = m;
    if (ring) ring[slot] = m;
  }
}

}  // namespace

template <typename T, bool EMBED, int NV>
void ln_fwd_launch(const float* x, const int32_t* tok, const float* wte, const float* wpe, int Tn, float* res0,
                   const float* g, const float* b, void* y, float* mu, float* rstd, int rows, int C, hipStream_t s,
                   int rms) {
  if (rms)
    hipLaunchKernelGGL((ln_fwd_kernel<T, EMBED, NV, true>), dim3(cdiv(rows, 4)), dim3(256), 0, s, x, tok, wte, wpe,
                       Tn, res0, g, b, (T*)y, mu, rstd, rows, C);
  else
    hipLaunchKernelGGL((ln_fwd_kernel<T, EMBED, NV, false>), dim3(cdiv(rows, 4)), dim3(256), 0, s, x, tok, wte, wpe,
                       Tn, res0, g, b, (T*)y, mu, rstd, rows, C);
}
template <typename T, bool EMBED>
hipError_t ln_fwd_nv(const float* x, const int32_t* tok, const float* wte, const float* wpe, int Tn, float* res0,
                     const float* g, const float* b, void* y, float* mu, float* rstd, int rows, int C, hipStream_t s,
                     int rms) {
  if (C % 4 || C > 4 * 64 * MAXV) return hipErrorInvalidValue;
  switch ((C / 4 + 63) / 64) {  // float4 slices per lane
    case 1: ln_fwd_launch<T, EMBED, 1>(x, tok, wte, wpe, Tn, res0, g, b, y, mu, rstd, rows, C, s, rms); break;
    case 2: ln_fwd_launch<T, EMBED, 2>(x, tok, wte, wpe, Tn, res0, g, b, y, mu, rstd, rows, C, s, rms); break;
    case 3: ln_fwd_launch<T, EMBED, 3>(x, tok, wte, wpe, Tn, res0, g, b, y, mu, rstd, rows, C, s, rms); break;
    case 4: ln_fwd_launch<T, EMBED, 4>(x, tok, wte, wpe, Tn, res0, g, b, y, mu, rstd, rows, C, s, rms); break;
    case 5:
    case 6: ln_fwd_launch<T, EMBED, 6>(x, tok, wte, wpe, Tn, res0, g, b, y, mu, rstd, rows, C, s, rms); break;
    default: ln_fwd_launch<T, EMBED, 8>(x, tok, wte, wpe, Tn, res0, g, b, y, mu, rstd, rows, C, s, rms); break;
  }
  return hipGetLastError();
}

hipError_t layernorm_fwd(int dtype, const float* x, const float* g, const float* b, void* y, float* mu,
                         float* rstd, int rows, int C, hipStream_t s, int rms) {
  if (dtype == BF16) return ln_fwd_nv<bf16, false>(x, nullptr, nullptr, nullptr, 1, nullptr, g, b, y, mu, rstd, rows, C, s, rms);
  return ln_fwd_nv<float, false>(x, nullptr, nullptr, nullptr, 1, nullptr, g, b, y, mu, rstd, rows, C, s, rms);
}

hipError_t embed_ln_fwd(int dtype, const int32_t* tok, const float* wte, const float* wpe, int Tn, float* res0,
                        const float* g, const float* b, void* y, float* mu, float* rstd, int rows, int C,
                        hipStream_t s, int rms) {
  if (dtype == BF16) return ln_fwd_nv<bf16, true>(nullptr, tok, wte, wpe, Tn, res0, g, b, y, mu, rstd, rows, C, s, rms);
  return ln_fwd_nv<float, true>(nullptr, tok, wte, wpe, Tn, res0, g, b, y, mu, rstd, rows, C, s, rms);
}

int layernorm_bwd_blocks(int rows) { return cdiv(rows, LNB_ROWS); }

// launch an instance of a LayerNorm-backward kernel with RMS chosen at run time
template <typename TY, typename T, int NV, bool DRES, typename... A>
void ln_bwd_launch(int rms, dim3 grid, hipStream_t s, A... args) {
  if (rms) hipLaunchKernelGGL((ln_bwd_kernel<TY, T, NV, DRES, true>), grid, dim3(256), 0, s, args...);
  else hipLaunchKernelGGL((ln_bwd_kernel<TY, T, NV, DRES, false>), grid, dim3(256), 0, s, args...);
}
template <typename TY, typename T, int WPR, bool DRES, typename... A>
void ln_bwd_rows_launch(int rms, dim3 grid, hipStream_t s, A... args) {
  if (rms) hipLaunchKernelGGL((ln_bwd_rows_kernel<TY, T, WPR, DRES, true>), grid, dim3(64 * WPR), 0, s, args...);
  else hipLaunchKernelGGL((ln_bwd_rows_kernel<TY, T, WPR, DRES, false>), grid, dim3(64 * WPR), 0, s, args...);
}

template <int NV, bool DRES>
hipError_t ln_bwd_nvd(int dtype, const void* dy, int dy_is_t, const float* x, const float* mu, const float* rstd,
                      const float* g, const float* dres_in, float* dres_out, void* dres_T, float* part, int rows,
                      int C, int nblk, hipStream_t s, int rms) {
  if (dtype == BF16 && dy_is_t)
    ln_bwd_launch<bf16, bf16, NV, DRES>(rms, dim3(nblk), s, (const bf16*)dy, x, mu, rstd, g, dres_in, dres_out,
                                        (bf16*)dres_T, part, rows, C);
  else if (dtype == BF16)
    ln_bwd_launch<float, bf16, NV, DRES>(rms, dim3(nblk), s, (const float*)dy, x, mu, rstd, g, dres_in, dres_out,
                                         (bf16*)dres_T, part, rows, C);
  else
    ln_bwd_launch<float, float, NV, DRES>(rms, dim3(nblk), s, (const float*)dy, x, mu, rstd, g, dres_in, dres_out,
                                          (float*)dres_T, part, rows, C);
  return hipGetLastError();
}
template <int NV>
hipError_t ln_bwd_nv(int dtype, const void* dy, int dy_is_t, const float* x, const float* mu, const float* rstd,
                     const float* g, const float* dres_in, float* dres_out, void* dres_T, float* part, int rows,
                     int C, int nblk, hipStream_t s, int rms) {
  return dres_in ? ln_bwd_nvd<NV, true>(dtype, dy, dy_is_t, x, mu, rstd, g, dres_in, dres_out, dres_T, part, rows, C,
                                        nblk, s, rms)
                 : ln_bwd_nvd<NV, false>(dtype, dy, dy_is_t, x, mu, rstd, g, dres_in, dres_out, dres_T, part, rows, C,
                                         nblk, s, rms);
}

template <int WPR, bool DRES>
hipError_t ln_bwd_rows_d(int dtype, const void* dy, int dy_is_t, const float* x, const float* mu, const float* rstd,
                         const float* g, const float* dres_in, float* dres_out, void* dres_T, float* part, int rows,
                         int nblk, hipStream_t s, int rms) {
  if (dtype == BF16 && dy_is_t)
    ln_bwd_rows_launch<bf16, bf16, WPR, DRES>(rms, dim3(nblk), s, (const bf16*)dy, x, mu, rstd, g, dres_in,
                                              dres_out, (bf16*)dres_T, part, rows);
  else if (dtype == BF16)
    ln_bwd_rows_launch<float, bf16, WPR, DRES>(rms, dim3(nblk), s, (const float*)dy, x, mu, rstd, g, dres_in,
                                               dres_out, (bf16*)dres_T, part, rows);
  else
    ln_bwd_rows_launch<float, float, WPR, DRES>(rms, dim3(nblk), s, (const float*)dy, x, mu, rstd, g, dres_in,
                                                dres_out, (float*)dres_T, part, rows);
  return hipGetLastError();
}
hipError_t layernorm_bwd(int dtype, const void* dy, int dy_is_t, const float* x, const float* mu,
                         const float* rstd, const float* g, const float* dres_in, float* dres_out, void* dres_T,
                         float* part, int rows, int C, int* nblk_out, hipStream_t s, int rms) {
  const int nblk = layernorm_bwd_blocks(rows);
  if (nblk_out) *nblk_out = nblk;
  if (C % 4 || C > 4 * 64 * MAXV) return hipErrorInvalidValue;
  // the split-row kernel for the final LayerNorm (fp32 dy from the LM head),
  // which runs beside the head's dW product (2 x 221 VGPRs per SIMD: only a
  // 64-VGPR wave fits beside it): 377 -> 129 us in the step.  Inside the
  // layers the one-wave-per-row kernel was faster in the step (same box,
  // 3 x 20 steps: +0.1 ms with the split-row kernel there).
  if (!dy_is_t && !dres_in) {
    if (C == 512) return ln_bwd_rows_d<2, false>(dtype, dy, dy_is_t, x, mu, rstd, g, dres_in, dres_out, dres_T, part, rows, nblk, s, rms);
    if (C == 768) return ln_bwd_rows_d<3, false>(dtype, dy, dy_is_t, x, mu, rstd, g, dres_in, dres_out, dres_T, part, rows, nblk, s, rms);
    if (C == 1024) return ln_bwd_rows_d<4, false>(dtype, dy, dy_is_t, x, mu, rstd, g, dres_in, dres_out, dres_T, part, rows, nblk, s, rms);
  }
  switch ((C / 4 + 63) / 64) {  // float4 slices per lane
    case 1: return ln_bwd_nv<1>(dtype, dy, dy_is_t, x, mu, rstd, g, dres_in, dres_out, dres_T, part, rows, C, nblk, s, rms);
    case 2: return ln_bwd_nv<2>(dtype, dy, dy_is_t, x, mu, rstd, g, dres_in, dres_out, dres_T, part, rows, C, nblk, s, rms);
    case 3: return ln_bwd_nv<3>(dtype, dy, dy_is_t, x, mu, rstd, g, dres_in, dres_out, dres_T, part, rows, C, nblk, s, rms);
    case 4: return ln_bwd_nv<4>(dtype, dy, dy_is_t, x, mu, rstd, g, dres_in, dres_out, dres_T, part, rows, C, nblk, s, rms);
    case 5:
    case 6: return ln_bwd_nv<6>(dtype, dy, dy_is_t, x, mu, rstd, g, dres_in, dres_out, dres_T, part, rows, C, nblk, s, rms);
    case 7: return ln_bwd_nv<7>(dtype, dy, dy_is_t, x, mu, rstd, g, dres_in, dres_out, dres_T, part, rows, C, nblk, s, rms);
    default: return ln_bwd_nv<8>(dtype, dy, dy_is_t, x, mu, rstd, g, dres_in, dres_out, dres_T, part, rows, C, nblk, s, rms);
  }
}

hipError_t reduce_jobs(const RedJob* jobs, int njobs, int nblocks, int accumulate, hipStream_t s) {
  if (njobs <= 0 || nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_jobs_kernel, dim3(nblocks), dim3(256), 0, s, jobs, njobs, accumulate);
  return hipGetLastError();
}

hipError_t reduce_rows_f32(const float* part, int nrows, int cols, int64_t ld, float* out, int accumulate,
                           hipStream_t s) {
  hipLaunchKernelGGL(reduce_rows_kernel, dim3(cdiv(cols, 16)), dim3(256), 0, s, part, nrows, cols, ld, out,
                     accumulate);
  return hipGetLastError();
}

hipError_t colsum_partial(int dtype, const void* x, int rows, int cols, float* part, hipStream_t s) {
  if (cols % 8) return hipErrorInvalidValue;
  dim3 grid(cdiv(cols / 8, 64), cdiv(rows, 256));
  if (dtype == BF16)
    hipLaunchKernelGGL(colsum_partial_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)x, rows, cols, part);
  else
    hipLaunchKernelGGL(colsum_partial_kernel<float>, grid, dim3(256), 0, s, (const float*)x, rows, cols, part);
  return hipGetLastError();
}


hipError_t mean_f32(const float* x, int n, float* out, float* ring, int slot, hipStream_t s) {
  hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, s, x, n, out, ring, slot);
  return hipGetLastError();
}

}  // namespace gk
