// The tied LM head fused with next-token cross-entropy, forward and backward,
// without ever storing a [rows, vocabulary] logits matrix ("GPT training"
// (Zero) page, output layer: the projection and the loss as one operator so
// that the [B*T, V] logits are not kept; CS336 page, section 1: the loss is
// the mean over rows of logsumexp(z) - z[y] with the row maximum taken out).
//
// With F the final-LayerNorm rows [N, C] and W the tied embedding [V, C],
// z = F W^T, p = softmax(z) per row, g = scale (p - onehot(y)):
//   dF = g W = scale (sum_v p_v W_v - W_y),   dW = g^T F.
// Two passes over the vocabulary, both streaming 32-row blocks of one operand
// through LDS while the other operand stays in registers:
//   pass 1 (per block of F rows): z tiles against every W block, a softmax
//     in one sweep (exponentials against a per-row reference, their running
//     sum), and sum_v p_v W_v accumulated - the forward pass of attention with
//     keys = values = W.  Its end gives the log-sum-exp, the row loss and dF.
//   pass 2 (per block of W rows): z tiles against every F block, recomputed,
//     g from the saved log-sum-exp, and dW accumulated.
// 8 N V C FLOPs against the algorithmic 6 N V C (the logits are computed
// twice); HBM traffic is F, W, dF, dW and per-row scalars.
//
// gfx950 layout of one workgroup (4 waves, one per SIMD):
//  * the contraction over C is split across the waves: wave w owns the
//    columns [c_lo, c_lo + 64 ng) (C / 64 column groups dealt out in order)
//    for both products, so it only ever reads its own slice of a streamed
//    block: it loads that slice itself (buffer_load ... lds, one wave
//    instruction = 1 KB) and refills its stage without waiting for the
//    other waves;
//  * z tiles are computed transposed (rows = streamed rows, columns = fixed
//    rows) so that a tile's accumulators are directly the B operand of the
//    second product; each wave's partial tile over its columns is summed with
//    the others' through LDS (each wave reduces one quarter of the tile's
//    accumulators in a fixed order, then every wave reads the whole sum), so
//    all waves hold the same bits of z and take the same softmax decisions;
//  * the second product reads the streamed block transposed with
//    ds_read_b64_tr_b16, so no transposed copy is stored;
//  * LDS rows of a slice are 128 ng bytes; their 16-byte chunks are
//    XOR-permuted by row so that the 16 rows of a ds_read_b128 pass and the
//    4 rows x 4 chunks of a transpose-read pass hit distinct banks.
#include "common.h"
#include "kernels.h"
#include "mfma_lds.h"

namespace gk {
namespace hd {
using namespace mx;

#define SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
constexpr int BV = 32;          // streamed rows per block
constexpr float HEADROOM = 64.f; // pass 1: p = 2^(z log2e - m) may reach 2^64 before a sweep is redone

struct Args {
  const bf16* fix;   // rows kept in registers: F (pass 1) or W (pass 2), [n_fix][C]
  const bf16* str;   // streamed rows: W (pass 1) or F (pass 2), [n_str][C]
  int n_fix, n_str, C;
  const int32_t* y;  // [N] targets
  const float* lse;  // pass 2: [N] natural-log log-sum-exp from pass 1
  float* loss;       // pass 1: [N] row losses
  float* lse_out;    // pass 1: [N]
  float* out;        // pass 1: dF [N][C]; pass 2: dW [V][C]
  int accumulate;    // pass 2: dW += instead of =
  float scale;       // gradients are those of scale * (sum of row losses)
  int* bad;          // pass 1: set to 1 when a target lies outside [0, V)
  int blk0;          // index of the launch's first block of fixed rows
  // pass 2's split of the streamed rows (nz > 1): workgroup z * tb + b takes
  // fixed block blk0 + b over streamed rows [z z_rows, (z + 1) z_rows) and
  // writes its partial dW to out + z z_stride, row f at (f - out_row0) C
  int nz, tb, z_rows, out_row0;
  int64_t z_stride;
  // pass 1 split over vocabulary segments (nz > 1): workgroup z * tb + b takes
  // fixed block blk0 + b against the streamed rows [z z_rows, (z + 1) z_rows)
  // and writes the segment's per-row reference, sum and target logit to
  // seg_s + z n_fix 4 and, when out is set, its unnormalised sum p W to
  // out + z z_stride; seg_combine_kernel then forms the row results
  float* seg_s;
};

// Column groups of 64 dealt to the 4 waves in order: wave w gets ng of them from column c_lo.
__device__ __forceinline__ void wave_range(int C, int w, int& ng, int& c_lo) {
  const int G = C >> 6, q = G >> 2, r = G & 3;
  ng = q + (w < r ? 1 : 0);
  c_lo = (w * q + min(w, r)) * 64;
}

// Physical 16-byte chunk of logical chunk ch in LDS row `row` of a slice whose
// rows are NG * 128 bytes.  NG odd: consecutive rows alternate between the two
// 128-byte halves of a 256-byte bank window, and the low 3 bits are XORed by a
// permutation of (row / 2) % 8; NG even: rows alias in the window and the low
// 4 bits are XORed by a permutation of row % 16.  Either way the 16 rows of a
// row-fragment pass and the 4 rows x 4 chunks of a transpose-read pass land on
// distinct 16-byte slots.  The map is its own inverse.
template <int NG>
__device__ __forceinline__ int phys(int ch, int row) {
  if constexpr (NG & 1) {
    const int i = (row >> 1) & 7;
    return ch ^ (((i & 1) << 2) | (i >> 1));
  } else {
    const int r = row & 15;
    return ch ^ (((r & 3) << 2) | (r >> 2));
  }
}

template <int NG>
struct Slice {
  static constexpr int RS = NG * 128;   // bytes per LDS row
  static constexpr int BYTES = BV * RS;  // one block's slice
  static constexpr int NLD = BYTES / 1024;  // wave load instructions per block
};

// row fragment (A operand of the z product): block row `row`, k-step ks (16 columns), lane half g
template <int NG>
__device__ __forceinline__ uint4 frag_row(const char* s, int row, int ks, int g) {
  const int ch = phys<NG>(ks * 2 + g, row);
  return *reinterpret_cast<const uint4*>(s + row * Slice<NG>::RS + ch * 16);
}
// transposed fragment (A operand of the second product): lane l holds column
// c0 + l % 32 of the slice and block rows r0 + 4 (l / 32) + j, then
// r0 + 8 + 4 (l / 32) + j (j = 0..3): the k order of pack_half over rows
// r0 .. r0 + 15.  In each 16-lane group G, lane s reads 4 consecutive columns
// of one row; the transpose read gives lane i element i % 4 of the row read by
// lane i / 4 + 4 j.
template <int NG>
__device__ __forceinline__ uint4 frag_tr(const char* s, int c0, int r0, int lane) {
  const int G = lane >> 4, sl = lane & 15;
  const int cc = c0 + 16 * (G & 1) + 4 * (sl & 3);
  const int ch = cc >> 3, sub = (cc & 7) * 2;
  const int ra = r0 + 4 * (G >> 1) + (sl >> 2), rb = ra + 8;
  constexpr int RS = Slice<NG>::RS;
  v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(s + ra * RS + phys<NG>(ch, ra) * 16 + sub));
  v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(s + rb * RS + phys<NG>(ch, rb) * 16 + sub));
  const uint2 a = bitcast<uint2>(lo), b = bitcast<uint2>(hi);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// LDS of a workgroup: per wave ST stages of its slice (+ 512 bytes of per-row
// scalars in pass 2); the partial z tiles [4 waves][NQT][4 quarters][64 lanes]
// (float4); the bf16 probabilities or gradients [NQT][4 quarters][64 lanes]
// (4 bf16 each); and per-wave column values [NQT][4 waves][64 lanes] (float).
template <int NG, int NQT, int ST, int MODE>
struct Lds {
  static constexpr int STAGE = Slice<NG>::BYTES + (MODE ? 512 : 0);
  static constexpr int PER_WAVE = ST * STAGE;
  static constexpr int PART = 4 * PER_WAVE;
  static constexpr int PQ = PART + 4 * NQT * 4 * 64 * 16;
  static constexpr int COLV = PQ + NQT * 4 * 64 * 8;
  static constexpr int TOTAL = COLV + NQT * 4 * 64 * 4;
};

// Per-lane state of a workgroup's pass (the same row statistics in every wave).
template <int NG, int NQT>
struct State {
  uint4 qf[NQT][NG * 4];    // fixed rows: B fragments of the z product over this wave's columns
  f32x16 O[NQT][NG * 2];    // second-product accumulators over this wave's columns
  float m[NQT], l[NQT], zy[NQT];  // pass 1: reference max (log2 units); this wave's quarter: sum of p, target logit
  float seen[NQT];                // pass 1: this wave's quarter: maximum so far (log2 units)
  int yq[NQT];              // pass 1: the fixed row's target
  int ng, f0, lane, w, g, c32;
};

// This wave's slice loads of a streamed block: instruction i, lane -> (block
// row, logical chunk) -> source byte offset; pass 2 also loads the block rows'
// log-sum-exps and targets (one dword instruction each, into the stage tail).
template <int NG, int MODE>
struct Loader {
  rsrc_t rs, rl, ry;
  uint32_t off[Slice<NG>::NLD];
  uint32_t blk_bytes;
  int lane;
  // load instruction i of block blk into stage st
  __device__ __forceinline__ void one(int i, int blk, char* st) const {
    dma16(rs, st + i * 1024, off[i] + (uint32_t)blk * blk_bytes);
  }
  __device__ __forceinline__ void tail(int blk, char* st) const {
    if constexpr (MODE == 1) {
      dma4(rl, st + Slice<NG>::BYTES, (uint32_t)(blk * BV + lane) * 4);
      dma4(ry, st + Slice<NG>::BYTES + 256, (uint32_t)(blk * BV + lane) * 4);
    }
  }
  __device__ __forceinline__ void all(int blk, char* st) const {
#pragma unroll
    for (int i = 0; i < Slice<NG>::NLD; ++i) one(i, blk, st);
    tail(blk, st);
  }
  static constexpr int PER_BLOCK = Slice<NG>::NLD + (MODE ? 2 : 0);  // load instructions per block

  // The same loads through descriptors that start at block blk (built with
  // scalar arithmetic once per block, so a load needs no address arithmetic):
  // rows past the end of the streamed rows, a whole block past it included,
  // read zeros.
  const bf16* str;
  const float* lse;
  const int32_t* yv;
  int n_str, C;
  struct Block {
    rsrc_t rs, rl, ry;
  };
  __device__ __forceinline__ Block block(int blk) const {
    const int left = max(n_str - blk * BV, 0);
    Block b;
    b.rs = make_rsrc(str + (int64_t)blk * BV * C, (int64_t)left * C * 2);
    if constexpr (MODE == 1) {
      b.rl = make_rsrc(lse + (int64_t)blk * BV, (int64_t)left * 4);
      b.ry = make_rsrc(yv + (int64_t)blk * BV, (int64_t)left * 4);
    }
    return b;
  }
  __device__ __forceinline__ void one(int i, const Block& b, char* st) const { dma16(b.rs, st + i * 1024, off[i]); }
  __device__ __forceinline__ void tail(const Block& b, char* st) const {
    if constexpr (MODE == 1) {
      dma4(b.rl, st + Slice<NG>::BYTES, (uint32_t)lane * 4);
      dma4(b.ry, st + Slice<NG>::BYTES + 256, (uint32_t)lane * 4);
    }
  }
};

// second product over this wave's columns: O^T[c][fixed] += (block^T)[c][streamed] P^T[streamed][fixed]
// (the tiles past a wave's own columns are computed too and never stored)
// Both halves of the streamed rows (hh) go over all column tiles in turn, so
// the two products into one accumulator are 2 NG NQT products apart (an MFMA
// result is not ready for a dependent product for several issue slots).  A
// ring of three fragments keeps the reads two (hh, ct) steps ahead of their
// products; the empty asm statements keep the compiler from hoisting every
// read to the top (registers).
template <int NG, int NQT>
__device__ __forceinline__ void second_product(const char* __restrict__ rd, const uint4 (&pb)[NQT][2],
                                               State<NG, NQT>& S) {
  constexpr int NT = NG * 2;
  uint4 f[3];
  f[0] = frag_tr<NG>(rd, 0, 0, S.lane);
  f[1] = frag_tr<NG>(rd, (1 % NT) * 32, (1 / NT) * 16, S.lane);
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i) {
    const int hh = i / NT, ct = i % NT;
    if (i + 2 < 2 * NT) f[(i + 2) % 3] = frag_tr<NG>(rd, ((i + 2) % NT) * 32, ((i + 2) / NT) * 16, S.lane);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) mma32(S.O[qt][ct], f[i % 3], pb[qt][hh]);
  }
}

// Partial z^T tiles of one streamed block over this wave's columns (z[qt][e]:
// streamed row r0 + crow(e, g), fixed row f0 + 32 qt + c32).  Block `refill`
// is loaded into wr meanwhile, one instruction per k-step (a wave that issues
// its loads back to back stalls at issue): when refill >= 0, or always with
// ALWAYS (a block past the end of the streamed rows loads zeros).
// Every k-step runs in every wave, also past a wave's own columns (fewer
// groups than NG): those k-steps have zero fixed fragments, and the slot data
// there is real memory from the loads, so it is finite; the waves meet at every
// block and wait for the widest one anyway.
template <int NG, int NQT, int MODE, bool ALWAYS>
__device__ __forceinline__ void z_partials(const char* __restrict__ rd, char* __restrict__ wr, int refill,
                                           const Loader<NG, MODE>& ld, const State<NG, NQT>& S,
                                           f32x16 (&z)[NQT]) {
  const int g = S.g, c32 = S.c32;
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) zero16(z[qt]);
  // the fragment of k-step ks + 2 is read while k-step ks's products run
  uint4 af[3];
  af[0] = frag_row<NG>(rd, c32, 0, g);
  af[1] = frag_row<NG>(rd, c32, 1, g);
#pragma unroll
  for (int ks = 0; ks < NG * 4; ++ks) {
    if (ks + 2 < NG * 4) af[(ks + 2) % 3] = frag_row<NG>(rd, c32, ks + 2, g);
    if (ALWAYS || refill >= 0) ld.one(ks, refill, wr);  // NLD == 4 NG == the number of k-steps
    asm volatile("" ::: "memory");
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) mma32(z[qt], af[ks % 3], S.qf[qt][ks]);  // serves every fixed tile
  }
  if (ALWAYS || refill >= 0) ld.tail(refill, wr);
}

template <int NQT>
__device__ __forceinline__ void write_part(float4* __restrict__ part, const f32x16 (&z)[NQT], int w, int lane) {
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4)
      part[((w * NQT + qt) * 4 + e4) * 64 + lane] =
          make_float4(z[qt][4 * e4], z[qt][4 * e4 + 1], z[qt][4 * e4 + 2], z[qt][4 * e4 + 3]);
}

// After the partial tiles of a block are in `part` (and a barrier): wave w adds
// accumulator quarter w (e = 4 w .. 4 w + 3, the streamed rows 8 w + 4 g + i)
// over the 4 waves, in wave order, and turns it into bf16 probabilities (pass
// 1, against the row's reference m) or gradients (pass 2, from the block rows'
// log-sum-exps l4 and targets y4 of those rows) in pq.  At block 0 of pass 1
// (first), the reference m of each fixed row is set to the block's maximum,
// exchanged through LDS.
// this wave's quarter of the 4 waves' partial tiles (pp[qt][v]: wave v's)
template <int NQT>
__device__ __forceinline__ void read_quarter(const float4* __restrict__ part, int w, int lane, float4 (&pp)[NQT][4]) {
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
    for (int v = 0; v < 4; ++v) pp[qt][v] = part[((v * NQT + qt) * 4 + w) * 64 + lane];
}


// Sum of the four waves' partial logit tiles of one quarter.
__device__ __forceinline__ float4 sum4(const float4 (&p)[4]) {
  float4 s = p[0];
#pragma unroll
  for (int u = 1; u < 4; ++u) {
    s.x += p[u].x;
    s.y += p[u].y;
    s.z += p[u].z;
    s.w += p[u].w;
  }
  return s;
}
template <int NG, int NQT, int MODE>
__device__ __forceinline__ void quarter_p(const float4 (&pp)[NQT][4], uint2* __restrict__ pq,
                                          float* __restrict__ colv, const Args& a, int r0, bool first,
                                          float4 l4, int4 y4, State<NG, NQT>& S) {
  const int lane = S.lane, w = S.w, g = S.g, c32 = S.c32;
  float q[NQT][4];  // this wave's quarter of z: streamed rows r0 + 8 w + 4 g + i
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    float4 s4 = pp[qt][0];
#pragma unroll
    for (int v = 1; v < 4; ++v) {
      const float4 p4 = pp[qt][v];
      s4.x += p4.x;
      s4.y += p4.y;
      s4.z += p4.z;
      s4.w += p4.w;
    }
    q[qt][0] = s4.x;
    q[qt][1] = s4.y;
    q[qt][2] = s4.z;
    q[qt][3] = s4.w;
  }
  const int rq = r0 + 8 * w + 4 * g;  // streamed row of q[.][0]
  if constexpr (MODE == 0) {
    float mx[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      float v = NEG_INF;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (rq + i >= a.n_str) q[qt][i] = NEG_INF;  // W rows past V are not classes
        v = fmaxf(v, q[qt][i]);
        if (rq + i == S.yq[qt]) S.zy[qt] = q[qt][i];
      }
      mx[qt] = v * LOG2E;
      S.seen[qt] = fmaxf(S.seen[qt], mx[qt]);
    }
    if (first) {  // the reference: each fixed row's maximum over this block
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) colv[(qt * 4 + w) * 64 + lane] = mx[qt];
      lds_barrier();
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        float v = colv[(qt * 4) * 64 + lane];
#pragma unroll
        for (int u = 1; u < 4; ++u) v = fmaxf(v, colv[(qt * 4 + u) * 64 + lane]);
        S.m[qt] = halves_max(v);
      }
    }
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      bf16x4 v;
      float ls = S.l[qt];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16 p = (bf16)hw_exp2(fmaf(q[qt][i], LOG2E, -S.m[qt]));
        v[i] = p;
        ls += (float)p;  // the sum of the rounded p the product uses
      }
      S.l[qt] = ls;
      pq[(qt * 4 + w) * 64 + lane] = bitcast<uint2>(v);
    }
  } else {
    // pass 2: g = scale (exp(z - lse) - [y == v]); F rows past N (loaded as zeros) give 0
    const float lv[4] = {l4.x * LOG2E, l4.y * LOG2E, l4.z * LOG2E, l4.w * LOG2E};
    const int yv[4] = {y4.x, y4.y, y4.z, y4.w};
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int vq = S.f0 + qt * 32 + c32;  // this lane's W row
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = hw_exp2(fmaf(q[qt][i], LOG2E, -lv[i])) - (yv[i] == vq ? 1.f : 0.f);
        if (rq + i >= a.n_str) p = 0.f;
        v[i] = (bf16)(p * a.scale);
      }
      pq[(qt * 4 + w) * 64 + lane] = bitcast<uint2>(v);
    }
  }
}

// the B fragments of the second product, assembled from the 4 quarters in pq
template <int NQT>
__device__ __forceinline__ void read_pb(const uint2* __restrict__ pq, int lane, uint4 (&pb)[NQT][2]) {
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint2 lo = pq[(qt * 4 + 2 * hh) * 64 + lane], hi = pq[(qt * 4 + 2 * hh + 1) * 64 + lane];
      pb[qt][hh] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
}

// the streamed rows' log-sum-exps and targets of this lane's quarter (pass 2: the stage tail)
template <int NG, int MODE>
__device__ __forceinline__ void quarter_tail(const char* rd, int w, int g, float4& l4, int4& y4) {
  if constexpr (MODE == 1) {
    const float* sl = reinterpret_cast<const float*>(rd + Slice<NG>::BYTES);
    const int* sy = reinterpret_cast<const int*>(rd + Slice<NG>::BYTES + 256);
    l4 = *reinterpret_cast<const float4*>(sl + 8 * w + 4 * g);
    y4 = *reinterpret_cast<const int4*>(sy + 8 * w + 4 * g);
  } else {
    l4 = make_float4(0.f, 0.f, 0.f, 0.f);
    y4 = make_int4(0, 0, 0, 0);
  }
}

// One streamed block (its slice in rd, streamed rows r0 ..), in sequence: the
// partial z tiles (loading block `refill` into wr meanwhile), their sum and
// softmax through LDS, and the B fragments of the second product.  The
// pointers are distinct and __restrict__, so the compiler need not wait for
// the loads into wr before the LDS accesses here.
template <int NG, int NQT, int MODE>
__device__ __forceinline__ void block_p(const char* __restrict__ rd, char* __restrict__ wr, int refill,
                                        const Loader<NG, MODE>& ld, float4* __restrict__ part,
                                        uint2* __restrict__ pq, float* __restrict__ colv, const Args& a, int r0,
                                        bool first, State<NG, NQT>& S, uint4 (&pb)[NQT][2]) {
  {
    f32x16 z[NQT];
    z_partials<NG, NQT, MODE, false>(rd, wr, refill, ld, S, z);
    write_part<NQT>(part, z, S.w, S.lane);
  }
  lds_barrier();
  float4 l4;
  int4 y4;
  quarter_tail<NG, MODE>(rd, S.w, S.g, l4, y4);
  float4 pp[NQT][4];
  read_quarter<NQT>(part, S.w, S.lane, pp);
  quarter_p<NG, NQT, MODE>(pp, pq, colv, a, r0, first, l4, y4, S);
  lds_barrier();
  read_pb<NQT>(pq, S.lane, pb);
}

// Element (qt, i) of this wave's quarter of a block past a pass's reference
// block (streamed row rq + i): the bf16 probability (pass 1, with the running
// sum, maximum and target logit) or gradient (pass 2, from the row's
// log-sum-exp lv in log2 units and target yv) into v[i]; the same arithmetic,
// in the same order, as quarter_p.
template <int NG, int NQT, int MODE>
__device__ __forceinline__ void quarter_elem(float qv, int qt, int i, int rq, const Args& a, float lv, int yv,
                                             State<NG, NQT>& S, bf16x4& v) {
  if constexpr (MODE == 0) {
    if (rq + i >= a.n_str) qv = NEG_INF;
    if (rq + i == S.yq[qt]) S.zy[qt] = qv;
    S.seen[qt] = fmaxf(S.seen[qt], qv * LOG2E);
    const bf16 p = (bf16)hw_exp2(fmaf(qv, LOG2E, -S.m[qt]));
    v[i] = p;
    S.l[qt] += (float)p;
  } else {
    const int vq = S.f0 + qt * 32 + S.c32;
    float p = hw_exp2(fmaf(qv, LOG2E, -lv)) - (yv == vq ? 1.f : 0.f);
    if (rq + i >= a.n_str) p = 0.f;
    v[i] = (bf16)(p * a.scale);
  }
}

// Software-pipelined step j of a sweep (block j in cur, block j + 1 in nxt;
// block j's transposed fragments T and its quarter's row scalars l4, y4 are
// already in registers, read during step j - 1):
//  phase 1: the partial z tiles of block j + 1 (NEXT) on the matrix cores,
//    loading block j + 2 into cur meanwhile, interleaved with the sum and
//    softmax of block j (its partials in `part`) on the vector ALUs;
//  phase 2: the second product of block j, interleaved with the reads of block
//    j + 1's transposed fragments and row scalars into T, l4, y4 and the
//    store of block j + 1's partials into `part`.
// Barrier 1 separates pq's writes from its reads and part's reads from its
// rewrite; barrier 2 ends the step (LDS reads of nxt complete, part written).
// Block j + 1's loads were issued in step j - 1; the loads of block j + 2 go to
// cur, whose reads ended with step j - 1.  A block past the end loads zeros.
template <int NG, int NQT, int MODE, bool FIRST, bool NEXT>
__device__ __forceinline__ void pipe_step(char* __restrict__ cur, const char* __restrict__ nxt, int j,
                                          const Loader<NG, MODE>& ld, float4* __restrict__ part,
                                          uint2* __restrict__ pq, float* __restrict__ colv, const Args& a,
                                          State<NG, NQT>& S, uint4 (&T)[NG * 4], float4& l4, int4& y4) {
  constexpr int NT = NG * 2, KS = NG * 4;
  const int lane = S.lane, g = S.g, c32 = S.c32;
  f32x16 zn[NQT];
  float4 pp[NQT][4];
  if constexpr (NEXT && !FIRST && KS >= 6 * NQT) {
    // Explicitly interleaved: k-step ks issues its fragment read, one slice
    // load and its MFMAs, and then a slice of block j's vector work (the sums
    // of quarter qt at ks = qt, element e at ks = NQT + e, the stores of quarter
    // qt at ks = 5 NQT + qt); scheduling barriers keep the slices in place.
    wait_vm<0>();  // block j + 1 has landed in nxt
    const typename Loader<NG, MODE>::Block nb = ld.block(j + 2);
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) zero16(zn[qt]);
    const int rq = j * BV + 8 * S.w + 4 * g;
    const float lv[4] = {l4.x * LOG2E, l4.y * LOG2E, l4.z * LOG2E, l4.w * LOG2E};
    const int yv[4] = {y4.x, y4.y, y4.z, y4.w};
    float4 q4[NQT];
    bf16x4 v[NQT];
    uint4 af[3];
    af[0] = frag_row<NG>(nxt, c32, 0, g);
    af[1] = frag_row<NG>(nxt, c32, 1, g);
    read_quarter<NQT>(part, S.w, lane, pp);  // ahead of the loads into cur, which the compiler may take to alias
    // Pass 1 sums the four waves' partials here, before the k-steps, so that
    // only the sums live through them: summed one quarter per k-step, the
    // partials stayed live and pass 1 spilled registers inside its loop (8
    // scratch accesses per two blocks, whose waits also wait on the block loads
    // issued before them; 3 this way). Pass 2 keeps the per-k-step sums: it
    // spills less either way and measured a little faster so.
    constexpr bool EARLY = MODE == 0;
    if constexpr (EARLY) {
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) q4[qt] = sum4(pp[qt]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 2 < KS) af[(ks + 2) % 3] = frag_row<NG>(nxt, c32, ks + 2, g);
      ld.one(ks, nb, cur);
      if (ks == KS - 1) ld.tail(nb, cur);
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) mma32(zn[qt], af[ks % 3], S.qf[qt][ks]);
      if (ks < NQT) {
        if constexpr (!EARLY) q4[ks] = sum4(pp[ks]);
      } else if (ks < 5 * NQT) {
        const int e = ks - NQT, qt = e >> 2, i = e & 3;
        const float qv = i == 0 ? q4[qt].x : i == 1 ? q4[qt].y : i == 2 ? q4[qt].z : q4[qt].w;
        quarter_elem<NG, NQT, MODE>(qv, qt, i, rq, a, lv[i], yv[i], S, v[qt]);
      } else if (ks < 6 * NQT) {
        const int qt = ks - 5 * NQT;
        pq[(qt * 4 + S.w) * 64 + lane] = bitcast<uint2>(v[qt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    read_quarter<NQT>(part, S.w, lane, pp);
    if constexpr (NEXT) {
      wait_vm<0>();  // block j + 1 has landed in nxt
      const typename Loader<NG, MODE>::Block nb = ld.block(j + 2);
      uint4 af[3];
      af[0] = frag_row<NG>(nxt, c32, 0, g);
      af[1] = frag_row<NG>(nxt, c32, 1, g);
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) zero16(zn[qt]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 2 < KS) af[(ks + 2) % 3] = frag_row<NG>(nxt, c32, ks + 2, g);
        ld.one(ks, nb, cur);
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) mma32(zn[qt], af[ks % 3], S.qf[qt][ks]);
      }
      ld.tail(nb, cur);
    }
    quarter_p<NG, NQT, MODE>(pp, pq, colv, a, j * BV, FIRST, l4, y4, S);
  }
  lds_barrier();
  uint4 pb[NQT][2];
  read_pb<NQT>(pq, lane, pb);
  if constexpr (NEXT) write_part<NQT>(part, zn, S.w, lane);
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i) {
    const int hh = i / NT, ct = i % NT;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) mma32(S.O[qt][ct], T[i], pb[qt][hh]);
    if constexpr (NEXT) T[i] = frag_tr<NG>(nxt, ct * 32, hh * 16, lane);
  }
  if constexpr (NEXT) {
    quarter_tail<NG, MODE>(nxt, S.w, g, l4, y4);
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) {
      SGB(0x008, NQT);
      SGB(0x100, 1);
      if (i < 8) SGB(0x200, 1);  // the partial-tile stores
    }
  }
  lds_barrier();
}

// Sum (or max) of a per-lane value over the 4 waves and the two lane halves,
// through LDS (after a barrier every wave holds the same result).
template <bool MAX>
__device__ __forceinline__ float wg_column(float v, float* __restrict__ colv, int w, int lane) {
  colv[w * 64 + lane] = v;
  lds_barrier();
  float t = colv[lane];
#pragma unroll
  for (int u = 1; u < 4; ++u) t = MAX ? fmaxf(t, colv[u * 64 + lane]) : t + colv[u * 64 + lane];
  lds_barrier();  // every wave has read colv before it is written again
  return MAX ? halves_max(t) : halves_sum(t);
}

template <int NG, int NQT, int ST, int MODE, bool PIPE, bool SEG = false>
__global__ __launch_bounds__(256, 1) void head_kernel(Args a) {
  using L = Lds<NG, NQT, ST, MODE>;
  using SL = Slice<NG>;
  static_assert(L::TOTAL <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  State<NG, NQT> S;
  const int t = threadIdx.x;
  S.lane = t & 63;
  S.w = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform in the wave: scalar LDS bases
  S.g = S.lane >> 5;
  S.c32 = S.lane & 31;
  const int lane = S.lane, w = S.w, g = S.g, c32 = S.c32;
  const int C = a.C;
  int c_lo, ng;
  wave_range(C, w, ng, c_lo);
  S.ng = __builtin_amdgcn_readfirstlane(ng);  // uniform in the wave: scalar branches
  c_lo = __builtin_amdgcn_readfirstlane(c_lo);
  int bidx = blockIdx.x;
  const int n_vocab = a.n_str;  // pass 1: targets are checked against the whole vocabulary
  int y_off = 0;                // pass 1: first vocabulary row of this workgroup's segment
  if constexpr (MODE == 0 && SEG) {
    {
      const int z = bidx / a.tb;
      bidx -= z * a.tb;
      y_off = z * a.z_rows;
      a.str += (int64_t)y_off * a.C;
      a.n_str = min(a.z_rows, a.n_str - y_off);
      if (a.out) a.out += (int64_t)z * a.z_stride;
      a.seg_s += (int64_t)z * a.n_fix * 4;
    }
  }
  if constexpr (MODE == 1) {
    if (a.nz > 1) {
      const int z = bidx / a.tb;
      bidx -= z * a.tb;
      const int r0 = z * a.z_rows;
      a.str += (int64_t)r0 * a.C;
      a.lse += r0;
      a.y += r0;
      a.n_str = min(a.z_rows, a.n_str - r0);
      a.out += (int64_t)z * a.z_stride;
    }
  }
  S.f0 = (a.blk0 + bidx) * (32 * NQT);  // first fixed row of the workgroup
  const int nblk = (a.n_str + BV - 1) / BV;

#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int fr = S.f0 + qt * 32 + c32;
    const bf16* src = a.fix + (int64_t)min(fr, a.n_fix - 1) * C + c_lo + g * 8;
#pragma unroll
    for (int ks = 0; ks < NG * 4; ++ks)
      S.qf[qt][ks] =
          (ks < S.ng * 4 && fr < a.n_fix) ? *reinterpret_cast<const uint4*>(src + ks * 16) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int ct = 0; ct < NG * 2; ++ct) zero16(S.O[qt][ct]);
    S.m[qt] = NEG_INF;
    S.l[qt] = 0.f;
    S.zy[qt] = 0.f;
    S.seen[qt] = NEG_INF;
    S.yq[qt] = 0;
    if constexpr (MODE == 0) {
      int yy = fr < a.n_fix ? a.y[fr] : 0;
      if (yy < 0 || yy >= n_vocab) {  // clamped into the row; reported through a.bad
        if (fr < a.n_fix && a.bad) *a.bad = 1;
        yy = yy < 0 ? 0 : n_vocab - 1;
      }
      yy -= y_off;  // a target outside this segment is never matched
      S.yq[qt] = (yy >= 0 && yy < a.n_str) ? yy : -1;
    }
  }

  Loader<NG, MODE> ld;
  ld.rs = make_rsrc(a.str, (int64_t)a.n_str * C * 2);
  ld.rl = make_rsrc(MODE == 1 ? (const void*)a.lse : nullptr, MODE == 1 ? (int64_t)a.n_str * 4 : 0);
  ld.ry = make_rsrc(MODE == 1 ? (const void*)a.y : nullptr, MODE == 1 ? (int64_t)a.n_str * 4 : 0);
  ld.lane = lane;
  ld.blk_bytes = (uint32_t)(BV * C * 2);
  ld.str = a.str;
  ld.lse = a.lse;
  ld.yv = a.y;
  ld.n_str = a.n_str;
  ld.C = C;
#pragma unroll
  for (int i = 0; i < SL::NLD; ++i) {
    const int q = i * 1024 + 16 * lane;
    const int row = q / SL::RS, pc = (q % SL::RS) >> 4;
    ld.off[i] = (uint32_t)(((int64_t)row * C + c_lo + phys<NG>(pc, row) * 8) * 2);
  }
  constexpr int LPB = Loader<NG, MODE>::PER_BLOCK;
  char* wbase = smem + w * L::PER_WAVE;
  float4* part = reinterpret_cast<float4*>(smem + L::PART);
  uint2* pq = reinterpret_cast<uint2*>(smem + L::PQ);
  float* colv = reinterpret_cast<float*>(smem + L::COLV);
  static_assert(SL::NLD == NG * 4, "one slice load per k-step");

  // Block j lives in stage j % ST.  Before block j is used, the stage block
  // j - 1 used (this wave alone reads its slice, and it is done with it) gets
  // block j + ST - 1, issued during block j's z product; so the loads still
  // outstanding when block j is needed are those of blocks j + 1 .. j + ST - 2.
  // With one stage the next block is loaded after the current one is consumed.
  auto wait_block = [&](int j) {
    if constexpr (ST == 3) {
      if (j + 1 < nblk) wait_vm<LPB>();
      else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
  };
  auto stage = [&](int sc) { return wbase + sc * L::STAGE; };
  auto prologue = [&]() {
    if constexpr (ST == 1) {
      ld.all(0, wbase);
    } else {
#pragma unroll
      for (int s2 = 0; s2 < ST - 1; ++s2)
        if (s2 < nblk) ld.all(s2, stage(s2));
    }
  };
  if constexpr (!PIPE) prologue();
  // the stage to refill while block j (in stage sc) is used, and the block it gets (-1: none)
  auto refill_of = [&](int j, int sc, char*& wr) {
    if constexpr (ST == 1) {
      wr = wbase + L::STAGE;  // unused: the single stage is refilled after the block
      return -1;
    } else {
      wr = stage(sc == 0 ? ST - 1 : sc - 1);
      return j + ST - 1 < nblk ? j + ST - 1 : -1;
    }
  };

  // The software-pipelined sweep over the streamed blocks; first: the pass's
  // first (pass 1 sets the reference m of each fixed row at its block 0).
  auto sweep_pipe = [&](bool first) {
    static_assert(!PIPE || ST == 2, "the pipelined sweep holds blocks j and j + 1 in two stages");
    ld.all(0, stage(0));
    ld.all(1, stage(1));  // past the end of the streamed rows: zeros, never read
    wait_vm<LPB>();       // block 0 has landed
    uint4 T[NG * 4];
    float4 l4;
    int4 y4;
    {
      f32x16 z[NQT];
      z_partials<NG, NQT, MODE, false>(stage(0), stage(1), -1, ld, S, z);
      write_part<NQT>(part, z, w, lane);
#pragma unroll
      for (int i = 0; i < NG * 4; ++i)
        T[i] = frag_tr<NG>(stage(0), (i % (NG * 2)) * 32, (i / (NG * 2)) * 16, lane);
      quarter_tail<NG, MODE>(stage(0), w, S.g, l4, y4);
    }
    lds_barrier();
    const bool f0 = MODE == 0 && first;
    if (nblk == 1) {
      if (f0) pipe_step<NG, NQT, MODE, true, false>(stage(0), stage(1), 0, ld, part, pq, colv, a, S, T, l4, y4);
      else pipe_step<NG, NQT, MODE, false, false>(stage(0), stage(1), 0, ld, part, pq, colv, a, S, T, l4, y4);
    } else {
      if (f0) pipe_step<NG, NQT, MODE, true, true>(stage(0), stage(1), 0, ld, part, pq, colv, a, S, T, l4, y4);
      else pipe_step<NG, NQT, MODE, false, true>(stage(0), stage(1), 0, ld, part, pq, colv, a, S, T, l4, y4);
      // two steps per trip, so that each step's stages are fixed offsets from the wave's base
      int j = 1;
      for (; j + 2 < nblk; j += 2) {
        pipe_step<NG, NQT, MODE, false, true>(stage(1), stage(0), j, ld, part, pq, colv, a, S, T, l4, y4);
        pipe_step<NG, NQT, MODE, false, true>(stage(0), stage(1), j + 1, ld, part, pq, colv, a, S, T, l4, y4);
      }
      if (j + 1 < nblk) {
        pipe_step<NG, NQT, MODE, false, true>(stage(1), stage(0), j, ld, part, pq, colv, a, S, T, l4, y4);
        ++j;
      }
      if (j & 1) pipe_step<NG, NQT, MODE, false, false>(stage(1), stage(0), j, ld, part, pq, colv, a, S, T, l4, y4);
      else pipe_step<NG, NQT, MODE, false, false>(stage(0), stage(1), j, ld, part, pq, colv, a, S, T, l4, y4);
    }
    wait_vm<0>();  // the loads past the end have landed before the stages are reloaded or released
  };

  uint4 pb[NQT][2];
  if constexpr (MODE == 0) {
    // Softmax against a fixed reference per row instead of a running maximum:
    // m is the row's maximum over the first W block (so p <= 2^(max - m)), and
    // the accumulators are never rescaled inside the sweep.  A row whose later
    // maximum exceeds m by more than HEADROOM (p could overflow) has the whole
    // sweep redone with m = that maximum; the maxima are combined over the
    // waves, so the decision is the same in all of them.
    for (int attempt = 0;; ++attempt) {
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
#pragma unroll
        for (int ct = 0; ct < NG * 2; ++ct) zero16(S.O[qt][ct]);
        S.l[qt] = 0.f;
        S.seen[qt] = NEG_INF;
      }
      if constexpr (PIPE) {
        sweep_pipe(attempt == 0);
      } else {
        if (attempt > 0) prologue();  // the sweep starts over: reload the first blocks
        int sc = 0;
        for (int j = 0; j < nblk; ++j) {
          char* wr;
          const int rf = refill_of(j, sc, wr);
          wait_block(j);
          block_p<NG, NQT, MODE>(stage(sc), wr, rf, ld, part, pq, colv, a, j * BV, j == 0 && attempt == 0,
                                 S, pb);
          second_product<NG, NQT>(stage(sc), pb, S);
          if constexpr (ST == 1)
            if (j + 1 < nblk) ld.all(j + 1, wbase);
          sc = sc + 1 == ST ? 0 : sc + 1;
        }
      }
      bool redo = false;
      float seen[NQT];
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        seen[qt] = wg_column<true>(S.seen[qt], colv, w, lane);
        redo |= seen[qt] > S.m[qt] + HEADROOM;
      }
      if (!__any(redo)) break;
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) S.m[qt] = fmaxf(S.m[qt], seen[qt]);
    }
    // totals over the waves' quarters and the lane halves
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      S.l[qt] = wg_column<false>(S.l[qt], colv, w, lane);
      S.zy[qt] = wg_column<false>(S.zy[qt], colv, w, lane);  // exactly one quarter saw the target
    }
  } else if constexpr (PIPE) {
    sweep_pipe(true);
  } else {
    int sc = 0;
    for (int j = 0; j < nblk; ++j) {
      char* wr;
      const int rf = refill_of(j, sc, wr);
      wait_block(j);
      block_p<NG, NQT, MODE>(stage(sc), wr, rf, ld, part, pq, colv, a, j * BV, false, S, pb);
      second_product<NG, NQT>(stage(sc), pb, S);
      if constexpr (ST == 1)
        if (j + 1 < nblk) ld.all(j + 1, wbase);
      sc = sc + 1 == ST ? 0 : sc + 1;
    }
  }

  // epilogue: tile ct of fixed tile qt holds columns c_lo + 32 ct + crow(e, g) of fixed row f0 + 32 qt + c32
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int fr = S.f0 + qt * 32 + c32;
    if (fr >= a.n_fix) continue;
    float* orow = a.out + (int64_t)(fr - a.out_row0) * C + c_lo;
    if constexpr (MODE == 0) {
      const float lt = S.l[qt], zt = S.zy[qt];
      if constexpr (SEG) {  // a vocabulary segment: its reference, sum, target logit and unnormalised sum p W
        if (w == 0 && g == 0) {
          a.seg_s[(int64_t)fr * 4] = S.m[qt];
          a.seg_s[(int64_t)fr * 4 + 1] = lt;
          a.seg_s[(int64_t)fr * 4 + 2] = zt;
        }
        if (a.out == nullptr) continue;
#pragma unroll
        for (int ct = 0; ct < NG * 2; ++ct) {
          if (ct >= S.ng * 2) continue;
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int c = ct * 32 + r4 * 8 + g * 4;
            const f32x16& o = S.O[qt][ct];
            store4(orow + c, make_float4(o[4 * r4], o[4 * r4 + 1], o[4 * r4 + 2], o[4 * r4 + 3]));
          }
        }
        continue;
      }
      const float lse = (S.m[qt] + hw_log2(lt)) * LN2;
      if (w == 0 && g == 0) {
        a.loss[fr] = lse - zt;
        a.lse_out[fr] = lse;
      }
      if (a.out == nullptr) continue;  // forward only
      const float inv = 1.f / lt, sc2 = a.scale;
      const bf16* wy = a.str + (int64_t)S.yq[qt] * C + c_lo;
#pragma unroll
      for (int ct = 0; ct < NG * 2; ++ct) {
        if (ct >= S.ng * 2) continue;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int c = ct * 32 + r4 * 8 + g * 4;
          const float4 wv = load4(wy + c);
          const f32x16& o = S.O[qt][ct];
          store4(orow + c, make_float4((o[4 * r4] * inv - wv.x) * sc2, (o[4 * r4 + 1] * inv - wv.y) * sc2,
                                       (o[4 * r4 + 2] * inv - wv.z) * sc2, (o[4 * r4 + 3] * inv - wv.w) * sc2));
        }
      }
    } else {
#pragma unroll
      for (int ct = 0; ct < NG * 2; ++ct) {
        if (ct >= S.ng * 2) continue;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int c = ct * 32 + r4 * 8 + g * 4;
          const f32x16& o = S.O[qt][ct];
          float4 v = make_float4(o[4 * r4], o[4 * r4 + 1], o[4 * r4 + 2], o[4 * r4 + 3]);
          if (a.accumulate) {
            const float4 p = load4(orow + c);
            v.x += p.x;
            v.y += p.y;
            v.z += p.z;
            v.w += p.w;
          }
          store4(orow + c, v);
        }
      }
    }
  }
}

// Pass 1 over vocabulary segments, combined per row in segment order.  With
// segment z's reference m_z (log2 units), sum l_z of 2^(z log2 e - m_z), target
// logit zy_z (zero outside the target's segment) and unnormalised sum O_z of
// p W: M = max_z m_z, f_z = 2^(m_z - M), l = sum_z f_z l_z,
// lse = (M + log2 l) ln 2, loss = lse - sum_z zy_z and
// dF = scale ((sum_z f_z O_z) / l - W_y).  One workgroup per row.
constexpr int MAX_SEG = 8;
__global__ __launch_bounds__(256) void seg_combine_kernel(const float* __restrict__ seg_s,
                                                          const float* __restrict__ seg_O, int nvs, int N, int V,
                                                          int C, const bf16* __restrict__ W,
                                                          const int32_t* __restrict__ y, float scale,
                                                          float* __restrict__ loss, float* __restrict__ lse_out,
                                                          float* __restrict__ dF) {
  __shared__ float fz[MAX_SEG];
  __shared__ float inv_l;
  const int n = blockIdx.x;
  if (threadIdx.x == 0) {
    float M = NEG_INF;
    for (int z = 0; z < nvs; ++z) M = fmaxf(M, seg_s[((int64_t)z * N + n) * 4]);
    float l = 0.f, zy = 0.f;
    for (int z = 0; z < nvs; ++z) {
      const float* sz = seg_s + ((int64_t)z * N + n) * 4;
      const float f = hw_exp2(sz[0] - M);
      fz[z] = f;
      l += f * sz[1];
      zy += sz[2];
    }
    const float lse = (M + hw_log2(l)) * LN2;
    loss[n] = lse - zy;
    lse_out[n] = lse;
    inv_l = 1.f / l;
  }
  __syncthreads();
  if (!dF) return;
  int yy = y[n];
  yy = yy < 0 ? 0 : (yy >= V ? V - 1 : yy);  // out-of-range targets were flagged by pass 1
  const float il = inv_l;
  for (int c = 4 * (int)threadIdx.x; c < C; c += 1024) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int z = 0; z < nvs; ++z) {
      const float4 o = load4(seg_O + ((int64_t)z * N + n) * C + c);
      const float f = fz[z];
      acc.x = fmaf(f, o.x, acc.x);
      acc.y = fmaf(f, o.y, acc.y);
      acc.z = fmaf(f, o.z, acc.z);
      acc.w = fmaf(f, o.w, acc.w);
    }
    const float4 wv = load4(W + (int64_t)yy * C + c);
    store4(dF + (int64_t)n * C + c, make_float4((acc.x * il - wv.x) * scale, (acc.y * il - wv.y) * scale,
                                                (acc.z * il - wv.z) * scale, (acc.w * il - wv.w) * scale));
  }
}

// ---------------------------------------------------------------------------
// fp32: the same two passes in plain fp32 FMAs (the tiny fp32 model; no
// tensor-core path), 256 threads and 8 rows per workgroup.
constexpr int FR = 8;      // rows per workgroup
constexpr int FCH = 256;   // streamed rows per chunk (one per thread)

// pass 1: per row, lse by an online max/sum over all W rows, then
// dF = scale (sum_v p_v W_v - W_y) from a second sweep.
__global__ __launch_bounds__(256) void head_f32_fwd(const float* __restrict__ F, const float* __restrict__ W, int N, int V,
                                                    int C, const int32_t* __restrict__ y, float scale,
                                                    float* __restrict__ loss, float* __restrict__ lse_out,
                                                    float* __restrict__ dF, int* bad) {
  extern __shared__ float fsm[];  // [FR][C] rows of F, then [FR][FCH] gradients of a chunk
  float* rowsF = fsm;
  float* gch = fsm + FR * C;
  __shared__ float rm[FR][4], rsum[FR][4], rzy[FR];
  const int t = threadIdx.x, n0 = blockIdx.x * FR;
  for (int i = t; i < FR * C; i += 256) {
    const int r = i / C;
    rowsF[i] = (n0 + r < N) ? F[(int64_t)(n0 + r) * C + i % C] : 0.f;
  }
  if (t < FR) rzy[t] = 0.f;
  int yr[FR];
#pragma unroll
  for (int r = 0; r < FR; ++r) {
    int yy = (n0 + r < N) ? y[n0 + r] : 0;
    if (yy < 0 || yy >= V) {
      if (n0 + r < N && bad && t == 0) *bad = 1;
      yy = yy < 0 ? 0 : V - 1;
    }
    yr[r] = yy;
  }
  __syncthreads();
  float m[FR], s[FR];
#pragma unroll
  for (int r = 0; r < FR; ++r) {
    m[r] = -__builtin_huge_valf();
    s[r] = 0.f;
  }
  for (int v = t; v < V; v += 256) {
    float z[FR];
#pragma unroll
    for (int r = 0; r < FR; ++r) z[r] = 0.f;
    for (int c = 0; c < C; ++c) {
      const float wv = W[(int64_t)v * C + c];
#pragma unroll
      for (int r = 0; r < FR; ++r) z[r] = fmaf(rowsF[r * C + c], wv, z[r]);
    }
#pragma unroll
    for (int r = 0; r < FR; ++r) {
      if (v == yr[r]) rzy[r] = z[r];
      if (z[r] > m[r]) {
        s[r] = s[r] * hw_exp2((m[r] - z[r]) * LOG2E);
        m[r] = z[r];
      }
      s[r] += hw_exp2((z[r] - m[r]) * LOG2E);
    }
  }
  // combine the threads' (max, sum) pairs: across the wave, then the 4 waves
  const int lane = t & 63, wv = t >> 6;
#pragma unroll
  for (int r = 0; r < FR; ++r) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float mo = __shfl_xor(m[r], o, WAVE), so = __shfl_xor(s[r], o, WAVE);
      const float mn = fmaxf(m[r], mo);
      s[r] = (mn == -__builtin_huge_valf()) ? 0.f : s[r] * hw_exp2((m[r] - mn) * LOG2E) + so * hw_exp2((mo - mn) * LOG2E);
      m[r] = mn;
    }
    if (lane == 0) {
      rm[r][wv] = m[r];
      rsum[r][wv] = s[r];
    }
  }
  __syncthreads();
  float lse[FR];
#pragma unroll
  for (int r = 0; r < FR; ++r) {
    const float M = fmaxf(fmaxf(rm[r][0], rm[r][1]), fmaxf(rm[r][2], rm[r][3]));
    float S = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) S += rsum[r][k] * hw_exp2((rm[r][k] - M) * LOG2E);
    lse[r] = M + hw_log2(S) * LN2;
  }
  if (t < FR && n0 + t < N) {
    loss[n0 + t] = lse[t] - rzy[t];
    lse_out[n0 + t] = lse[t];
  }
  if (dF == nullptr) return;  // forward only (the whole workgroup leaves together)
  // second sweep: chunk of FCH W rows -> g[r][v] in LDS -> dF[r][c] += sum_v g[r][v] W[v][c]
  constexpr int CMAX = 4;  // columns per thread: C <= 1024
  float acc[FR][CMAX];
#pragma unroll
  for (int r = 0; r < FR; ++r)
#pragma unroll
    for (int k = 0; k < CMAX; ++k) acc[r][k] = 0.f;
  for (int v0 = 0; v0 < V; v0 += FCH) {
    const int v = v0 + t;
    float z[FR];
#pragma unroll
    for (int r = 0; r < FR; ++r) z[r] = 0.f;
    if (v < V)
      for (int c = 0; c < C; ++c) {
        const float wv2 = W[(int64_t)v * C + c];
#pragma unroll
        for (int r = 0; r < FR; ++r) z[r] = fmaf(rowsF[r * C + c], wv2, z[r]);
      }
    __syncthreads();  // the previous chunk's gradients are consumed
#pragma unroll
    for (int r = 0; r < FR; ++r)
      gch[r * FCH + t] = (v < V) ? (hw_exp2((z[r] - lse[r]) * LOG2E) - (v == yr[r] ? 1.f : 0.f)) * scale : 0.f;
    __syncthreads();
    const int nv = min(FCH, V - v0);
    for (int k = 0; k < nv; ++k) {
      const float* wr = W + (int64_t)(v0 + k) * C;
#pragma unroll
      for (int kc = 0; kc < CMAX; ++kc) {
        const int c = t + 256 * kc;
        if (c < C) {
          const float wv2 = wr[c];
#pragma unroll
          for (int r = 0; r < FR; ++r) acc[r][kc] = fmaf(gch[r * FCH + k], wv2, acc[r][kc]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < FR; ++r) {
    if (n0 + r >= N) continue;
#pragma unroll
    for (int kc = 0; kc < CMAX; ++kc) {
      const int c = t + 256 * kc;
      if (c < C) dF[(int64_t)(n0 + r) * C + c] = acc[r][kc];
    }
  }
}

// pass 2: per W row v, dW[v] (+)= sum_n scale (exp(z_nv - lse_n) - [y_n == v]) F_n
__global__ __launch_bounds__(256) void head_f32_dw(const float* __restrict__ F, const float* __restrict__ W, int N, int V,
                                                   int C, const int32_t* __restrict__ y, const float* __restrict__ lse,
                                                   float scale, float* __restrict__ dW, int accumulate) {
  extern __shared__ float fsm[];  // [FR][C] rows of W, then [FR][FCH] gradients of a chunk
  float* rowsW = fsm;
  float* gch = fsm + FR * C;
  const int t = threadIdx.x, v0 = blockIdx.x * FR;
  for (int i = t; i < FR * C; i += 256) {
    const int r = i / C;
    rowsW[i] = (v0 + r < V) ? W[(int64_t)(v0 + r) * C + i % C] : 0.f;
  }
  constexpr int CMAX = 4;
  float acc[FR][CMAX];
#pragma unroll
  for (int r = 0; r < FR; ++r)
#pragma unroll
    for (int k = 0; k < CMAX; ++k) acc[r][k] = 0.f;
  __syncthreads();
  for (int n0 = 0; n0 < N; n0 += FCH) {
    const int n = n0 + t;
    float z[FR];
#pragma unroll
    for (int r = 0; r < FR; ++r) z[r] = 0.f;
    if (n < N)
      for (int c = 0; c < C; ++c) {
        const float fv = F[(int64_t)n * C + c];
#pragma unroll
        for (int r = 0; r < FR; ++r) z[r] = fmaf(rowsW[r * C + c], fv, z[r]);
      }
    const float ln = n < N ? lse[n] : 0.f;
    const int yn = n < N ? y[n] : -1;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < FR; ++r)
      gch[r * FCH + t] = (n < N) ? (hw_exp2((z[r] - ln) * LOG2E) - (yn == v0 + r ? 1.f : 0.f)) * scale : 0.f;
    __syncthreads();
    const int nn = min(FCH, N - n0);
    for (int k = 0; k < nn; ++k) {
      const float* fr = F + (int64_t)(n0 + k) * C;
#pragma unroll
      for (int kc = 0; kc < CMAX; ++kc) {
        const int c = t + 256 * kc;
        if (c < C) {
          const float fv = fr[c];
#pragma unroll
          for (int r = 0; r < FR; ++r) acc[r][kc] = fmaf(gch[r * FCH + k], fv, acc[r][kc]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < FR; ++r) {
    if (v0 + r >= V) continue;
#pragma unroll
    for (int kc = 0; kc < CMAX; ++kc) {
      const int c = t + 256 * kc;
      if (c < C) {
        float* o = dW + (int64_t)(v0 + r) * C + c;
        *o = accumulate ? *o + acc[r][kc] : acc[r][kc];
      }
    }
  }
}

// launch a bf16 pass with the register/LDS shape for C
template <int MODE, bool SEG = false>
hipError_t launch_bf16_range(const Args& a, int ngmax, dim3 grid, hipStream_t s);

template <int MODE>
hipError_t launch_bf16(const Args& a, hipStream_t s, int max_wgs) {
  const int G = a.C / 64;
  const int ngmax = (G + 3) / 4;
  // fixed rows per workgroup: 64 (two 32-row tiles) while a wave's 64-column groups are <= 3, else 32.
  // max_wgs > 0 splits the pass into launches of at most that many workgroups
  // (blocks blk0 .. blk0 + grid - 1 each), queued one after another on s, so
  // no more than max_wgs of them are resident at once
  const int rows = ngmax <= 3 ? 64 : 32;
  const int nfix = (a.n_fix + rows - 1) / rows;
  const int step = max_wgs > 0 && max_wgs < nfix ? max_wgs : nfix;
  for (int b0 = 0; b0 < nfix; b0 += step) {
    Args ab = a;
    ab.blk0 = b0;
    if (hipError_t e = launch_bf16_range<MODE>(ab, ngmax, dim3(std::min(step, nfix - b0)), s)) return e;
  }
  return hipSuccess;
}

template <int MODE, bool SEG>
hipError_t launch_bf16_range(const Args& a, int ngmax, dim3 grid, hipStream_t s) {
  // the software-pipelined sweep where its registers fit (GPT_HEAD_PIPE=0: the sequential one)
  const char* e = getenv("GPT_HEAD_PIPE");
  const bool pipe = !(e && e[0] == '0');
  switch (ngmax) {
    case 1: hipLaunchKernelGGL((head_kernel<1, 2, 3, MODE, false, SEG>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((head_kernel<2, 2, 3, MODE, false, SEG>), grid, dim3(256), 0, s, a); break;
    case 3:
      if (pipe) hipLaunchKernelGGL((head_kernel<3, 2, 2, MODE, true, SEG>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((head_kernel<3, 2, 2, MODE, false, SEG>), grid, dim3(256), 0, s, a);
      break;
    case 4:
      if (pipe) hipLaunchKernelGGL((head_kernel<4, 1, 2, MODE, true, SEG>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((head_kernel<4, 1, 2, MODE, false, SEG>), grid, dim3(256), 0, s, a);
      break;
    case 5: hipLaunchKernelGGL((head_kernel<5, 1, 1, MODE, false, SEG>), grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL((head_kernel<6, 1, 1, MODE, false, SEG>), grid, dim3(256), 0, s, a); break;
    case 7: hipLaunchKernelGGL((head_kernel<7, 1, 1, MODE, false, SEG>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Pass 2's last round: with nfix blocks of W rows over the 256 CUs, a last
// round of t <= 128 blocks would run nearly alone (V = 50304, 64-row blocks:
// 786 = 3 x 256 + 18).  Those t blocks instead split the streamed rows into Z
// parts (Z t about 256 workgroups) whose partial dW go to a workspace and are
// summed in order afterwards.
struct TailPlan {
  int t = 0, Z = 1, z_rows = 0, row0 = 0, rows_valid = 0;
  int64_t floats = 0;
};
TailPlan tail_plan(int N, int V, int C) {
  TailPlan p;
  const int ngmax = (C / 64 + 3) / 4;
  const int rows = ngmax <= 3 ? 64 : 32;
  const int nfix = (V + rows - 1) / rows;
  const int t = nfix % 256;
  if (nfix <= 256 || t == 0 || t > 128) return p;
  const int Z = std::min(256 / t, std::max(1, N / (8 * BV)));  // at least 8 streamed blocks per part
  if (Z < 2) return p;
  p.t = t;
  p.row0 = (nfix - t) * rows;
  p.rows_valid = V - p.row0;
  p.z_rows = ((N + Z - 1) / Z + BV - 1) / BV * BV;
  p.Z = (N + p.z_rows - 1) / p.z_rows;
  p.floats = (int64_t)p.Z * p.rows_valid * C;
  return p;
}

// Pass 1 over vocabulary segments when its row blocks would leave CUs idle:
// with fewer than 256 blocks of fixed rows, the vocabulary is cut into nvs
// segments of vs_rows rows (at most 8, each at least 8 streamed blocks), so
// that about 256 workgroups run; the segments' partial results (nvs * N *
// (4 + C) floats) are combined per row afterwards.
struct SegPlan {
  int nvs = 1, vs_rows = 0, nfix = 0;
  int64_t floats = 0;
};
SegPlan seg_plan(int N, int V, int C) {
  SegPlan p;
  const int ngmax = (C / 64 + 3) / 4;
  const int rows = ngmax <= 3 ? 64 : 32;
  const int nfix = (N + rows - 1) / rows;
  if (nfix >= 256) return p;
  const int nvs = std::min(std::min(MAX_SEG, (256 + nfix - 1) / nfix), V / (8 * BV));
  if (nvs < 2) return p;
  p.vs_rows = ((V + nvs - 1) / nvs + BV - 1) / BV * BV;
  p.nvs = (V + p.vs_rows - 1) / p.vs_rows;
  if (p.nvs < 2) return SegPlan{};
  p.nfix = nfix;
  p.floats = (int64_t)p.nvs * N * (4 + C);
  return p;
}

// Row statistics of one block of logit columns for the GEMM form of pass 1
// (the same softmax, reached a column block at a time): z holds the block's
// logits [N][ldz] for vocabulary columns v0 .. v0 + n - 1.  One wave per row:
// each lane keeps a running maximum and sum of exp over its columns, the
// lanes' pairs are combined by the usual rescaling, and the block's pair is
// merged into the row's (m, l) the same way (block 0 starts them).  The block
// holding the row's target records its logit; the last block writes
// lse = m + ln l and the row loss lse - z_y.  A target outside [0, V) is
// clamped into the row and sets *bad.
__device__ __forceinline__ void ml_merge(float& m, float& l, float m2, float l2) {
  const float M = fmaxf(m, m2);
  const float a = m == NEG_INF ? 0.f : l * hw_exp(m - M);
  const float b = m2 == NEG_INF ? 0.f : l2 * hw_exp(m2 - M);
  m = M;
  l = a + b;
}
__global__ __launch_bounds__(256) void block_stats_kernel(const float* __restrict__ z, int ldz, int N, int n, int v0,
                                                          int V, const int32_t* __restrict__ y, float* __restrict__ ml,
                                                          float* __restrict__ zy, float* __restrict__ loss,
                                                          float* __restrict__ lse, int first, int last,
                                                          int* __restrict__ bad) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= N) return;
  const float* zr = z + (int64_t)row * ldz;
  float m = NEG_INF, l = 0.f;
  for (int c = lane * 4; c < n; c += 256) {
    if (c + 3 < n) {
      const float4 v = *reinterpret_cast<const float4*>(zr + c);
      ml_merge(m, l, v.x, 1.f);
      ml_merge(m, l, v.y, 1.f);
      ml_merge(m, l, v.z, 1.f);
      ml_merge(m, l, v.w, 1.f);
    } else {
      for (int k = c; k < n; ++k) ml_merge(m, l, zr[k], 1.f);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    ml_merge(m, l, m2, l2);
  }
  if (lane != 0) return;
  float* mlr = ml + 2 * (int64_t)row;
  float rm = m, rl = l;
  if (!first) {
    rm = mlr[0];
    rl = mlr[1];
    ml_merge(rm, rl, m, l);
  }
  int t = y[row];
  if (t < 0 || t >= V) {
    if (bad) *bad = 1;
    t = t < 0 ? 0 : V - 1;
  }
  if (t >= v0 && t < v0 + n) zy[row] = zr[t - v0];
  if (last) {
    const float s = rm + hw_log2(rl) * LN2;
    lse[row] = s;
    loss[row] = s - zy[row];
  } else {
    mlr[0] = rm;
    mlr[1] = rl;
  }
}

}  // namespace hd

hipError_t lmhead_block_stats(const float* z, int ldz, int N, int n, int v0, int V, const int32_t* y, float* ml,
                              float* zy, float* loss, float* lse, int first, int last, int* bad, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (n <= 0 || ldz < n || ((uintptr_t)z & 15) || (ldz & 3)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(hd::block_stats_kernel, dim3((N + 3) / 4), dim3(256), 0, s, z, ldz, N, n, v0, V, y, ml, zy,
                     loss, lse, first, last, bad);
  return hipGetLastError();
}

int64_t lmhead_fwd_seg_floats(int dtype, int N, int V, int C) {
  return dtype == BF16 ? hd::seg_plan(N, V, C).floats : 0;
}

int64_t lmhead_dw_tail_floats(int dtype, int N, int V, int C) {
  return dtype == BF16 ? hd::tail_plan(N, V, C).floats : 0;
}

// bf16: up to 7 column groups of 64 per wave; fp32: the plain kernels keep 8 rows of C floats
// plus a 256-row gradient chunk in LDS (40 KB at C = 1024)
int lmhead_max_embd(int dtype) { return dtype == BF16 ? 7 * 4 * 64 : 1024; }

hipError_t lmhead_fwd(int dtype, const void* F, const void* W, int N, int V, int C, const int32_t* y, float scale,
                      float* loss, float* lse, float* dF, int* bad, hipStream_t s, float* seg_ws,
                      int64_t seg_floats) {
  if (N <= 0) return hipSuccess;
  if (V <= 0 || C <= 0 || C % 64 || C > lmhead_max_embd(dtype)) return hipErrorInvalidValue;
  if (dtype == BF16) {
    // 32-bit buffer offsets into the streamed W (the last block's rows run up to 31 past V)
    if ((int64_t)(V + 32) * C * 2 >= (1ll << 32)) return hipErrorInvalidValue;
    hd::Args a{};
    a.fix = (const bf16*)F;
    a.str = (const bf16*)W;
    a.n_fix = N;
    a.n_str = V;
    a.C = C;
    a.y = y;
    a.loss = loss;
    a.lse_out = lse;
    a.out = dF;
    a.scale = scale;
    a.bad = bad;
    const hd::SegPlan sp = seg_ws ? hd::seg_plan(N, V, C) : hd::SegPlan{};
    if (sp.nvs < 2 || sp.floats > seg_floats) return hd::launch_bf16<0>(a, s, 0);
    hd::Args b = a;  // segment z of every block of rows, then the per-row combination
    b.nz = sp.nvs;
    b.tb = sp.nfix;
    b.z_rows = sp.vs_rows;
    b.seg_s = seg_ws;
    b.out = dF ? seg_ws + (int64_t)sp.nvs * N * 4 : nullptr;
    b.z_stride = (int64_t)N * C;
    if (hipError_t e = hd::launch_bf16_range<0, true>(b, (C / 64 + 3) / 4, dim3(sp.nvs * sp.nfix), s)) return e;
    hipLaunchKernelGGL(hd::seg_combine_kernel, dim3(N), dim3(256), 0, s, seg_ws, b.out, sp.nvs, N, V, C,
                       (const bf16*)W, y, scale, loss, lse, dF);
    return hipGetLastError();
  }
  const size_t sh = (size_t)(hd::FR * C + hd::FR * hd::FCH) * 4;
  hipLaunchKernelGGL(hd::head_f32_fwd, dim3((N + hd::FR - 1) / hd::FR), dim3(256), sh, s, (const float*)F,
                     (const float*)W, N, V, C, y, scale, loss, lse, dF, bad);
  return hipGetLastError();
}

hipError_t lmhead_dw(int dtype, const void* F, const void* W, int N, int V, int C, const int32_t* y, const float* lse,
                     float scale, float* dW, int accumulate, hipStream_t s, int max_wgs, float* tail_ws,
                     int64_t tail_floats) {
  if (V <= 0) return hipSuccess;
  if (N <= 0 || C <= 0 || C % 64 || C > lmhead_max_embd(dtype)) return hipErrorInvalidValue;
  if (dtype == BF16) {
    if ((int64_t)(N + 32) * C * 2 >= (1ll << 32)) return hipErrorInvalidValue;
    hd::Args a{};
    a.fix = (const bf16*)W;
    a.str = (const bf16*)F;
    a.n_fix = V;
    a.n_str = N;
    a.C = C;
    a.y = y;
    a.lse = lse;
    a.out = dW;
    a.accumulate = accumulate;
    a.scale = scale;
    const hd::TailPlan tp = tail_ws ? hd::tail_plan(N, V, C) : hd::TailPlan{};
    if (tp.t == 0 || tp.floats > tail_floats) return hd::launch_bf16<1>(a, s, max_wgs);
    hd::Args m = a;  // the full rounds: W rows [0, row0)
    m.n_fix = tp.row0;
    if (hipError_t e = hd::launch_bf16<1>(m, s, max_wgs)) return e;
    hd::Args t = a;  // the last blocks, split over the rows of F
    const int ngmax = (C / 64 + 3) / 4, rows = ngmax <= 3 ? 64 : 32;
    t.blk0 = tp.row0 / rows;
    t.nz = tp.Z;
    t.tb = tp.t;
    t.z_rows = tp.z_rows;
    t.out = tail_ws;
    t.out_row0 = tp.row0;
    t.z_stride = (int64_t)tp.rows_valid * C;
    t.accumulate = 0;
    if (hipError_t e = hd::launch_bf16_range<1>(t, ngmax, dim3(tp.Z * tp.t), s)) return e;
    return splits_reduce(tail_ws, tp.Z, tp.rows_valid, C, dW + (int64_t)tp.row0 * C, C, accumulate, s);
  }
  const size_t sh = (size_t)(hd::FR * C + hd::FR * hd::FCH) * 4;
  hipLaunchKernelGGL(hd::head_f32_dw, dim3((V + hd::FR - 1) / hd::FR), dim3(256), sh, s, (const float*)F,
                     (const float*)W, N, V, C, y, lse, scale, dW, accumulate);
  return hipGetLastError();
}

}  // namespace gk
