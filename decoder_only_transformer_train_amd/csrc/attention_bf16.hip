// Causal flash attention for bf16, head size 64, on gfx950 32x32x16 MFMAs.
//
// Same method as the fp32 kernels in attention.hip (online softmax over
// 64-key blocks, log-sum-exp saved for a recomputing backward, dK/dV and dQ
// by separate atomic-free workgroups), laid out for the 32x32 MFMA and the LDS
// direct-load path:
//  * Every streamed operand block is 64 rows x 64 d of a row-major [T][ld]
//    tensor, moved by buffer_load_dwordx4 ... lds straight into an 8 KB LDS
//    tile (one wave instruction = 8 rows); the next blocks are in flight while
//    the current one is consumed.  The 16-byte chunks of row r sit XOR-permuted
//    by swz(r), which keeps both read forms below free of bank conflicts.
//  * A block is read two ways: as row fragments (ds_read_b128: lane = row,
//    8 consecutive d) when its rows index the MFMA's output rows, and as
//    transposed fragments (two ds_read_b64_tr_b16: lane = d, 8 rows) when its
//    rows are the contraction index, so no transposed copy is ever stored.
//  * Scores are computed in the orientation whose C tile feeds the next
//    product as its B operand: lane l of a 32x32 C tile holds column l % 32
//    and rows (e / 4) * 8 + (l / 32) * 4 + e % 4, e = 0..15; the 8 values of
//    one 16-row half are a 32x32x16 B fragment whose k order the transposed
//    reads reproduce.
//  * Forward and dQ workgroups take a 256-query block; wave w owns the
//    32-row tiles w and 7 - w, so every wave has one early and one late tile
//    and the causal work is balanced.  A dK/dV workgroup takes 128 keys, one
//    32-key tile per wave.
//  * Workgroup order: the grids are one-dimensional, longest blocks first,
//    with (batch, head) varying fastest.  The hardware deals workgroup i to
//    XCD i % 8, so every XCD gets the same mix of long and short causal
//    blocks (a [blocks][heads] grid put all of one block index on the same
//    XCDs, up to 1.8x the mean load on one of them), and the blocks of one
//    head land on one XCD, whose L2 then serves their shared rows.  The
//    backward's dK/dV and dQ blocks share one launch and one such order, so
//    a single tail ends both.
//  * Forward softmax: the two tiles of a wave share one read of the K and V
//    fragments of a block.  The running maximum is updated lazily: the
//    output is rescaled only when a block's maximum exceeds it by more than
//    2^TAU, so p stays below 2^TAU (exact in bf16 range and fp32 sums) and
//    the rescale branch is rare after a row's first block.  Each lane half
//    keeps its own running sum of the bf16-rounded p (the values the PV
//    product uses), added once at the end.
//  * Stage refills: iteration j waits for its block, passes the barrier
//    (every wave is done with block j - 1), refills block j - 1's stage with
//    block j + ST - 1 and consumes block j.  The stage pointers are distinct
//    and passed as __restrict__, which lets the compiler drop its blanket wait
//    on outstanding direct-to-LDS loads before LDS reads; the real
//    dependencies are the explicit vmcnt wait and the barrier.
#include <algorithm>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace gk {
namespace fa {

constexpr int HD = 64;             // head size
constexpr int TILE = 64 * HD * 2;  // bytes of one 64-row block
constexpr int ST = 3;              // LDS stages
constexpr float NEG_INF = -__builtin_huge_valf();

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
// one wave instruction: lane i's 16 (4) bytes at voff land at lds + 16 i (4 i);
// loads past the descriptor's range write zeros
__device__ __forceinline__ void dma16(rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, 0, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt simm16 on gfx9: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt at their maxima
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// wait until at most n (0 or 1) blocks' loads, NL instructions each, are outstanding
template <int NL>
__device__ __forceinline__ void wait_blocks(int n) {
  if (n >= 1) wait_vm<NL>();
  else wait_vm<0>();
}

__device__ __forceinline__ void mma32(f32x16& c, const uint4& a, const uint4& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0, 0, 0);
}
__device__ __forceinline__ void zero16(f32x16& c) {
#pragma unroll
  for (int e = 0; e < 16; ++e) c[e] = 0.f;
}
// row offset (within a 32-row C tile) of accumulator e for lane group g
__device__ __forceinline__ int crow(int e, int g) { return (e >> 2) * 8 + g * 4 + (e & 3); }

// chunk permutation of row r (8 chunks of 16 bytes per 128-byte row): for the
// 16 rows one ds_read_b128 pass touches, and for the 4 rows x 4 chunks one
// transpose-read pass touches, every 16-byte slot of a 256-byte bank window
// is hit once
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// Per-lane source offsets of one wave's 2 instructions (rows 8 i .. 8 i + 7 of
// a block, i = 2 w + ii): lane L loads chunk (L % 8) ^ swz(row) of row L / 8.
struct BlockLoad {
  uint32_t off[2];
  __device__ __forceinline__ void init(int64_t ld, int col0, int w, int lane) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int r = (w * 2 + ii) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      off[ii] = (uint32_t)(((int64_t)r * ld + col0 + c * 8) * 2);
    }
  }
  // the block starting row0_bytes into the operand; rows past it read as zero
  __device__ __forceinline__ void issue(rsrc_t r, char* s, uint32_t row0_bytes, int w) const {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) dma16(r, s + (w * 2 + ii) * 1024, off[ii] + row0_bytes);
  }
};

// A fragment of block row `row`, d = 16 kk .. 16 kk + 15 (lane half g takes 8 of them)
__device__ __forceinline__ uint4 frag_row(const char* s, int row, int kk, int g) {
  const int c = (kk * 2 + g) ^ swz(row);
  return *reinterpret_cast<const uint4*>(s + row * 128 + c * 16);
}
// A fragment of the transposed block: lane l holds d = d0 + l % 32 and block
// rows r0 + 4 (l / 32) + j, then r0 + 8 + 4 (l / 32) + j (j = 0..3) - the k
// order of pack_half over a C tile's 16-row half starting at r0.  In each
// 16-lane group G, lane s reads 4 consecutive d of one row; the transpose read
// hands lane i element i % 4 of the row read by lane i / 4 + 4 j.
__device__ __forceinline__ uint4 frag_tr(const char* s, int d0, int r0, int lane) {
  const int G = lane >> 4, sl = lane & 15;
  const int dd = d0 + 16 * (G & 1) + 4 * (sl & 3);
  const int c = dd >> 3, sub = (dd & 7) * 2;
  const int ra = r0 + 4 * (G >> 1) + (sl >> 2), rb = ra + 8;
  v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(s + ra * 128 + ((c ^ swz(ra)) * 16) + sub));
  v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(s + rb * 128 + ((c ^ swz(rb)) * 16) + sub));
  const uint2 a = bitcast<uint2>(lo), b = bitcast<uint2>(hi);
  return make_uint4(a.x, a.y, b.x, b.y);
}
// B fragment from half hh of a 32x32 C tile (accumulators 8 hh .. 8 hh + 7)
__device__ __forceinline__ uint4 pack_half(const f32x16& c, int hh) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (bf16)c[8 * hh + j];
  return bitcast<uint4>(v);
}

// ---------------------------------------------------------------------------
// Forward.  Stage = K block + V block (16 KB).  A wave owns two 32-query tiles
// (A early, B late); both read the same K and V fragments of a block.
constexpr float TAU = 8.0f;  // lazy rescale: the running max may lag the true one by up to 2^8

struct QTile {
  uint4 qf[4];
  f32x16 o[2];
  float m, l;  // running max (scaled log2 units), this lane half's running sum
};

__device__ __forceinline__ void read_kf(uint4 (&kf)[2][4], const char* sK, int c32, int g) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf[kt][kk] = frag_row(sK, kt * 32 + c32, kk, g);
}
__device__ __forceinline__ void read_vf(uint4 (&vf)[4][2], const char* sV, int lane) {
#pragma unroll
  for (int hh = 0; hh < 4; ++hh)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) vf[hh][dt] = frag_tr(sV, dt * 32, hh * 16, lane);
}
__device__ __forceinline__ void scores(f32x16 (&s)[2], const uint4 (&kf)[2][4], const uint4 (&qf)[4]) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    zero16(s[kt]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) mma32(s[kt], kf[kt][kk], qf[kk]);
  }
}
// keys after the query (or past the sequence: qc = min(q, T - 1)) -> -inf
__device__ __forceinline__ void mask_keys(f32x16 (&s)[2], int key0, int qc, int g) {
  int rel = qc - key0 - g * 4;  // query minus the lane half's first key
  asm volatile("" : "+v"(rel));  // keep the compares in the block that uses them
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kt][e] = (kt * 32 + (e >> 2) * 8 + (e & 3) <= rel) ? s[kt][e] : NEG_INF;
}
__device__ __forceinline__ float swap_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// the query's maximum raw score over the block (both lane halves)
__device__ __forceinline__ float rowmax(const f32x16 (&s)[2]) {
  float a = NEG_INF, b = NEG_INF;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    a = fmaxf(a, s[0][e]);
    b = fmaxf(b, s[1][e]);
  }
  return swap_halves(fmaxf(a, b));
}
__device__ __forceinline__ void rescale(QTile& T, float mxs) {
  const float mnew = fmaxf(T.m, mxs);
  const float alpha = hw_exp2(T.m - mnew);
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) T.o[dt] *= alpha;
  T.l *= alpha;
  T.m = mnew;
}
// p = 2^(s cs - m) packed to bf16 as the B fragments of the PV product; the
// running sum adds the rounded p (the same values the product uses)
__device__ __forceinline__ void probs(QTile& T, const f32x16 (&s)[2], uint4 (&p)[4], float cs) {
  float l = T.l;
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (bf16)hw_exp2(fmaf(s[hh >> 1][8 * (hh & 1) + j], cs, -T.m));
    p[hh] = bitcast<uint4>(v);
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t one = {(bf16)1.0f, (bf16)1.0f};
    l = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(p[hh].x), one, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(p[hh].y), one, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(p[hh].z), one, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(p[hh].w), one, l, false);
  }
  T.l = l;
}
__device__ __forceinline__ void pv(QTile& T, const uint4 (&vf)[4][2], const uint4 (&p)[4]) {
#pragma unroll
  for (int hh = 0; hh < 4; ++hh)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) mma32(T.o[dt], vf[hh][dt], p[hh]);
}

// both tiles against one block; MASK: the block is the last of A (and of B if mB)
template <bool MASK>
__device__ __forceinline__ void fwd_both(const char* sK, const char* sV, QTile& A, QTile& B, int key0, int qcA,
                                         int qcB, bool mB, int lane) {
  const int g = lane >> 5, c32 = lane & 31;
  const float cs = LOG2E / 8.0f;
  uint4 kf[2][4];
  read_kf(kf, sK, c32, g);
  f32x16 sA[2], sB[2];
  scores(sA, kf, A.qf);
  scores(sB, kf, B.qf);
  if (MASK) {
    mask_keys(sA, key0, qcA, g);
    if (mB) mask_keys(sB, key0, qcB, g);
  }
  const float mxA = rowmax(sA) * cs, mxB = rowmax(sB) * cs;
  uint4 vf[4][2];
  read_vf(vf, sV, lane);
  if (__any((mxA > A.m + TAU) | (mxB > B.m + TAU))) {
    rescale(A, mxA);
    rescale(B, mxB);
  }
  uint4 p[4];
  probs(A, sA, p, cs);
  pv(A, vf, p);
  probs(B, sB, p, cs);
  pv(B, vf, p);
}
template <bool MASK>
__device__ __forceinline__ void fwd_one(const char* sK, const char* sV, QTile& B, int key0, int qcB, int lane) {
  const int g = lane >> 5, c32 = lane & 31;
  const float cs = LOG2E / 8.0f;
  uint4 kf[2][4];
  read_kf(kf, sK, c32, g);
  f32x16 sB[2];
  scores(sB, kf, B.qf);
  if (MASK) mask_keys(sB, key0, qcB, g);
  const float mxB = rowmax(sB) * cs;
  uint4 vf[4][2];
  read_vf(vf, sV, lane);
  if (__any(mxB > B.m + TAU)) rescale(B, mxB);
  uint4 p[4];
  probs(B, sB, p, cs);
  pv(B, vf, p);
}

// one key block: wait for it, refill the stage freed by the previous block, then
// the tiles that still need this block (distinct __restrict__ stage pointers
// keep the compiler from waiting on every outstanding direct-to-LDS load)
__device__ __forceinline__ void fwd_iter(const char* __restrict__ rd, char* __restrict__ wr, int kb, int nkb, rsrc_t r,
                                         const BlockLoad& lk, const BlockLoad& lv, uint32_t blk_bytes, QTile& A,
                                         QTile& B, int lastA, int lastB, int qcA, int qcB, int w, int lane) {
  wait_blocks<4>(min(ST - 2, nkb - 1 - kb));
  __syncthreads();
  if (kb + ST - 1 < nkb) {
    lk.issue(r, wr, (uint32_t)(kb + ST - 1) * blk_bytes, w);
    lv.issue(r, wr + TILE, (uint32_t)(kb + ST - 1) * blk_bytes, w);
  }
  if (kb < lastA) fwd_both<false>(rd, rd + TILE, A, B, kb * 64, qcA, qcB, false, lane);
  else if (kb == lastA) fwd_both<true>(rd, rd + TILE, A, B, kb * 64, qcA, qcB, lastB == lastA, lane);
  else if (kb < lastB) fwd_one<false>(rd, rd + TILE, B, kb * 64, qcB, lane);
  else if (kb == lastB) fwd_one<true>(rd, rd + TILE, B, kb * 64, qcB, lane);
}

__global__ __launch_bounds__(256, 2) void fwd_kernel(const bf16* __restrict__ qkv, bf16* __restrict__ o,
                                                     float* __restrict__ lse2, int Tn, int H) {
  __shared__ __attribute__((aligned(16))) char smem[ST * 2 * TILE];
  const int nqb = (Tn + 255) / 256;
  const int BH = gridDim.x / nqb;
  const int qb = nqb - 1 - (int)blockIdx.x / BH;  // latest (longest) query blocks first
  const int bh = (int)blockIdx.x % BH, b = bh / H, h = bh % H;
  const int Cc = H * HD;
  const int64_t ld = 3 * (int64_t)Cc;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const rsrc_t r = make_rsrc(base, (int64_t)Tn * ld * 2);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 5, c32 = lane & 31;
  const int q0 = qb * 256;
  const int nkb = (min(Tn, q0 + 256) + 63) / 64;
  QTile A, B;
  QTile* tl[2] = {&A, &B};
  const int qlo[2] = {q0 + w * 32, q0 + (7 - w) * 32};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    QTile& Q = *tl[i];
    const int q = qlo[i] + c32;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      Q.qf[kk] = (q < Tn) ? *reinterpret_cast<const uint4*>(base + (int64_t)q * ld + h * HD + kk * 16 + g * 8)
                          : make_uint4(0, 0, 0, 0);
    zero16(Q.o[0]);
    zero16(Q.o[1]);
    Q.m = NEG_INF;
    Q.l = 0.f;
  }
  // each tile's last block (the only one that needs the causal mask)
  const int lastA = min((qlo[0] + 31) / 64, nkb - 1), lastB = min((qlo[1] + 31) / 64, nkb - 1);
  const int qcA = min(qlo[0] + c32, Tn - 1), qcB = min(qlo[1] + c32, Tn - 1);
  BlockLoad lk, lv;
  lk.init(ld, Cc + h * HD, w, lane);
  lv.init(ld, 2 * Cc + h * HD, w, lane);
  const uint32_t blk_bytes = (uint32_t)(64 * ld * 2);
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nkb) {
      lk.issue(r, smem + s * 2 * TILE, (uint32_t)s * blk_bytes, w);
      lv.issue(r, smem + s * 2 * TILE + TILE, (uint32_t)s * blk_bytes, w);
    }
  int sc = 0;
  for (int kb = 0; kb < nkb; ++kb) {
    const int sw = sc == 0 ? ST - 1 : sc - 1;
    fwd_iter(smem + sc * 2 * TILE, smem + sw * 2 * TILE, kb, nkb, r, lk, lv, blk_bytes, A, B, lastA, lastB, qcA, qcB,
             w, lane);
    sc = sc + 1 == ST ? 0 : sc + 1;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    QTile& Q = *tl[i];
    const int q = qlo[i] + c32;
    const float lsum = Q.l + __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(Q.l), __float_as_uint(Q.l), false, false)[g == 0 ? 1 : 0]);
    if (q >= Tn) continue;
    const float inv = 1.f / lsum;
    bf16* orow = o + (int64_t)(b * Tn + q) * Cc + h * HD;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        store4(orow + dt * 32 + r4 * 8 + g * 4,
               make_float4(Q.o[dt][4 * r4] * inv, Q.o[dt][4 * r4 + 1] * inv, Q.o[dt][4 * r4 + 2] * inv,
                           Q.o[dt][4 * r4 + 3] * inv));
    if (g == 0) lse2[(int64_t)bh * Tn + q] = Q.m + hw_log2(lsum);
  }
}

// ---------------------------------------------------------------------------
// dK, dV for a 128-key block (one 32-key tile per wave): streams the 64-query
// blocks from the block's diagonal to the end.  Stage = Q block + dO block +
// 64 log-sum-exps + 64 D values (16 KB + 512 B); the two dword loads go to
// waves 0 and 1, so those waves count 5 load instructions per block, the
// others 4.
constexpr int KV_STAGE = 2 * TILE + 512;

struct KvState {
  uint4 kf[4], vf[4];
  f32x16 dk[2], dv[2];
  int key, klo;
};

struct KvLoads {
  rsrc_t rq, rdo, rl, rdv;
  BlockLoad lq, ldo;
  uint32_t qblk_bytes, dblk_bytes;
  __device__ __forceinline__ void issue(char* st, int qb, int w, int lane) const {
    lq.issue(rq, st, (uint32_t)qb * qblk_bytes, w);
    ldo.issue(rdo, st + TILE, (uint32_t)qb * dblk_bytes, w);
    if (w < 2) dma4(w == 0 ? rl : rdv, st + 2 * TILE + w * 256, (uint32_t)(qb * 64 + lane) * 4);
  }
};

template <bool MASK>
__device__ __forceinline__ void kv_block(const char* __restrict__ rd, char* __restrict__ wr, int j, int nblk,
                                         int qb0, const KvLoads& L, KvState& S, int Tn, int w, int lane) {
  const int g = lane >> 5, c32 = lane & 31;
  const int n_out = min(ST - 2, nblk - 1 - j);
  if (w < 2) wait_blocks<5>(n_out);
  else wait_blocks<4>(n_out);
  __syncthreads();
  if (j + ST - 1 < nblk) L.issue(wr, qb0 + j + ST - 1, w, lane);
  const int qb = qb0 + j;
  if (MASK && qb * 64 + 63 < S.klo) return;  // every query of the block is before every key of the tile
  const char* sQ = rd;
  const char* sdO = rd + TILE;
  const float* slse = reinterpret_cast<const float*>(rd + 2 * TILE);
  const float* sDv = slse + 64;
  const float cs = LOG2E / 8.0f;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    f32x16 s, dp;
    zero16(s);
    zero16(dp);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      mma32(s, frag_row(sQ, qt * 32 + c32, kk, g), S.kf[kk]);
      mma32(dp, frag_row(sdO, qt * 32 + c32, kk, g), S.vf[kk]);
    }
    // Rows past the sequence need no mask: their Q and dO rows load as zeros, so
    // their dS = p (dO.V - D) = p (0 - 0) and their P^T dO terms vanish.  Only the
    // causal mask is left, and only on tiles that reach past the diagonal.
    const bool diag = MASK && S.klo + 31 > qb * 64 + qt * 32;
    float lv[16], dv[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int qi0 = qt * 32 + r4 * 8 + g * 4;  // rows crow(4 r4 .. 4 r4 + 3, g)
      const float4 l4 = *reinterpret_cast<const float4*>(slse + qi0);
      const float4 d4 = *reinterpret_cast<const float4*>(sDv + qi0);
      lv[4 * r4] = l4.x; lv[4 * r4 + 1] = l4.y; lv[4 * r4 + 2] = l4.z; lv[4 * r4 + 3] = l4.w;
      dv[4 * r4] = d4.x; dv[4 * r4 + 1] = d4.y; dv[4 * r4 + 2] = d4.z; dv[4 * r4 + 3] = d4.w;
    }
    if (diag) {
      // keep s <= 0 mask inputs: score -> -inf for keys after the query, so p = 0
      const int rel = qb * 64 + qt * 32 - S.key;  // query row of crow(e) minus this lane's key
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = (rel + crow(e, g) >= 0) ? s[e] : NEG_INF;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = hw_exp2(fmaf(s[e], cs, -lv[e]));
      s[e] = p;
      dp[e] = p * (dp[e] - dv[e]);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint4 bp = pack_half(s, hh);
      const uint4 bds = pack_half(dp, hh);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        mma32(S.dv[dt], frag_tr(sdO, dt * 32, qt * 32 + hh * 16, lane), bp);
        mma32(S.dk[dt], frag_tr(sQ, dt * 32, qt * 32 + hh * 16, lane), bds);
      }
    }
  }
}

__device__ __forceinline__ void dkdv_item(char* smem, int kb, int bh, const bf16* __restrict__ qkv,
                                          const bf16* __restrict__ dO, const float* __restrict__ lse2,
                                          const float* __restrict__ Dv, bf16* __restrict__ dqkv, int Tn, int H) {
  const int nqb = (Tn + 63) / 64;
  const int b = bh / H, h = bh % H;
  const int Cc = H * HD;
  const int64_t ld = 3 * (int64_t)Cc;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const bf16* dob = dO + (int64_t)b * Tn * Cc;
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), g = lane >> 5, c32 = lane & 31;
  KvLoads L;
  L.rq = make_rsrc(base, (int64_t)Tn * ld * 2);
  L.rdo = make_rsrc(dob, (int64_t)Tn * Cc * 2);
  L.rl = make_rsrc(lse2 + (int64_t)bh * Tn, (int64_t)Tn * 4);
  L.rdv = make_rsrc(Dv + (int64_t)bh * Tn, (int64_t)Tn * 4);
  L.lq.init(ld, h * HD, w, lane);
  L.ldo.init(Cc, h * HD, w, lane);
  L.qblk_bytes = (uint32_t)(64 * ld * 2);
  L.dblk_bytes = (uint32_t)(64 * Cc * 2);
  const int k0 = kb * 128;
  KvState S;
  S.klo = k0 + w * 32;
  S.key = S.klo + c32;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const bool ok = S.key < Tn;
    const int64_t off = (int64_t)S.key * ld + h * HD + kk * 16 + g * 8;
    S.kf[kk] = ok ? *reinterpret_cast<const uint4*>(base + Cc + off) : make_uint4(0, 0, 0, 0);
    S.vf[kk] = ok ? *reinterpret_cast<const uint4*>(base + 2 * Cc + off) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    zero16(S.dk[dt]);
    zero16(S.dv[dt]);
  }
  const int qb0 = k0 / 64;
  const int nblk = nqb - qb0;  // this workgroup streams query blocks qb0 .. nqb - 1
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nblk) L.issue(smem + s * KV_STAGE, qb0 + s, w, lane);
  // Only the first two query blocks reach the diagonal of this workgroup's
  // keys; the rest run a copy of the block without the mask and its branches,
  // so that one tile's softmax and the next tile's products share one
  // straight-line stretch of code the compiler can interleave.
  int sc = 0, j = 0;
  for (; j < min(2, nblk); ++j) {
    const int sw = sc == 0 ? ST - 1 : sc - 1;
    kv_block<true>(smem + sc * KV_STAGE, smem + sw * KV_STAGE, j, nblk, qb0, L, S, Tn, w, lane);
    sc = sc + 1 == ST ? 0 : sc + 1;
  }
  for (; j < nblk; ++j) {
    const int sw = sc == 0 ? ST - 1 : sc - 1;
    kv_block<false>(smem + sc * KV_STAGE, smem + sw * KV_STAGE, j, nblk, qb0, L, S, Tn, w, lane);
    sc = sc + 1 == ST ? 0 : sc + 1;
  }
  if (S.key < Tn) {
    bf16* krow = dqkv + (int64_t)(b * Tn + S.key) * ld + Cc + h * HD;
    bf16* vrow = krow + Cc;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = dt * 32 + r4 * 8 + g * 4;
        store4(krow + d, make_float4(S.dk[dt][4 * r4] * 0.125f, S.dk[dt][4 * r4 + 1] * 0.125f,
                                     S.dk[dt][4 * r4 + 2] * 0.125f, S.dk[dt][4 * r4 + 3] * 0.125f));
        store4(vrow + d,
               make_float4(S.dv[dt][4 * r4], S.dv[dt][4 * r4 + 1], S.dv[dt][4 * r4 + 2], S.dv[dt][4 * r4 + 3]));
      }
  }
}

// ---------------------------------------------------------------------------
// dQ for a 256-query block: streams 64-key blocks up to the block's diagonal.
// Stage = K block + V block (16 KB).
struct DqState {
  uint4 qf[2][4], dof[2][4];
  f32x16 dq[2][2];
  float lq[2], dd[2];
  int q[2], qlo[2];
};

template <bool MASK>
__device__ __forceinline__ void dq_block(const char* __restrict__ rd, char* __restrict__ wr, int kb, int nkb, rsrc_t r,
                                         const BlockLoad& lk, const BlockLoad& lv, uint32_t blk_bytes, DqState& S,
                                         int w, int lane) {
  const int g = lane >> 5, c32 = lane & 31;
  wait_blocks<4>(min(ST - 2, nkb - 1 - kb));
  __syncthreads();
  if (kb + ST - 1 < nkb) {
    lk.issue(r, wr, (uint32_t)(kb + ST - 1) * blk_bytes, w);
    lv.issue(r, wr + TILE, (uint32_t)(kb + ST - 1) * blk_bytes, w);
  }
  const char* sK = rd;
  const char* sV = rd + TILE;
  const float cs = LOG2E / 8.0f;
  // one 32-key half at a time (its K and V fragments serve both query tiles):
  // scores, dP, dS, then its two 16-key dQ steps
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (MASK && kb * 64 > S.qlo[i] + 31) continue;
      f32x16 s, dp;
      zero16(s);
      zero16(dp);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        mma32(s, frag_row(sK, kt * 32 + c32, kk, g), S.qf[i][kk]);
        mma32(dp, frag_row(sV, kt * 32 + c32, kk, g), S.dof[i][kk]);
      }
      // a query past the sequence has lse = D = 0 and its dQ is never stored;
      // keys past the sequence come after every valid query
      // Only the causal mask, only where this half reaches past the tile's
      // first query (keys past the sequence load as zeros and contribute nothing).
      if (MASK && kb * 64 + kt * 32 + 31 > S.qlo[i]) {
        const int rel = S.q[i] - (kb * 64 + kt * 32);  // this lane's query minus the half's first key
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = (crow(e, g) <= rel) ? s[e] : NEG_INF;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = hw_exp2(fmaf(s[e], cs, -S.lq[i])) * (dp[e] - S.dd[i]);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint4 bds = pack_half(s, hh);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
          mma32(S.dq[i][dt], frag_tr(sK, dt * 32, kt * 32 + hh * 16, lane), bds);
      }
    }
  }
}

__device__ __forceinline__ void dq_item(char* smem, int qb, int bh, const bf16* __restrict__ qkv,
                                        const bf16* __restrict__ dO, const float* __restrict__ lse2,
                                        const float* __restrict__ Dv, bf16* __restrict__ dqkv, int Tn, int H) {
  const int b = bh / H, h = bh % H;
  const int Cc = H * HD;
  const int64_t ld = 3 * (int64_t)Cc;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const rsrc_t r = make_rsrc(base, (int64_t)Tn * ld * 2);
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), g = lane >> 5, c32 = lane & 31;
  const int q0 = qb * 256;
  DqState S;
  const int qt[2] = {w, 7 - w};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    S.qlo[i] = q0 + qt[i] * 32;
    S.q[i] = S.qlo[i] + c32;
    const bool ok = S.q[i] < Tn;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      S.qf[i][kk] = ok ? *reinterpret_cast<const uint4*>(base + (int64_t)S.q[i] * ld + h * HD + kk * 16 + g * 8)
                       : make_uint4(0, 0, 0, 0);
      S.dof[i][kk] =
          ok ? *reinterpret_cast<const uint4*>(dO + (int64_t)(b * Tn + S.q[i]) * Cc + h * HD + kk * 16 + g * 8)
             : make_uint4(0, 0, 0, 0);
    }
    S.lq[i] = ok ? lse2[(int64_t)bh * Tn + S.q[i]] : 0.f;
    S.dd[i] = ok ? Dv[(int64_t)bh * Tn + S.q[i]] : 0.f;
    zero16(S.dq[i][0]);
    zero16(S.dq[i][1]);
  }
  BlockLoad lk, lv;
  lk.init(ld, Cc + h * HD, w, lane);
  lv.init(ld, 2 * Cc + h * HD, w, lane);
  const uint32_t blk_bytes = (uint32_t)(64 * ld * 2);
  const int nkb = (min(Tn, q0 + 256) + 63) / 64;
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nkb) {
      lk.issue(r, smem + s * 2 * TILE, (uint32_t)s * blk_bytes, w);
      lv.issue(r, smem + s * 2 * TILE + TILE, (uint32_t)s * blk_bytes, w);
    }
  // key blocks before the query block's first row need no mask (see dkdv_item)
  int sc = 0, kb = 0;
  for (; kb < min(nkb, q0 / 64); ++kb) {
    const int sw = sc == 0 ? ST - 1 : sc - 1;
    dq_block<false>(smem + sc * 2 * TILE, smem + sw * 2 * TILE, kb, nkb, r, lk, lv, blk_bytes, S, w, lane);
    sc = sc + 1 == ST ? 0 : sc + 1;
  }
  for (; kb < nkb; ++kb) {
    const int sw = sc == 0 ? ST - 1 : sc - 1;
    dq_block<true>(smem + sc * 2 * TILE, smem + sw * 2 * TILE, kb, nkb, r, lk, lv, blk_bytes, S, w, lane);
    sc = sc + 1 == ST ? 0 : sc + 1;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (S.q[i] >= Tn) continue;
    bf16* qrow = dqkv + (int64_t)(b * Tn + S.q[i]) * ld + h * HD;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        store4(qrow + dt * 32 + r4 * 8 + g * 4,
               make_float4(S.dq[i][dt][4 * r4] * 0.125f, S.dq[i][dt][4 * r4 + 1] * 0.125f,
                           S.dq[i][dt][4 * r4 + 2] * 0.125f, S.dq[i][dt][4 * r4 + 3] * 0.125f));
  }
}

// The dK/dV and dQ work of one backward in one launch: class c of the grid
// (blockIdx.x / BH) is a dK/dV key block or a dQ query block, the classes in
// decreasing order of work, (batch, head) varying fastest within a class.
constexpr int MAX_CLASSES = 256;
struct BwdOrder {
  unsigned short cls[MAX_CLASSES];  // bit 15: dQ query block, else dK/dV key block; low bits: block index
};

__global__ __launch_bounds__(256, 2) void bwd_kernel(const bf16* __restrict__ qkv, const bf16* __restrict__ dO,
                                                     const float* __restrict__ lse2, const float* __restrict__ Dv,
                                                     bf16* __restrict__ dqkv, int Tn, int H, int BH, BwdOrder ord) {
  __shared__ __attribute__((aligned(16))) char smem[ST * KV_STAGE > ST * 2 * TILE ? ST * KV_STAGE : ST * 2 * TILE];
  const int c = (int)blockIdx.x / BH, bh = (int)blockIdx.x % BH;
  const int e = ord.cls[c];
  if (e & 0x8000) dq_item(smem, e & 0x7fff, bh, qkv, dO, lse2, Dv, dqkv, Tn, H);
  else dkdv_item(smem, e, bh, qkv, dO, lse2, Dv, dqkv, Tn, H);
}

}  // namespace fa

hipError_t attn_fwd_bf16_d64(const void* qkv, void* o, float* lse, int B, int Tn, int H, hipStream_t s) {
  // buffer offsets are 32-bit: one sequence of qkv must stay under 4 GB
  if ((int64_t)Tn * 3 * H * fa::HD * 2 >= (1ll << 32)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fa::fwd_kernel, dim3((Tn + 255) / 256 * B * H), dim3(256), 0, s, (const bf16*)qkv, (bf16*)o,
                     lse, Tn, H);
  return hipGetLastError();
}

hipError_t attn_bwd_bf16_d64(const void* qkv, const void* dO, const float* lse, const float* Dv, void* dqkv, int B,
                             int Tn, int H, hipStream_t s) {
  if ((int64_t)Tn * 3 * H * fa::HD * 2 >= (1ll << 32)) return hipErrorInvalidValue;
  // classes and their work in streamed blocks: a dK/dV key block (128 keys) streams
  // the 64-query blocks from its diagonal on (32 MFMAs per wave each); a dQ query
  // block (256 queries) streams the 64-key blocks up to its end (48 per wave each)
  const int nkv = (Tn + 127) / 128, nq64 = (Tn + 63) / 64, nqd = (Tn + 255) / 256;
  if (nkv + nqd > fa::MAX_CLASSES) return hipErrorInvalidValue;
  int cost[fa::MAX_CLASSES];
  fa::BwdOrder ord;
  int n = 0;
  for (int kb = 0; kb < nkv; ++kb) { ord.cls[n] = (unsigned short)kb; cost[n++] = 2 * (nq64 - 2 * kb); }
  for (int qb = 0; qb < nqd; ++qb) {
    ord.cls[n] = (unsigned short)(0x8000 | qb);
    cost[n++] = 3 * ((std::min(Tn, qb * 256 + 256) + 63) / 64);
  }
  for (int i = 1; i < n; ++i)  // insertion sort, decreasing work (stable)
    for (int j = i; j > 0 && cost[j] > cost[j - 1]; --j) {
      std::swap(cost[j], cost[j - 1]);
      std::swap(ord.cls[j], ord.cls[j - 1]);
    }
  hipLaunchKernelGGL(fa::bwd_kernel, dim3(n * B * H), dim3(256), 0, s, (const bf16*)qkv, (const bf16*)dO, lse, Dv,
                     (bf16*)dqkv, Tn, H, B * H, ord);
  return hipGetLastError();
}

}  // namespace gk
