// Host-side launchers of the gfx950 kernels (internal to libgpt.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gk {

enum Dtype { F32 = 0, BF16 = 1 };

// ---- GEMM: C[m][n] = sum_k A(m,k) B(n,k) ----
// a_trans == 0: A stored [M][lda] (k contiguous); 1: A stored [K][lda] (m contiguous).
// b_trans == 0: B stored [N][ldb] (k contiguous); 1: B stored [K][ldb] (n contiguous).
enum Epi {
  EPI_STORE = 0,     // C(T) = acc + bias
  EPI_RESID = 1,     // C(f32) = R(f32) + acc + bias
  EPI_GELU = 2,      // u = acc + bias: C(T) = gelu'(u) (kept for the backward), C2(T) = gelu(u)
  EPI_GELU_BWD = 3,  // C(T) = acc * aux(T) (aux = gelu'(u) from the forward)
  EPI_F32 = 4,       // C(f32) = (accumulate ? C : 0) + acc
  // C(T) = acc (no bias), and dv[b][h][t] = sum over head h's 64 columns of row
  // m = b * tn + t of C(T) * aux(T): attention's D = rowsum(dO * O) computed
  // where dO is produced (bf16, N a multiple of 64, 256- or 128-column tiles)
  EPI_STORE_ODOT = 5,
  // C(T) = scale (exp(acc - lse[m]) - [col0 + n == rowi[m]]): the softmax
  // cross-entropy gradient of a block of logit columns col0 .. col0 + N - 1
  EPI_CE_GRAD = 6,
};

struct Gemm {
  int dtype;  // element type of A, B, and of T-typed outputs
  int a_trans, b_trans, epi;
  const void* A;
  const void* B;
  int64_t lda, ldb;
  int M, N, K;
  void* C;
  int64_t ldc;
  const float* bias = nullptr;
  const float* R = nullptr;
  void* C2 = nullptr;
  const void* aux = nullptr;
  int accumulate = 0;
  float* dv = nullptr;  // EPI_STORE_ODOT: [rows / tn][heads][tn] row sums
  int tn = 0, heads = 0;
  const float* lse = nullptr;     // EPI_CE_GRAD: [M] per-row log-sum-exp
  const int32_t* rowi = nullptr;  // EPI_CE_GRAD: [M] per-row target class
  int col0 = 0;                   // EPI_CE_GRAD
  float scale = 1.f;              // EPI_CE_GRAD
  // split-K (EPI_F32 only): when > 1, partial sums go to ws [splits][M][N] and are reduced in order;
  // ws holds ws_floats floats and the split count is lowered until splits * M * N fits
  int splits = 1;
  float* ws = nullptr;
  int64_t ws_floats = 0;
};
// after_main (nullable) is recorded right after the main kernel, before any split-K reduction;
// with before_main too, both are attached to the main kernel's dispatch (its start and end)
hipError_t gemm(const Gemm& g, hipStream_t s, hipEvent_t after_main = nullptr, hipEvent_t before_main = nullptr);
// split count a GEMM of this shape with an fp32 output would use (its split-K
// workspace is gemm_pick_splits(...) * M * N floats when that is > 1)
int gemm_pick_splits(int M, int N, int K, int a_trans, int b_trans);
// out[m][n] (+)= sum over z < splits of ws[z][m][n] (fixed order); ws [splits][M][N], out row stride ldc
hipError_t splits_reduce(const float* ws, int splits, int M, int N, float* out, int64_t ldc, int accumulate,
                         hipStream_t s);

// ---- LayerNorm (rms = 1: RMSNorm, mu = 0 and no shift; b may be null) ----
// y = (x - mu) * rstd * g + b per row of C; x fp32 [rows][C]; y T; mu, rstd fp32 [rows]
hipError_t layernorm_fwd(int dtype, const float* x, const float* g, const float* b, void* y,
                         float* mu, float* rstd, int rows, int C, hipStream_t s, int rms = 0);
// embedding (wte[tok] + wpe[t], wpe nullable) -> res0 (f32), fused with the first LayerNorm
hipError_t embed_ln_fwd(int dtype, const int32_t* tok, const float* wte, const float* wpe, int T,
                        float* res0, const float* g, const float* b, void* y, float* mu,
                        float* rstd, int rows, int C, hipStream_t s, int rms = 0);
// LayerNorm backward: dres_out = dres_in + dx (f32, may alias dres_in), dres_T = T(dres_out);
// part [nblk][3C]: per-block column sums of dy*xhat, dy and dres_out
// dy is T when dy_is_t (bf16 or fp32 as dtype), else fp32
hipError_t layernorm_bwd(int dtype, const void* dy, int dy_is_t, const float* x, const float* mu,
                         const float* rstd, const float* g, const float* dres_in, float* dres_out, void* dres_T,
                         float* part, int rows, int C, int* nblk_out, hipStream_t s, int rms = 0);
int layernorm_bwd_blocks(int rows);

// ---- the second block variant's elementwise steps ----
// RoPE on the q and k thirds of qkv [rows][3C] (T, in place), head size D,
// position t = row % Tn; tab [Tmax][D/2] holds (cos, sin) of the pair angles;
// inverse rotates by minus the angles (the backward, on dqkv)
hipError_t rope_qk(int dtype, void* qkv, int rows, int C, int Tn, int D, const float2* tab, int inverse, hipStream_t s);
// SwiGLU: u [rows][2F] = [gate | up] (T) -> h [rows][F] = silu(gate) * up (T)
hipError_t swiglu_fwd(int dtype, const void* u, void* h, int rows, int F, hipStream_t s);
// backward: dh [rows][F] (T) -> du [rows][2F] = [dh up silu'(gate) | dh silu(gate)] (T)
hipError_t swiglu_bwd(int dtype, const void* u, const void* dh, void* du, int rows, int F, hipStream_t s);
// One column reduction of a batch: out[c] (+)= sum_r part[r * ld + c], c < cols;
// blocks [first_block, first_block + cdiv(cols, 16)) of the batch launch serve it.
struct RedJob {
  const float* part;
  float* out;
  int nrows, cols, ld, first_block;
};
// all jobs (device array, first_block increasing) in one launch of nblocks blocks
hipError_t reduce_jobs(const RedJob* jobs, int njobs, int nblocks, int accumulate, hipStream_t s);
// out[c] = (acc ? out[c] : 0) + sum_r part[r][c] for c < cols (fixed order)
hipError_t reduce_rows_f32(const float* part, int nrows, int cols, int64_t ld, float* out,
                           int accumulate, hipStream_t s);
// column sums of a T matrix [rows][cols] -> part [cdiv(rows,256)][cols] (f32)
hipError_t colsum_partial(int dtype, const void* x, int rows, int cols, float* part,
                          hipStream_t s);

// ---- attention (causal, flash) ----
// qkv T [B*T][3C] (q | k | v, head h at channels h*D..), o T [B*T][C], lse f32 [B][H][T]
hipError_t attn_fwd(int dtype, const void* qkv, void* o, float* lse, int B, int T, int H, int D,
                    hipStream_t s);
// bf16, head size 64 kernels on 32x32x16 MFMAs (attention_bf16.hip); Dv precomputed
hipError_t attn_fwd_bf16_d64(const void* qkv, void* o, float* lse, int B, int T, int H, hipStream_t s);
hipError_t attn_bwd_bf16_d64(const void* qkv, const void* dO, const float* lse, const float* Dv,
                             void* dqkv, int B, int T, int H, hipStream_t s);
// dO T [B*T][C] -> dqkv T [B*T][3C]; Dv f32 [B][H][T] workspace
hipError_t attn_bwd(int dtype, const void* qkv, const void* o, const void* dO, const float* lse,
                    float* Dv, void* dqkv, int B, int T, int H, int D, hipStream_t s);

// ---- LM head fused with cross-entropy (head.hip) ----
// F T [N][C] rows, W T [V][C], y int32 [N]; nothing of size [N][V] is stored.
// Pass 1: loss[n] = lse_n - z_n,y_n, lse[n] (natural log), and, when dF != null,
// dF [N][C] (f32) = scale (softmax(z_n) W - W_y).  A target outside [0, V) is
// clamped into the row (never read out of it) and, when bad != null, sets
// *bad = 1 (the caller clears it first).
// Pass 2 (needs pass 1's lse): dW [V][C] (f32) (+)= scale (softmax(z) - onehot(y))^T F.
// C a multiple of 64, at most lmhead_max_embd(dtype); bf16 needs V*C*2 and
// N*C*2 below 4 GB (32-bit buffer offsets).
int lmhead_max_embd(int dtype);
// seg_ws (bf16, nullable): at least lmhead_fwd_seg_floats(...) floats; with it a pass whose
// blocks of rows would leave CUs idle runs over vocabulary segments, combined per row after
hipError_t lmhead_fwd(int dtype, const void* F, const void* W, int N, int V, int C, const int32_t* y, float scale,
                      float* loss, float* lse, float* dF, int* bad, hipStream_t s, float* seg_ws = nullptr,
                      int64_t seg_floats = 0);
int64_t lmhead_fwd_seg_floats(int dtype, int N, int V, int C);
// Pass 1 a block of vocabulary columns at a time (fp32 GEMM form): given the
// block's logits z [N][ldz] (columns v0 .. v0 + n - 1, ldz a multiple of 4, z
// 16-byte aligned), merge each row's maximum and sum of exp into ml [N][2]
// (first: start them), record the target's logit in zy [N] from the block
// holding it, and on the last block write lse [N] (natural log) and
// loss [N] = lse - z_y.  Targets outside [0, V) are clamped and set *bad.
hipError_t lmhead_block_stats(const float* z, int ldz, int N, int n, int v0, int V, const int32_t* y, float* ml,
                              float* zy, float* loss, float* lse, int first, int last, int* bad, hipStream_t s);
// max_wgs > 0 (bf16): launches of at most that many workgroups.  tail_ws (bf16, nullable): at
// least lmhead_dw_tail_floats(...) floats; with it the last partial round of W-row blocks is
// split over the rows of F (partial sums there, then added in order)
hipError_t lmhead_dw(int dtype, const void* F, const void* W, int N, int V, int C, const int32_t* y, const float* lse,
                     float scale, float* dW, int accumulate, hipStream_t s, int max_wgs = 0,
                     float* tail_ws = nullptr, int64_t tail_floats = 0);
int64_t lmhead_dw_tail_floats(int dtype, int N, int V, int C);
// mean of n floats in fixed order -> out[0] (and ring[slot] if ring != null)
hipError_t mean_f32(const float* x, int n, float* out, float* ring, int slot, hipStream_t s);

// ---- embedding backward ----
// sort the (tok[i], i) keys, u32 [n]: one workgroup up to 16384 keys; above that
// 16384-key chunks side by side in tmp (u32 [n]), merged by rank into keys
constexpr int SORT_MAX_TOKENS = 262144;
hipError_t sort_tokens(const int32_t* tok, int n, uint32_t* keys, uint32_t* tmp, hipStream_t s);
// dwte[tok] += sum of dres rows with that token, in sorted order (deterministic);
// part: workspace f32 [n][C]
hipError_t embed_bwd_ws(const uint32_t* keys, int n, const float* dres, int C, float* part,
                        float* dwte, hipStream_t s);
// dwpe[t] (+)= sum_b dres[b][t]
hipError_t wpe_bwd(const float* dres, int B, int T, int C, float* dwpe, int accumulate,
                   hipStream_t s);

// ---- optimiser ----
// partial sums of squares of g [n] -> part[nblk]; then norm (and clip scale) into scal
hipError_t sumsq_partial(const float* g, int64_t n, float* part, int* nblk, hipStream_t s);
int sumsq_blocks(int64_t n);
// scal[0] = norm, scal[1] = clip scale (1 if clip <= 0), scal[2] = finite flag,
// scal[3] = AdamW step size, scal[4] = sticky non-finite flag
hipError_t norm_finish(const float* part, int nblk, float clip, float* scal, hipStream_t s);
// AdamW over [0, n) (n % 4 == 0); decay applies to [0, n_decay); shadow (bf16) may be null;
// step_dev: device int update counter, advanced only when the norm is finite
hipError_t adamw(float* p, const float* g, float* m, float* v, void* shadow, int64_t n,
                 int64_t n_decay, float* scal, float lr, float b1, float b2, float eps, float wd,
                 int* step_dev, hipStream_t s);
// the same in pieces: adamw_prep once (advances step_dev, sets scal[3]), then
// adamw_range over [lo, hi) (multiples of 4; decay below n_decay) in any order
hipError_t adamw_prep(float* scal, float lr, float b1, float b2, int* step_dev, hipStream_t s);
hipError_t adamw_range(float* p, const float* g, float* m, float* v, void* shadow, int64_t lo, int64_t hi,
                       int64_t n_decay, const float* scal, float lr, float b1, float b2, float eps, float wd,
                       hipStream_t s);
// fp32 -> bf16 copy
hipError_t to_bf16(const float* x, void* y, int64_t n, hipStream_t s);
// x[i] = value
hipError_t fill_f32(float* x, int64_t n, float value, hipStream_t s);
// Philox4x32-10 + Box-Muller normals: x[i] = std * N(0,1) with counter (offset + i), key seed
hipError_t init_normal(float* x, int64_t n, float std, uint64_t seed, uint64_t offset,
                       hipStream_t s);

}  // namespace gk
