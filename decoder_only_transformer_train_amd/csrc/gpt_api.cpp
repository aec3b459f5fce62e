// Host side of libgpt.so: configuration, arena layout, launch sequences of
// the training step, tensor access and kernel timing.  See include/gpt.h.
#include "gpt.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

namespace {

thread_local std::string g_err = "no error";

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIPCHK(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(GPT_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_));        \
  } while (0)

constexpr int RING = 4096;
constexpr int64_t ALIGN = 256;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct TensorDesc {
  std::string name;
  int64_t rows, cols;  // cols == 0: vector of `rows`
  int decays;
  int kind;            // 0: N(0,0.02), 1: N(0,0.02/sqrt(2L)), 2: zero, 3: one
  int64_t off;         // element offset in the flat parameter buffer
  int64_t numel() const { return cols ? rows * cols : rows; }
};

// Bump allocator over the arena; with base == nullptr it only measures.
struct Carver {
  char* base;
  int64_t used = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename P> P* take(int64_t bytes) {
    used = align_up(used, ALIGN);
    P* p = base ? reinterpret_cast<P*>(base + used) : nullptr;
    used += bytes;
    return p;
  }
};

struct Layer {
  void* ln1;  // T [N][C]
  float *mu1, *rs1;
  void* qkv;  // T [N][3C]
  void* att;  // T [N][C]
  float* lse; // [B][H][T] (log2 domain)
  float* res_mid;  // f32 [N][C]
  void* ln2;
  float *mu2, *rs2;
  void* fcdg;   // T [N][4C]: GELU'(FC pre-activation), kept for the backward
  void* fcact;  // T [N][4C]
  // backward column-sum partials, reduced in one batch at the end of backward
  float *ln1_part, *ln2_part;   // [N / 32][3C]: ln gain, ln shift, residual-gradient column sums
  float *fcb_part, *attb_part;  // [N / 256][4C], [N / 256][3C]: fc and qkv bias gradients
};

struct Prof {
  std::string cls;
  std::vector<hipEvent_t> ev;  // start/stop pairs
  size_t used = 0;
  double flops = 0, bytes = 0;
  int64_t launches = 0;
};

}  // namespace

struct gpt_ctx {
  gpt_config cfg;
  hipStream_t stream;
  int dt, es;  // dtype, element size of T
  int64_t N, C, L, H, D, V, Vp, T, B;
  int blk = GPT_BLOCK_GPT2;  // block type
  int64_t F = 0;             // SwiGLU width (GPT_BLOCK_RMS_ROPE_SWIGLU)
  float2* rope_tab = nullptr;  // [max_seq][D/2] (cos, sin) of the RoPE angles
  void* dh = nullptr;          // T [N][F]: gradient at the SwiGLU output
  std::vector<TensorDesc> tensors;  // logical (ABI) order
  int64_t P, P_decay;               // flat parameter floats
  float *params, *grads, *m, *v;
  void* shadow;  // bf16 copy of params (bf16 mode) or null
  int32_t* win;  // [N + 1] tokens
  // two pinned host buffers the batch windows are copied through, so that the
  // host-to-device copy is asynchronous; stage_ev[k]: the last copy out of buffer k
  int32_t* stage_host[2] = {nullptr, nullptr};
  hipEvent_t stage_ev[2] = {nullptr, nullptr};
  int stage_i = 0;
  std::vector<float*> res;  // L + 1 residual streams
  std::vector<Layer> layers;
  void* lnf;
  float *muf, *rsf;
  // head: per-row losses and log-sum-exps, the gradient at the final LayerNorm output
  float *tok_loss, *tok_lse, *dF, *loss;
  void* gchunk = nullptr;  // GEMM form of the head dW: T [N][head_cols], one column block's logit gradient
  int64_t head_cols = 0;
  float* head_skws = nullptr;  // split-K workspace of the head's dW blocks (head_skn floats)
  // GEMM form of pass 1 (fp32): running row maximum and sum of exp [N][2], target logits [N]
  float* head_ml = nullptr;
  float* head_zy = nullptr;
  int64_t head_skn = 0;
  float* head_tail = nullptr;  // partial sums of the head dW pass's split last round (head_tail_n floats)
  int64_t head_tail_n = 0;
  float* head_seg = nullptr;  // the head pass 1's vocabulary-segment results (head_seg_n floats; in-model only)
  int64_t head_seg_n = 0;
  float* ring;
  int ring_wr = 0, ring_rd = 0;
  // backward
  float *dres, *dln;
  void* dlnT;  // T [N][C]: gradient at a LayerNorm output
  void *dresT2[2], *dfc, *datt, *dqkv;  // dresT2: two T copies of the residual gradient (see gpt_backward)
  // weight-gradient products run on a second stream, ordered by events
  hipStream_t side = nullptr;
  std::vector<hipEvent_t> sev;
  hipEvent_t head_fork = nullptr, side_tail = nullptr;  // head_fork: pass 1 done, the tied dW may start
  // the head's tied-weight gradient blocks run on a stream of their own, so
  // they never queue in front of the layers' weight gradients on `side`
  // (whose completion the data-gradient chain waits for)
  hipStream_t hside = nullptr;
  hipEvent_t hside_tail = nullptr;
  hipEvent_t fwd_start = nullptr;  // the forward's start, for side-stream work that needs only the batch
  // AdamW runs on the side stream in pieces (all vectors, wte + wpe, then each
  // layer's matrices); the next forward waits for each piece where it first
  // reads it.  adam_ev[k] marks piece k done; adam_pending: pieces queued
  // since the last forward (the side stream holds nothing else then)
  std::vector<hipEvent_t> adam_ev;
  hipEvent_t norm_done = nullptr;
  bool adam_pending = false;
  float *Dv, *lnf_part, *splitk_ws = nullptr;
  int64_t splitk_n = 0;  // floats in splitk_ws
  gk::RedJob* jobs_dev;
  std::vector<gk::RedJob> jobs;
  int nred_blocks = 0;
  uint32_t* keys;
  uint32_t* keys_tmp = nullptr;
  float *norm_part, *scal;
  int* step_dev;
  bool wte_fresh = true, others_fresh = true, have_fwd = false, fwd_grad = false;
  float last_scale = 0.f;
  Prof prof;
  // parameter pointers by logical id
  float* P_(int id) { return params + tensors[id].off; }
  float* G_(int id) { return grads + tensors[id].off; }
  const void* W_(int id) {  // GEMM operand view of a parameter
    return shadow ? (const void*)((uint16_t*)shadow + tensors[id].off) : (const void*)(params + tensors[id].off);
  }
};

namespace {

enum { T_WTE = 0, T_WPE = 1 };
inline int tid(int l, int k) { return 2 + 12 * l + k; }  // k: 0 ln1.g .. 11 mlp_proj.b
enum { K_LN1G, K_LN1B, K_ATTW, K_ATTB, K_PROJW, K_PROJB, K_LN2G, K_LN2B, K_FCW, K_FCB, K_MPW, K_MPB };
inline int tid_lnf(int L, int k) { return 2 + 12 * L + k; }
// GPT_BLOCK_RMS_ROPE_SWIGLU: wte, 7 tensors per block, rmsf.g, lm_head
enum { VK_RMS1, VK_ATTW, VK_PROJW, VK_RMS2, VK_W1, VK_W3, VK_W2 };
inline int vt(int l, int k) { return 1 + 7 * l + k; }
inline int vt_rmsf(int L) { return 1 + 7 * L; }
inline int vt_head(int L) { return 2 + 7 * L; }

int check_cfg(const gpt_config* c) {
  if (!c) return fail(GPT_EINVAL, "null config");
  if (c->dtype != GPT_F32 && c->dtype != GPT_BF16) return fail(GPT_EINVAL, "dtype must be GPT_F32 or GPT_BF16");
  if (c->n_layer < 1 || c->n_embd < 64 || c->n_head < 1 || c->vocab < 1 || c->batch < 1 || c->seq < 1)
    return fail(GPT_EINVAL, "sizes must be positive (n_embd >= 64)");
  if (c->n_embd % 64 != 0 || c->n_embd > gk::lmhead_max_embd(c->dtype))
    return fail(GPT_EINVAL, "n_embd must be a multiple of 64, <= 1792 (bf16) or 1024 (fp32)");
  if (c->n_embd % c->n_head != 0) return fail(GPT_EINVAL, "n_embd % n_head != 0");
  const int D = c->n_embd / c->n_head;
  if (c->dtype == GPT_BF16 && D != 64) return fail(GPT_EINVAL, "bf16 head size must be 64");
  if (c->dtype == GPT_F32 && D != 16 && D != 32 && D != 64) return fail(GPT_EINVAL, "fp32 head size must be 16, 32 or 64");
  if (c->padded_vocab < c->vocab) return fail(GPT_EINVAL, "padded_vocab < vocab");
  if (c->block != GPT_BLOCK_GPT2 && c->block != GPT_BLOCK_RMS_ROPE_SWIGLU) return fail(GPT_EINVAL, "unknown block type");
  if (c->block == GPT_BLOCK_RMS_ROPE_SWIGLU) {
    if (c->d_ff < 64 || c->d_ff % 64) return fail(GPT_EINVAL, "d_ff must be a positive multiple of 64");
    if (!(c->rope_theta > 0.f) || !std::isfinite(c->rope_theta)) return fail(GPT_EINVAL, "rope_theta must be > 0");
  }
  if (c->seq > c->max_seq) return fail(GPT_EINVAL, "seq > max_seq");
  const int64_t N = (int64_t)c->batch * c->seq;
  if (N > gk::SORT_MAX_TOKENS) return fail(GPT_EINVAL, "batch * seq must be <= 262144");
  int shift = 0;
  while ((1 << shift) < N) ++shift;
  if (((uint64_t)c->padded_vocab << shift) > 0xFFFFFFFFull) return fail(GPT_EINVAL, "padded_vocab too large for this batch");
  // GEMM operands are read through buffer descriptors with 32-bit byte
  // offsets: the widest activation ([N, 4C], or [N, 2 d_ff] for the gate and
  // up projections of the variant block) and the embedding must stay below 4 GiB
  const int64_t es = c->dtype == GPT_BF16 ? 2 : 4, C = c->n_embd;
  const int64_t wide = c->block == GPT_BLOCK_RMS_ROPE_SWIGLU ? std::max<int64_t>(3 * C, 2 * (int64_t)c->d_ff) : 4 * C;
  if (N * wide * es >= (1ll << 32) || (int64_t)c->padded_vocab * C * es >= (1ll << 32))
    return fail(GPT_EINVAL, "an activation or the embedding reaches 4 GiB (32-bit buffer offsets)");
  return 0;
}

std::vector<TensorDesc> make_tensors(const gpt_config* c, int64_t* P, int64_t* P_decay) {
  const int64_t C = c->n_embd, L = c->n_layer;
  std::vector<TensorDesc> t;
  auto add = [&](const std::string& n, int64_t r, int64_t cc, int dec, int kind) {
    t.push_back(TensorDesc{n, r, cc, dec, kind, 0});
  };
  add("wte", c->padded_vocab, C, 1, 0);
  if (c->block == GPT_BLOCK_RMS_ROPE_SWIGLU) {
    const int64_t F = c->d_ff;
    for (int64_t l = 0; l < L; ++l) {  // w1 and w3 adjacent: one [2F, C] operand
      const std::string p = "h" + std::to_string(l) + ".";
      add(p + "rms1.g", C, 0, 0, 3);
      add(p + "attn.w", 3 * C, C, 1, 0);
      add(p + "proj.w", C, C, 1, 1);
      add(p + "rms2.g", C, 0, 0, 3);
      add(p + "w1", F, C, 1, 0);
      add(p + "w3", F, C, 1, 0);
      add(p + "w2", C, F, 1, 1);
    }
    add("rmsf.g", C, 0, 0, 3);
    add("lm_head", c->padded_vocab, C, 1, 0);
  } else {
  add("wpe", c->max_seq, C, 1, 0);
  for (int64_t l = 0; l < L; ++l) {
    const std::string p = "h" + std::to_string(l) + ".";
    add(p + "ln1.g", C, 0, 0, 3);
    add(p + "ln1.b", C, 0, 0, 2);
    add(p + "attn.w", 3 * C, C, 1, 0);
    add(p + "attn.b", 3 * C, 0, 0, 2);
    add(p + "proj.w", C, C, 1, 1);
    add(p + "proj.b", C, 0, 0, 2);
    add(p + "ln2.g", C, 0, 0, 3);
    add(p + "ln2.b", C, 0, 0, 2);
    add(p + "fc.w", 4 * C, C, 1, 0);
    add(p + "fc.b", 4 * C, 0, 0, 2);
    add(p + "mlp_proj.w", C, 4 * C, 1, 1);
    add(p + "mlp_proj.b", C, 0, 0, 2);
  }
  add("lnf.g", C, 0, 0, 3);
  add("lnf.b", C, 0, 0, 2);
  }
  // memory order: every decayed (2-D) tensor first, then the vectors
  int64_t off = 0;
  for (auto& d : t)
    if (d.decays) { d.off = off; off += align_up(d.numel(), 64); }
  *P_decay = off;
  for (auto& d : t)
    if (!d.decays) { d.off = off; off += align_up(d.numel(), 64); }
  *P = off;
  return t;
}

int64_t splitk_floats(int64_t N, int64_t C, int64_t F) {
  int64_t best = 0;
  // weight-gradient shapes: qkv, projection, MLP in and out ([2F, C] and [C, F] for SwiGLU)
  const int64_t shapes[6][2] = {{3 * C, C}, {C, C}, {4 * C, C}, {C, 4 * C}, {2 * F, C}, {C, F}};
  for (auto& s : shapes) {
    const int sp = gk::gemm_pick_splits((int)s[0], (int)s[1], (int)N, 1, 1);
    if (sp > 1) best = std::max(best, (int64_t)sp * s[0] * s[1]);
  }
  return best;
}

// The head's weight gradient by column-block GEMMs instead of the single
// recompute kernel: GPT_HEAD_DW=gemm, read at every use (contexts and
// workspaces sized under one setting keep working under the other: without a
// block buffer the single kernel runs).
bool head_gemm_mode() {
  const char* e = getenv("GPT_HEAD_DW");
  return e && std::string(e) == "gemm";
}
// A model context's choice: fp32 contexts take the GEMM form of both passes
// unless GPT_HEAD_DW=kernel (their products run on the fp32 MFMAs, the fused
// kernels' fp32 variant on plain FMAs: the CS336 TinyStories step in fp32,
// 23.7 ms with the fused kernels, 18.8 ms with the GEMM-form dW, 11.1 ms with
// both passes, same box).  bf16 contexts take the GEMM form of dW from
// C = 1024 up (same box each: GPT-2 350M, C = 1024, 28.28-28.31 -> 27.87-27.94
// ms per step; GPT-2 1.5B, C = 1600, where the fused dW kernel has no
// software-pipelined sweep, 244.8-245.0 -> 241.2-241.5 ms) and keep the fused
// kernels at C = 768 (GPT-2 124M: 18.43-18.50 ms against 19.19-19.22 ms with
// the GEMM form); GPT_HEAD_DW=gemm or =kernel forces either.  The public head entry points size their workspace by
// head_gemm_mode() alone, so their default stays the kernel.
bool head_gemm_ctx(int dtype, int64_t C) {
  const char* e = getenv("GPT_HEAD_DW");
  if (e && std::string(e) == "kernel") return false;
  if (e && std::string(e) == "gemm") return true;
  return dtype == GPT_F32 || C >= 1024;
}

// Vocabulary columns per block of the GEMM form of the head's weight gradient:
// the block's logit gradient [N][cols] (T) is about 128 MB, a multiple of 256
// columns (the GEMM tile) between 256 and V rounded up (4096 columns at N =
// 16384 in bf16: 19.9 ms per 124M step against 20.7 ms with 2048, same box).
// GPT_HEAD_COLS overrides it for tuning runs.
int64_t head_block_cols(int64_t N, int64_t V, int64_t es) {
  static const int64_t forced = [] {
    const char* e = getenv("GPT_HEAD_COLS");
    return e ? std::max<int64_t>(0, atoll(e)) : 0;
  }();
  const int64_t vmax = (V + 255) / 256 * 256;
  int64_t c = forced ? forced : (128ll << 20) / (N * es) / 256 * 256;
  return std::min(vmax, std::max<int64_t>(256, c / 256 * 256));
}

// Lays out (base == nullptr: measures) everything the context needs.
int64_t carve(gpt_ctx* x, void* base) {
  Carver cv(base);
  const int64_t N = x->N, C = x->C, es = x->es;
  x->params = cv.take<float>(x->P * 4);
  x->grads = cv.take<float>(x->P * 4);
  x->m = cv.take<float>(x->P * 4);
  x->v = cv.take<float>(x->P * 4);
  x->shadow = (x->dt == GPT_BF16) ? cv.take<void>(x->P * 2) : nullptr;
  x->win = cv.take<int32_t>((N + 1) * 4);
  x->res.assign(x->L + 1, nullptr);
  for (auto& r : x->res) r = cv.take<float>(N * C * 4);
  x->layers.assign(x->L, Layer{});
  const int64_t nh = x->B * x->H * x->T;
  const int64_t nlnb = gk::layernorm_bwd_blocks((int)N), ncs = (N + 255) / 256;
  for (auto& l : x->layers) {
    l.ln1_part = cv.take<float>(nlnb * 3 * C * 4);
    l.ln2_part = cv.take<float>(nlnb * 3 * C * 4);
    const bool gpt2 = x->blk == GPT_BLOCK_GPT2;
    l.fcb_part = cv.take<float>(gpt2 ? ncs * 4 * C * 4 : 0);
    l.attb_part = cv.take<float>(gpt2 ? ncs * 3 * C * 4 : 0);
    l.ln1 = cv.take<void>(N * C * es);
    l.mu1 = cv.take<float>(N * 4);
    l.rs1 = cv.take<float>(N * 4);
    l.qkv = cv.take<void>(N * 3 * C * es);
    l.att = cv.take<void>(N * C * es);
    l.lse = cv.take<float>(nh * 4);
    l.res_mid = cv.take<float>(N * C * 4);
    l.ln2 = cv.take<void>(N * C * es);
    l.mu2 = cv.take<float>(N * 4);
    l.rs2 = cv.take<float>(N * 4);
    // GPT-2: GELU' and GELU output [N][4C]; SwiGLU: [gate | up] [N][2F] and its output [N][F]
    l.fcdg = cv.take<void>(N * (gpt2 ? 4 * C : 2 * x->F) * es);
    l.fcact = cv.take<void>(N * (gpt2 ? 4 * C : x->F) * es);
  }
  x->lnf = cv.take<void>(N * C * es);
  x->muf = cv.take<float>(N * 4);
  x->rsf = cv.take<float>(N * 4);
  x->tok_loss = cv.take<float>(N * 4);
  x->tok_lse = cv.take<float>(N * 4);
  x->dF = cv.take<float>(N * C * 4);
  x->head_tail_n = gk::lmhead_dw_tail_floats(x->dt, (int)N, (int)x->Vp, (int)C);
  x->head_tail = x->head_tail_n ? cv.take<float>(x->head_tail_n * 4) : nullptr;
  x->head_seg_n = gk::lmhead_fwd_seg_floats(x->dt, (int)N, (int)x->Vp, (int)C);
  x->head_seg = x->head_seg_n ? cv.take<float>(x->head_seg_n * 4) : nullptr;
  if (head_gemm_ctx(x->dt, C)) {
    x->head_cols = head_block_cols(N, x->Vp, es);
    x->gchunk = cv.take<void>(N * x->head_cols * es);
    const int sp = gk::gemm_pick_splits((int)x->head_cols, (int)C, (int)N, 1, 1);
    x->head_skn = sp > 1 ? (int64_t)sp * x->head_cols * C : 0;
    x->head_skws = x->head_skn ? cv.take<float>(x->head_skn * 4) : nullptr;
    x->head_ml = x->dt == GPT_F32 ? cv.take<float>(N * 8) : nullptr;
    x->head_zy = x->dt == GPT_F32 ? cv.take<float>(N * 4) : nullptr;
  } else {
    x->gchunk = nullptr;
    x->head_skws = nullptr;
    x->head_ml = x->head_zy = nullptr;
    x->head_cols = x->head_skn = 0;
  }
  x->loss = cv.take<float>(64);
  x->ring = cv.take<float>(RING * 4);
  x->dres = cv.take<float>(N * C * 4);
  x->dln = cv.take<float>(N * C * 4);
  x->dlnT = cv.take<void>(N * C * es);
  x->dresT2[0] = cv.take<void>(N * C * es);
  x->dresT2[1] = cv.take<void>(N * C * es);
  x->dfc = cv.take<void>(N * std::max(4 * C, 2 * x->F) * es);
  x->dh = x->blk == GPT_BLOCK_RMS_ROPE_SWIGLU ? cv.take<void>(N * x->F * es) : nullptr;
  x->rope_tab = x->blk == GPT_BLOCK_RMS_ROPE_SWIGLU ? cv.take<float2>(x->cfg.max_seq * (x->D / 2) * 8) : nullptr;
  x->datt = cv.take<void>(N * C * es);
  x->dqkv = cv.take<void>(N * 3 * C * es);
  x->Dv = cv.take<float>(nh * 4);
  x->lnf_part = cv.take<float>(nlnb * 3 * C * 4);
  x->jobs_dev = cv.take<gk::RedJob>((8 * x->L + 3) * (int64_t)sizeof(gk::RedJob));
  x->splitk_n = std::max<int64_t>(1, splitk_floats(N, C, x->F));
  x->splitk_ws = cv.take<float>(x->splitk_n * 4);
  x->keys = cv.take<uint32_t>(N * 4);
  x->keys_tmp = N > 16384 ? cv.take<uint32_t>(N * 4) : nullptr;  // the chunked sort's sorted chunks
  x->norm_part = cv.take<float>(gk::sumsq_blocks(x->P) * 4);
  x->scal = cv.take<float>(64);
  x->step_dev = cv.take<int>(64);
  return align_up(cv.used, ALIGN);
}

// The batched end-of-backward reduction: every LayerNorm gain/shift gradient
// and every bias gradient, each the fixed-order sum of its partial rows.
void build_jobs(gpt_ctx* x) {
  const int C = (int)x->C, N = (int)x->N, L = (int)x->L;
  const int nlnb = gk::layernorm_bwd_blocks(N), ncs = (N + 255) / 256;
  x->jobs.clear();
  int blocks = 0;
  auto add = [&](const float* part, int nrows, int cols, int ld, float* out) {
    x->jobs.push_back(gk::RedJob{part, out, nrows, cols, ld, blocks});
    blocks += (cols + 15) / 16;
  };
  if (x->blk == GPT_BLOCK_RMS_ROPE_SWIGLU) {  // RMSNorm gains only (no shifts, no biases)
    add(x->lnf_part, nlnb, C, 3 * C, x->G_(vt_rmsf(L)));
    for (int l = 0; l < L; ++l) {
      add(x->layers[l].ln2_part, nlnb, C, 3 * C, x->G_(vt(l, VK_RMS2)));
      add(x->layers[l].ln1_part, nlnb, C, 3 * C, x->G_(vt(l, VK_RMS1)));
    }
    x->nred_blocks = blocks;
    return;
  }
  // final LayerNorm; its residual-gradient column sums are the last MLP output bias gradient
  add(x->lnf_part, nlnb, C, 3 * C, x->G_(tid_lnf(L, 0)));
  add(x->lnf_part + C, nlnb, C, 3 * C, x->G_(tid_lnf(L, 1)));
  add(x->lnf_part + 2 * C, nlnb, C, 3 * C, x->G_(tid(L - 1, K_MPB)));
  for (int l = 0; l < L; ++l) {
    const Layer& ly = x->layers[l];
    add(ly.ln2_part, nlnb, C, 3 * C, x->G_(tid(l, K_LN2G)));
    add(ly.ln2_part + C, nlnb, C, 3 * C, x->G_(tid(l, K_LN2B)));
    add(ly.ln2_part + 2 * C, nlnb, C, 3 * C, x->G_(tid(l, K_PROJB)));
    add(ly.ln1_part, nlnb, C, 3 * C, x->G_(tid(l, K_LN1G)));
    add(ly.ln1_part + C, nlnb, C, 3 * C, x->G_(tid(l, K_LN1B)));
    if (l > 0) add(ly.ln1_part + 2 * C, nlnb, C, 3 * C, x->G_(tid(l - 1, K_MPB)));
    add(ly.fcb_part, ncs, 4 * C, 4 * C, x->G_(tid(l, K_FCB)));
    add(ly.attb_part, ncs, 3 * C, 3 * C, x->G_(tid(l, K_ATTB)));
  }
  x->nred_blocks = blocks;
}

void setup_dims(gpt_ctx* x, const gpt_config* c) {
  x->cfg = *c;
  x->dt = c->dtype;
  x->es = (c->dtype == GPT_BF16) ? 2 : 4;
  x->L = c->n_layer;
  x->C = c->n_embd;
  x->H = c->n_head;
  x->D = x->C / x->H;
  x->V = c->vocab;
  x->Vp = c->padded_vocab;
  x->T = c->seq;
  x->B = c->batch;
  x->N = x->B * x->T;
  x->blk = c->block;
  x->F = c->block == GPT_BLOCK_RMS_ROPE_SWIGLU ? c->d_ff : 4 * c->n_embd;
  x->tensors = make_tensors(c, &x->P, &x->P_decay);
}

// ---- profiling (HIP events around launches of one kernel class) ----
struct ProfScope {
  gpt_ctx* x;
  bool on;
  hipStream_t st;
  // attach: the caller hands start_event() and stop_event() to the launch itself
  ProfScope(gpt_ctx* x_, const char* cls, double flops, double bytes, hipStream_t s_ = nullptr, bool attach = false)
      : x(x_), st(s_ ? s_ : x_->stream) {
    on = !x->prof.cls.empty() && (x->prof.cls == "any" || x->prof.cls == cls);
    if (!on) return;
    if (x->prof.used + 2 > x->prof.ev.size()) {
      for (int i = 0; i < 64; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) { on = false; return; }
        x->prof.ev.push_back(e);
      }
    }
    if (!attach) (void)hipEventRecord(x->prof.ev[x->prof.used], st);
    x->prof.flops += flops;
    x->prof.bytes += bytes;
    x->prof.launches += 1;
  }
  // the events, for a caller that records them itself (nullptr when not profiling)
  hipEvent_t start_event() { return on ? x->prof.ev[x->prof.used] : nullptr; }
  hipEvent_t stop_event() { return on ? x->prof.ev[x->prof.used + 1] : nullptr; }
  ~ProfScope() {
    if (!on) return;
    if (!stopped) (void)hipEventRecord(x->prof.ev[x->prof.used + 1], st);
    x->prof.used += 2;
  }
  bool stopped = false;
};

// GEMM classes time only the main kernel (a split-K reduction is not
// included), with the events attached to its dispatch: no marker packets
// between it and its neighbours
int run_gemm(gpt_ctx* x, const char* cls, const gk::Gemm& g, hipStream_t st = nullptr) {
  if (!st) st = x->stream;
  ProfScope ps(x, cls, 2.0 * g.M * g.N * (double)g.K, 0.0, st, true);
  hipEvent_t stop = ps.stop_event();
  HIPCHK(gk::gemm(g, st, stop, ps.start_event()));
  ps.stopped = stop != nullptr;
  return 0;
}

gk::Gemm mk(gpt_ctx* x, int at, int bt, int epi, const void* A, int64_t lda, const void* B, int64_t ldb,
            int64_t M, int64_t N, int64_t K, void* C, int64_t ldc) {
  gk::Gemm g;
  g.dtype = x->dt;
  g.a_trans = at;
  g.b_trans = bt;
  g.epi = epi;
  g.A = A;
  g.B = B;
  g.lda = lda;
  g.ldb = ldb;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.C = C;
  g.ldc = ldc;
  return g;
}

inline void* off_T(gpt_ctx* x, void* p, int64_t elems) { return (char*)p + elems * x->es; }

// weight gradient dW[M][N] (+)= sum_n A(m, n) B(n-th col): both operands token-major
// (runs on the side stream in the backward; the split-K workspace is only used there)
int wgrad(gpt_ctx* x, const char* cls, const void* dY, int64_t ldy, const void* Xin, int64_t ldx, int64_t M,
          int64_t Nn, float* dW, int acc) {
  gk::Gemm g = mk(x, 1, 1, gk::EPI_F32, dY, ldy, Xin, ldx, M, Nn, x->N, dW, Nn);
  g.accumulate = acc;
  g.splits = gk::gemm_pick_splits((int)M, (int)Nn, (int)x->N, 1, 1);
  g.ws = x->splitk_ws;
  g.ws_floats = x->splitk_n;
  return run_gemm(x, cls, g, x->side);
}

// column partial sums of a bias gradient (reduced with the others at the end of backward)
int bias_colsum(gpt_ctx* x, int dtype, const void* dY, int64_t cols, float* part) {
  ProfScope ps(x, "bias_colsum", 0.0, (double)x->N * cols * (dtype == GPT_BF16 ? 2 : 4), x->side);
  HIPCHK(gk::colsum_partial(dtype, dY, (int)x->N, (int)cols, part, x->side));
  return 0;
}

// LayerNorm backward into x->dres (+ its T copy); gain/shift/residual column
// partials into part
int ln_bwd(gpt_ctx* x, const void* dy, bool dy_is_t, const float* xin, const float* mu, const float* rs, int g_id,
           const float* dres_in, float* part, void* dresT) {
  ProfScope ps(x, "layernorm_bwd", 0.0, (double)x->N * x->C * ((dy_is_t ? x->es : 4) + 4 + 4 + 4 + x->es) + 8.0 * x->N);
  HIPCHK(gk::layernorm_bwd(x->dt, dy, dy_is_t ? 1 : 0, xin, mu, rs, x->P_(g_id), dres_in, x->dres, dresT, part,
                           (int)x->N, (int)x->C, nullptr, x->stream, x->blk == GPT_BLOCK_RMS_ROPE_SWIGLU ? 1 : 0));
  return 0;
}

// LayerNorm (GPT_BLOCK_GPT2) or RMSNorm (b_id < 0: GPT_BLOCK_RMS_ROPE_SWIGLU) forward
int ln_fwd(gpt_ctx* x, const float* in, int g_id, int b_id, void* out, float* mu, float* rs) {
  ProfScope ps(x, "layernorm_fwd", 0.0, (double)x->N * x->C * (4 + x->es) + 8.0 * x->N);
  HIPCHK(gk::layernorm_fwd(x->dt, in, x->P_(g_id), b_id >= 0 ? x->P_(b_id) : nullptr, out, mu, rs, (int)x->N,
                           (int)x->C, x->stream, b_id < 0 ? 1 : 0));
  return 0;
}

// main stream waits for all work queued on the side streams so far
int join_side(gpt_ctx* x) {
  if (x->side) {
    HIPCHK(hipEventRecord(x->side_tail, x->side));
    HIPCHK(hipStreamWaitEvent(x->stream, x->side_tail, 0));
  }
  if (x->hside) {
    HIPCHK(hipEventRecord(x->hside_tail, x->hside));
    HIPCHK(hipStreamWaitEvent(x->stream, x->hside_tail, 0));
  }
  return 0;
}

// The tied head fused with the cross-entropy (no [N, V] logits anywhere):
// one pass gives the per-row loss and log-sum-exp and, with gradients, dF -
// on the context stream - then the fixed-order mean of the row losses.  The
// head's part of the tied weight's gradient, which only the embedding step of
// the backward reads, runs on a stream of its own when there is one, beside
// the backward of the blocks.  By default one kernel recomputes each vocabulary
// block's logits from the row log-sum-exps and contracts their gradient with F
// without it leaving the CU.  The GEMM form (GPT_HEAD_DW=gemm, when a block
// buffer exists) instead runs, per block of head_cols vocabulary columns, one
// product that recomputes the block's logits and turns them into their
// gradient (exp(z - lse) - onehot) * scale in its epilogue (T, [N][cols]), and a
// second that contracts it with F over the rows into those rows of dW.  Same
// box, 124M step: 20.25 ms with the single kernel against 20.47 ms with the
// GEMM form, which also moves the [N, V] logit gradient through memory once
// each way (about 6 GB per step).
// Pass 1 in GEMM form (fp32 model contexts): the logits of one block of
// head_cols vocabulary columns at a time go to the block buffer through an
// fp32 product, and lmhead_block_stats merges the block into each row's
// maximum and sum of exp (after the last block: log-sum-exp and row loss).
// For dF each block's logit gradient (exp(z - lse) - onehot) * scale is then
// formed again by the product's cross-entropy-gradient epilogue and
// dF += G_blk W_blk.  The same softmax as the fused kernel, on the fp32 MFMAs
// instead of plain FMAs; the buffer holds one block, never [N, V].
int head_fwd_gemm(gpt_ctx* x, const void* Fin, const void* W, int64_t V, const int32_t* y, int64_t N, int64_t C,
                  float scale, float* tok_loss, float* tok_lse, float* dF, int* bad) {
  const int64_t cols = x->head_cols;
  const char* Wb = (const char*)W;
  for (int64_t v0 = 0; v0 < V; v0 += cols) {
    const int64_t n = std::min(cols, V - v0);
    gk::Gemm g = mk(x, 0, 0, gk::EPI_STORE, Fin, C, Wb + v0 * C * 4, C, N, n, C, x->gchunk, cols);
    g.dtype = GPT_F32;
    if (int e = run_gemm(x, "head_z", g)) return e;
    HIPCHK(gk::lmhead_block_stats((const float*)x->gchunk, (int)cols, (int)N, (int)n, (int)v0, (int)V, y, x->head_ml,
                                  x->head_zy, tok_loss, tok_lse, v0 == 0, v0 + n >= V, bad, x->stream));
  }
  if (!dF) return 0;
  for (int64_t v0 = 0; v0 < V; v0 += cols) {
    const int64_t n = std::min(cols, V - v0);
    gk::Gemm g = mk(x, 0, 0, gk::EPI_CE_GRAD, Fin, C, Wb + v0 * C * 4, C, N, n, C, x->gchunk, cols);
    g.dtype = GPT_F32;
    g.lse = tok_lse;
    g.rowi = y;
    g.col0 = (int)v0;
    g.scale = scale;
    if (int e = run_gemm(x, "head_dz", g)) return e;
    g = mk(x, 0, 1, gk::EPI_F32, x->gchunk, cols, Wb + v0 * C * 4, C, N, C, n, dF, C);
    g.dtype = GPT_F32;
    g.accumulate = v0 > 0;
    if (int e = run_gemm(x, "head_df", g)) return e;
  }
  return 0;
}

int head(gpt_ctx* x, const void* Fin, const void* W, int64_t V, const int32_t* y, int64_t N, int64_t C, float scale,
         float* tok_loss, float* tok_lse, float* dF, float* dW, int dW_acc, int dtype, float* loss, float* ring,
         int slot, int* bad, bool fused_dw = false) {
  if (dtype == GPT_F32 && !fused_dw && x->gchunk && x->head_ml && head_gemm_ctx(dtype, C)) {
    ProfScope ps(x, "head_fwd", (dF ? 4.0 : 2.0) * N * V * C, 0.0);
    if (int e = head_fwd_gemm(x, Fin, W, V, y, N, C, scale, tok_loss, tok_lse, dF, bad)) return e;
  } else {
    ProfScope ps(x, "head_fwd", (dF ? 4.0 : 2.0) * N * V * C, 0.0);
    HIPCHK(gk::lmhead_fwd(dtype, Fin, W, (int)N, (int)V, (int)C, y, scale, tok_loss, tok_lse, dF, bad, x->stream,
                          x->head_seg, x->head_seg_n));
  }
  HIPCHK(gk::mean_f32(tok_loss, (int)N, loss, ring, slot, x->stream));
  if (!dW) return 0;
  hipStream_t ds = x->hside ? x->hside : x->stream;
  if (x->hside) {
    HIPCHK(hipEventRecord(x->head_fork, x->stream));
    HIPCHK(hipStreamWaitEvent(x->hside, x->head_fork, 0));
  }
  if (fused_dw || !x->gchunk || !head_gemm_ctx(dtype, C)) {
    ProfScope ps(x, "head_dw", 2.0 * N * V * C, 0.0, ds);
    // GPT_HEAD_DW_WGS caps its grid (tuning runs): fewer resident workgroups
    // leave more CUs to the backward running beside it
    const char* cap = x->hside ? getenv("GPT_HEAD_DW_WGS") : nullptr;
    HIPCHK(gk::lmhead_dw(dtype, Fin, W, (int)N, (int)V, (int)C, y, tok_lse, scale, dW, dW_acc, ds,
                         cap ? atoi(cap) : 0, getenv("GPT_HEAD_DW_NOTAIL") ? nullptr : x->head_tail,
                         x->head_tail_n));
    return 0;
  }
  const int64_t es = dtype == GPT_BF16 ? 2 : 4, cols = x->head_cols;
  for (int64_t v0 = 0; v0 < V; v0 += cols) {
    const int64_t n = std::min(cols, V - v0);
    gk::Gemm g = mk(x, 0, 0, gk::EPI_CE_GRAD, Fin, C, (const char*)W + v0 * C * es, C, N, n, C, x->gchunk, cols);
    g.dtype = dtype;
    g.lse = tok_lse;
    g.rowi = y;
    g.col0 = (int)v0;
    g.scale = scale;
    if (int e = run_gemm(x, "head_dw_dz", g, ds)) return e;
    g = mk(x, 1, 1, gk::EPI_F32, x->gchunk, cols, Fin, C, n, C, N, dW + v0 * C, C);
    g.dtype = dtype;
    g.accumulate = dW_acc;
    if (x->head_skws) {
      g.splits = gk::gemm_pick_splits((int)n, (int)C, (int)N, 1, 1);
      g.ws = x->head_skws;
      g.ws_floats = x->head_skn;
    }
    if (int e = run_gemm(x, "head_dw", g, ds)) return e;
  }
  return 0;
}

// ---- GPT_BLOCK_RMS_ROPE_SWIGLU (CS336 pretraining page, the second block variant) ----

// Forward of the embedding and the blocks into lnf: embedding + RMSNorm, then
// per block QKV (no bias) -> RoPE on q and k (in place) -> causal attention ->
// out-projection + residual -> RMSNorm -> [gate | up] = x [W1; W3]^T ->
// SwiGLU -> down-projection + residual; the final RMSNorm.
int forward_variant(gpt_ctx* x, bool adam) {
  hipStream_t s = x->stream;
  const int64_t N = x->N, C = x->C, F = x->F;
  const int L = (int)x->L;
  {
    ProfScope ps(x, "layernorm_fwd", 0.0, (double)N * C * (4 + 4 + x->es) + 8.0 * N);
    HIPCHK(gk::embed_ln_fwd(x->dt, x->win, x->P_(0), nullptr, (int)x->T, x->res[0], x->P_(vt(0, VK_RMS1)), nullptr,
                            x->layers[0].ln1, x->layers[0].mu1, x->layers[0].rs1, (int)N, (int)C, s, 1));
  }
  for (int l = 0; l < L; ++l) {
    Layer& ly = x->layers[l];
    if (adam && l <= 2) HIPCHK(hipStreamWaitEvent(s, x->adam_ev[l < 2 ? 2 + l : L + 1], 0));
    gk::Gemm g = mk(x, 0, 0, gk::EPI_STORE, ly.ln1, C, x->W_(vt(l, VK_ATTW)), C, N, 3 * C, C, ly.qkv, 3 * C);
    if (int e = run_gemm(x, "gemm_qkv_fwd", g)) return e;
    {
      ProfScope ps(x, "rope", 0.0, (double)N * 2 * C * 2 * x->es);
      HIPCHK(gk::rope_qk(x->dt, ly.qkv, (int)N, (int)C, (int)x->T, (int)x->D, x->rope_tab, 0, s));
    }
    {
      const double pairs = (double)x->B * x->H * x->T * (x->T + 1) / 2.0;
      ProfScope ps(x, "attn_fwd", 4.0 * x->D * pairs, 0.0);
      HIPCHK(gk::attn_fwd(x->dt, ly.qkv, ly.att, ly.lse, (int)x->B, (int)x->T, (int)x->H, (int)x->D, s));
    }
    g = mk(x, 0, 0, gk::EPI_RESID, ly.att, C, x->W_(vt(l, VK_PROJW)), C, N, C, C, ly.res_mid, C);
    g.R = x->res[l];
    if (int e = run_gemm(x, "gemm_proj_fwd", g)) return e;
    if (int e = ln_fwd(x, ly.res_mid, vt(l, VK_RMS2), -1, ly.ln2, ly.mu2, ly.rs2)) return e;
    g = mk(x, 0, 0, gk::EPI_STORE, ly.ln2, C, x->W_(vt(l, VK_W1)), C, N, 2 * F, C, ly.fcdg, 2 * F);
    if (int e = run_gemm(x, "gemm_fc_fwd", g)) return e;
    {
      ProfScope ps(x, "swiglu", 0.0, (double)N * F * 3 * x->es);
      HIPCHK(gk::swiglu_fwd(x->dt, ly.fcdg, ly.fcact, (int)N, (int)F, s));
    }
    g = mk(x, 0, 0, gk::EPI_RESID, ly.fcact, F, x->W_(vt(l, VK_W2)), F, N, C, F, x->res[l + 1], C);
    g.R = ly.res_mid;
    if (int e = run_gemm(x, "gemm_mlpproj_fwd", g)) return e;
    if (l + 1 < L) {
      Layer& nx = x->layers[l + 1];
      if (int e = ln_fwd(x, x->res[l + 1], vt(l + 1, VK_RMS1), -1, nx.ln1, nx.mu1, nx.rs1)) return e;
    } else {
      if (int e = ln_fwd(x, x->res[l + 1], vt_rmsf(L), -1, x->lnf, x->muf, x->rsf)) return e;
    }
  }
  return 0;
}

// Backward of the blocks and the embedding (the head already wrote dF and
// G(lm_head)).  Same two-stream schedule as the GPT-2 blocks: weight
// gradients on the side stream, started by events on the data-gradient chain,
// which waits for them before reusing their inputs.  dqkv is rotated back
// (RoPE's transpose) before the QKV products read it.
int backward_variant(gpt_ctx* x) {
  hipStream_t s = x->stream, ss = x->side;
  const int64_t N = x->N, C = x->C, F = x->F;
  const int acc = x->others_fresh ? 0 : 1;
  const int L = (int)x->L;
  auto ev = [&](int l, int k) { return x->sev[(size_t)l * 8 + k]; };
  auto fork = [&](int l, int k) -> int {
    HIPCHK(hipEventRecord(ev(l, k), s));
    HIPCHK(hipStreamWaitEvent(ss, ev(l, k), 0));
    return 0;
  };
  auto done = [&](int l, int k) -> int {
    HIPCHK(hipEventRecord(ev(l, 4 + k), ss));
    return 0;
  };
  auto wait_side = [&](int l, int k) -> int {
    HIPCHK(hipStreamWaitEvent(s, ev(l, 4 + k), 0));
    return 0;
  };
  void* T0 = x->dresT2[0];
  void* T1 = x->dresT2[1];
  if (int e = ln_bwd(x, x->dF, false, x->res[L], x->muf, x->rsf, vt_rmsf(L), nullptr, x->lnf_part, T0)) return e;
  for (int l = L - 1; l >= 0; --l) {
    Layer& ly = x->layers[l];
    // SwiGLU down-projection: dW2 on the side stream, dh = dY W2 on s
    if (int e = fork(l, 0)) return e;
    if (int e = wgrad(x, "gemm_wgrad_mlp", T0, C, ly.fcact, F, C, F, x->G_(vt(l, VK_W2)), acc)) return e;
    if (int e = done(l, 0)) return e;
    gk::Gemm g = mk(x, 0, 1, gk::EPI_STORE, T0, C, x->W_(vt(l, VK_W2)), F, N, F, C, x->dh, F);
    if (int e = run_gemm(x, "gemm_dgrad_mlp", g)) return e;
    if (l + 1 < L)
      if (int e = wait_side(l + 1, 1)) return e;  // previous layer's W1/W3 dW finished reading dfc
    {
      ProfScope ps(x, "swiglu", 0.0, (double)N * F * 5 * x->es);
      HIPCHK(gk::swiglu_bwd(x->dt, ly.fcdg, x->dh, x->dfc, (int)N, (int)F, s));
    }
    // [W1; W3]: one [2F, C] product each way
    if (int e = fork(l, 1)) return e;
    if (int e = wgrad(x, "gemm_wgrad_mlp", x->dfc, 2 * F, ly.ln2, C, 2 * F, C, x->G_(vt(l, VK_W1)), acc)) return e;
    if (int e = done(l, 1)) return e;
    g = mk(x, 0, 1, gk::EPI_STORE, x->dfc, 2 * F, x->W_(vt(l, VK_W1)), C, N, C, 2 * F, x->dlnT, C);
    if (int e = run_gemm(x, "gemm_dgrad_mlp", g)) return e;
    if (l + 1 < L)
      if (int e = wait_side(l + 1, 2)) return e;  // previous layer's proj dW finished reading T1
    if (int e = ln_bwd(x, x->dlnT, true, ly.res_mid, ly.mu2, ly.rs2, vt(l, VK_RMS2), x->dres, ly.ln2_part, T1))
      return e;
    // attention output projection
    if (int e = fork(l, 2)) return e;
    if (int e = wgrad(x, "gemm_wgrad_attn", T1, C, ly.att, C, C, C, x->G_(vt(l, VK_PROJW)), acc)) return e;
    if (int e = done(l, 2)) return e;
    g = mk(x, 0, 1, gk::EPI_STORE, T1, C, x->W_(vt(l, VK_PROJW)), C, N, C, C, x->datt, C);
    const bool fused_dv = x->dt == GPT_BF16 && x->D == 64;
    if (fused_dv) {
      g.epi = gk::EPI_STORE_ODOT;
      g.aux = ly.att;
      g.dv = x->Dv;
      g.tn = (int)x->T;
      g.heads = (int)x->H;
    }
    if (int e = run_gemm(x, "gemm_dgrad_attn", g)) return e;
    if (l + 1 < L)
      if (int e = wait_side(l + 1, 3)) return e;  // previous layer's qkv dW finished reading dqkv
    {
      const double pairs = (double)x->B * x->H * x->T * (x->T + 1) / 2.0;
      ProfScope ps(x, "attn_bwd", 8.0 * x->D * pairs, 0.0);
      if (fused_dv)
        HIPCHK(gk::attn_bwd_bf16_d64(ly.qkv, x->datt, ly.lse, x->Dv, x->dqkv, (int)x->B, (int)x->T, (int)x->H, s));
      else
        HIPCHK(gk::attn_bwd(x->dt, ly.qkv, ly.att, x->datt, ly.lse, x->Dv, x->dqkv, (int)x->B, (int)x->T, (int)x->H,
                            (int)x->D, s));
    }
    {
      ProfScope ps(x, "rope", 0.0, (double)N * 2 * C * 2 * x->es);
      HIPCHK(gk::rope_qk(x->dt, x->dqkv, (int)N, (int)C, (int)x->T, (int)x->D, x->rope_tab, 1, s));
    }
    // QKV projection
    if (int e = fork(l, 3)) return e;
    if (int e = wgrad(x, "gemm_wgrad_attn", x->dqkv, 3 * C, ly.ln1, C, 3 * C, C, x->G_(vt(l, VK_ATTW)), acc)) return e;
    if (int e = done(l, 3)) return e;
    g = mk(x, 0, 1, gk::EPI_STORE, x->dqkv, 3 * C, x->W_(vt(l, VK_ATTW)), C, N, C, 3 * C, x->dlnT, C);
    if (int e = run_gemm(x, "gemm_dgrad_attn", g)) return e;
    if (int e = wait_side(l, 0)) return e;  // this layer's W2 dW finished reading T0
    if (int e = ln_bwd(x, x->dlnT, true, x->res[l], ly.mu1, ly.rs1, vt(l, VK_RMS1), x->dres, ly.ln1_part, T0))
      return e;
  }
  if (int e = join_side(x)) return e;
  if (ss) {
    HIPCHK(hipEventRecord(x->fwd_start, s));
    HIPCHK(hipStreamWaitEvent(ss, x->fwd_start, 0));
  }
  hipStream_t s2 = ss ? ss : s;
  {
    // the token rows are the only gradient of wte here (the head has its own tensor)
    ProfScope ps(x, "embed_bwd", 0.0, (double)N * C * 12);
    if (x->wte_fresh) HIPCHK(gk::fill_f32(x->G_(0), x->tensors[0].numel(), 0.f, s));
    HIPCHK(gk::embed_bwd_ws(x->keys, (int)N, x->dres, (int)C, x->dln, x->G_(0), s));
    x->wte_fresh = false;
  }
  {
    ProfScope ps(x, "param_reduce", 0.0, 0.0, s2);
    HIPCHK(gk::reduce_jobs(x->jobs_dev, (int)x->jobs.size(), x->nred_blocks, acc, s2));
  }
  x->others_fresh = false;
  x->fwd_grad = false;
  return 0;
}

}  // namespace

extern "C" {

size_t gpt_arena_bytes(const gpt_config* cfg) {
  if (check_cfg(cfg)) return 0;
  gpt_ctx tmp;
  setup_dims(&tmp, cfg);
  return (size_t)carve(&tmp, nullptr);
}

int gpt_init(const gpt_config* cfg, void* arena, size_t arena_bytes, void* hip_stream, uint64_t seed, gpt_ctx** out) {
  if (int e = check_cfg(cfg)) return e;
  if (!arena || !out) return fail(GPT_EINVAL, "null arena or out pointer");
  if (((uintptr_t)arena) % ALIGN) return fail(GPT_EINVAL, "arena must be 256-byte aligned");
  gpt_ctx* x = new gpt_ctx();
  setup_dims(x, cfg);
  const int64_t need = carve(x, nullptr);
  if ((int64_t)arena_bytes < need) {
    delete x;
    return fail(GPT_ENOMEM, "arena too small: need " + std::to_string(need) + " bytes");
  }
  carve(x, arena);
  x->stream = (hipStream_t)hip_stream;
  hipStream_t s = x->stream;
  int rc = 0;
  auto chk = [&](hipError_t e) {
    if (e != hipSuccess && !rc) rc = fail(GPT_EHIP, std::string("init: ") + hipGetErrorString(e));
  };
  chk(gk::fill_f32(x->params, x->P, 0.f, s));
  chk(gk::fill_f32(x->grads, x->P, 0.f, s));
  chk(gk::fill_f32(x->m, x->P, 0.f, s));
  chk(gk::fill_f32(x->v, x->P, 0.f, s));
  chk(gk::fill_f32(x->scal, 16, 0.f, s));
  chk(gk::fill_f32((float*)x->step_dev, 16, 0.f, s));
  chk(gk::fill_f32(x->ring, RING, 0.f, s));
  // the head's block buffer is read past a short last block's columns (k-tile
  // padding, multiplied by zeros): it must hold finite values from the start
  if (x->gchunk && x->dt == GPT_F32) chk(gk::fill_f32((float*)x->gchunk, x->N * x->head_cols, 0.f, s));
  const float std_r = 0.02f / std::sqrt(2.0f * (float)x->L);
  uint64_t logical = 0;
  for (auto& d : x->tensors) {
    float* p = x->params + d.off;
    if (d.kind == 0) chk(gk::init_normal(p, d.numel(), 0.02f, seed, logical, s));
    else if (d.kind == 1) chk(gk::init_normal(p, d.numel(), std_r, seed, logical, s));
    else if (d.kind == 3) chk(gk::fill_f32(p, d.numel(), 1.f, s));
    logical += (uint64_t)d.numel();
  }
  if (x->shadow) chk(gk::to_bf16(x->params, x->shadow, x->P, s));
  build_jobs(x);
  chk(hipMemcpyAsync(x->jobs_dev, x->jobs.data(), x->jobs.size() * sizeof(gk::RedJob), hipMemcpyHostToDevice, s));
  if (x->rope_tab) {
    // RoPE angles t * theta^(-2i/D) for every position the context can see, in
    // double, stored as fp32 (cos, sin) pairs
    const int64_t Tm = x->cfg.max_seq, half = x->D / 2;
    std::vector<float2> tab((size_t)(Tm * half));
    for (int64_t t = 0; t < Tm; ++t)
      for (int64_t i = 0; i < half; ++i) {
        const double a = (double)t * std::pow((double)x->cfg.rope_theta, -2.0 * (double)i / (double)x->D);
        tab[(size_t)(t * half + i)] = make_float2((float)std::cos(a), (float)std::sin(a));
      }
    chk(hipMemcpyAsync(x->rope_tab, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice, s));
    chk(hipStreamSynchronize(s));
  }
  // side stream (default priority) and its ordering events
  chk(hipStreamCreateWithFlags(&x->side, hipStreamNonBlocking));
  chk(hipStreamCreateWithFlags(&x->hside, hipStreamNonBlocking));
  chk(hipEventCreateWithFlags(&x->hside_tail, hipEventDisableTiming));
  x->sev.assign((size_t)x->L * 8, nullptr);
  for (auto& e : x->sev) chk(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  chk(hipEventCreateWithFlags(&x->head_fork, hipEventDisableTiming));
  chk(hipEventCreateWithFlags(&x->side_tail, hipEventDisableTiming));
  chk(hipEventCreateWithFlags(&x->fwd_start, hipEventDisableTiming));
  chk(hipEventCreateWithFlags(&x->norm_done, hipEventDisableTiming));
  x->adam_ev.assign((size_t)x->L + 2, nullptr);
  for (auto& e : x->adam_ev) chk(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  for (int k = 0; k < 2; ++k) {
    chk(hipHostMalloc((void**)&x->stage_host[k], (size_t)(x->N + 1) * 4, hipHostMallocDefault));
    chk(hipEventCreateWithFlags(&x->stage_ev[k], hipEventDisableTiming));
  }
  if (rc) {
    gpt_destroy(x);
    return rc;
  }
  *out = x;
  return 0;
}

int gpt_destroy(gpt_ctx* x) {
  if (!x) return 0;
  for (auto e : x->prof.ev) (void)hipEventDestroy(e);
  if (x->side) (void)hipStreamSynchronize(x->side);
  if (x->hside) (void)hipStreamSynchronize(x->hside);
  for (auto e : x->sev)
    if (e) (void)hipEventDestroy(e);
  for (auto e : x->adam_ev)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : {x->head_fork, x->side_tail, x->hside_tail, x->fwd_start, x->norm_done})
    if (e) (void)hipEventDestroy(e);
  for (int k = 0; k < 2; ++k) {
    if (x->stage_ev[k]) {
      (void)hipEventSynchronize(x->stage_ev[k]);
      (void)hipEventDestroy(x->stage_ev[k]);
    }
    if (x->stage_host[k]) (void)hipHostFree(x->stage_host[k]);
  }
  if (x->side) (void)hipStreamDestroy(x->side);
  if (x->hside) (void)hipStreamDestroy(x->hside);
  delete x;
  return 0;
}

int gpt_make_batch(gpt_ctx* x, const int32_t* host_tokens, int64_t n_tokens, int64_t start) {
  if (!x || !host_tokens) return fail(GPT_EINVAL, "null argument");
  const int64_t need = x->N + 1;
  if (start < 0 || start + need > n_tokens) return fail(GPT_ERANGE, "window past the end of the token stream");
  for (int64_t i = 0; i < need; ++i) {
    const int32_t t = host_tokens[start + i];
    if (t < 0 || t >= x->V)
      return fail(GPT_ERANGE, "token " + std::to_string(t) + " at " + std::to_string(start + i) + " outside [0, vocab)");
  }
  // the side stream's token sort may still read the previous batch (not when
  // it holds only AdamW pieces: the update joined everything queued before them)
  if (!x->adam_pending)
    if (int e = join_side(x)) return e;
  // the window goes through a pinned buffer whose previous copy (two batches
  // ago) has completed, so the copy needs no wait on the stream: the host can
  // queue the forward while the GPU still runs the previous step
  const int k = x->stage_i;
  HIPCHK(hipEventSynchronize(x->stage_ev[k]));
  std::memcpy(x->stage_host[k], host_tokens + start, (size_t)need * 4);
  HIPCHK(hipMemcpyAsync(x->win, x->stage_host[k], need * 4, hipMemcpyHostToDevice, x->stream));
  HIPCHK(hipEventRecord(x->stage_ev[k], x->stream));
  x->stage_i = k ^ 1;
  return 0;
}

int64_t gpt_next_start(int64_t pos, int64_t n_tokens, int32_t B, int32_t T, int32_t rank, int32_t world) {
  if (B < 1 || T < 1 || world < 1 || rank < 0 || rank >= world || n_tokens < 1)
    return fail(GPT_EINVAL, "bad cursor arguments");
  const int64_t step = (int64_t)B * T * world;
  int64_t p = pos + step;
  if (p + step + 1 > n_tokens) p = (int64_t)B * T * rank;
  return p;
}

int gpt_forward_loss(gpt_ctx* x, float loss_scale, float* loss_host) {
  if (!x) return fail(GPT_EINVAL, "null context");
  if (!(loss_scale >= 0.f) || !std::isfinite(loss_scale)) return fail(GPT_EINVAL, "loss_scale must be >= 0");
  hipStream_t s = x->stream;
  const int64_t N = x->N, C = x->C;
  const int32_t* xt = x->win;
  const int32_t* yt = x->win + 1;
  // a previous call's head dW may still read lnf and the log-sum-exps and write
  // G(wte); after an update the side stream holds only AdamW pieces, waited for
  // piece by piece
  const bool adam = x->adam_pending;
  x->adam_pending = false;
  if (adam) HIPCHK(hipStreamWaitEvent(s, x->adam_ev[1], 0));  // vectors, then wte and wpe
  else if (int e = join_side(x)) return e;
  if (loss_scale > 0.f) {
    // the embedding backward's token sort needs only the batch: it runs on the
    // side stream beside the forward (its keys are read after backward's join)
    HIPCHK(hipEventRecord(x->fwd_start, s));
    HIPCHK(hipStreamWaitEvent(x->side, x->fwd_start, 0));
    HIPCHK(gk::sort_tokens(x->win, (int)N, x->keys, x->keys_tmp, x->side));
  }
  if (x->blk == GPT_BLOCK_RMS_ROPE_SWIGLU) {
    if (int e = forward_variant(x, adam)) return e;
  } else {
  {
    ProfScope ps(x, "layernorm_fwd", 0.0, (double)N * C * (4 + 4 + 4 + x->es) + 8.0 * N);
    HIPCHK(gk::embed_ln_fwd(x->dt, xt, x->P_(T_WTE), x->P_(T_WPE), (int)x->T, x->res[0], x->P_(tid(0, K_LN1G)),
                            x->P_(tid(0, K_LN1B)), x->layers[0].ln1, x->layers[0].mu1, x->layers[0].rs1, (int)N,
                            (int)C, s));
  }
  for (int l = 0; l < x->L; ++l) {
    Layer& ly = x->layers[l];
    // layer 0 and 1's matrices, then all the rest (they finish long before layer 2)
    if (adam && l <= 2) HIPCHK(hipStreamWaitEvent(s, x->adam_ev[l < 2 ? 2 + l : x->L + 1], 0));
    gk::Gemm g = mk(x, 0, 0, gk::EPI_STORE, ly.ln1, C, x->W_(tid(l, K_ATTW)), C, N, 3 * C, C, ly.qkv, 3 * C);
    g.bias = x->P_(tid(l, K_ATTB));
    if (int e = run_gemm(x, "gemm_qkv_fwd", g)) return e;
    {
      const double pairs = (double)x->B * x->H * x->T * (x->T + 1) / 2.0;
      ProfScope ps(x, "attn_fwd", 4.0 * x->D * pairs, 0.0);
      HIPCHK(gk::attn_fwd(x->dt, ly.qkv, ly.att, ly.lse, (int)x->B, (int)x->T, (int)x->H, (int)x->D, s));
    }
    g = mk(x, 0, 0, gk::EPI_RESID, ly.att, C, x->W_(tid(l, K_PROJW)), C, N, C, C, ly.res_mid, C);
    g.bias = x->P_(tid(l, K_PROJB));
    g.R = x->res[l];
    if (int e = run_gemm(x, "gemm_proj_fwd", g)) return e;
    if (int e = ln_fwd(x, ly.res_mid, tid(l, K_LN2G), tid(l, K_LN2B), ly.ln2, ly.mu2, ly.rs2)) return e;
    g = mk(x, 0, 0, gk::EPI_GELU, ly.ln2, C, x->W_(tid(l, K_FCW)), C, N, 4 * C, C, ly.fcdg, 4 * C);
    g.bias = x->P_(tid(l, K_FCB));
    g.C2 = ly.fcact;
    if (int e = run_gemm(x, "gemm_fc_fwd", g)) return e;
    g = mk(x, 0, 0, gk::EPI_RESID, ly.fcact, 4 * C, x->W_(tid(l, K_MPW)), 4 * C, N, C, 4 * C, x->res[l + 1], C);
    g.bias = x->P_(tid(l, K_MPB));
    g.R = ly.res_mid;
    if (int e = run_gemm(x, "gemm_mlpproj_fwd", g)) return e;
    if (l + 1 < x->L) {
      Layer& nx = x->layers[l + 1];
      if (int e = ln_fwd(x, x->res[l + 1], tid(l + 1, K_LN1G), tid(l + 1, K_LN1B), nx.ln1, nx.mu1, nx.rs1)) return e;
    } else {
      if (int e = ln_fwd(x, x->res[l + 1], tid_lnf(x->L, 0), tid_lnf(x->L, 1), x->lnf, x->muf, x->rsf)) return e;
    }
  }
  }
  const float scale = loss_scale / (float)N;
  const bool grad = loss_scale > 0.f;
  // the GPT-2 head is tied to wte; the variant's head is a tensor of its own
  const bool tied = x->blk == GPT_BLOCK_GPT2;
  const int hw = tied ? T_WTE : vt_head((int)x->L);
  const bool fresh = tied ? x->wte_fresh : x->others_fresh;
  if (int e = head(x, x->lnf, x->W_(hw), x->Vp, yt, N, C, grad ? scale : 0.f, x->tok_loss, x->tok_lse,
                   grad ? x->dF : nullptr, grad ? x->G_(hw) : nullptr, fresh ? 0 : 1, x->dt, x->loss, x->ring,
                   (int)(x->ring_wr % RING), nullptr))
    return e;
  if (grad && tied) x->wte_fresh = false;
  x->ring_wr++;
  x->have_fwd = true;
  x->fwd_grad = grad;
  x->last_scale = loss_scale;
  if (loss_host) {
    HIPCHK(hipMemcpyAsync(loss_host, x->loss, 4, hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
    if (!std::isfinite(*loss_host)) return fail(GPT_ENONFINITE, "non-finite loss");
  }
  return 0;
}

int gpt_backward(gpt_ctx* x) {
  if (!x) return fail(GPT_EINVAL, "null context");
  if (!x->have_fwd || !x->fwd_grad) return fail(GPT_EINVAL, "gpt_backward needs a gpt_forward_loss with loss_scale > 0");
  if (x->blk == GPT_BLOCK_RMS_ROPE_SWIGLU) return backward_variant(x);
  hipStream_t s = x->stream, ss = x->side;
  const int64_t N = x->N, C = x->C;
  const int acc = x->others_fresh ? 0 : 1;
  const int L = (int)x->L;
  // The four weight-gradient products of a layer (and the fc/qkv bias column
  // sums) run on the side stream ss, off the data-gradient chain on s.  Each
  // side product starts after an event that s records when its input is
  // written; s waits for the side product's completion event before it
  // overwrites that input: dfc (next layer's GELU backward), dqkv (next
  // layer's attention backward) and the residual-gradient T copies, which
  // alternate between two buffers - T0 enters a layer, LN2 writes T1, LN1 T0.
  // Events per layer: 0-3 mark the inputs ready, 4-7 the side products done.
  auto ev = [&](int l, int k) { return x->sev[(size_t)l * 8 + k]; };
  auto fork = [&](int l, int k) -> int {
    HIPCHK(hipEventRecord(ev(l, k), s));
    HIPCHK(hipStreamWaitEvent(ss, ev(l, k), 0));
    return 0;
  };
  auto done = [&](int l, int k) -> int {
    HIPCHK(hipEventRecord(ev(l, 4 + k), ss));
    return 0;
  };
  auto wait_side = [&](int l, int k) -> int {
    HIPCHK(hipStreamWaitEvent(s, ev(l, 4 + k), 0));
    return 0;
  };
  void* T0 = x->dresT2[0];
  void* T1 = x->dresT2[1];
  if (int e = ln_bwd(x, x->dF, false, x->res[L], x->muf, x->rsf, tid_lnf(L, 0), nullptr, x->lnf_part, T0)) return e;
  for (int l = L - 1; l >= 0; --l) {
    Layer& ly = x->layers[l];
    // MLP output projection: dW on the side stream, GELU backward on s
    if (int e = fork(l, 0)) return e;
    if (int e = wgrad(x, "gemm_wgrad_mlp", T0, C, ly.fcact, 4 * C, C, 4 * C, x->G_(tid(l, K_MPW)), acc)) return e;
    if (int e = done(l, 0)) return e;
    if (l + 1 < L)
      if (int e = wait_side(l + 1, 1)) return e;  // previous layer's fc dW finished reading dfc
    gk::Gemm g = mk(x, 0, 1, gk::EPI_GELU_BWD, T0, C, x->W_(tid(l, K_MPW)), 4 * C, N, 4 * C, C, x->dfc, 4 * C);
    g.aux = ly.fcdg;
    if (int e = run_gemm(x, "gemm_dgrad_mlp", g)) return e;
    // MLP input projection
    if (int e = fork(l, 1)) return e;
    if (int e = wgrad(x, "gemm_wgrad_mlp", x->dfc, 4 * C, ly.ln2, C, 4 * C, C, x->G_(tid(l, K_FCW)), acc)) return e;
    if (int e = bias_colsum(x, x->dt, x->dfc, 4 * C, ly.fcb_part)) return e;
    if (int e = done(l, 1)) return e;
    g = mk(x, 0, 1, gk::EPI_STORE, x->dfc, 4 * C, x->W_(tid(l, K_FCW)), C, N, C, 4 * C, x->dlnT, C);
    if (int e = run_gemm(x, "gemm_dgrad_mlp", g)) return e;
    if (l + 1 < L)
      if (int e = wait_side(l + 1, 2)) return e;  // previous layer's proj dW finished reading T1
    if (int e = ln_bwd(x, x->dlnT, true, ly.res_mid, ly.mu2, ly.rs2, tid(l, K_LN2G), x->dres, ly.ln2_part, T1))
      return e;
    // attention output projection
    if (int e = fork(l, 2)) return e;
    if (int e = wgrad(x, "gemm_wgrad_attn", T1, C, ly.att, C, C, C, x->G_(tid(l, K_PROJW)), acc)) return e;
    if (int e = done(l, 2)) return e;
    g = mk(x, 0, 1, gk::EPI_STORE, T1, C, x->W_(tid(l, K_PROJW)), C, N, C, C, x->datt, C);
    // bf16, D = 64: the attention backward's row sums D = rowsum(dO * O) come
    // out of this product's epilogue, where dO is produced
    const bool fused_dv = x->dt == GPT_BF16 && x->D == 64;
    if (fused_dv) {
      g.epi = gk::EPI_STORE_ODOT;
      g.aux = ly.att;
      g.dv = x->Dv;
      g.tn = (int)x->T;
      g.heads = (int)x->H;
    }
    if (int e = run_gemm(x, "gemm_dgrad_attn", g)) return e;
    if (l + 1 < L)
      if (int e = wait_side(l + 1, 3)) return e;  // previous layer's qkv dW finished reading dqkv
    {
      const double pairs = (double)x->B * x->H * x->T * (x->T + 1) / 2.0;
      ProfScope ps(x, "attn_bwd", 8.0 * x->D * pairs, 0.0);
      if (fused_dv)
        HIPCHK(gk::attn_bwd_bf16_d64(ly.qkv, x->datt, ly.lse, x->Dv, x->dqkv, (int)x->B, (int)x->T, (int)x->H, s));
      else
        HIPCHK(gk::attn_bwd(x->dt, ly.qkv, ly.att, x->datt, ly.lse, x->Dv, x->dqkv, (int)x->B, (int)x->T, (int)x->H,
                            (int)x->D, s));
    }
    // QKV projection
    if (int e = fork(l, 3)) return e;
    if (int e = wgrad(x, "gemm_wgrad_attn", x->dqkv, 3 * C, ly.ln1, C, 3 * C, C, x->G_(tid(l, K_ATTW)), acc)) return e;
    if (int e = bias_colsum(x, x->dt, x->dqkv, 3 * C, ly.attb_part)) return e;
    if (int e = done(l, 3)) return e;
    g = mk(x, 0, 1, gk::EPI_STORE, x->dqkv, 3 * C, x->W_(tid(l, K_ATTW)), C, N, C, 3 * C, x->dlnT, C);
    if (int e = run_gemm(x, "gemm_dgrad_attn", g)) return e;
    if (int e = wait_side(l, 0)) return e;  // this layer's MLP-output dW finished reading T0
    if (int e = ln_bwd(x, x->dlnT, true, x->res[l], ly.mu1, ly.rs1, tid(l, K_LN1G), x->dres, ly.ln1_part, T0))
      return e;
  }
  // join: every side product (the head's dW among them) is done before the
  // embedding backward adds into G(wte), the parameter reduction and AdamW
  if (int e = join_side(x)) return e;
  // embeddings: token rows (deterministic segmented sum) on s; positions and
  // the batched reduction of the bias / LayerNorm partials (which write other
  // tensors) beside it on the side stream, which every later reader joins
  if (ss) {
    HIPCHK(hipEventRecord(x->fwd_start, s));
    HIPCHK(hipStreamWaitEvent(ss, x->fwd_start, 0));
  }
  hipStream_t s2 = ss ? ss : s;
  {
    ProfScope ps(x, "embed_bwd", 0.0, (double)N * C * 12);
    HIPCHK(gk::embed_bwd_ws(x->keys, (int)N, x->dres, (int)C, x->dln, x->G_(T_WTE), s));
    HIPCHK(gk::wpe_bwd(x->dres, (int)x->B, (int)x->T, (int)C, x->G_(T_WPE), acc, s2));
  }
  {
    ProfScope ps(x, "param_reduce", 0.0, 0.0, s2);
    HIPCHK(gk::reduce_jobs(x->jobs_dev, (int)x->jobs.size(), x->nred_blocks, acc, s2));
  }
  x->others_fresh = false;
  x->fwd_grad = false;
  return 0;
}

int gpt_adamw_step(gpt_ctx* x, float lr, float beta1, float beta2, float eps, float weight_decay, float grad_clip,
                   float* grad_norm_host) {
  if (!x) return fail(GPT_EINVAL, "null context");
  if (!(lr >= 0.f) || !(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f) || !(eps >= 0.f) ||
      !(weight_decay >= 0.f))
    return fail(GPT_EINVAL, "bad AdamW hyper-parameters");
  if (int e = join_side(x)) return e;  // gradients still being written on the side stream
  if (x->wte_fresh || x->others_fresh) {
    // some gradients were never written since the last update: they are zero
    if (x->wte_fresh) HIPCHK(gk::fill_f32(x->G_(T_WTE), x->tensors[T_WTE].numel(), 0.f, x->stream));
    if (x->others_fresh) {
      // wte comes first in memory; every other tensor (and padding) follows it
      const int64_t rest = align_up(x->tensors[T_WTE].numel(), 64);
      HIPCHK(gk::fill_f32(x->grads + rest, x->P - rest, 0.f, x->stream));
    }
  }
  hipStream_t s = x->stream;
  int nblk = 0;
  if (!x->side) {
    ProfScope ps(x, "adamw", 0.0, (double)x->P * (4.0 + (x->shadow ? 30.0 : 28.0)));
    HIPCHK(gk::sumsq_partial(x->grads, x->P, x->norm_part, &nblk, s));
    HIPCHK(gk::norm_finish(x->norm_part, nblk, grad_clip, x->scal, s));
    HIPCHK(gk::adamw(x->params, x->grads, x->m, x->v, x->shadow, x->P, x->P_decay, x->scal, lr, beta1, beta2, eps,
                     weight_decay, x->step_dev, s));
  } else {
    // the gradient norm on s; the update on the side stream in pieces, in the
    // order the next forward reads them (memory order: every matrix - wte,
    // wpe, then each layer's - before the vectors): the vectors, wte + wpe,
    // then layer by layer.  The forward waits for each piece (adam_ev) instead
    // of the whole update, so most of it runs beside the forward's products.
    ProfScope ps(x, "adamw", 0.0, (double)x->P * (4.0 + (x->shadow ? 30.0 : 28.0)), x->side);
    HIPCHK(gk::sumsq_partial(x->grads, x->P, x->norm_part, &nblk, s));
    HIPCHK(gk::norm_finish(x->norm_part, nblk, grad_clip, x->scal, s));
    // the step counter and step size on s too: gpt_step_count reads them there
    HIPCHK(gk::adamw_prep(x->scal, lr, beta1, beta2, x->step_dev, s));
    HIPCHK(hipEventRecord(x->norm_done, s));
    HIPCHK(hipStreamWaitEvent(x->side, x->norm_done, 0));
    auto piece = [&](int64_t lo, int64_t hi, int k) -> int {
      HIPCHK(gk::adamw_range(x->params, x->grads, x->m, x->v, x->shadow, lo, hi, x->P_decay, x->scal, lr, beta1,
                             beta2, eps, weight_decay, x->side));
      HIPCHK(hipEventRecord(x->adam_ev[k], x->side));
      return 0;
    };
    const int L = (int)x->L;
    auto first = [&](int l) {  // layer l's matrices (the variant's lm_head rides with the last layer's)
      return l < L ? x->tensors[x->blk == GPT_BLOCK_GPT2 ? tid(l, K_ATTW) : vt(l, VK_ATTW)].off : x->P_decay;
    };
    if (int e = piece(x->P_decay, x->P, 0)) return e;  // LayerNorm gains/shifts and biases of every layer
    if (int e = piece(0, first(0), 1)) return e;       // wte, wpe (GPT-2) or wte
    for (int l = 0; l < L; ++l)
      if (int e = piece(first(l), first(l + 1), 2 + l)) return e;
    x->adam_pending = true;
  }
  x->wte_fresh = x->others_fresh = true;
  x->have_fwd = false;
  if (grad_norm_host) {
    float sc[8];
    HIPCHK(hipMemcpyAsync(sc, x->scal, sizeof(sc), hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
    *grad_norm_host = sc[0];
    if (sc[4] != 0.f) {
      HIPCHK(gk::fill_f32(x->scal + 4, 1, 0.f, s));
      x->wte_fresh = x->others_fresh = false;  // the skipped step's gradients stay readable
      return fail(GPT_ENONFINITE, "non-finite gradient norm: update skipped");
    }
  }
  return 0;
}

size_t gpt_lmhead_ce_ws_bytes(int64_t N, int64_t V, int64_t C, int32_t dtype) {
  if (N < 1 || V < 1 || C < 64 || C % 64 || (dtype != GPT_F32 && dtype != GPT_BF16)) return 0;
  if (N > 0x7fffffff || V > 0x7fffffff || C > gk::lmhead_max_embd(dtype)) return 0;
  if (dtype == GPT_BF16 && ((N + 32) * C * 2 >= (1ll << 32) || (V + 32) * C * 2 >= (1ll << 32))) return 0;
  // per-row losses and log-sum-exps, the out-of-range target flag; for the GEMM
  // form of dW also the logit gradient of one block of vocabulary columns and a
  // split-K workspace
  size_t b = (size_t)(2 * align_up(N * 4, ALIGN) + ALIGN);
  // the dW pass's split last round (bf16)
  b += (size_t)align_up(gk::lmhead_dw_tail_floats(dtype, (int)N, (int)V, (int)C) * 4, ALIGN);
  if (head_gemm_mode()) {
    const int64_t es = dtype == GPT_BF16 ? 2 : 4, cols = head_block_cols(N, V, es);
    b += (size_t)align_up(N * cols * es, ALIGN);
    const int sp = gk::gemm_pick_splits((int)cols, (int)C, (int)N, 1, 1);
    if (sp > 1) b += (size_t)align_up((int64_t)sp * cols * C * 4, ALIGN);
  }
  return b;
}

int gpt_lmhead_ce(const void* X, const void* W, const int32_t* y, int64_t N, int64_t V, int64_t C, int32_t dtype,
                  float* loss_dev, float* dX, float* dW, void* ws, size_t ws_bytes, void* hip_stream) {
  const size_t need = gpt_lmhead_ce_ws_bytes(N, V, C, dtype);
  if (!need || !X || !W || !y || !loss_dev) return fail(GPT_EINVAL, "bad lmhead_ce arguments");
  if (!ws || ws_bytes < need) return fail(GPT_ENOMEM, "lmhead_ce workspace too small");
  if (((uintptr_t)ws) % ALIGN) return fail(GPT_EINVAL, "lmhead_ce workspace must be 256-byte aligned");
  gpt_ctx tmp;  // launch helpers only use the stream and the profiling fields; no side stream
  tmp.stream = (hipStream_t)hip_stream;
  Carver cv(ws);
  float* tl = cv.take<float>(N * 4);
  float* tlse = cv.take<float>(N * 4);
  int* bad = cv.take<int>(ALIGN);
  tmp.head_tail_n = gk::lmhead_dw_tail_floats(dtype, (int)N, (int)V, (int)C);
  tmp.head_tail = tmp.head_tail_n ? cv.take<float>(tmp.head_tail_n * 4) : nullptr;
  if (head_gemm_mode()) {
    const int64_t es = dtype == GPT_BF16 ? 2 : 4;
    tmp.head_cols = head_block_cols(N, V, es);
    tmp.gchunk = cv.take<void>(N * tmp.head_cols * es);
    const int sp = gk::gemm_pick_splits((int)tmp.head_cols, (int)C, (int)N, 1, 1);
    if (sp > 1) {
      tmp.head_skn = (int64_t)sp * tmp.head_cols * C;
      tmp.head_skws = cv.take<float>(tmp.head_skn * 4);
    }
  }
  HIPCHK(gk::fill_f32((float*)bad, 1, 0.f, tmp.stream));
  if (int e = head(&tmp, X, W, V, y, N, C, 1.0f / (float)N, tl, tlse, dX, dW, 0, dtype, loss_dev, nullptr, 0, bad))
    return e;
  // out-of-range targets were clamped on the device; report them here
  int flag = 0;
  HIPCHK(hipMemcpyAsync(&flag, bad, 4, hipMemcpyDeviceToHost, tmp.stream));
  HIPCHK(hipStreamSynchronize(tmp.stream));
  if (flag) return fail(GPT_ERANGE, "a target id is outside [0, V)");
  return 0;
}

}  // extern "C"

// ---- gpt_lmhead_ce without allocation: a file-scope device scratch array ----
namespace {
constexpr int64_t NOALLOC_MAX_ROWS = 65536;
// per-row losses [NOALLOC_MAX_ROWS], per-row log-sum-exps [NOALLOC_MAX_ROWS], the out-of-range flag
constexpr size_t NOALLOC_BYTES = 2 * NOALLOC_MAX_ROWS * 4 + 256;
__device__ __align__(256) char scratch[NOALLOC_BYTES];
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[MAX_DEVICES] = {};

// The current device's copy of `scratch`, looked up once per device with that
// device current.  Host code uses this address, never the array's name.
int scratch_for_current_device(void** out) {
  int dev = -1;
  HIPCHK(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(GPT_EINVAL, "device index out of range");
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return 0;
}
}  // namespace

extern "C" {

int gpt_lmhead_ce_noalloc(const void* X, const void* W, const int32_t* y, int64_t N, int64_t V, int64_t C,
                          int32_t dtype, float* loss_dev, float* dX, float* dW, void* hip_stream) {
  if (!X || !W || !y || !loss_dev || gpt_lmhead_ce_ws_bytes(N, V, C, dtype) == 0)
    return fail(GPT_EINVAL, "bad lmhead_ce arguments");
  if (N > NOALLOC_MAX_ROWS)
    return fail(GPT_EINVAL, "gpt_lmhead_ce_noalloc: N = " + std::to_string(N) + " rows exceeds its scratch of " +
                                std::to_string(NOALLOC_MAX_ROWS) + " rows (use gpt_lmhead_ce with a workspace)");
  void* sp = nullptr;
  if (int e = scratch_for_current_device(&sp)) return e;
  gpt_ctx tmp;  // stream and profiling fields only; no side stream, no workspace
  tmp.stream = (hipStream_t)hip_stream;
  float* tl = (float*)sp;
  float* tlse = tl + NOALLOC_MAX_ROWS;
  int* bad = (int*)(tlse + NOALLOC_MAX_ROWS);
  HIPCHK(gk::fill_f32((float*)bad, 1, 0.f, tmp.stream));  // the scratch keeps the previous call's flag
  // dW by the single-kernel recompute (whatever GPT_HEAD_DW says), which needs
  // only the per-row log-sum-exps
  if (int e = head(&tmp, X, W, V, y, N, C, 1.0f / (float)N, tl, tlse, dX, dW, 0, dtype, loss_dev, nullptr, 0, bad,
                   /*fused_dw=*/true))
    return e;
  int flag = 0;
  HIPCHK(hipMemcpyAsync(&flag, bad, 4, hipMemcpyDeviceToHost, tmp.stream));
  HIPCHK(hipStreamSynchronize(tmp.stream));
  if (flag) return fail(GPT_ERANGE, "a target id is outside [0, V)");
  return 0;
}

int gpt_num_tensors(const gpt_ctx* x) { return x ? (int)x->tensors.size() : fail(GPT_EINVAL, "null context"); }

int gpt_tensor_info(const gpt_ctx* x, int id, const char** name, int64_t shape[2], int* decays) {
  if (!x || id < 0 || id >= (int)x->tensors.size()) return fail(GPT_EINVAL, "bad tensor id");
  const TensorDesc& d = x->tensors[id];
  if (name) *name = d.name.c_str();
  if (shape) {
    shape[0] = d.rows;
    shape[1] = d.cols;
  }
  if (decays) *decays = d.decays;
  return 0;
}

static float* kind_ptr(gpt_ctx* x, int kind) {
  switch (kind) {
    case GPT_PARAM: return x->params;
    case GPT_GRAD: return x->grads;
    case GPT_ADAM_M: return x->m;
    case GPT_ADAM_V: return x->v;
    default: return nullptr;
  }
}

int gpt_get_tensor(gpt_ctx* x, int kind, int id, float* host, int64_t n) {
  if (!x || !host || id < 0 || id >= (int)x->tensors.size()) return fail(GPT_EINVAL, "bad tensor access");
  float* base = kind_ptr(x, kind);
  if (!base) return fail(GPT_EINVAL, "bad tensor kind");
  const TensorDesc& d = x->tensors[id];
  if (n != d.numel()) return fail(GPT_EINVAL, "element count mismatch for " + d.name);
  if (int e = join_side(x)) return e;  // gradients may still be written on the side stream
  if (kind == GPT_GRAD && (id == T_WTE ? x->wte_fresh : x->others_fresh)) {
    std::memset(host, 0, n * 4);  // cleared since the last update
    return 0;
  }
  HIPCHK(hipMemcpyAsync(host, base + d.off, n * 4, hipMemcpyDeviceToHost, x->stream));
  HIPCHK(hipStreamSynchronize(x->stream));
  return 0;
}

int gpt_set_tensor(gpt_ctx* x, int kind, int id, const float* host, int64_t n) {
  if (!x || !host || id < 0 || id >= (int)x->tensors.size()) return fail(GPT_EINVAL, "bad tensor access");
  float* base = kind_ptr(x, kind);
  if (!base) return fail(GPT_EINVAL, "bad tensor kind");
  const TensorDesc& d = x->tensors[id];
  if (n != d.numel()) return fail(GPT_EINVAL, "element count mismatch for " + d.name);
  if (int e = join_side(x)) return e;  // side-stream products read activations and write gradients
  if (kind == GPT_GRAD) {
    // materialise the cleared state before writing part of it
    if (id == T_WTE && x->wte_fresh) {
      HIPCHK(gk::fill_f32(x->G_(T_WTE), d.numel(), 0.f, x->stream));
      x->wte_fresh = false;
    } else if (id != T_WTE && x->others_fresh) {
      const int64_t rest = align_up(x->tensors[T_WTE].numel(), 64);  // everything after wte
      HIPCHK(gk::fill_f32(x->grads + rest, x->P - rest, 0.f, x->stream));
      x->others_fresh = false;
    }
  }
  HIPCHK(hipMemcpyAsync(base + d.off, host, n * 4, hipMemcpyHostToDevice, x->stream));
  if (kind == GPT_PARAM && x->shadow)
    HIPCHK(gk::to_bf16(base + d.off, (uint16_t*)x->shadow + d.off, n, x->stream));
  HIPCHK(hipStreamSynchronize(x->stream));
  return 0;
}

int gpt_get_batch(gpt_ctx* x, int32_t* xh, int32_t* yh, int64_t n) {
  if (!x || !xh || !yh || n != x->N) return fail(GPT_EINVAL, "need B*T ints for x and y");
  HIPCHK(hipMemcpyAsync(xh, x->win, n * 4, hipMemcpyDeviceToHost, x->stream));
  HIPCHK(hipMemcpyAsync(yh, x->win + 1, n * 4, hipMemcpyDeviceToHost, x->stream));
  HIPCHK(hipStreamSynchronize(x->stream));
  return 0;
}

int gpt_get_token_losses(gpt_ctx* x, float* host, int64_t n) {
  if (!x || !host || n != x->N) return fail(GPT_EINVAL, "need B*T floats");
  HIPCHK(hipMemcpyAsync(host, x->tok_loss, n * 4, hipMemcpyDeviceToHost, x->stream));
  HIPCHK(hipStreamSynchronize(x->stream));
  return 0;
}

int gpt_read_losses(gpt_ctx* x, float* host, int max) {
  if (!x || !host || max < 0) return fail(GPT_EINVAL, "bad arguments");
  std::vector<float> all(RING);
  HIPCHK(hipMemcpyAsync(all.data(), x->ring, RING * 4, hipMemcpyDeviceToHost, x->stream));
  float sc[8];
  HIPCHK(hipMemcpyAsync(sc, x->scal, sizeof(sc), hipMemcpyDeviceToHost, x->stream));
  HIPCHK(hipStreamSynchronize(x->stream));
  int k = 0;
  if (x->ring_wr - x->ring_rd > RING) x->ring_rd = x->ring_wr - RING;
  while (x->ring_rd < x->ring_wr && k < max) host[k++] = all[(x->ring_rd++) % RING];
  if (sc[4] != 0.f) {
    HIPCHK(gk::fill_f32(x->scal + 4, 1, 0.f, x->stream));
    HIPCHK(hipStreamSynchronize(x->stream));
    return fail(GPT_ENONFINITE, "a non-finite gradient norm skipped an update");
  }
  return k;
}

int64_t gpt_step_count(const gpt_ctx* xc) {
  gpt_ctx* x = const_cast<gpt_ctx*>(xc);
  if (!x) return fail(GPT_EINVAL, "null context");
  int t = 0;
  if (hipMemcpyAsync(&t, x->step_dev, 4, hipMemcpyDeviceToHost, x->stream) != hipSuccess) return fail(GPT_EHIP, "copy");
  if (hipStreamSynchronize(x->stream) != hipSuccess) return fail(GPT_EHIP, "sync");
  return t;
}

int gpt_set_step_count(gpt_ctx* x, int64_t t) {
  if (!x) return fail(GPT_EINVAL, "null context");
  if (t < 0 || t > 0x7fffffff) return fail(GPT_EINVAL, "step count outside [0, 2^31)");
  if (int e = join_side(x)) return e;  // an update still queued on the side stream reads the counter's step size
  const int v = (int)t;
  HIPCHK(hipMemcpyAsync(x->step_dev, &v, 4, hipMemcpyHostToDevice, x->stream));
  HIPCHK(hipStreamSynchronize(x->stream));
  return 0;
}

int gpt_profile_begin(gpt_ctx* x, const char* cls) {
  if (!x || !cls) return fail(GPT_EINVAL, "null argument");
  x->prof.cls = cls;
  x->prof.used = 0;
  x->prof.flops = x->prof.bytes = 0;
  x->prof.launches = 0;
  return 0;
}

int gpt_profile_end(gpt_ctx* x, double* total_ms, int64_t* launches, double* flops, double* bytes) {
  if (!x) return fail(GPT_EINVAL, "null context");
  HIPCHK(hipStreamSynchronize(x->stream));
  if (x->side) HIPCHK(hipStreamSynchronize(x->side));
  if (x->hside) HIPCHK(hipStreamSynchronize(x->hside));
  double ms = 0;
  for (size_t i = 0; i + 1 < x->prof.used; i += 2) {
    float t = 0;
    HIPCHK(hipEventElapsedTime(&t, x->prof.ev[i], x->prof.ev[i + 1]));
    ms += t;
  }
  if (total_ms) *total_ms = ms;
  if (launches) *launches = x->prof.launches;
  if (flops) *flops = x->prof.flops;
  if (bytes) *bytes = x->prof.bytes;
  x->prof.cls.clear();
  x->prof.used = 0;
  return 0;
}

const char* gpt_last_error(void) { return g_err.c_str(); }

}  // extern "C"
