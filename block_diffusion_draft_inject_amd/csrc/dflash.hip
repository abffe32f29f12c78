// libdflash C ABI: argument validation, workspace layout and launch sequencing.
// Every entry point checks its host-visible arguments before any HIP call, then only enqueues
// kernels on the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <vector>

#include "../../include/dflash.h"
#include "kernels.h"
#include "rowops.h"

using namespace dfl;

static thread_local char g_err[512] = "";

// Scratch of dflash_draft_block_static (the allocation-free draft): one copy per GPU the library
// runs on, alive until the process ends.  Host code uses its device address from
// hipGetSymbolAddress (kept per device in g_scratch), never the array's name.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
static std::atomic<void*> g_scratch[MAX_DEVICES];

static dflash_status fail(dflash_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

#define HIP_TRY(call)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) return fail(DFLASH_E_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

namespace {

constexpr uint32_t HANDLE_MAGIC = 0xDF1A5401u;

size_t esize(const dflash_config* c) { return c->dtype == DFLASH_BF16 ? 2 : 4; }

// Workspace regions (byte offsets), a pure function of (config, max_batch, max_inject_rows).
struct WsLayout {
  size_t h0, h1, act_y, act_o, act_s, qb, hsplit, kb, vb, act_a, act_z, ctx, part, o_part, m_part, l_part, tk_val, tk_id;
  size_t ubar, cbuf, meta_seq, meta_pos, row_off, row_start, row_skip, total, counters, sel_part, sel_cnt;
  size_t bytes;
  size_t part_floats;
  int chunks_max;
};

struct Handle {
  uint32_t magic;
  dflash_config cfg;
  const void* g_embed;
  const void* g_lm;
  const void* g_cnorm;
  const void* g_fc;
  const void* g_fnorm;
  const void* g_A;
  const void* g_B;
  const void* g_WH;
  const unsigned char* lm_fp8;       // E4M3 lm_head codes [V][d] (NULL: the bf16 lm_head)
  const float* lm_fp8_scale;         // [V] per-row power-of-two scales
  const unsigned char* lm_fp4;       // MXFP4 lm_head codes [V][d/2] (NULL: not in use)
  const unsigned char* lm_fp4_scale; // [V][d/32] block scale bytes
  struct QuantMlp {                  // per layer: [gate; up] [2 ffn][d] and down [d][ffn] as E4M3 codes
    const unsigned char *gu, *dn;    // with row scales, or MXFP4 codes (half the bytes) with block
    const float *gu_s, *dn_s;        // scale bytes [rows][cols / 32] (NULL gu: the bf16 matrices)
    const unsigned char *gu_b, *dn_b;
  };
  std::vector<QuantMlp> mlp_q;
  struct QuantAttn {                 // per layer: quantised [wq; wk; wv] (qw + 2 kvw rows) and wo (d rows):
    const unsigned char *qkv, *o;      // codes; E4M3 with row scales, or MXFP4 with block scale bytes
    const float *qkv_s, *o_s;
    const unsigned char *qkv_b, *o_b;
  };
  std::vector<QuantAttn> attn_q;
  const unsigned char *inj_fc8, *inj_kv8;   // injection: fc [d][concat], K/V stack [L (wk, wv)][d] codes
  const float *inj_fc8_s, *inj_kv8_s;       // E4M3 row scales, or
  const unsigned char *inj_fc_b, *inj_kv_b; // MXFP4 block scale bytes
  std::vector<const void*> layers;   // n_layers * DFLASH_LAYER_TENSORS
  // 16-row-blocked copies of the bf16 weight matrices for the MFMA tiles (NULL: row-major only)
  const void* blk_lm = nullptr;
  const void* blk_fc = nullptr;
  std::vector<const void*> blk_layers;   // empty, or n_layers * DFLASH_LAYER_TENSORS
  int max_seqs, max_batch, max_inject_rows;
  char* kv;
  dflash_kv_layout kvl;
  char* ws;
  WsLayout wl;
  // timing
  int t_cap, t_next, t_count;
  std::vector<hipEvent_t> t_ev;
  bool sel_cnt_clear = false;   // the selector's arrival counters have been zeroed on the device
};

bool bf(const dflash_config* c) { return c->dtype == DFLASH_BF16; }
// the pages' per-channel conv: coefficients from a base per channel plus a correction per conv_group channels
bool per_channel_conv(const dflash_config* c) { return c->use_conv && c->conv_group > 0; }

int attn_chunks(const dflash_config* c, int n_seq) {
  const int max_chunks = (c->window + c->block_size + 63) / 64;
  int ch = 512 / (n_seq * c->n_kv_heads);
  if (ch < 1) ch = 1;
  if (ch > max_chunks) ch = max_chunks;
  if (ch > 256) ch = 256;
  return ch;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Largest partial buffer (floats) any GEMM of a draft call with n_seq sequences, or an
// injection pass of `rows` rows, needs.
size_t draft_part_floats(const dflash_config* c, int n_seq) {
  const bool b = bf(c);
  const int M = n_seq * c->block_size, d = c->hidden, qw = c->n_heads * c->head_dim, kvw = c->n_kv_heads * c->head_dim;
  size_t mx = 0;
  auto upd = [&](int mode, int N, int K) {
    GemmPlan pl = gemm_plan(b, mode, M, N, K);
    size_t f = gemm_part_floats(pl, mode, M, N);
    if (f > mx) mx = f;
  };
  upd(GEMM_PARTIAL, qw + 2 * kvw, d);
  upd(GEMM_PARTIAL, d, qw);
  if (b && M <= 64) upd(GEMM_SWIGLU, 2 * c->ffn, d);
  else upd(GEMM_PARTIAL, 2 * c->ffn, d);
  upd(GEMM_PARTIAL, d, c->ffn);
  if (b) {   // an MXFP4 down projection runs on the skinny kernels at any row count
    size_t f = gemm_part_floats(gemm_plan_skinny(GEMM_PARTIAL, M, d, c->ffn), GEMM_PARTIAL, M, d);
    if (f > mx) mx = f;
  }
  if (per_channel_conv(c)) upd(GEMM_PARTIAL, 2 * d / c->conv_group, d);   // conv corrections
  if (!b) {
    size_t f = (size_t)M * c->vocab;   // fp32 path keeps full logits
    if (f > mx) mx = f;
  }
  return mx;
}

size_t inject_part_floats(const dflash_config* c, int rows) {
  const bool b = bf(c);
  const int d = c->hidden, kvw = c->n_kv_heads * c->head_dim;
  GemmPlan p1 = gemm_plan(b, GEMM_PARTIAL, rows, d, c->n_taps * c->target_hidden);
  GemmPlan p2 = gemm_plan(b, GEMM_PARTIAL, rows, c->n_layers * 2 * kvw, d);
  size_t a = gemm_part_floats(p1, GEMM_PARTIAL, rows, d);
  size_t e = gemm_part_floats(p2, GEMM_PARTIAL, rows, c->n_layers * 2 * kvw);
  return a > e ? a : e;
}

// partial top-16 lists per row: the most any top-16 kernel may write (a quantised lm_head can
// run on the skinny kernels instead of the plain plan's)
int topk_groups(const dflash_config* c, int n_seq) {
  const int M = n_seq * c->block_size;
  const int g0 = gemm_plan(true, GEMM_TOPK, M, c->vocab, c->hidden).groups;
  const int g1 = gemm_plan_skinny(GEMM_TOPK, M, c->vocab, c->hidden).groups;
  return g0 > g1 ? g0 : g1;
}

WsLayout ws_layout(const dflash_config* c, int max_batch, int max_inject_rows, int max_seqs) {
  WsLayout L{};
  const size_t es = esize(c);
  const int K = c->block_size, d = c->hidden;
  const size_t M = (size_t)max_batch * K;
  const int qw = c->n_heads * c->head_dim, kvw = c->n_kv_heads * c->head_dim;
  const int G = c->n_heads / c->n_kv_heads, R = G * K;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  L.h0 = take(M * d * 4);
  L.h1 = take(M * d * 4);
  // activations: fp32, or two bf16 planes (hi, lo) -- 4 bytes per element either way
  L.act_y = take(M * d * 4);
  L.act_o = take(M * qw * 4);
  L.act_s = take(M * c->ffn * 4);
  L.qb = take(M * qw * 4);
  L.hsplit = take(M * d * 4);
  L.kb = take(M * kvw * es);
  L.vb = take(M * kvw * es);
  // per-channel conv: the sublayer output a and the normed rows z as GEMM operands
  L.act_a = per_channel_conv(c) ? take(M * d * 4) : 0;
  L.act_z = per_channel_conv(c) ? take(M * d * 4) : 0;
  L.ctx = take((size_t)max_batch * sizeof(SeqCtx));
  size_t pf = 0;
  int chmax = 1;
  size_t attn_f = 0, tk_f = 0;
  for (int n = 1; n <= max_batch; ++n) {
    size_t f = draft_part_floats(c, n);
    if (f > pf) pf = f;
    int ch = attn_chunks(c, n);
    size_t af = (size_t)n * c->n_kv_heads * ch * R;
    if (af > attn_f) attn_f = af;
    if (ch > chmax) chmax = ch;
    if (bf(c)) {
      size_t tf = (size_t)n * K * topk_groups(c, n) * TOPK;
      if (tf > tk_f) tk_f = tf;
    }
  }
  for (int r = 1; r <= max_inject_rows; ++r) {
    size_t f = inject_part_floats(c, r);
    if (f > pf) pf = f;
  }
  L.part_floats = pf;
  L.part = take(pf * 4);
  L.o_part = take(attn_f * c->head_dim * 4);
  L.m_part = take(attn_f * 4);
  L.l_part = take(attn_f * 4);
  L.chunks_max = chmax;
  L.tk_val = take(tk_f * 4);
  L.tk_id = take(tk_f * 4);
  const size_t Ri = (size_t)max_inject_rows;
  L.ubar = take(Ri * c->n_taps * c->target_hidden * 4);
  L.cbuf = take(Ri * d * 4);
  L.meta_seq = take(Ri * 4);
  L.meta_pos = take(Ri * 4);
  L.row_off = take(((size_t)max_seqs + 1) * 4);
  L.row_start = take((size_t)max_seqs * 4);
  L.row_skip = take((size_t)max_seqs * 4);
  L.total = take(4);
  L.counters = take(NCOUNTERS * 4);
  // selector: partial pair scores per (sequence, slot, chunk of 32 ranks) and arrival counters
  L.sel_part = take((size_t)max_batch * (K - 1) * ((c->sel_rank + 31) / 32) * TOPK * TOPK * 4);
  L.sel_cnt = take((size_t)max_batch * 4);
  L.bytes = off;
  return L;
}

dflash_status check_cfg(const dflash_config* c) {
  if (!c) return fail(DFLASH_E_INVALID, "config is NULL");
  if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16) return fail(DFLASH_E_INVALID, "dtype %d", (int)c->dtype);
  if (c->n_layers < 1 || c->n_layers > MAX_LAYERS) return fail(DFLASH_E_UNSUPPORTED, "n_layers must be 1..%d", MAX_LAYERS);
  if (c->hidden < 64 || c->hidden > 4096 || c->hidden % 64) return fail(DFLASH_E_UNSUPPORTED, "hidden must be a multiple of 64 in [64, 4096]");
  if (c->n_heads < 1 || c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads)
    return fail(DFLASH_E_UNSUPPORTED, "n_heads must be a positive multiple of n_kv_heads");
  if (c->head_dim < 2 || c->head_dim > 128 || c->head_dim % 2) return fail(DFLASH_E_UNSUPPORTED, "head_dim must be even and <= 128");
  if (c->block_size < 2 || c->block_size > 32) return fail(DFLASH_E_UNSUPPORTED, "block_size must be 2..32");
  const int R = (c->n_heads / c->n_kv_heads) * c->block_size;
  if (R > 64) return fail(DFLASH_E_UNSUPPORTED, "(n_heads/n_kv_heads)*block_size must be <= 64");
  if (c->topk != 16) return fail(DFLASH_E_UNSUPPORTED, "topk must be 16");
  if (c->sel_rank < 8 || c->sel_rank > 256 || c->sel_rank % 8)
    return fail(DFLASH_E_UNSUPPORTED, "sel_rank must be a multiple of 8 in [8, 256]");
  if (c->window < 1) return fail(DFLASH_E_INVALID, "window must be >= 1");
  if (c->vocab < 16) return fail(DFLASH_E_INVALID, "vocab must be >= 16");
  if (c->mask_id < 0 || c->mask_id >= c->vocab) return fail(DFLASH_E_INVALID, "mask_id outside the vocabulary");
  if (c->n_taps < 1 || c->target_hidden < 1) return fail(DFLASH_E_INVALID, "n_taps and target_hidden must be positive");
  if (c->ffn < 1) return fail(DFLASH_E_INVALID, "ffn must be positive");
  if ((c->n_taps * c->target_hidden) % 8) return fail(DFLASH_E_UNSUPPORTED, "n_taps*target_hidden must be a multiple of 8");
  if (c->n_taps * c->target_hidden > (c->dtype == DFLASH_BF16 ? 65536 : 32768))
    return fail(DFLASH_E_UNSUPPORTED, "n_taps*target_hidden must be <= 65536 (bf16) or 32768 (fp32)");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 1.f)) return fail(DFLASH_E_INVALID, "rms_eps >= 0 and rope_theta > 1 required");
  if (c->conv_group < 0) return fail(DFLASH_E_INVALID, "conv_group must be >= 0");
  if (c->conv_group > 0 && (c->hidden % c->conv_group || c->conv_group % 4))
    return fail(DFLASH_E_UNSUPPORTED, "conv_group must divide hidden and be a multiple of 4");
  if (c->dtype == DFLASH_BF16) {
    if (c->head_dim != 128) return fail(DFLASH_E_UNSUPPORTED, "bf16 attention needs head_dim 128");
    const int qw = c->n_heads * c->head_dim, kvw = c->n_kv_heads * c->head_dim;
    if (c->ffn % 128 || qw % 64 || (c->n_taps * c->target_hidden) % 64)
      return fail(DFLASH_E_UNSUPPORTED, "bf16 GEMMs need ffn a multiple of 128, n_heads*head_dim and the concat width multiples of 64");
    if (qw % kvw) return fail(DFLASH_E_UNSUPPORTED, "n_heads*head_dim must be a multiple of n_kv_heads*head_dim");
    // the O and down projections feed the sublayer epilogue, which sums at most 8 k-splits: the
    // streaming plan reaches 8 splits of 2048 at K = 16384
    if (c->ffn > 16384 || qw > 16384)
      return fail(DFLASH_E_UNSUPPORTED, "bf16 drafters need ffn and n_heads*head_dim <= 16384");
    if ((qw / kvw) + 2 > MAX_SEG || 2 * c->n_layers > MAX_SEG) return fail(DFLASH_E_UNSUPPORTED, "too many weight segments");
  } else {
    if (256 % R || c->head_dim % (256 / R)) return fail(DFLASH_E_UNSUPPORTED, "fp32 attention needs 256 %% R == 0 and head_dim %% (256/R) == 0");
    const int qw = c->n_heads * c->head_dim, kvw = c->n_kv_heads * c->head_dim;
    if ((qw / kvw) + 2 > MAX_SEG || 2 * c->n_layers > MAX_SEG) return fail(DFLASH_E_UNSUPPORTED, "too many weight segments");
  }
  return DFLASH_OK;
}

dflash_kv_layout kv_layout(const dflash_config* c, int max_seqs) {
  dflash_kv_layout k{};
  const size_t one = (size_t)c->n_layers * max_seqs * c->n_kv_heads * c->window * c->head_dim * esize(c);
  k.k_offset = 0;
  k.v_offset = align_up(one);
  k.seq_len_offset = align_up(k.v_offset + one);
  k.seq_base_offset = align_up(k.seq_len_offset + (size_t)max_seqs * 4);
  k.device_error_offset = align_up(k.seq_base_offset + (size_t)max_seqs * 4);
  k.total_bytes = align_up(k.device_error_offset + 4);
  return k;
}

Handle* as_handle(dflash_handle* h) {
  Handle* H = reinterpret_cast<Handle*>(h);
  if (!H || H->magic != HANDLE_MAGIC) return nullptr;
  return H;
}

template <typename P>
P* wsp(Handle* H, size_t off) { return reinterpret_cast<P*>(H->ws + off); }
template <typename P>
P* wsp(char* ws, size_t off) { return reinterpret_cast<P*>(ws + off); }

const void* LW(Handle* H, int l, int t) { return H->layers[(size_t)l * DFLASH_LAYER_TENSORS + t]; }
const void* LWB(Handle* H, int l, int t) {
  return H->blk_layers.empty() ? nullptr : H->blk_layers[(size_t)l * DFLASH_LAYER_TENSORS + t];
}

// Points a GEMM that runs on the bf16 MFMA tiles at the 16-row-blocked weight copies: segment i
// moves from its matrix base[i] to the same byte offset in that matrix's copy blk[i] (a 16-row
// group takes the same bytes in both forms).  Nothing changes unless the plan runs the bf16 tiles,
// the segments hold whole 16-row groups and every segment's matrix has a copy.
void use_blocked(GemmParams& g, const GemmPlan& pl, int nseg, const void* const* base, const void* const* blk) {
  if (pl.kind != 5 || g.row_scale || g.blk_scale || g.seg_rows % 16 || g.ldb % 32) return;
  for (int i = 0; i < nseg; ++i)
    if (!blk[i]) return;
  for (int i = 0; i < nseg; ++i)
    g.seg[i] = reinterpret_cast<const char*>(blk[i]) +
               (reinterpret_cast<const char*>(g.seg[i]) - reinterpret_cast<const char*>(base[i]));
  g.b_blocked = 1;
}

int* seq_len(Handle* H) { return reinterpret_cast<int*>(H->kv + H->kvl.seq_len_offset); }
int* seq_base(Handle* H) { return reinterpret_cast<int*>(H->kv + H->kvl.seq_base_offset); }
int* dev_err(Handle* H) { return reinterpret_cast<int*>(H->kv + H->kvl.device_error_offset); }

GemmParams gemm_base(const void* A, int lda, int M, int N, int K) {
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A = A;
  p.lda = lda;
  p.M = M;
  p.N = N;
  p.K = K;
  p.ldb = K;
  p.block = 1;
  return p;
}

// One draft pass over the workspace at `ws` with regions `W`, whose activation planes hold `Mmax`
// rows.  Host checks of the FP8 row limits come first (before anything is enqueued).
dflash_status draft_impl(Handle* H, char* ws, const WsLayout& W, size_t Mmax, int32_t n_seq, const int32_t* seq_ids,
                         const int32_t* anchor_ids, int32_t* topk_ids, float* topk_logits, float* h_final,
                         float* logits, hipStream_t st) {
  const dflash_config* c = &H->cfg;
  const bool b = bf(c);
  const int K = c->block_size, d = c->hidden, M = n_seq * K;
  // E4M3 and MXFP4 weights: each GEMM takes the plain plan's kernel when that kernel takes the
  // format, else the skinny kernels (gemm_plan_wf: a quantised top-16 GEMM of at most 16 rows that
  // the streaming kernel would take; MXFP4 tiles with more than 2048 k a workgroup).  A skinny
  // top-16 pass keeps one work counter per row tile of 64 rows.
  const int lm_wf = H->lm_fp4 ? 2 : (H->lm_fp8 ? 1 : 0);
  const GemmPlan lm_plan = gemm_plan_wf(b, b ? GEMM_TOPK : GEMM_PARTIAL, M, c->vocab, d, lm_wf);
  if (b && lm_plan.kind == 0 && (int)lm_plan.grid.y > NCOUNTERS)
    return fail(DFLASH_E_UNSUPPORTED, "an MXFP4 lm_head with a hidden size above 2048 runs on the skinny kernels, "
                "which take at most %d draft rows (n_seq * block_size = %d)", NCOUNTERS * 64, M);
  const int qw = c->n_heads * c->head_dim, kvw = c->n_kv_heads * c->head_dim;
  float* part = wsp<float>(ws, W.part);
  SeqCtx* ctx = wsp<SeqCtx>(ws, W.ctx);
  int* counters = wsp<int>(ws, W.counters);
  float* hA = wsp<float>(ws, W.h0);
  float* hB = wsp<float>(ws, W.h1);
  char* act_y = ws + W.act_y;
  char* act_o = ws + W.act_o;
  char* act_s = ws + W.act_s;
  RowArgs ra{};
  ra.K = K;
  ra.d = d;
  ra.mask_id = c->mask_id;
  ra.use_conv = c->use_conv;
  ra.eps = c->rms_eps;
  ra.anchor = anchor_ids;
  ra.vocab = c->vocab;
  ra.dev_err = dev_err(H);
  ra.embed = H->g_embed;
  ra.h_out = hA;
  ra.pre_gain = LW(H, 0, DFLASH_L_ATTN_NORM);
  ra.pre_w = LW(H, 0, DFLASH_L_CONV_ATTN_PRE_W);
  ra.pre_b = LW(H, 0, DFLASH_L_CONV_ATTN_PRE_B);
  ra.y = act_y;
  ra.ldy = d;
  ra.y_plane = Mmax * d;
  ra.plan = PlanArgs{H->max_seqs, c->window, seq_ids, seq_len(H), seq_base(H), ctx, counters};
  // Per-channel conv: each conv takes a correction GEMM (rows x [2 d/G][d]) on its input first.
  // A post-conv runs as: reduce the sublayer's k-split partials into activation planes a, the
  // correction GEMM on a, then the residual + post-conv + RMSNorm kernel, which writes z; a
  // pre-conv as: the correction GEMM on z, then the conv itself, which writes the GEMM input y.
  const bool pc = per_channel_conv(c);
  const int Ncorr = pc ? 2 * d / c->conv_group : 0;
  char* act_a = ws + W.act_a;
  char* act_z = ws + W.act_z;
  auto pc_corr = [&](const char* x, const void* wc, int& splits) -> dflash_status {
    GemmParams gc = gemm_base(x, d, M, Ncorr, d);
    gc.a_plane = Mmax * d;
    gc.seg[0] = wc;
    gc.seg_rows = Ncorr;
    gc.part = part;
    GemmPlan pl = gemm_plan(b, GEMM_PARTIAL, M, Ncorr, d);
    HIP_TRY(gemm_launch(b, pl, GEMM_PARTIAL, gc, st));
    splits = pl.splits;
    return DFLASH_OK;
  };
  auto pc_pre = [&](const void* wc, const void* base) -> dflash_status {
    int sp = 1;
    dflash_status s2 = pc_corr(act_z, wc, sp);
    if (s2 != DFLASH_OK) return s2;
    PcArgs pa{};
    pa.K = K; pa.d = d; pa.G = c->conv_group; pa.splits = sp; pa.part_rows = M; pa.ldo = d;
    pa.plane = Mmax * d;
    pa.x = act_z; pa.part = part; pa.base = base; pa.out = act_y;
    HIP_TRY(launch_conv_apply(b, pa, M, st));
    return DFLASH_OK;
  };
  auto pc_post = [&](int splits, float* h_in, float* h_out, const void* wc, const void* base, const void* gain,
                     bool final) -> dflash_status {
    ReduceArgs rd{M, d, splits, M, Mmax * d, nullptr, 0, part, act_a};
    HIP_TRY(launch_reduce_store(b, rd, st));
    int sp = 1;
    dflash_status s2 = pc_corr(act_a, wc, sp);
    if (s2 != DFLASH_OK) return s2;
    PcArgs pa{};
    pa.K = K; pa.d = d; pa.G = c->conv_group; pa.splits = sp; pa.part_rows = M; pa.ldo = d;
    pa.plane = Mmax * d; pa.eps = c->rms_eps;
    pa.h_in = h_in; pa.h_out = h_out; pa.x = act_a; pa.part = part; pa.base = base; pa.gain = gain;
    pa.final_norm = final ? 1 : 0;
    pa.out = final ? (void*)h_final : (void*)act_z;
    pa.out2 = final ? (void*)(ws + W.hsplit) : nullptr;
    HIP_TRY(launch_post_pre_pc(b, pa, M, st));
    return DFLASH_OK;
  };
  if (pc) {   // h = E[x], z = RMSNorm(h) (the embed kernel without its conv), then the pre-conv
    RowArgs re = ra;
    re.use_conv = 0;
    re.y = act_z;
    HIP_TRY(launch_embed_pre(b, re, M, st));
    dflash_status s2 = pc_pre(LW(H, 0, DFLASH_L_CONV_ATTN_PRE_W), LW(H, 0, DFLASH_L_CONV_ATTN_PRE_B));
    if (s2 != DFLASH_OK) return s2;
  } else {
    HIP_TRY(launch_embed_pre(b, ra, M, st));
  }
  ra.plan = PlanArgs{};
  const int chunks = attn_chunks(c, n_seq);
  for (int l = 0; l < c->n_layers; ++l) {
    // q, k, v = y [W_q; W_k; W_v]^T
    const int G = qw / kvw;
    GemmParams gq = gemm_base(act_y, d, M, qw + 2 * kvw, d);
    gq.a_plane = Mmax * d;
    for (int i = 0; i < G; ++i)
      gq.seg[i] = reinterpret_cast<const char*>(LW(H, l, DFLASH_L_WQ)) + (size_t)i * kvw * d * esize(c);
    gq.seg[G] = LW(H, l, DFLASH_L_WK);
    gq.seg[G + 1] = LW(H, l, DFLASH_L_WV);
    gq.seg_rows = kvw;
    gq.part = part;
    const Handle::QuantAttn* a8 = (size_t)l < H->attn_q.size() && H->attn_q[l].qkv ? &H->attn_q[l] : nullptr;
    const int awf = a8 ? (a8->qkv_b ? 2 : 1) : 0;
    if (a8) {   // one stacked [wq; wk; wv] segment of E4M3 or MXFP4 codes
      gq.seg[0] = a8->qkv;
      gq.seg_rows = qw + 2 * kvw;
      gq.ldb = awf == 2 ? d / 2 : d;
      gq.row_scale = a8->qkv_s;
      gq.blk_scale = a8->qkv_b;
    }
    GemmPlan pq = gemm_plan_wf(b, GEMM_PARTIAL, M, qw + 2 * kvw, d, awf);
    if (!a8) {
      const void *qb[MAX_SEG], *qk[MAX_SEG];
      for (int i = 0; i < G; ++i) { qb[i] = LW(H, l, DFLASH_L_WQ); qk[i] = LWB(H, l, DFLASH_L_WQ); }
      qb[G] = LW(H, l, DFLASH_L_WK); qk[G] = LWB(H, l, DFLASH_L_WK);
      qb[G + 1] = LW(H, l, DFLASH_L_WV); qk[G + 1] = LWB(H, l, DFLASH_L_WV);
      use_blocked(gq, pq, G + 2, qb, qk);
    }
    HIP_TRY(gemm_launch(b, pq, GEMM_PARTIAL, gq, st));
    QkvArgs qa{};
    qa.K = K;
    qa.nh = c->n_heads;
    qa.nkv = c->n_kv_heads;
    qa.dh = c->head_dim;
    qa.N = qw + 2 * kvw;
    qa.splits = pq.splits;
    qa.part_rows = M;
    qa.eps = c->rms_eps;
    qa.log_theta = log((double)c->rope_theta);
    qa.ctx = ctx;
    qa.part = part;
    qa.q_gain = LW(H, l, DFLASH_L_Q_NORM);
    qa.k_gain = LW(H, l, DFLASH_L_K_NORM);
    qa.q = ws + W.qb;
    qa.q_plane = Mmax * qw;
    qa.k = ws + W.kb;
    qa.v = ws + W.vb;
    HIP_TRY(launch_qkv_post(b, qa, M, st));
    AttnArgs aa{};
    aa.K = K;
    aa.nh = c->n_heads;
    aa.nkv = c->n_kv_heads;
    aa.dh = c->head_dim;
    aa.window = c->window;
    aa.max_seqs = H->max_seqs;
    aa.chunks = chunks;
    aa.layer = l;
    aa.scale = 1.0f / sqrtf((float)c->head_dim);
    aa.ctx = ctx;
    aa.q = qa.q;
    aa.kb = qa.k;
    aa.vb = qa.v;
    aa.kcache = H->kv + H->kvl.k_offset;
    aa.vcache = H->kv + H->kvl.v_offset;
    aa.o_part = wsp<float>(ws, W.o_part);
    aa.m_part = wsp<float>(ws, W.m_part);
    aa.l_part = wsp<float>(ws, W.l_part);
    aa.o = act_o;
    aa.q_plane = Mmax * qw;
    aa.o_plane = Mmax * qw;
    HIP_TRY(launch_attention(b, aa, n_seq, st));
    // a = o W_o^T
    GemmParams go = gemm_base(act_o, qw, M, d, qw);
    go.a_plane = Mmax * qw;
    go.seg[0] = LW(H, l, DFLASH_L_WO);
    go.seg_rows = d;
    go.part = part;
    if (a8) {
      go.seg[0] = a8->o;
      go.ldb = awf == 2 ? qw / 2 : qw;
      go.row_scale = a8->o_s;
      go.blk_scale = a8->o_b;
    }
    GemmPlan po = gemm_plan_wf(b, GEMM_PARTIAL, M, d, qw, awf);
    if (!a8) {
      const void *ob = LW(H, l, DFLASH_L_WO), *ok = LWB(H, l, DFLASH_L_WO);
      use_blocked(go, po, 1, &ob, &ok);
    }
    HIP_TRY(gemm_launch(b, po, GEMM_PARTIAL, go, st));
    RowArgs rp = ra;
    rp.h_in = hA;
    rp.h_out = hB;
    rp.part = part;
    rp.splits = po.splits;
    rp.part_rows = M;
    rp.post_w = LW(H, l, DFLASH_L_CONV_ATTN_POST_W);
    rp.post_b = LW(H, l, DFLASH_L_CONV_ATTN_POST_B);
    rp.pre_gain = LW(H, l, DFLASH_L_MLP_NORM);
    rp.pre_w = LW(H, l, DFLASH_L_CONV_MLP_PRE_W);
    rp.pre_b = LW(H, l, DFLASH_L_CONV_MLP_PRE_B);
    rp.final_norm = 0;
    rp.y = act_y;
    rp.ldy = d;
    if (pc) {
      dflash_status s2 = pc_post(po.splits, hA, hB, rp.post_w, rp.post_b, rp.pre_gain, false);
      if (s2 == DFLASH_OK) s2 = pc_pre(rp.pre_w, rp.pre_b);
      if (s2 != DFLASH_OK) return s2;
    } else {
      HIP_TRY(launch_post_pre(b, rp, M, st));
    }
    // s = silu(y W_gate^T) * (y W_up^T)
    GemmParams gg = gemm_base(act_y, d, M, 2 * c->ffn, d);
    gg.a_plane = Mmax * d;
    gg.seg[0] = LW(H, l, DFLASH_L_W_GATE);
    gg.seg[1] = LW(H, l, DFLASH_L_W_UP);
    gg.seg_rows = c->ffn;
    gg.half = c->ffn;
    gg.out = act_s;
    gg.out_plane = Mmax * c->ffn;
    gg.part = part;
    const Handle::QuantMlp* mq = (size_t)l < H->mlp_q.size() && H->mlp_q[l].gu ? &H->mlp_q[l] : nullptr;
    if (mq) {   // one stacked [gate; up] segment of codes (MXFP4: checked up front, the stream kernel)
      gg.seg[0] = mq->gu;
      gg.seg[1] = nullptr;
      gg.seg_rows = 2 * c->ffn;
      gg.ldb = mq->gu_b ? d / 2 : d;
      gg.row_scale = mq->gu_s;
      gg.blk_scale = mq->gu_b;
    }
    const int mwf = mq ? (mq->gu_b ? 2 : 1) : 0;
    if (b && M <= 64) {   // the SwiGLU epilogue inside the GEMM
      GemmPlan pg = gemm_plan_wf(b, GEMM_SWIGLU, M, 2 * c->ffn, d, mwf);
      HIP_TRY(gemm_launch(b, pg, GEMM_SWIGLU, gg, st));
    } else {
      gg.half = 0;
      GemmPlan pg = gemm_plan_wf(b, GEMM_PARTIAL, M, 2 * c->ffn, d, mwf);
      if (!mq) {
        const void* gb[2] = {LW(H, l, DFLASH_L_W_GATE), LW(H, l, DFLASH_L_W_UP)};
        const void* gk[2] = {LWB(H, l, DFLASH_L_W_GATE), LWB(H, l, DFLASH_L_W_UP)};
        use_blocked(gg, pg, 2, gb, gk);
      }
      HIP_TRY(gemm_launch(b, pg, GEMM_PARTIAL, gg, st));
      SwigluArgs sa{M, c->ffn, pg.splits, M, Mmax * c->ffn, part, act_s};
      HIP_TRY(launch_swiglu(b, sa, st));
    }
    // m = s W_down^T
    GemmParams gd = gemm_base(act_s, c->ffn, M, d, c->ffn);
    gd.a_plane = Mmax * c->ffn;
    gd.seg[0] = LW(H, l, DFLASH_L_W_DOWN);
    gd.seg_rows = d;
    gd.part = part;
    if (mq) {
      gd.seg[0] = mq->dn;
      gd.ldb = mq->dn_b ? c->ffn / 2 : c->ffn;
      gd.row_scale = mq->dn_s;
      gd.blk_scale = mq->dn_b;
    }
    GemmPlan pd = gemm_plan_wf(b, GEMM_PARTIAL, M, d, c->ffn, mwf);
    if (!mq) {
      const void *db = LW(H, l, DFLASH_L_W_DOWN), *dk = LWB(H, l, DFLASH_L_W_DOWN);
      use_blocked(gd, pd, 1, &db, &dk);
    }
    HIP_TRY(gemm_launch(b, pd, GEMM_PARTIAL, gd, st));
    RowArgs rm = ra;
    rm.h_in = hB;
    rm.h_out = hA;
    rm.part = part;
    rm.splits = pd.splits;
    rm.part_rows = M;
    rm.post_w = LW(H, l, DFLASH_L_CONV_MLP_POST_W);
    rm.post_b = LW(H, l, DFLASH_L_CONV_MLP_POST_B);
    if (l + 1 < c->n_layers) {
      rm.pre_gain = LW(H, l + 1, DFLASH_L_ATTN_NORM);
      rm.pre_w = LW(H, l + 1, DFLASH_L_CONV_ATTN_PRE_W);
      rm.pre_b = LW(H, l + 1, DFLASH_L_CONV_ATTN_PRE_B);
      rm.final_norm = 0;
      rm.y = act_y;
      rm.ldy = d;
    } else {
      rm.pre_gain = H->g_fnorm;
      rm.final_norm = 1;
      rm.y = h_final;
      rm.y2 = ws + W.hsplit;
      rm.ldy = d;
    }
    if (pc) {
      const bool last = l + 1 == c->n_layers;
      dflash_status s2 = pc_post(pd.splits, hB, hA, rm.post_w, rm.post_b, rm.pre_gain, last);
      if (s2 == DFLASH_OK && !last) s2 = pc_pre(rm.pre_w, rm.pre_b);
      if (s2 != DFLASH_OK) return s2;
    } else {
      HIP_TRY(launch_post_pre(b, rm, M, st));
    }
  }
  // shared lm_head + top-16 per draft slot
  GemmParams gl = gemm_base(b ? (const void*)(ws + W.hsplit) : (const void*)h_final, d, M, c->vocab, d);
  gl.a_plane = Mmax * d;
  gl.seg[0] = H->g_lm;
  gl.seg_rows = c->vocab;
  gl.block = K;
  MergeArgs ma{};
  ma.K = K;
  ma.out_ids = topk_ids;
  ma.out_vals = topk_logits;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (H->t_cap > 0) {
    ev0 = H->t_ev[2 * H->t_next];
    ev1 = H->t_ev[2 * H->t_next + 1];
    H->t_next = (H->t_next + 1) % H->t_cap;
    if (H->t_count < H->t_cap) H->t_count++;
    HIP_TRY(hipEventRecord(ev0, st));
  }
  if (b) {
    gl.tk_val = wsp<float>(ws, W.tk_val);
    gl.tk_id = wsp<int>(ws, W.tk_id);
    gl.logits = logits;
    gl.counter = counters;
    const GemmPlan& pl = lm_plan;
    if (H->lm_fp4) {   // MXFP4 lm_head: the independent-wave kernel (<= 16 rows) or the skinny ones
      gl.seg[0] = H->lm_fp4;
      gl.ldb = d / 2;                 // bytes per weight row
      gl.blk_scale = H->lm_fp4_scale;
    } else if (H->lm_fp8) {   // FP8 lm_head: every top-16 kernel but the batch-1 streaming one
      gl.seg[0] = H->lm_fp8;
      gl.ldb = d;                     // bytes per weight row
      gl.row_scale = H->lm_fp8_scale;
    } else {
      use_blocked(gl, pl, 1, &H->g_lm, &H->blk_lm);
    }
    HIP_TRY(gemm_launch(b, pl, GEMM_TOPK, gl, st));
    if (ev1) HIP_TRY(hipEventRecord(ev1, st));
    ma.ncand = pl.groups * TOPK;
    ma.vals = gl.tk_val;
    ma.ids = gl.tk_id;
  } else {
    gl.part = part;
    GemmPlan pl = gemm_plan(b, GEMM_PARTIAL, M, c->vocab, d);
    HIP_TRY(gemm_launch(b, pl, GEMM_PARTIAL, gl, st));
    if (ev1) HIP_TRY(hipEventRecord(ev1, st));
    ma.ncand = c->vocab;
    ma.vals = part;
    ma.ids = nullptr;
    ma.logits_out = logits;
  }
  ma.counters = counters;
  HIP_TRY(launch_topk_merge(ma, n_seq * (K - 1), st));
  return DFLASH_OK;
}

}  // namespace

extern "C" {

const char* dflash_status_string(dflash_status s) {
  switch (s) {
    case DFLASH_OK: return "ok";
    case DFLASH_E_INVALID: return "invalid argument";
    case DFLASH_E_SHAPE: return "size outside the handle's limits";
    case DFLASH_E_UNSUPPORTED: return "unsupported configuration";
    case DFLASH_E_HIP: return "HIP runtime error";
    case DFLASH_E_STATE: return "invalid handle state";
  }
  return "unknown status";
}

const char* dflash_last_error(void) { return g_err; }

dflash_status dflash_config_check(const dflash_config* cfg) { return check_cfg(cfg); }

size_t dflash_kv_cache_bytes(const dflash_config* cfg, int32_t max_seqs) {
  if (check_cfg(cfg) != DFLASH_OK || max_seqs < 1) return 0;
  return kv_layout(cfg, max_seqs).total_bytes;
}

dflash_status dflash_kv_cache_layout(const dflash_config* cfg, int32_t max_seqs, dflash_kv_layout* out) {
  dflash_status s = check_cfg(cfg);
  if (s != DFLASH_OK) return s;
  if (max_seqs < 1) return fail(DFLASH_E_INVALID, "max_seqs must be >= 1");
  if (!out) return fail(DFLASH_E_INVALID, "out is NULL");
  *out = kv_layout(cfg, max_seqs);
  return DFLASH_OK;
}

size_t dflash_workspace_bytes(const dflash_config* cfg, int32_t max_seqs, int32_t max_batch, int32_t max_inject_rows) {
  if (check_cfg(cfg) != DFLASH_OK || max_seqs < 1 || max_batch < 1 || max_inject_rows < 1) return 0;
  if (max_batch > 4096 || max_seqs > (1 << 20) || max_inject_rows > (1 << 16)) return 0;
  return ws_layout(cfg, max_batch, max_inject_rows, max_seqs).bytes;
}

dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* w, int32_t max_seqs, int32_t max_batch,
                            int32_t max_inject_rows, void* kv_cache, size_t kv_bytes, void* workspace, size_t ws_bytes,
                            dflash_handle** out) {
  dflash_status s = check_cfg(cfg);
  if (s != DFLASH_OK) return s;
  if (!w || !out || !kv_cache || !workspace) return fail(DFLASH_E_INVALID, "NULL weights, output, kv_cache or workspace");
  if (max_seqs < 1 || max_batch < 1 || max_inject_rows < 1) return fail(DFLASH_E_INVALID, "max_seqs, max_batch, max_inject_rows must be >= 1");
  if (max_batch > 4096) return fail(DFLASH_E_UNSUPPORTED, "max_batch must be <= 4096");
  if (max_seqs > 1 << 20) return fail(DFLASH_E_UNSUPPORTED, "max_seqs must be <= 2^20");
  if (max_inject_rows > 1 << 16) return fail(DFLASH_E_UNSUPPORTED, "max_inject_rows must be <= 65536");
  const void* globals[] = {w->embed, w->lm_head, w->concat_norm, w->fc, w->final_norm, w->sel_A, w->sel_B, w->sel_WH};
  for (const void* p : globals)
    if (!p) return fail(DFLASH_E_INVALID, "a global weight pointer is NULL");
  if (!w->layers) return fail(DFLASH_E_INVALID, "layers is NULL");
  for (int i = 0; i < cfg->n_layers * DFLASH_LAYER_TENSORS; ++i)
    if (!w->layers[i]) return fail(DFLASH_E_INVALID, "layer tensor %d of layer %d is NULL", i % DFLASH_LAYER_TENSORS, i / DFLASH_LAYER_TENSORS);
  const dflash_kv_layout kvl = kv_layout(cfg, max_seqs);
  if (kv_bytes < kvl.total_bytes) return fail(DFLASH_E_SHAPE, "kv_cache has %zu bytes, needs %zu", kv_bytes, kvl.total_bytes);
  // the workspace also holds per-sequence injection offsets, sized by max_seqs
  const WsLayout wl = ws_layout(cfg, max_batch, max_inject_rows, max_seqs);
  if (ws_bytes < wl.bytes) return fail(DFLASH_E_SHAPE, "workspace has %zu bytes, needs %zu", ws_bytes, wl.bytes);
  Handle* H = new Handle();
  H->magic = HANDLE_MAGIC;
  H->cfg = *cfg;
  H->g_embed = w->embed;
  H->g_lm = w->lm_head;
  H->g_cnorm = w->concat_norm;
  H->g_fc = w->fc;
  H->g_fnorm = w->final_norm;
  H->g_A = w->sel_A;
  H->g_B = w->sel_B;
  H->g_WH = w->sel_WH;
  H->layers.assign(w->layers, w->layers + (size_t)cfg->n_layers * DFLASH_LAYER_TENSORS);
  H->max_seqs = max_seqs;
  H->max_batch = max_batch;
  H->max_inject_rows = max_inject_rows;
  H->kv = reinterpret_cast<char*>(kv_cache);
  H->kvl = kvl;
  H->ws = reinterpret_cast<char*>(workspace);
  H->wl = wl;
  H->t_cap = H->t_next = H->t_count = 0;
  *out = reinterpret_cast<dflash_handle*>(H);
  return DFLASH_OK;
}

dflash_status dflash_destroy(dflash_handle* h) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  for (hipEvent_t e : H->t_ev) (void)hipEventDestroy(e);
  H->magic = 0;
  delete H;
  return DFLASH_OK;
}

dflash_status dflash_reset_seqs(dflash_handle* h, int32_t n_seq, const int32_t* seq_ids, void* stream) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  if (n_seq < 0 || n_seq > H->max_seqs) return fail(DFLASH_E_SHAPE, "n_seq %d outside [0, max_seqs=%d]", n_seq, H->max_seqs);
  if (n_seq > 0 && !seq_ids) return fail(DFLASH_E_INVALID, "seq_ids is NULL");
  ResetArgs a{n_seq, H->max_seqs, seq_ids, seq_len(H), seq_base(H), dev_err(H)};
  HIP_TRY(launch_reset(a, (hipStream_t)stream));
  return DFLASH_OK;
}

dflash_status dflash_inject_kv(dflash_handle* h, int32_t n_seq, const int32_t* seq_ids, const int32_t* start_pos,
                               const int32_t* n_new, int32_t max_new, const void* target_hidden, void* stream) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  const dflash_config* c = &H->cfg;
  if (n_seq < 0 || n_seq > H->max_seqs) return fail(DFLASH_E_SHAPE, "n_seq %d outside [0, max_seqs=%d]", n_seq, H->max_seqs);
  if (max_new < 0) return fail(DFLASH_E_INVALID, "max_new must be >= 0");
  if (n_seq == 0 || max_new == 0) return DFLASH_OK;
  if (!seq_ids || !n_new || !target_hidden) return fail(DFLASH_E_INVALID, "NULL seq_ids, n_new or target_hidden");
  if ((long long)n_seq * max_new > (1ll << 30)) return fail(DFLASH_E_SHAPE, "n_seq * max_new too large");
  hipStream_t st = (hipStream_t)stream;
  const bool b = bf(c);
  const int d = c->hidden, concat = c->n_taps * c->target_hidden, kvw = c->n_kv_heads * c->head_dim;
  const int Nkv = c->n_layers * 2 * kvw;
  const int Ri = H->max_inject_rows;
  InjectArgs ia{};
  ia.n_seq = n_seq;
  ia.max_new = max_new;
  ia.max_seqs = H->max_seqs;
  ia.concat = concat;
  ia.eps = c->rms_eps;
  ia.seq_ids = seq_ids;
  ia.start_pos = start_pos;
  ia.n_new = n_new;
  ia.seq_len = seq_len(H);
  ia.seq_base = seq_base(H);
  ia.dev_err = dev_err(H);
  ia.row_off = wsp<int>(H, H->wl.row_off);
  ia.row_start = wsp<int>(H, H->wl.row_start);
  ia.row_skip = wsp<int>(H, H->wl.row_skip);
  ia.window = c->window;
  ia.total = wsp<int>(H, H->wl.total);
  ia.states = target_hidden;
  ia.gain = H->g_cnorm;
  ia.ubar = H->ws + H->wl.ubar;
  ia.ubar_plane = (size_t)H->max_inject_rows * concat;
  ia.meta_seq = wsp<int>(H, H->wl.meta_seq);
  ia.meta_pos = wsp<int>(H, H->wl.meta_pos);
  const long long max_rows = (long long)n_seq * max_new;
  HIP_TRY(launch_inject_plan(ia, st));
  float* part = wsp<float>(H, H->wl.part);
  for (long long r0 = 0; r0 < max_rows; r0 += Ri) {
    const int rows = (int)((max_rows - r0) < Ri ? (max_rows - r0) : Ri);
    ia.chunk0 = (int)r0;
    HIP_TRY(launch_concat_norm(b, ia, rows, st));
    // rows valid in this pass = clamp(total - r0, 0, rows): kernels read it from meta/total
    // fc: c = u_bar W_fc^T
    GemmParams g1 = gemm_base(H->ws + H->wl.ubar, concat, rows, d, concat);
    g1.a_plane = ia.ubar_plane;
    g1.m_dev = ia.total;
    g1.m_off = (int)r0;
    g1.seg[0] = H->g_fc;
    g1.seg_rows = d;
    g1.part = part;
    const int iwf = H->inj_fc8 ? (H->inj_fc_b ? 2 : 1) : 0;
    if (H->inj_fc8) {
      g1.seg[0] = H->inj_fc8;
      g1.ldb = iwf == 2 ? concat / 2 : concat;
      g1.row_scale = H->inj_fc8_s;
      g1.blk_scale = H->inj_fc_b;
    }
    GemmPlan p1 = gemm_plan_wf(b, GEMM_PARTIAL, rows, d, concat, iwf);
    if (!H->inj_fc8) use_blocked(g1, p1, 1, &H->g_fc, &H->blk_fc);
    HIP_TRY(gemm_launch(b, p1, GEMM_PARTIAL, g1, st));
    const size_t c_plane = (size_t)H->max_inject_rows * d;
    ReduceArgs ra{rows, d, p1.splits, rows, c_plane, ia.total, (int)r0, part, H->ws + H->wl.cbuf};
    HIP_TRY(launch_reduce_store(b, ra, st));
    // layer-batched K/V projection of every layer
    GemmParams g2 = gemm_base(H->ws + H->wl.cbuf, d, rows, Nkv, d);
    g2.a_plane = c_plane;
    g2.m_dev = ia.total;
    g2.m_off = (int)r0;
    for (int l = 0; l < c->n_layers; ++l) {
      g2.seg[2 * l] = LW(H, l, DFLASH_L_WK);
      g2.seg[2 * l + 1] = LW(H, l, DFLASH_L_WV);
    }
    g2.seg_rows = kvw;
    g2.part = part;
    if (H->inj_kv8) {   // the stacked codes in the same row order: layer l's wk rows, then its wv rows
      g2.seg[0] = H->inj_kv8;
      g2.seg_rows = Nkv;
      g2.ldb = iwf == 2 ? d / 2 : d;
      g2.row_scale = H->inj_kv8_s;
      g2.blk_scale = H->inj_kv_b;
    }
    GemmPlan p2 = gemm_plan_wf(b, GEMM_PARTIAL, rows, Nkv, d, iwf);
    if (!H->inj_kv8) {
      const void *kb[MAX_SEG], *kk[MAX_SEG];
      for (int l = 0; l < c->n_layers; ++l) {
        kb[2 * l] = LW(H, l, DFLASH_L_WK); kk[2 * l] = LWB(H, l, DFLASH_L_WK);
        kb[2 * l + 1] = LW(H, l, DFLASH_L_WV); kk[2 * l + 1] = LWB(H, l, DFLASH_L_WV);
      }
      use_blocked(g2, p2, 2 * c->n_layers, kb, kk);
    }
    HIP_TRY(gemm_launch(b, p2, GEMM_PARTIAL, g2, st));
    KvPostArgs ka{};
    ka.N = Nkv;
    ka.splits = p2.splits;
    ka.part_rows = rows;
    ka.nkv = c->n_kv_heads;
    ka.dh = c->head_dim;
    ka.window = c->window;
    ka.max_seqs = H->max_seqs;
    ka.eps = c->rms_eps;
    ka.log_theta = log((double)c->rope_theta);
    ka.part = part;
    ka.meta_seq = ia.meta_seq;
    ka.meta_pos = ia.meta_pos;
    for (int l = 0; l < c->n_layers; ++l) ka.k_gain[l] = LW(H, l, DFLASH_L_K_NORM);
    ka.kcache = H->kv + H->kvl.k_offset;
    ka.vcache = H->kv + H->kvl.v_offset;
    HIP_TRY(launch_kv_post(b, ka, rows, c->n_layers * 2 * c->n_kv_heads, st));
  }
  return DFLASH_OK;
}

dflash_status dflash_draft_block(dflash_handle* h, int32_t n_seq, const int32_t* seq_ids, const int32_t* anchor_ids,
                                 int32_t* topk_ids, float* topk_logits, float* h_final, float* logits, void* stream) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  const dflash_config* c = &H->cfg;
  if (n_seq < 1 || n_seq > H->max_batch) return fail(DFLASH_E_SHAPE, "n_seq %d outside [1, max_batch=%d]", n_seq, H->max_batch);
  if (!seq_ids || !anchor_ids || !topk_ids || !topk_logits || !h_final)
    return fail(DFLASH_E_INVALID, "NULL seq_ids, anchor_ids, topk_ids, topk_logits or h_final");
  hipStream_t st = (hipStream_t)stream;
  return draft_impl(H, H->ws, H->wl, (size_t)H->max_batch * c->block_size, n_seq, seq_ids, anchor_ids, topk_ids,
                    topk_logits, h_final, logits, st);
}

dflash_status dflash_draft_block_static(dflash_handle* h, int32_t n_seq, const int32_t* seq_ids, const int32_t* anchor_ids,
                                        int32_t* topk_ids, float* topk_logits, float* h_final, float* logits,
                                        void* stream) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  const dflash_config* c = &H->cfg;
  if (n_seq < 1 || n_seq > 4096) return fail(DFLASH_E_SHAPE, "n_seq %d outside [1, 4096]", n_seq);
  if (!seq_ids || !anchor_ids || !topk_ids || !topk_logits || !h_final)
    return fail(DFLASH_E_INVALID, "NULL seq_ids, anchor_ids, topk_ids, topk_logits or h_final");
  // the draft's regions laid out for exactly n_seq sequences (injection regions at their minimum)
  const WsLayout wl = ws_layout(c, n_seq, 1, 1);
  if (wl.bytes > STATIC_SCRATCH_BYTES)
    return fail(DFLASH_E_SHAPE, "a draft of %d sequences needs %zu bytes of scratch; the static scratch holds %zu",
                n_seq, wl.bytes, STATIC_SCRATCH_BYTES);
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(DFLASH_E_UNSUPPORTED, "device %d: at most %d devices", dev, MAX_DEVICES);
  void* base = g_scratch[dev].load(std::memory_order_acquire);
  if (!base) {   // first call on this device: the array's address there (two racing first calls agree)
    HIP_TRY(hipGetSymbolAddress(&base, HIP_SYMBOL(scratch)));
    g_scratch[dev].store(base, std::memory_order_release);
  }
  return draft_impl(H, reinterpret_cast<char*>(base), wl, (size_t)n_seq * c->block_size, n_seq, seq_ids, anchor_ids,
                    topk_ids, topk_logits, h_final, logits, (hipStream_t)stream);
}

// The selector's workspace; the first selector call of a handle zeroes its arrival counters
// (a fill kernel on the call's stream; afterwards every launch leaves them at zero).
static hipError_t select_prepare(Handle* H, SelectArgs& sa, hipStream_t st) {
  sa.spart = wsp<float>(H->ws, H->wl.sel_part);
  sa.sel_cnt = wsp<unsigned>(H->ws, H->wl.sel_cnt);
  if (!H->sel_cnt_clear) {
    const hipError_t e = launch_fill_u32(sa.sel_cnt, H->max_batch, 0u, st);
    if (e != hipSuccess) return e;
    H->sel_cnt_clear = true;
  }
  return hipSuccess;
}

dflash_status dflash_select_path(dflash_handle* h, int32_t n_seq, const int32_t* anchor_ids, const int32_t* topk_ids,
                                 const float* topk_logits, const float* h_final, dflash_select_mode mode,
                                 int32_t* path_ids, float* path_score, float* margin, void* stream) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  const dflash_config* c = &H->cfg;
  if (n_seq < 1 || n_seq > H->max_batch) return fail(DFLASH_E_SHAPE, "n_seq %d outside [1, max_batch=%d]", n_seq, H->max_batch);
  if (mode != DFLASH_SELECT_VITERBI && mode != DFLASH_SELECT_GREEDY) return fail(DFLASH_E_INVALID, "mode %d", (int)mode);
  if (!anchor_ids || !topk_ids || !topk_logits || !h_final || !path_ids)
    return fail(DFLASH_E_INVALID, "NULL anchor_ids, topk_ids, topk_logits, h_final or path_ids");
  SelectArgs sa{c->block_size, c->hidden, c->sel_rank, (int)mode, c->vocab, dev_err(H), anchor_ids, topk_ids,
                topk_logits, h_final, H->g_A, H->g_B, H->g_WH, path_ids, path_score, margin,
                1.0f, 1.0f, nullptr, nullptr, nullptr};
  HIP_TRY(select_prepare(H, sa, (hipStream_t)stream));
  HIP_TRY(launch_select(bf(c), sa, n_seq, (hipStream_t)stream));
  return DFLASH_OK;
}

dflash_status dflash_select_sample(dflash_handle* h, int32_t n_seq, const int32_t* anchor_ids, const int32_t* topk_ids,
                                   const float* topk_logits, const float* h_final, float temperature,
                                   float top_p, const float* uniforms, int32_t* path_ids, float* q_path,
                                   float* q_cand, void* stream) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  const dflash_config* c = &H->cfg;
  if (n_seq < 1 || n_seq > H->max_batch) return fail(DFLASH_E_SHAPE, "n_seq %d outside [1, max_batch=%d]", n_seq, H->max_batch);
  if (!(temperature >= 1e-6f && temperature <= 1e6f)) return fail(DFLASH_E_INVALID, "temperature must be in [1e-6, 1e6]");
  if (!(top_p > 0.f && top_p <= 1.f)) return fail(DFLASH_E_INVALID, "top_p must be in (0, 1]");
  if (!anchor_ids || !topk_ids || !topk_logits || !h_final || !uniforms || !path_ids || !q_path)
    return fail(DFLASH_E_INVALID, "NULL anchor_ids, topk_ids, topk_logits, h_final, uniforms, path_ids or q_path");
  SelectArgs sa{c->block_size, c->hidden, c->sel_rank, 2, c->vocab, dev_err(H), anchor_ids, topk_ids,
                topk_logits, h_final, H->g_A, H->g_B, H->g_WH, path_ids, nullptr, nullptr,
                1.0f / temperature, top_p, uniforms, q_path, q_cand};
  HIP_TRY(select_prepare(H, sa, (hipStream_t)stream));
  HIP_TRY(launch_select(bf(c), sa, n_seq, (hipStream_t)stream));
  return DFLASH_OK;
}

dflash_status dflash_verify_rejection(int32_t n_seq, int32_t block_size, int32_t vocab, const int32_t* draft_ids,
                                      const float* q_path, const int32_t* topk_ids, const float* q_cand,
                                      const float* target_probs, const float* u_accept, const float* u_resample,
                                      int32_t* n_accepted, int32_t* n_commit, int32_t* committed, int32_t* next_anchor,
                                      void* stream) {
  if (n_seq < 0) return fail(DFLASH_E_INVALID, "n_seq must be >= 0");
  if (block_size < 2 || block_size > 64) return fail(DFLASH_E_INVALID, "block_size must be in [2, 64]");
  if (vocab < 2) return fail(DFLASH_E_INVALID, "vocab must be >= 2");
  if (n_seq == 0) return DFLASH_OK;
  if (!draft_ids || !q_path || !topk_ids || !q_cand || !target_probs || !u_accept || !u_resample || !n_accepted ||
      !committed || !next_anchor)
    return fail(DFLASH_E_INVALID, "NULL input or output pointer");
  RejectArgs ra{n_seq, block_size, vocab, draft_ids, q_path, topk_ids, q_cand, target_probs, u_accept, u_resample,
                n_accepted, n_commit, committed, next_anchor};
  HIP_TRY(launch_verify_rejection(ra, (hipStream_t)stream));
  return DFLASH_OK;
}

dflash_status dflash_verify_greedy(int32_t n_seq, int32_t block_size, const int32_t* draft_ids, const int32_t* target_argmax,
                                   int32_t* n_accepted, int32_t* n_commit, int32_t* committed, int32_t* next_anchor,
                                   void* stream) {
  if (n_seq < 0) return fail(DFLASH_E_INVALID, "n_seq must be >= 0");
  if (block_size < 2) return fail(DFLASH_E_INVALID, "block_size must be >= 2");
  if (n_seq == 0) return DFLASH_OK;
  if (!draft_ids || !target_argmax || !n_accepted || !committed || !next_anchor)
    return fail(DFLASH_E_INVALID, "NULL draft_ids, target_argmax, n_accepted, committed or next_anchor");
  VerifyArgs va{n_seq, block_size, draft_ids, target_argmax, n_accepted, n_commit, committed, next_anchor};
  HIP_TRY(launch_verify(va, (hipStream_t)stream));
  return DFLASH_OK;
}

dflash_status dflash_quantize_fp8_rows(const void* src, int32_t rows, int32_t cols, uint8_t* codes, float* row_scales,
                                      void* stream) {
  if (rows < 0 || cols <= 0 || cols % 8) return fail(DFLASH_E_SHAPE, "rows must be >= 0 and cols a positive multiple of 8");
  if (rows > 0 && (!src || !codes || !row_scales)) return fail(DFLASH_E_INVALID, "NULL src, codes or row_scales");
  HIP_TRY(launch_quantize_fp8_rows(src, rows, cols, codes, row_scales, (hipStream_t)stream));
  return DFLASH_OK;
}

dflash_status dflash_block_weights(const void* src, int64_t rows, int64_t cols, void* dst, void* stream) {
  if (rows <= 0 || cols <= 0 || rows % 16 || cols % 32)
    return fail(DFLASH_E_SHAPE, "rows must be a positive multiple of 16 and cols of 32");
  if (!src || !dst) return fail(DFLASH_E_INVALID, "NULL src or dst");
  if (src == dst) return fail(DFLASH_E_INVALID, "src and dst must not be the same buffer");
  HIP_TRY(launch_block_weights(src, (long)rows, (long)cols, dst, (hipStream_t)stream));
  return DFLASH_OK;
}

dflash_status dflash_set_blocked_weights(dflash_handle* h, const dflash_weights* blocked) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  const dflash_config* c = &H->cfg;
  if (!blocked) {
    H->blk_lm = H->blk_fc = nullptr;
    H->blk_layers.clear();
    return DFLASH_OK;
  }
  if (!bf(c)) return fail(DFLASH_E_UNSUPPORTED, "blocked weights are for bf16 drafters");
  const int d = c->hidden, qw = c->n_heads * c->head_dim, kvw = c->n_kv_heads * c->head_dim;
  const int concat = c->n_taps * c->target_hidden;
  // (rows, cols) of each matrix that may come blocked: rows a multiple of 16, cols of 32
  auto shape_ok = [](const void* p, long rows, long cols) { return !p || (rows % 16 == 0 && cols % 32 == 0); };
  if (!shape_ok(blocked->lm_head, c->vocab, d)) return fail(DFLASH_E_SHAPE, "a blocked lm_head needs vocab % 16 == 0");
  if (!shape_ok(blocked->fc, d, concat)) return fail(DFLASH_E_SHAPE, "a blocked fc needs n_taps*target_hidden % 32 == 0");
  std::vector<const void*> lay;
  if (blocked->layers) {
    lay.assign(blocked->layers, blocked->layers + (size_t)c->n_layers * DFLASH_LAYER_TENSORS);
    for (int l = 0; l < c->n_layers; ++l) {
      const void* const* t = &lay[(size_t)l * DFLASH_LAYER_TENSORS];
      if (!shape_ok(t[DFLASH_L_WQ], qw, d) || !shape_ok(t[DFLASH_L_WK], kvw, d) || !shape_ok(t[DFLASH_L_WV], kvw, d) ||
          !shape_ok(t[DFLASH_L_WO], d, qw) || !shape_ok(t[DFLASH_L_W_GATE], c->ffn, d) ||
          !shape_ok(t[DFLASH_L_W_UP], c->ffn, d) || !shape_ok(t[DFLASH_L_W_DOWN], d, c->ffn))
        return fail(DFLASH_E_SHAPE, "a blocked layer matrix needs rows % 16 == 0 and cols % 32 == 0");
    }
  }
  H->blk_lm = blocked->lm_head;
  H->blk_fc = blocked->fc;
  H->blk_layers.swap(lay);
  return DFLASH_OK;
}

dflash_status dflash_set_lm_head_fp8(dflash_handle* h, const uint8_t* codes, const float* row_scales) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  if (!codes != !row_scales) return fail(DFLASH_E_INVALID, "codes and row_scales must both be set or both be NULL");
  if (codes && !bf(&H->cfg)) return fail(DFLASH_E_UNSUPPORTED, "the FP8 lm_head is for bf16 drafters");
  H->lm_fp8 = codes;
  H->lm_fp8_scale = row_scales;
  if (codes) H->lm_fp4 = H->lm_fp4_scale = nullptr;
  return DFLASH_OK;
}

dflash_status dflash_quantize_mxfp4_rows(const void* src, int32_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                                         void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32) return fail(DFLASH_E_INVALID, "rows >= 0 and cols a positive multiple of 32 required");
  if (rows > 0 && (!src || !codes || !scales)) return fail(DFLASH_E_INVALID, "NULL src, codes or scales");
  HIP_TRY(launch_quantize_mxfp4_rows(src, rows, cols, codes, scales, (hipStream_t)stream));
  return DFLASH_OK;
}

dflash_status dflash_set_lm_head_mxfp4(dflash_handle* h, const uint8_t* codes, const uint8_t* scales) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  if (!codes != !scales) return fail(DFLASH_E_INVALID, "codes and scales must both be set or both be NULL");
  if (codes && !bf(&H->cfg)) return fail(DFLASH_E_UNSUPPORTED, "the MXFP4 lm_head is for bf16 drafters");
  H->lm_fp4 = codes;
  H->lm_fp4_scale = scales;
  if (codes) H->lm_fp8 = nullptr, H->lm_fp8_scale = nullptr;
  return DFLASH_OK;
}

dflash_status dflash_set_mlp_fp8(dflash_handle* h, int32_t layer, const uint8_t* gate_up_codes,
                                const float* gate_up_scales, const uint8_t* down_codes, const float* down_scales) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  if (layer < 0 || layer >= H->cfg.n_layers) return fail(DFLASH_E_INVALID, "layer %d outside [0, n_layers)", layer);
  const int set = !!gate_up_codes + !!gate_up_scales + !!down_codes + !!down_scales;
  if (set != 0 && set != 4) return fail(DFLASH_E_INVALID, "all four pointers set, or all NULL");
  if (set && !bf(&H->cfg)) return fail(DFLASH_E_UNSUPPORTED, "FP8 weights are for bf16 drafters");
  if (H->mlp_q.size() < (size_t)H->cfg.n_layers) H->mlp_q.resize(H->cfg.n_layers, Handle::QuantMlp{});
  H->mlp_q[layer] = Handle::QuantMlp{gate_up_codes, down_codes, gate_up_scales, down_scales, nullptr, nullptr};
  return DFLASH_OK;
}

dflash_status dflash_set_mlp_mxfp4(dflash_handle* h, int32_t layer, const uint8_t* gate_up_codes,
                                   const uint8_t* gate_up_scales, const uint8_t* down_codes,
                                   const uint8_t* down_scales) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  if (layer < 0 || layer >= H->cfg.n_layers) return fail(DFLASH_E_INVALID, "layer %d outside [0, n_layers)", layer);
  const int set = !!gate_up_codes + !!gate_up_scales + !!down_codes + !!down_scales;
  if (set != 0 && set != 4) return fail(DFLASH_E_INVALID, "all four pointers set, or all NULL");
  if (set && !bf(&H->cfg)) return fail(DFLASH_E_UNSUPPORTED, "MXFP4 weights are for bf16 drafters");
  if (set && (H->cfg.hidden % 128 || H->cfg.ffn % 128))
    return fail(DFLASH_E_UNSUPPORTED, "MXFP4 MLP weights need hidden and ffn sizes that are multiples of 128");
  if (H->mlp_q.size() < (size_t)H->cfg.n_layers) H->mlp_q.resize(H->cfg.n_layers, Handle::QuantMlp{});
  H->mlp_q[layer] = Handle::QuantMlp{gate_up_codes, down_codes, nullptr, nullptr, gate_up_scales, down_scales};
  return DFLASH_OK;
}

dflash_status dflash_set_attn_fp8(dflash_handle* h, int32_t layer, const uint8_t* qkv_codes, const float* qkv_scales,
                                 const uint8_t* o_codes, const float* o_scales) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  if (layer < 0 || layer >= H->cfg.n_layers) return fail(DFLASH_E_INVALID, "layer %d outside [0, n_layers)", layer);
  const int set = !!qkv_codes + !!qkv_scales + !!o_codes + !!o_scales;
  if (set != 0 && set != 4) return fail(DFLASH_E_INVALID, "all four pointers set, or all NULL");
  if (set && !bf(&H->cfg)) return fail(DFLASH_E_UNSUPPORTED, "FP8 weights are for bf16 drafters");
  if (H->attn_q.size() < (size_t)H->cfg.n_layers) H->attn_q.resize(H->cfg.n_layers, Handle::QuantAttn{});
  H->attn_q[layer] = Handle::QuantAttn{qkv_codes, o_codes, qkv_scales, o_scales, nullptr, nullptr};
  return DFLASH_OK;
}

dflash_status dflash_set_attn_mxfp4(dflash_handle* h, int32_t layer, const uint8_t* qkv_codes, const uint8_t* qkv_scales,
                                    const uint8_t* o_codes, const uint8_t* o_scales) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  if (layer < 0 || layer >= H->cfg.n_layers) return fail(DFLASH_E_INVALID, "layer %d outside [0, n_layers)", layer);
  const int set = !!qkv_codes + !!qkv_scales + !!o_codes + !!o_scales;
  if (set != 0 && set != 4) return fail(DFLASH_E_INVALID, "all four pointers set, or all NULL");
  if (set && !bf(&H->cfg)) return fail(DFLASH_E_UNSUPPORTED, "MXFP4 weights are for bf16 drafters");
  if (set && (H->cfg.hidden % 128 || (H->cfg.n_heads * H->cfg.head_dim) % 128))
    return fail(DFLASH_E_UNSUPPORTED, "MXFP4 attention weights need hidden and n_heads*head_dim multiples of 128");
  if (H->attn_q.size() < (size_t)H->cfg.n_layers) H->attn_q.resize(H->cfg.n_layers, Handle::QuantAttn{});
  H->attn_q[layer] = Handle::QuantAttn{qkv_codes, o_codes, nullptr, nullptr, qkv_scales, o_scales};
  return DFLASH_OK;
}

dflash_status dflash_set_inject_fp8(dflash_handle* h, const uint8_t* fc_codes, const float* fc_scales,
                                   const uint8_t* kv_codes, const float* kv_scales) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  const int set = !!fc_codes + !!fc_scales + !!kv_codes + !!kv_scales;
  if (set != 0 && set != 4) return fail(DFLASH_E_INVALID, "all four pointers set, or all NULL");
  if (set && !bf(&H->cfg)) return fail(DFLASH_E_UNSUPPORTED, "FP8 weights are for bf16 drafters");
  H->inj_fc8 = fc_codes;
  H->inj_fc8_s = fc_scales;
  H->inj_kv8 = kv_codes;
  H->inj_kv8_s = kv_scales;
  H->inj_fc_b = H->inj_kv_b = nullptr;
  return DFLASH_OK;
}

dflash_status dflash_set_inject_mxfp4(dflash_handle* h, const uint8_t* fc_codes, const uint8_t* fc_scales,
                                      const uint8_t* kv_codes, const uint8_t* kv_scales) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  const int set = !!fc_codes + !!fc_scales + !!kv_codes + !!kv_scales;
  if (set != 0 && set != 4) return fail(DFLASH_E_INVALID, "all four pointers set, or all NULL");
  if (set && !bf(&H->cfg)) return fail(DFLASH_E_UNSUPPORTED, "MXFP4 weights are for bf16 drafters");
  if (set && (H->cfg.hidden % 128 || (H->cfg.n_taps * H->cfg.target_hidden) % 128))
    return fail(DFLASH_E_UNSUPPORTED, "MXFP4 injection weights need hidden and n_taps*target_hidden multiples of 128");
  H->inj_fc8 = fc_codes;
  H->inj_kv8 = kv_codes;
  H->inj_fc8_s = H->inj_kv8_s = nullptr;
  H->inj_fc_b = fc_scales;
  H->inj_kv_b = kv_scales;
  return DFLASH_OK;
}

dflash_status dflash_synth_target_argmax(int32_t n_seq, int32_t block_size, int32_t vocab, const int32_t* draft_ids,
                                         float match_prob, uint64_t seed, int64_t* counter, int32_t* target_argmax,
                                         void* stream) {
  if (n_seq < 0 || n_seq > 1024) return fail(DFLASH_E_SHAPE, "n_seq must be 0..1024");
  if (block_size < 2 || vocab < 2) return fail(DFLASH_E_INVALID, "block_size and vocab must be >= 2");
  if (!((match_prob >= 0.f && match_prob <= 1.f) || match_prob == -1.f))
    return fail(DFLASH_E_INVALID, "match_prob must be in [0, 1], or -1");
  if (n_seq == 0) return DFLASH_OK;
  if (!draft_ids || !counter || !target_argmax) return fail(DFLASH_E_INVALID, "NULL draft_ids, counter or target_argmax");
  SynthArgs a{n_seq, block_size, vocab, match_prob, (unsigned long long)seed, reinterpret_cast<long long*>(counter),
              draft_ids, target_argmax};
  HIP_TRY(launch_synth(a, (hipStream_t)stream));
  return DFLASH_OK;
}

dflash_status dflash_timing_enable(dflash_handle* h, int32_t capacity) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  if (capacity < 0 || capacity > 100000) return fail(DFLASH_E_INVALID, "capacity must be 0..100000");
  for (hipEvent_t e : H->t_ev) (void)hipEventDestroy(e);
  H->t_ev.clear();
  H->t_cap = H->t_next = H->t_count = 0;
  if (capacity == 0) return DFLASH_OK;
  H->t_ev.resize(2 * (size_t)capacity, nullptr);
  for (auto& e : H->t_ev) HIP_TRY(hipEventCreate(&e));
  H->t_cap = capacity;
  return DFLASH_OK;
}

dflash_status dflash_timing_read(dflash_handle* h, double* total_ms, int32_t* count) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  if (!total_ms || !count) return fail(DFLASH_E_INVALID, "NULL output");
  double tot = 0.0;
  const int n = H->t_count;
  for (int i = 0; i < n; ++i) {
    HIP_TRY(hipEventSynchronize(H->t_ev[2 * i + 1]));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, H->t_ev[2 * i], H->t_ev[2 * i + 1]));
    tot += ms;
  }
  *total_ms = tot;
  *count = n;
  return DFLASH_OK;
}

dflash_status dflash_get_device_error(dflash_handle* h, int32_t* code) {
  Handle* H = as_handle(h);
  if (!H) return fail(DFLASH_E_STATE, "not a live handle");
  if (!code) return fail(DFLASH_E_INVALID, "code is NULL");
  HIP_TRY(hipDeviceSynchronize());
  HIP_TRY(hipMemcpy(code, dev_err(H), 4, hipMemcpyDeviceToHost));
  return DFLASH_OK;
}

}  // extern "C"
