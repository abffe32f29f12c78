/*
 * libdflash -- the DFlash drafter's single-pass block draft on one AMD Instinct MI355X (gfx950).
 *
 * A cycle of block-diffusion speculative decoding, as the pages state it ("Architecture",
 * kb.ekarisky.com, DFlash 2: sequence diagram "One Cycle, Step by Step" and flowchart
 * "Draft-Verify Cycle"):
 *   (1) inject target hidden states into the drafter's KV cache       -> dflash_inject_kv
 *   (2) predict the whole block in one pass, top-16 per position      -> dflash_draft_block
 *   (3) candidate lists + last verified token -> one coherent path    -> dflash_select_path
 *   (4) accept the longest valid prefix plus one bonus token          -> dflash_verify_greedy
 * The target model's own verify pass is not part of this library: step (4) takes the target's
 * argmax tokens as input.
 *
 * Conventions for every call below
 *   - Pointers are DEVICE pointers unless marked (host).  Arrays are dense, row-major.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls only
 *     enqueue work; results are valid once the stream has been synchronised.  No call
 *     synchronises, allocates or frees device memory; all scratch lives in the caller's
 *     workspace buffer.  Calls on one handle must be serialised by the caller (one stream,
 *     or explicit ordering); concurrent calls that share a handle race on its workspace.
 *   - Ids are int32.  Logits, scores, margins and hidden states are fp32.  Weights, target
 *     states and the KV cache use the handle's dtype (fp32 or bf16).  Activations are carried
 *     in fp32; for bf16 drafters every activation that feeds a bf16 matrix core operation is
 *     split into two bf16 terms (hi + lo, about 16 mantissa bits), so the only bf16 rounding
 *     of computed values is the K/V written to (or read as) the cache.
 *   - Linear weights are [out][in] (one output row per line).
 *   - Errors: every check that the host can make (null pointers, sizes, counts above the
 *     handle's maxima, unsupported shapes) returns a negative status BEFORE anything is
 *     enqueued; dflash_last_error() then gives a message.  Nothing throws across this ABI.
 *     Problems only the device can see (a sequence id or n_new out of range) are clamped
 *     or skipped and recorded in a device error word (dflash_get_device_error).
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define DFLASH_API __attribute__((visibility("default")))
#else
#define DFLASH_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH_OK = 0,
  DFLASH_E_INVALID = -1,     /* null pointer, bad enum, inconsistent argument            */
  DFLASH_E_SHAPE = -2,       /* a size outside what the handle was created for           */
  DFLASH_E_UNSUPPORTED = -3, /* a configuration the kernels do not implement              */
  DFLASH_E_HIP = -4,         /* a HIP runtime call failed (message has the HIP error)     */
  DFLASH_E_STATE = -5        /* handle misuse (e.g. destroyed twice)                      */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

typedef enum { DFLASH_SELECT_VITERBI = 0, DFLASH_SELECT_GREEDY = 1 } dflash_select_mode;

/* Drafter shape (host struct, copied by dflash_create).
 *  - hidden d, n_heads x head_dim query heads, n_kv_heads KV heads (grouped-query attention:
 *    query head i reads KV head floor(i * n_kv_heads / n_heads)), ffn = SwiGLU width, vocab V.
 *  - n_taps tapped target layers of width target_hidden each; their concatenation
 *    (n_taps * target_hidden wide) is RMS-normalised and projected to d ("Z Lab releases
 *    DFlash 2 ...", section "Persistent Conditioning Through Target KV Injection").
 *  - block_size K: slot 0 holds the anchor (last verified token), slots 1..K-1 hold MASK
 *    ("Architecture", Component Breakdown row "Block attention mask").  K-1 drafts per block.
 *  - window W: the block sees the last min(L, W) injected positions ("Architecture",
 *    Component Breakdown row "DFlash drafter backbone": sliding window 1024).
 *  - topk must be 16 ("Architecture", flowchart "Drafter": top-16 candidates per position).
 *  - sel_rank r: width of the selector's A/B token tables and context gate.
 *  - use_conv: 1 = two-tap dynamic convolution around every attention and MLP sublayer
 *    ("Architecture", section "Problem 2 -- Suffix decay is local").
 *  - rope_theta: rotary base for the rotate-half RoPE applied after the per-head q/k norm.
 *  - conv_group: form of the conv coefficients.  0: one scalar per tap and position,
 *    k_t = sigmoid(W_c x_t + b_c) in R^2 (the conv weight of a sublayer is [2][d], its bias [2]).
 *    G > 0: per-channel (depthwise) coefficients ("Architecture", section "Problem 2": a learned
 *    base kernel per channel plus a small correction from the current hidden state shared per
 *    16 channels), k_tj[c] = sigmoid(base_j[c] + (W_c x_t)[j d/G + c/G]): the conv weight is the
 *    correction matrix [2 d/G][d] and the "bias" the base kernel [2][d].  G must divide hidden
 *    and be a multiple of 4; G = hidden with a constant base row is the scalar form. */
typedef struct {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab;
  int32_t n_taps, target_hidden;
  int32_t block_size, window, topk, sel_rank, mask_id, use_conv;
  float rms_eps, rope_theta;
  dflash_dtype dtype;
  int32_t conv_group;
} dflash_config;

/* Per-layer weight tensors, in this order, in dflash_weights.layers[l * DFLASH_LAYER_TENSORS + i]. */
typedef enum {
  DFLASH_L_ATTN_NORM = 0,   /* [d]                 pre-attention RMSNorm gain               */
  DFLASH_L_WQ,              /* [n_heads*head_dim][d]                                          */
  DFLASH_L_WK,              /* [n_kv*head_dim][d]  also projects the injected context        */
  DFLASH_L_WV,              /* [n_kv*head_dim][d]  also projects the injected context        */
  DFLASH_L_Q_NORM,          /* [head_dim]          per-head q RMSNorm gain                   */
  DFLASH_L_K_NORM,          /* [head_dim]          per-head k RMSNorm gain (block and ctx)   */
  DFLASH_L_WO,              /* [d][n_heads*head_dim]                                          */
  DFLASH_L_MLP_NORM,        /* [d]                                                            */
  DFLASH_L_W_GATE,          /* [ffn][d]                                                       */
  DFLASH_L_W_UP,            /* [ffn][d]                                                       */
  DFLASH_L_W_DOWN,          /* [d][ffn]                                                       */
  DFLASH_L_CONV_ATTN_PRE_W, /* [2][d]  conv taps k_t = sigmoid(W x_t + b): before attention   */
  DFLASH_L_CONV_ATTN_PRE_B, /* [2]     (conv_group G > 0: W is [2 d/G][d], b is [2][d])       */
  DFLASH_L_CONV_ATTN_POST_W,/* [2][d]  after attention (on the O-projection output)           */
  DFLASH_L_CONV_ATTN_POST_B,/* [2]                                                            */
  DFLASH_L_CONV_MLP_PRE_W,  /* [2][d]  before the MLP                                          */
  DFLASH_L_CONV_MLP_PRE_B,  /* [2]                                                            */
  DFLASH_L_CONV_MLP_POST_W, /* [2][d]  after the MLP                                           */
  DFLASH_L_CONV_MLP_POST_B, /* [2]                                                            */
  DFLASH_LAYER_TENSORS
} dflash_layer_tensor;

/* Borrowed device pointers (host struct, copied by dflash_create; the caller keeps the memory
 * alive and unchanged for the handle's life).  embed and lm_head are [V][d] (shared with the
 * target, "Architecture", Component Breakdown row "Target LLM"); sel_A / sel_B are [V][r]
 * token tables and sel_WH is [r][d] (context gate) of the path selector. */
typedef struct {
  const void* embed;        /* [V][d]                       */
  const void* lm_head;      /* [V][d]                       */
  const void* concat_norm;  /* [n_taps*target_hidden]       */
  const void* fc;           /* [d][n_taps*target_hidden]    */
  const void* final_norm;   /* [d]                          */
  const void* sel_A;        /* [V][r]                       */
  const void* sel_B;        /* [V][r]                       */
  const void* sel_WH;       /* [r][d]                       */
  const void* const* layers;/* (host) n_layers*DFLASH_LAYER_TENSORS device pointers */
} dflash_weights;

/* Where things sit inside the caller's kv_cache buffer (byte offsets).
 * K and V caches are [n_layers][max_seqs][n_kv_heads][window][head_dim] of dtype: position p
 * of a sequence lives in ring slot p mod window.  seq_len[s] is one past the last injected
 * position (= the anchor position of the next draft); seq_base[s] is the first position
 * injected since the sequence was last (re)started.  device_error is one int32 word. */
typedef struct {
  size_t k_offset, v_offset, seq_len_offset, seq_base_offset, device_error_offset, total_bytes;
} dflash_kv_layout;

typedef struct dflash_handle dflash_handle;

/* Validates a configuration; DFLASH_OK if the kernels support it, else DFLASH_E_UNSUPPORTED or
 * DFLASH_E_INVALID with the reason in dflash_last_error().  Supported: 1..16 layers; hidden a
 * multiple of 64 up to 4096; n_heads a multiple of n_kv_heads with (n_heads/n_kv_heads) *
 * block_size <= 64; block_size 2..32; topk 16; sel_rank a multiple of 8 in [8, 256]; the concat
 * width n_taps*target_hidden a multiple of 8 (of 64 for bf16) and at most 65536 (bf16) or 32768
 * (fp32); bf16 drafters need head_dim 128, ffn a multiple of 128 and n_heads*head_dim a multiple
 * of 64, both at most 16384. */
DFLASH_API dflash_status dflash_config_check(const dflash_config* cfg);

/* Size of the caller-owned KV cache buffer for `max_seqs` sequences (0 on invalid input). */
DFLASH_API size_t dflash_kv_cache_bytes(const dflash_config* cfg, int32_t max_seqs);
DFLASH_API dflash_status dflash_kv_cache_layout(const dflash_config* cfg, int32_t max_seqs, dflash_kv_layout* out /* host */);

/* Size of the caller-owned workspace for up to `max_seqs` sequences, blocks of up to `max_batch`
 * sequences and injection passes of up to `max_inject_rows` rows (an injection call with more
 * rows is processed in several passes).  0 on invalid input. */
DFLASH_API size_t dflash_workspace_bytes(const dflash_config* cfg, int32_t max_seqs, int32_t max_batch, int32_t max_inject_rows);

/* Creates a handle.  kv_cache (kv_bytes) and workspace (ws_bytes) are caller-owned device
 * buffers of at least the sizes above.  The caller must zero the seq_len/seq_base/device_error
 * words of kv_cache before first use (or call dflash_reset_seqs).  Host-side only: enqueues
 * nothing.  Calls of one handle share its workspace, so they must not overlap (one stream, or
 * ordered by events).  Several handles, each with its own workspace, may share one kv_cache and
 * run at the same time on different streams as long as their calls touch disjoint sequences
 * (e.g. a prefill injection of a new sequence beside the draft cycles of running ones); they
 * then share the device error word, which dflash_reset_seqs clears. */
DFLASH_API dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* w, int32_t max_seqs,
                            int32_t max_batch, int32_t max_inject_rows, void* kv_cache, size_t kv_bytes,
                            void* workspace, size_t ws_bytes, dflash_handle** out /* host */);
DFLASH_API dflash_status dflash_destroy(dflash_handle* h);   /* frees host state only */

/* Marks n_seq sequences empty (seq_len = seq_base = 0) and clears the device error word. */
DFLASH_API dflash_status dflash_reset_seqs(dflash_handle* h, int32_t n_seq, const int32_t* seq_ids, void* stream);

/* (1) KV injection.  For each i < n_seq, appends n_new[i] (device, 0..max_new) target-state rows
 * of sequence seq_ids[i] at absolute positions start_pos[i] .. start_pos[i]+n_new[i]-1.
 * start_pos may be NULL: append at the sequence's current length.  A start position other
 * than the current length restarts that sequence's context there.  seq_ids within one call
 * must be distinct.  Only the last `window` rows of a sequence in one call are projected (the
 * earlier ones fall outside the window by the end of the call).
 * target_hidden: [n_seq][max_new][n_taps*target_hidden] (dtype): row (i, r) is the
 * concatenation of the tapped target layers at that position.
 * Computes u_bar = RMSNorm(row) * concat_norm, c = fc u_bar, then for every layer
 * K = RoPE_p(RMSNorm_head(W_k c) * k_norm), V = W_v c into ring slot p mod window
 * ("Z Lab releases DFlash 2 ...", section "Persistent Conditioning Through Target KV
 * Injection"; "Architecture", section "Internals Worth Knowing": projection ahead of the
 * draft pass with fused norm + RoPE). */
DFLASH_API dflash_status dflash_inject_kv(dflash_handle* h, int32_t n_seq, const int32_t* seq_ids, const int32_t* start_pos,
                               const int32_t* n_new, int32_t max_new, const void* target_hidden, void* stream);

/* (2) One forward pass over the block [anchor_ids[i], MASK x (K-1)] of each sequence at
 * positions L..L+K-1 (L = the sequence's current length): embed, then per layer
 * h += Conv(Attn(Conv(RMSNorm h))), h += Conv(MLP(Conv(RMSNorm h))) with non-causal attention
 * over the K block slots plus the last min(L - base, window) injected positions, final
 * RMSNorm, shared lm_head, top-16 per draft slot ("Architecture", flowchart "Drafter" and
 * Component Breakdown).  Outputs (slot t = 1..K-1 at index t-1):
 *   topk_ids / topk_logits [n_seq][K-1][16], ordered by (logit desc, id asc);
 *   h_final [n_seq][K][d] fp32 -- final-normed hidden states, input of the selector;
 *   logits  [n_seq][K-1][V] fp32 or NULL -- full logits for checking only (extra HBM writes). */
DFLASH_API dflash_status dflash_draft_block(dflash_handle* h, int32_t n_seq, const int32_t* seq_ids, const int32_t* anchor_ids,
                                 int32_t* topk_ids, float* topk_logits, float* h_final, float* logits, void* stream);

/* Allocation-free variant of dflash_draft_block, for callers that cannot allocate device memory or
 * hand out a workspace per call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The same pass, arguments and outputs; every scratch buffer of the pass
 * (activations, GEMM k-split partials, attention partials, top-16 partial lists, work counters)
 * lives in the library's own static device array of 32 MiB on the current device instead of the
 * handle's workspace (the KV cache is still the handle's).  The current device must be the one
 * the stream, the handle's buffers and the outputs belong to.  The array is shared by every call
 * on that GPU and keeps the last call's contents (the pass itself zeroes what must start at zero),
 * so calls that overlap in time on one GPU -- several streams, several handles, several threads --
 * race on it: the caller must serialise them.  n_seq is limited by the array's size, not by the
 * handle's max_batch: dflash_workspace_bytes(cfg, 1, n_seq, 1) must not exceed 32 MiB (4 sequences
 * at block 16 and hidden 2048, 8 at block 8); a larger call returns DFLASH_E_SHAPE before anything
 * is enqueued.  No call allocates or frees device memory. */
DFLASH_API dflash_status dflash_draft_block_static(dflash_handle* h, int32_t n_seq, const int32_t* seq_ids,
                                                   const int32_t* anchor_ids, int32_t* topk_ids, float* topk_logits,
                                                   float* h_final, float* logits, void* stream);

/* (3) Path selection over the candidate lattice ("Architecture", section "Problem 1 --
 * Independent picks are incoherent"): S_t(a, b) = U_t(b) + sum_j A[a,j] * H_t[j] * B[b,j] with
 * U_t the drafter logit, H_t = sigmoid(W_H h_final[t]); slot 1's predecessor is the anchor.
 * VITERBI: the max-scoring path (margin = best - second-best complete path score, exact).
 * GREEDY: follow the best successor from the anchor (margin = smallest best-minus-second gap).
 * Ties go to the smaller candidate index.  path_ids [n_seq][K-1]; path_score, margin [n_seq]
 * may be NULL.  Works in the handle's workspace (partial pair scores and one arrival counter
 * per sequence), so it must not overlap the handle's other calls; the first selector call of a
 * handle also enqueues a small kernel that zeroes the counters (each launch leaves them zero). */
DFLASH_API dflash_status dflash_select_path(dflash_handle* h, int32_t n_seq, const int32_t* anchor_ids, const int32_t* topk_ids,
                                 const float* topk_logits, const float* h_final, dflash_select_mode mode,
                                 int32_t* path_ids, float* path_score, float* margin, void* stream);

/* (3s) Sampling walk over the same lattice ("Architecture", section "Problem 1 -- Independent
 * picks are incoherent": sampling draws from the same pair scores).  At slot t the pick b is
 * drawn from q_t(b) = softmax_b(S_t(a, b) / temperature) over the slot's 16 candidates given
 * the previous pick a (the anchor for slot 1), cut to its top-p nucleus when top_p < 1 (rank
 * by probability, ties to the lower candidate index; a candidate stays while the mass ranked
 * ahead of it is below top_p; renormalise): the first b, in candidate order, whose
 * cumulative probability exceeds uniforms[t-1] times the total.  uniforms [n_seq][K-1] in
 * [0, 1) are the caller's random numbers.  Outputs: path_ids [n_seq][K-1]; q_path
 * [n_seq][K-1] = q_t(pick); q_cand [n_seq][K-1][16] = q_t over the candidates after the cut (may be NULL;
 * dflash_verify_rejection needs it).  Device pointers; temperature in [1e-6, 1e6] (the walk's
 * picks are the greedy walk's as it goes to 0); top_p in (0, 1].  Workspace use as for
 * dflash_select_path. */
DFLASH_API dflash_status dflash_select_sample(dflash_handle* h, int32_t n_seq, const int32_t* anchor_ids, const int32_t* topk_ids,
                                   const float* topk_logits, const float* h_final, float temperature,
                                   float top_p, const float* uniforms, int32_t* path_ids, float* q_path,
                                   float* q_cand, void* stream);

/* (4s) Rejection-sampling verification ("Architecture", section "Speculative Decoding Context"
 * and flowchart "Verification": rejection sampling restores the exact target distribution).
 * draft_ids [n_seq][K-1] with the drafter's q_path [n_seq][K-1] and its distribution at every
 * slot, q_cand [n_seq][K-1][16] over topk_ids [n_seq][K-1][16] (zero elsewhere), as written by
 * dflash_select_sample; target_probs [n_seq][K][vocab]: row i-1 = the target's distribution for
 * slot i, row K-1 = the bonus distribution.  Draft i is accepted iff
 * u_accept[i-1] * q_path[i-1] < p_i(d_i), in order, up to the first rejection.  The committed
 * token after the accepted prefix is drawn with u_resample [n_seq] (inverse CDF in token
 * order) from max(0, p_i - q_i) normalised at a rejection at slot i, else from the bonus row.
 * Rows of target_probs need not be normalised; where max(0, p_i - q_i) has no positive mass the
 * token is drawn from p_i itself.  A slot's 16 candidate ids are distinct; a draft id outside
 * [0, vocab) counts as rejected.  Outputs as dflash_verify_greedy (n_commit may be NULL).
 * 2 <= block_size <= 64; one workgroup per sequence. */
DFLASH_API dflash_status dflash_verify_rejection(int32_t n_seq, int32_t block_size, int32_t vocab, const int32_t* draft_ids,
                                      const float* q_path, const int32_t* topk_ids, const float* q_cand,
                                      const float* target_probs, const float* u_accept, const float* u_resample,
                                      int32_t* n_accepted, int32_t* n_commit, int32_t* committed, int32_t* next_anchor,
                                      void* stream);

/* (4) Greedy longest-prefix verification ("Architecture", section "Speculative Decoding
 * Context" and the sequence diagram's last step: accepted prefix + 1 bonus token).
 * draft_ids [n_seq][K-1] = d_1..d_{K-1}; target_argmax [n_seq][K] = g_0..g_{K-1} (g_i is the
 * target's choice after slot i).  n = largest m with d_i == g_{i-1} for all i <= m.
 * Outputs: n_accepted [n_seq] = n; n_commit [n_seq] = n+1 (may be NULL; usable as the next
 * call's n_new); committed [n_seq][K] = d_1..d_n, g_n, then -1; next_anchor [n_seq] = g_n. */
DFLASH_API dflash_status dflash_verify_greedy(int32_t n_seq, int32_t block_size, const int32_t* draft_ids,
                                   const int32_t* target_argmax, int32_t* n_accepted, int32_t* n_commit,
                                   int32_t* committed, int32_t* next_anchor, void* stream);

/* FP8 weight-only lm_head (an option beside the bf16 pass; the pages run drafts with quantised
 * weights on one backend, "z-lab/dflash" README mirror, section "MLX (Apple Silicon)", and fix no
 * format).  dflash_quantize_fp8_rows writes, for a bf16 matrix src [rows][cols] (device, cols a
 * positive multiple of 8), the OCP FP8 E4M3 code of every weight (codes [rows][cols], device,
 * caller-owned) and one power-of-two scale per row (row_scales [rows] fp32, device): with a the
 * row's largest magnitude, scale = 2^k for the smallest integer k with a <= 448 * 2^k, and each
 * code is the E4M3 value nearest to w / scale (ties to even; the sign of w kept, so -0 is 0x80).
 * A row with a < 2^-64 gets zero codes and scale 1.  Asynchronous on stream; no allocation.
 * dflash_set_lm_head_fp8 makes a handle's dflash_draft_block read the shared lm_head as those codes
 * times their row scales (exact in bf16) instead of the bf16 matrix; NULL for both reverts to bf16.
 * The codes are borrowed like the weights.  Every batch size: at most 16 draft rows
 * (n_seq * block_size) the independent-wave kernel widens the codes in registers (hidden a
 * multiple of 512 up to 2048; other hidden sizes take the skinny kernel), 17..64 rows the skinny
 * MFMA kernel, more rows the LDS tile kernels (each 1 KiB LDS-DMA block 16 rows x 64 k of codes). */
DFLASH_API dflash_status dflash_quantize_fp8_rows(const void* src, int32_t rows, int32_t cols, uint8_t* codes,
                                                  float* row_scales, void* stream);
DFLASH_API dflash_status dflash_set_lm_head_fp8(dflash_handle* h, const uint8_t* codes, const float* row_scales);   /* clears an MXFP4 lm_head */
/* MXFP4 weight-only lm_head (4-bit weights, as in the pages' 4-bit drafts on one backend, "z-lab/dflash"
 * README mirror, section "MLX (Apple Silicon)"; the format is the OCP Microscaling MXFP4 encoding).
 * dflash_quantize_mxfp4_rows writes, for a bf16 matrix src [rows][cols] (device, 16-byte aligned,
 * cols a positive multiple of 32), per block of 32 consecutive weights of a row one scale byte
 * E = s + 127 (scales [rows][cols/32], device) with s = floor(log2 a) - 2 for the block's largest
 * magnitude a, and per weight the 4-bit E2M1 code of the magnitude nearest to |w| / 2^s among
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 (ties to the even code, larger magnitudes saturating to 6) with the
 * sign of w as bit 3 (codes [rows][cols/2], device, 8-byte aligned: weight 2j in the low nibble of
 * byte j).  A block with a < 2^-64 is stored as signed zeros with E = 127.  Asynchronous on stream;
 * no allocation.  dflash_set_lm_head_mxfp4 makes a handle's dflash_draft_block read the shared
 * lm_head as those codes, each standing for value(code) * 2^(E - 127) (exact in bf16), instead of the
 * bf16 matrix (and instead of an FP8 lm_head, which it clears); NULL for both reverts to bf16.
 * Borrowed like the weights.  Every batch size: at most 16 draft rows the independent-wave kernel
 * (hidden a multiple of 512 up to 2048), 17..64 rows the skinny kernel (codes streamed into
 * registers), more rows the LDS tile kernels (each 1 KiB LDS-DMA block 32 rows x 64 k of codes,
 * the block scales of a tile staged in LDS) when the hidden size is at most 2048, else the skinny
 * kernels over row tiles of 64 rows, which keep one work counter per row tile: such a draft call
 * of more than 4096 rows returns DFLASH_E_UNSUPPORTED before anything is enqueued. */
DFLASH_API dflash_status dflash_quantize_mxfp4_rows(const void* src, int32_t rows, int32_t cols, uint8_t* codes,
                                                    uint8_t* scales, void* stream);
DFLASH_API dflash_status dflash_set_lm_head_mxfp4(dflash_handle* h, const uint8_t* codes, const uint8_t* scales);
/* The same for one layer's MLP: gate_up_codes [2*ffn][d] are the codes of the stacked matrix
 * [W_gate; W_up] (gate rows first), down_codes [d][ffn] those of W_down, each with its row scales
 * (as written by dflash_quantize_fp8_rows); all four NULL reverts the layer to its bf16 matrices.
 * Borrowed like the weights.  Every batch size (the streaming, skinny and tile GEMM kernels all
 * take E4M3 codes). */
DFLASH_API dflash_status dflash_set_mlp_fp8(dflash_handle* h, int32_t layer, const uint8_t* gate_up_codes,
                                            const float* gate_up_scales, const uint8_t* down_codes,
                                            const float* down_scales);
/* The same for one layer's MLP in MXFP4: gate_up_codes [2*ffn][d/2] and down_codes [d][ffn/2] as
 * written by dflash_quantize_mxfp4_rows, with their block scale bytes gate_up_scales [2*ffn][d/32]
 * and down_scales [d][ffn/32].  Replaces the layer's FP8 MLP weights if any (and
 * dflash_set_mlp_fp8 replaces these); all four NULL reverts the layer to bf16.  hidden and ffn must
 * be multiples of 128 (else DFLASH_E_UNSUPPORTED).  Every batch size: at most 16 draft rows the
 * streaming kernels (the skinny ones where the streaming plan does not apply), 17..64 rows the
 * skinny kernels, more rows the LDS tile kernels (the skinny ones over row tiles of 64 rows where
 * a tile workgroup's k-range would exceed 2048). */
DFLASH_API dflash_status dflash_set_mlp_mxfp4(dflash_handle* h, int32_t layer, const uint8_t* gate_up_codes,
                                              const uint8_t* gate_up_scales, const uint8_t* down_codes,
                                              const uint8_t* down_scales);
/* The same for one layer's attention projections: qkv_codes [n_heads*head_dim + 2*n_kv_heads*head_dim][d]
 * are the codes of the stacked [W_q; W_k; W_v], o_codes [d][n_heads*head_dim] those of W_o.  Every
 * batch size. */
DFLASH_API dflash_status dflash_set_attn_fp8(dflash_handle* h, int32_t layer, const uint8_t* qkv_codes,
                                             const float* qkv_scales, const uint8_t* o_codes, const float* o_scales);
/* The same for the injection: fc_codes [d][n_taps*target_hidden] (W_fc) and kv_codes
 * [n_layers*2*n_kv_heads*head_dim][d], the stacked [W_k^0; W_v^0; W_k^1; W_v^1; ...].  Every
 * injection size, a prefill included. */
DFLASH_API dflash_status dflash_set_inject_fp8(dflash_handle* h, const uint8_t* fc_codes, const float* fc_scales,
                                               const uint8_t* kv_codes, const float* kv_scales);
/* MXFP4 forms of the last two (the 4-bit reading of the same passage; codes and block scale bytes
 * as written by dflash_quantize_mxfp4_rows: qkv_codes [n_heads*head_dim + 2*n_kv_heads*head_dim][d/2]
 * with qkv_scales [..][d/32], o_codes [d][n_heads*head_dim/2] with o_scales [d][n_heads*head_dim/32];
 * fc_codes [d][n_taps*target_hidden/2] with fc_scales [d][n_taps*target_hidden/32], kv_codes
 * [n_layers*2*n_kv_heads*head_dim][d/2] with kv_scales [..][d/32]).  Each replaces the FP8 weights
 * of the same GEMMs and is replaced by them; all four NULL reverts to bf16.  Borrowed like the
 * weights.  The widths these GEMMs read along k (hidden, n_heads*head_dim, n_taps*target_hidden)
 * must be multiples of 128, else DFLASH_E_UNSUPPORTED.  Every batch and injection size: the
 * streaming kernels at most 16 rows, the skinny ones 17..64, the LDS tile kernels above (their
 * block scales staged in LDS 2048 k at a time). */
DFLASH_API dflash_status dflash_set_attn_mxfp4(dflash_handle* h, int32_t layer, const uint8_t* qkv_codes,
                                               const uint8_t* qkv_scales, const uint8_t* o_codes,
                                               const uint8_t* o_scales);
DFLASH_API dflash_status dflash_set_inject_mxfp4(dflash_handle* h, const uint8_t* fc_codes, const uint8_t* fc_scales,
                                                 const uint8_t* kv_codes, const uint8_t* kv_scales);

/* A second layout of the bf16 weight matrices for the batched GEMMs (more than 64 rows), which run
 * on MFMA tiles whose weight operand is loaded 16 rows x 32 k at a time.  The operations are the
 * drafter's weight projections ("Architecture", kb.ekarisky.com, Component Breakdown); the layout
 * is this library's own, for its tile loads, and changes no result.
 *
 * dflash_block_weights: writes dst, the blocked copy of src, a row-major bf16 [rows][cols] matrix
 * (device pointers; dst is caller-owned, the same size as src and not overlapping it; rows a
 * positive multiple of 16, cols of 32), enqueued on `stream`.  Block (g, c) -- rows 16 g .. 16 g +
 * 15, k = 32 c .. 32 c + 31 -- is the KiB at byte offset (g * cols / 32 + c) * 1024 of dst; its
 * 16 bytes at offset 16 l hold row r = 16 g + l / 4, k = 32 c + 8 ((l mod 4) XOR s) .. + 7, with
 * s = ((l / 4) / 2 XOR (l / 4) / 8) mod 4.  A 16-row group therefore takes the same bytes in both
 * forms.  Errors: DFLASH_E_SHAPE (rows or cols), DFLASH_E_INVALID (NULL or src == dst), DFLASH_E_HIP.
 *
 * dflash_set_blocked_weights: registers blocked copies of the handle's matrices, borrowed like the
 * weights and holding the same values: blocked->lm_head [V][d], blocked->fc [d][n_taps *
 * target_hidden] and, in blocked->layers (host array indexed like dflash_weights.layers), the
 * entries DFLASH_L_WQ, WK, WV, WO, W_GATE, W_UP and W_DOWN; every other field and entry is ignored,
 * and a NULL leaves that matrix row-major only.  A GEMM that runs on the bf16 tiles (not one whose
 * weights are FP8 or MXFP4 codes) reads the copies when every matrix it spans has one; results are
 * the same bits.  blocked == NULL removes them.  Errors: DFLASH_E_STATE, DFLASH_E_UNSUPPORTED (fp32
 * drafter), DFLASH_E_SHAPE (a given matrix with rows not a multiple of 16 or cols of 32); on error
 * nothing changes. */
DFLASH_API dflash_status dflash_block_weights(const void* src, int64_t rows, int64_t cols, void* dst, void* stream);
DFLASH_API dflash_status dflash_set_blocked_weights(dflash_handle* h, const dflash_weights* blocked);

/* Benchmark workload helper, not part of the drafter: stands in for a target model's verify
 * pass.  For i = 1..K-1, g_{i-1} = d_i with probability match_prob, else a different token;
 * g_{K-1} is uniform.  match_prob = -1 instead draws the committed count tau uniform on {1..K}
 * and matches exactly drafts 1..tau-1 (greedy verification then commits tau tokens).  Randomness: splitmix64 of (seed, *counter, sequence, slot); *counter
 * (device int64) is incremented once per call.  Runs as one workgroup: n_seq <= 1024. */
DFLASH_API dflash_status dflash_synth_target_argmax(int32_t n_seq, int32_t block_size, int32_t vocab, const int32_t* draft_ids,
                                         float match_prob, uint64_t seed, int64_t* counter,
                                         int32_t* target_argmax, void* stream);

/* Kernel timing for measurement: while enabled, each dflash_draft_block records a pair of HIP
 * events around its lm_head + top-16 kernel on the call's stream (pair index advances modulo
 * capacity).  Disable it (capacity 0) before capturing a graph: events recorded inside a
 * captured graph cannot be read back.  dflash_timing_read waits for the pairs recorded so far
 * (at most capacity) and returns their summed milliseconds and count.  dflash_timing_enable
 * re-creates the events and clears the count; capacity 0 disables. */
DFLASH_API dflash_status dflash_timing_enable(dflash_handle* h, int32_t capacity);
DFLASH_API dflash_status dflash_timing_read(dflash_handle* h, double* total_ms /* host */, int32_t* count /* host */);

/* Reads (and keeps) the device error word; synchronises the device.  0 = none.
 * Bits: 1 = sequence id out of range, 2 = n_new outside [0, max_new], 4 = negative start_pos,
 * 8 = anchor token id outside [0, vocab), 16 = candidate id (dflash_select_path's topk_ids)
 * outside [0, vocab): the selector reads row 0 of A and B for it and still reports that id. */
DFLASH_API dflash_status dflash_get_device_error(dflash_handle* h, int32_t* code /* host */);

DFLASH_API const char* dflash_status_string(dflash_status s);
DFLASH_API const char* dflash_last_error(void);   /* thread-local message of the last failing call */

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
