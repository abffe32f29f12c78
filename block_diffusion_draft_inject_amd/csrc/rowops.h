// Argument structs and launchers of the non-GEMM kernels (internal).
#pragma once
#include "common.h"

namespace dfl {

// Per-sequence context of one draft call, written by the block-embed kernel.
struct SeqCtx {
  int sid;     // sequence id (clamped into range)
  int L;       // anchor position = current length
  int n_ctx;   // number of context positions visible: min(L - base, window)
  int slot0;   // ring slot of the oldest visible position
};

// Per-call sequence plan, done by the block-embed kernel (the workgroup of each sequence's
// slot 0 writes its SeqCtx; workgroup 0 zeroes the lm_head fragment counters).
struct PlanArgs {
  int max_seqs, window;
  const int* seq_ids;
  const int* seq_len;
  const int* seq_base;
  SeqCtx* ctx;
  int* counters;       // lm_head work-stealing counters, zeroed here
};

struct RowArgs {
  PlanArgs plan;       // block embed only
  int K, d, mask_id, use_conv, final_norm, splits, part_rows, ldy, vocab;
  size_t y_plane;      // activation planes of y (bf16 drafters)
  void* y2;            // final norm only: split copy of the output for the lm_head GEMM
  int* dev_err;
  float eps;
  const int* anchor;
  const void* embed;
  const float* h_in;
  float* h_out;
  const float* part;
  const void* post_w;
  const void* post_b;
  const void* pre_gain;
  const void* pre_w;
  const void* pre_b;
  void* y;
};

struct QkvArgs {
  int K, nh, nkv, dh, N, splits, part_rows;
  size_t q_plane;
  float eps;
  double log_theta;
  const SeqCtx* ctx;
  const float* part;
  const void* q_gain;
  const void* k_gain;
  void* q;
  void* k;
  void* v;
};

struct SwigluArgs {
  int M, f, splits, part_rows;
  size_t out_plane;
  const float* part;
  void* out;
};

struct ReduceArgs {
  int M, N, splits, part_rows;
  size_t out_plane;
  const int* m_dev;    // optional: rows valid = min(M, *m_dev - m_off)
  int m_off;
  const float* part;
  void* out;
};

struct InjectArgs {
  int n_seq, max_new, max_seqs, concat, chunk0, window;
  size_t ubar_plane;
  float eps;
  const int* seq_ids;
  const int* start_pos;
  const int* n_new;
  int* seq_len;
  int* seq_base;
  int* dev_err;
  int* row_off;     // [n_seq + 1]
  int* row_start;   // [n_seq] absolute position of the first projected row
  int* row_skip;    // [n_seq] leading rows not projected (they would leave the window)
  int* total;
  const void* states;
  const void* gain;
  void* ubar;
  int* meta_seq;
  int* meta_pos;
};

constexpr int MAX_LAYERS = 16;

struct KvPostArgs {
  int N, splits, part_rows, nkv, dh, window, max_seqs;
  float eps;
  double log_theta;
  const float* part;
  const int* meta_seq;
  const int* meta_pos;
  const void* k_gain[MAX_LAYERS];
  void* kcache;
  void* vcache;
};

struct ResetArgs {
  int n, max_seqs;
  const int* seq_ids;
  int* seq_len;
  int* seq_base;
  int* dev_err;
};

struct MergeArgs {
  int K, ncand;
  const float* vals;   // [n_seq*K][ncand]
  const int* ids;      // same shape or nullptr (id = index)
  int* out_ids;        // [n_seq][K-1][16]
  float* out_vals;
  float* logits_out;   // raw mode only: optional copy of the candidate row [n_seq][K-1][ncand]
  int* counters;       // lm_head work-stealing counters, zeroed here for the next call
};

struct AttnArgs {
  int K, nh, nkv, dh, window, max_seqs, chunks, n_layers_stride, layer;
  size_t q_plane, o_plane;
  float scale;
  const SeqCtx* ctx;
  const void* q;       // [rows][nh*dh]
  const void* kb;      // [rows][nkv*dh]
  const void* vb;
  const void* kcache;  // [layers][max_seqs][nkv][window][dh]
  const void* vcache;
  float* o_part;       // [n_seq][nkv][chunks][R][dh]
  float* m_part;       // [n_seq][nkv][chunks][R]
  float* l_part;
  void* o;             // [rows][nh*dh]
};

// Row handled by workgroup b of a launch of n one-row workgroups.  A launch deals its workgroups
// to the eight XCDs round-robin (workgroup b to XCD b mod 8); this gives each XCD one contiguous
// range of rows (XCD x: rows x*q + min(x, r) onwards, q = n / 8, r = n mod 8), so that a row
// reading its neighbours' inputs (the two-tap conv reads rows t-1 and t-2) finds them in the
// L2 of its own XCD, where the neighbours' workgroups fetched them.  A bijection for every n.
__device__ __forceinline__ int xcd_row(int b, int n) {
  const int x = b & 7, q = n >> 3, r = n & 7;
  return x * q + min(x, r) + (b >> 3);
}

// Hand-off from n workgroups to the one that arrives last at `counter` (device memory, zero
// before the first of the n arrivals).  Returns true in every thread of that workgroup, which
// then sees every global store the other n - 1 made before they arrived, and leaves the counter
// at zero for the next launch.  The workgroups may sit on different XCDs, whose L2 caches are
// separate: the workgroup barrier completes every wave's stores (into this XCD's L2), then
// one agent-scope release by the counting thread writes the L2 back (one write-back per
// workgroup, not per wave), the count itself is a system-scope atomic (performed past the
// L2s), and the last workgroup acquires at agent scope after it (L2 invalidated).  No
// workgroup waits for another.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned n, int* flag_lds) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const int last = prev + 1 == n;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    *flag_lds = last;
  }
  __syncthreads();
  const bool last = *flag_lds != 0;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

struct SelectArgs {
  int K, d, r, mode, vocab;   // mode 0 = Viterbi, 1 = greedy, 2 = sampling walk
  int* dev_err;
  const int* anchor;
  const int* topk_ids;
  const float* topk_logits;
  const float* h_final;   // [n_seq][K][d]
  const void* A;
  const void* B;
  const void* WH;
  int* path;
  float* score;
  float* margin;
  // sampling walk only
  float inv_temp;
  float top_p;            // nucleus cut, >= 1 keeps all 16
  const float* uniforms;  // [n_seq][K-1]
  float* q_path;          // [n_seq][K-1]
  float* q_cand;          // [n_seq][K-1][16] or null
  // workspace
  float* spart;           // [n_seq][K-1][rank chunks of 32][16][16] partial pair scores
  unsigned* sel_cnt;      // [n_seq] arrival counters: zero between launches (the last arrival resets)
  int spw;                // slots per workgroup (set by the launcher)
};

struct RejectArgs {
  int n_seq, K, V;
  const int* draft;        // [n_seq][K-1]
  const float* q_path;     // [n_seq][K-1]
  const int* cand;         // [n_seq][K-1][16]
  const float* q_cand;     // [n_seq][K-1][16]
  const float* p;          // [n_seq][K][V]
  const float* u_accept;   // [n_seq][K-1]
  const float* u_resample; // [n_seq]
  int* n_acc;
  int* n_commit;
  int* committed;          // [n_seq][K]
  int* next_anchor;
};

struct VerifyArgs {
  int n_seq, K;
  const int* draft;
  const int* target;
  int* n_acc;
  int* n_commit;
  int* committed;
  int* next_anchor;
};

struct SynthArgs {
  int n_seq, K, vocab;
  float p;
  unsigned long long seed;
  long long* counter;
  const int* draft;
  int* target;
};

// Per-channel two-tap conv (conv_group G > 0): coefficient vectors k_tj[c] = sigmoid(base_j[c] +
// corr_tj[c / G]), corr_t = W_c x_t in R^(2 d / G) given as k-split GEMM partials.
struct PcArgs {
  int K, d, G, splits, part_rows, final_norm, ldo;
  size_t plane;        // activation planes of x and out (bf16 drafters)
  float eps;
  const float* h_in;   // post-conv + norm only: residual in/out
  float* h_out;
  const void* x;       // conv input rows (activation planes): the sublayer output a, or the normed z
  const float* part;   // corrections [splits][part_rows][2 d / G], tap 0's groups first
  const void* base;    // [2][d]
  const void* gain;    // RMSNorm gain (post-conv + norm only)
  void* out;           // z planes / y planes / final: h_final fp32
  void* out2;          // final only: the lm_head's bf16 input rows
};

hipError_t launch_embed_pre(bool bf, const RowArgs& a, int rows, hipStream_t st);
hipError_t launch_post_pre_pc(bool bf, const PcArgs& a, int rows, hipStream_t st);
hipError_t launch_conv_apply(bool bf, const PcArgs& a, int rows, hipStream_t st);
hipError_t launch_post_pre(bool bf, const RowArgs& a, int rows, hipStream_t st);
hipError_t launch_qkv_post(bool bf, const QkvArgs& a, int rows, hipStream_t st);
hipError_t launch_swiglu(bool bf, const SwigluArgs& a, hipStream_t st);
hipError_t launch_reduce_store(bool bf, const ReduceArgs& a, hipStream_t st);
hipError_t launch_inject_plan(const InjectArgs& a, hipStream_t st);
hipError_t launch_concat_norm(bool bf, const InjectArgs& a, int rows, hipStream_t st);
hipError_t launch_kv_post(bool bf, const KvPostArgs& a, int rows, int heads, hipStream_t st);
hipError_t launch_reset(const ResetArgs& a, hipStream_t st);
hipError_t launch_topk_merge(const MergeArgs& a, int out_rows, hipStream_t st);
hipError_t launch_attention(bool bf, const AttnArgs& a, int n_seq, hipStream_t st);
hipError_t launch_select(bool bf, const SelectArgs& a, int n_seq, hipStream_t st);
hipError_t launch_fill_u32(unsigned* p, int n, unsigned v, hipStream_t st);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t st);
hipError_t launch_verify_rejection(const RejectArgs& a, hipStream_t st);
hipError_t launch_synth(const SynthArgs& a, hipStream_t st);
hipError_t launch_quantize_fp8_rows(const void* src, int rows, int cols, unsigned char* codes, float* scales,
                                    hipStream_t st);
hipError_t launch_quantize_mxfp4_rows(const void* src, int rows, int cols, unsigned char* codes, unsigned char* scales,
                                      hipStream_t st);

}  // namespace dfl
