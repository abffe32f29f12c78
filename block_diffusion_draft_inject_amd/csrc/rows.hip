// Row-wise kernels of the drafter: embedding, RMSNorm + two-tap conv + residual, per-head
// q/k RMSNorm + RoPE, SwiGLU, the injection pipeline's norm/plan/scatter, and the top-16 merge.
//
// Two-tap dynamic convolution ("Architecture", kb.ekarisky.com, section "Problem 2 -- Suffix
// decay is local"): Conv(x)_t = k_t0 x_t + k_t1 x_{t-1}, with per-position taps
// k_t = sigmoid(W_c x_t + b_c) computed from the conv's own input row; slot 0 of a block has
// no predecessor (x_{-1} = 0).  Rows of a block are consecutive (row = seq * K + slot).
#include "rowops.h"
#include <math.h>

namespace dfl {

constexpr int MAXV = 16;   // hidden <= 16 * 256

template <typename T>
__device__ __forceinline__ float ldw(const void* p, size_t i) {
  return ldv(reinterpret_cast<const T*>(p), i);
}

// RoPE angle for pair index i of head_dim dh at position pos, in double precision
// (pos * theta^(-2i/dh) can reach ~3e4 rad; a float product would be off by ~2e-3 rad).
__device__ __forceinline__ void rope_cs(long pos, int i, int dh, double log_theta, float& c, float& s) {
  const double inv = exp(-2.0 * (double)i / (double)dh * log_theta);
  double ang = (double)pos * inv;
  double sd, cd;
  sincos(ang, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// ------------------------------------------------------------------------ draft plan
// Per sequence of a draft call: clamp the id, read its length and base, and derive the
// visible context: positions max(base, L - window) .. L-1, which sit in consecutive ring
// slots (mod window) starting at slot0.
__global__ __launch_bounds__(256) void draft_plan_kernel(PlanArgs a) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= a.n_seq) return;
  int sid = a.seq_ids[b];
  if (sid < 0 || sid >= a.max_seqs) {
    atomicOr(a.dev_err, 1);
    sid = 0;
  }
  const int L = a.seq_len[sid], base = a.seq_base[sid];
  const int first = max(base, L - a.window);
  SeqCtx c;
  c.sid = sid;
  c.L = L;
  c.n_ctx = max(0, L - first);
  c.slot0 = first % a.window;
  a.ctx[b] = c;
}

// ------------------------------------------------------------------------ embed + pre
template <typename T>
__global__ __launch_bounds__(256) void embed_pre_kernel(RowArgs a) {
  __shared__ float red[4 * 4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int b = row / a.K, t = row % a.K;
  const int d = a.d;
  int anchor = a.anchor[b];
  if (anchor < 0 || anchor >= a.vocab) {   // out-of-range token: record and read row 0
    if (tid == 0 && t == 0) atomicOr(a.dev_err, 8);
    anchor = 0;
  }
  const int id_t = (t == 0) ? anchor : a.mask_id;
  const int id_p = (t <= 1) ? anchor : a.mask_id;
  float e[2][MAXV];
  float ss[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int k = i * 256 + tid;
    e[0][i] = e[1][i] = 0.f;
    if (k < d) {
      e[0][i] = ldw<T>(a.embed, (size_t)id_t * d + k);
      e[1][i] = (t > 0) ? ldw<T>(a.embed, (size_t)id_p * d + k) : 0.f;
      ss[0] += e[0][i] * e[0][i];
      ss[1] += e[1][i] * e[1][i];
      a.h_out[(size_t)row * d + k] = e[0][i];
    }
  }
  block_sum256<2>(ss, red);
  const float r0 = rsqrtf(ss[0] / d + a.eps), r1 = rsqrtf(ss[1] / d + a.eps);
  float dot[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int k = i * 256 + tid;
    if (k < d) {
      const float g = ldw<T>(a.pre_gain, k);
      e[0][i] *= r0 * g;
      e[1][i] *= r1 * g;
      if (a.use_conv) {
        dot[0] += ldw<T>(a.pre_w, k) * e[0][i];
        dot[1] += ldw<T>(a.pre_w, d + k) * e[0][i];
      }
    }
  }
  float k0 = 1.f, k1 = 0.f;
  if (a.use_conv) {
    block_sum256<2>(dot, red);
    k0 = sigmoidf_(dot[0] + ldw<T>(a.pre_b, 0));
    k1 = sigmoidf_(dot[1] + ldw<T>(a.pre_b, 1));
  }
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int k = i * 256 + tid;
    if (k < d) stv(reinterpret_cast<T*>(a.y), (size_t)row * a.ldy + k, k0 * e[0][i] + k1 * e[1][i]);
  }
}

// ------------------------------------------------------------------------ post + pre
// h_out[t] = h_in[t] + Conv_post(a)_t with a = sum of `splits` partials of the sublayer output,
// then y[t] = Conv_pre(RMSNorm(h_out))_t  (or, final: y[t] = RMSNorm(h_out[t]) * final gain).
template <typename T>
__global__ __launch_bounds__(256) void post_pre_kernel(RowArgs a) {
  __shared__ float red[4 * 4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int t = row % a.K;
  const int d = a.d;
  const bool conv = a.use_conv != 0;
  // rows t-2, t-1, t of the sublayer output (index 0, 1, 2)
  float s[3][MAXV];
  float hv[2][MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int k = i * 256 + tid;
#pragma unroll
    for (int q = 0; q < 3; ++q) s[q][i] = 0.f;
    hv[0][i] = hv[1][i] = 0.f;
    if (k >= d) continue;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int tt = t - 2 + q;
      if (tt < 0 || (!conv && q < 2)) continue;
      const int rr = row - 2 + q;
      float acc = 0.f;
      for (int sp = 0; sp < a.splits; ++sp) acc += a.part[((size_t)sp * a.part_rows + rr) * d + k];
      s[q][i] = acc;
    }
    if (t >= 1 && conv) hv[0][i] = a.h_in[(size_t)(row - 1) * d + k];
    hv[1][i] = a.h_in[(size_t)row * d + k];
  }
  // post-conv taps of rows t-1 and t
  float kp[2][2] = {{1.f, 0.f}, {1.f, 0.f}};
  if (conv) {
    float dot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int k = i * 256 + tid;
      if (k >= d) continue;
      const float w0 = ldw<T>(a.post_w, k), w1 = ldw<T>(a.post_w, d + k);
      dot[0] += w0 * s[1][i];
      dot[1] += w1 * s[1][i];
      dot[2] += w0 * s[2][i];
      dot[3] += w1 * s[2][i];
    }
    block_sum256<4>(dot, red);
    const float b0 = ldw<T>(a.post_b, 0), b1 = ldw<T>(a.post_b, 1);
    kp[0][0] = sigmoidf_(dot[0] + b0);
    kp[0][1] = sigmoidf_(dot[1] + b1);
    kp[1][0] = sigmoidf_(dot[2] + b0);
    kp[1][1] = sigmoidf_(dot[3] + b1);
  }
  float ss[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int k = i * 256 + tid;
    if (k >= d) continue;
    if (conv) {
      hv[0][i] += kp[0][0] * s[1][i] + kp[0][1] * s[0][i];   // row t-1 (s[0] is t-2, zero if absent)
      hv[1][i] += kp[1][0] * s[2][i] + kp[1][1] * s[1][i];
    } else {
      hv[1][i] += s[2][i];
    }
    a.h_out[(size_t)row * d + k] = hv[1][i];
    ss[0] += hv[0][i] * hv[0][i];
    ss[1] += hv[1][i] * hv[1][i];
  }
  block_sum256<2>(ss, red);
  const float r0 = rsqrtf(ss[0] / d + a.eps), r1 = rsqrtf(ss[1] / d + a.eps);
  if (a.final_norm) {
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int k = i * 256 + tid;
      if (k < d) stv(reinterpret_cast<T*>(a.y), (size_t)row * a.ldy + k, hv[1][i] * r1 * ldw<T>(a.pre_gain, k));
    }
    return;
  }
  float dot[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int k = i * 256 + tid;
    if (k >= d) continue;
    const float g = ldw<T>(a.pre_gain, k);
    hv[0][i] = (t >= 1) ? hv[0][i] * r0 * g : 0.f;
    hv[1][i] = hv[1][i] * r1 * g;
    if (conv) {
      dot[0] += ldw<T>(a.pre_w, k) * hv[1][i];
      dot[1] += ldw<T>(a.pre_w, d + k) * hv[1][i];
    }
  }
  float k0 = 1.f, k1 = 0.f;
  if (conv) {
    block_sum256<2>(dot, red);
    k0 = sigmoidf_(dot[0] + ldw<T>(a.pre_b, 0));
    k1 = sigmoidf_(dot[1] + ldw<T>(a.pre_b, 1));
  }
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int k = i * 256 + tid;
    if (k < d) stv(reinterpret_cast<T*>(a.y), (size_t)row * a.ldy + k, k0 * hv[1][i] + k1 * hv[0][i]);
  }
}

// ------------------------------------------------------------------------ q/k/v post
// One wave per (row, head).  Heads 0..nh-1 are q, nh..nh+nkv-1 k, then v.  Lane l holds
// elements l and l + dh/2, which is exactly a rotate-half RoPE pair.
template <typename T>
__global__ __launch_bounds__(64) void qkv_post_kernel(QkvArgs a) {
  const int row = blockIdx.x, head = blockIdx.y, lane = threadIdx.x;
  const int dh = a.dh, half = dh / 2;
  const int b = row / a.K, t = row % a.K;
  const int nq = a.nh * dh, nkvw = a.nkv * dh;
  const int col0 = head * dh;   // column in the fused [q | k | v] output
  float x0 = 0.f, x1 = 0.f;
  const bool act = lane < half;
  if (act) {
    for (int sp = 0; sp < a.splits; ++sp) {
      const float* pr = a.part + ((size_t)sp * a.part_rows + row) * a.N + col0;
      x0 += pr[lane];
      x1 += pr[lane + half];
    }
  }
  T* dst;
  int gain_kind;   // 0 = q, 1 = k, 2 = v
  size_t off;
  if (head < a.nh) {
    dst = reinterpret_cast<T*>(a.q);
    off = (size_t)row * nq + head * dh;
    gain_kind = 0;
  } else if (head < a.nh + a.nkv) {
    dst = reinterpret_cast<T*>(a.k);
    off = (size_t)row * nkvw + (head - a.nh) * dh;
    gain_kind = 1;
  } else {
    dst = reinterpret_cast<T*>(a.v);
    off = (size_t)row * nkvw + (head - a.nh - a.nkv) * dh;
    gain_kind = 2;
  }
  if (gain_kind < 2) {
    const float ss = wave_sum(act ? x0 * x0 + x1 * x1 : 0.f);
    const float r = rsqrtf(ss / dh + a.eps);
    const void* g = gain_kind == 0 ? a.q_gain : a.k_gain;
    if (act) {
      x0 *= r * ldw<T>(g, lane);
      x1 *= r * ldw<T>(g, lane + half);
      const long pos = (long)a.ctx[b].L + t;
      float c, s;
      rope_cs(pos, lane, dh, a.log_theta, c, s);
      const float y0 = x0 * c - x1 * s, y1 = x1 * c + x0 * s;
      x0 = y0;
      x1 = y1;
    }
  }
  if (act) {
    stv(dst, off + lane, x0);
    stv(dst, off + lane + half, x1);
  }
}

// ------------------------------------------------------------------------ swiglu from partials
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(SwigluArgs a) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)a.M * a.f) return;
  const size_t m = i / a.f, j = i % a.f;
  float g = 0.f, u = 0.f;
  for (int sp = 0; sp < a.splits; ++sp) {
    const float* pr = a.part + ((size_t)sp * a.part_rows + m) * (2 * a.f);
    g += pr[j];
    u += pr[a.f + j];
  }
  stv(reinterpret_cast<T*>(a.out), m * a.f + j, g / (1.f + __expf(-g)) * u);
}

// ------------------------------------------------------------------------ sum partials -> T
template <typename T>
__global__ __launch_bounds__(256) void reduce_store_kernel(ReduceArgs a) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int Mv = a.m_dev ? max(0, min(a.M, *a.m_dev - a.m_off)) : a.M;
  if (i >= (size_t)Mv * a.N) return;
  float acc = 0.f;
  for (int sp = 0; sp < a.splits; ++sp) acc += a.part[(size_t)sp * a.part_rows * a.N + i];
  stv(reinterpret_cast<T*>(a.out), i, acc);
}

// ------------------------------------------------------------------------ injection
// One workgroup: per-sequence row offsets of this call (exclusive scan of the projected row
// counts), and the sequences' length update.  Of n rows for one sequence only the last
// min(n, window) are projected: earlier ones are outside the window once the call completes,
// and their ring slots would collide with the later rows'.
__global__ __launch_bounds__(256) void inject_plan_kernel(InjectArgs a) {
  __shared__ int scan[256];
  __shared__ int carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int i0 = 0; i0 < a.n_seq; i0 += 256) {
    const int i = i0 + tid;
    int n = 0;
    if (i < a.n_seq) {
      n = a.n_new[i];
      const int sid = a.seq_ids[i];
      int err = 0;
      if (n < 0 || n > a.max_new) { err |= 2; n = n < 0 ? 0 : a.max_new; }
      if (sid < 0 || sid >= a.max_seqs) { err |= 1; n = 0; }
      int sp = 0;
      if (n > 0) {
        sp = a.start_pos ? a.start_pos[i] : a.seq_len[sid];
        if (sp < 0) { err |= 4; n = 0; }
      }
      int skip = 0;
      if (n > 0) {
        const int len = a.seq_len[sid];
        if (len == 0 || sp != len) a.seq_base[sid] = sp;   // fresh or restarted
        a.seq_len[sid] = sp + n;
        if (n > a.window) skip = n - a.window;
      }
      if (err) atomicOr(a.dev_err, err);
      a.row_start[i] = sp + skip;
      a.row_skip[i] = skip;
      n -= skip;
    }
    scan[tid] = n;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {   // inclusive Hillis-Steele scan
      const int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    if (i < a.n_seq) a.row_off[i] = carry + scan[tid] - n;
    __syncthreads();
    if (tid == 255) carry += scan[255];
    __syncthreads();
  }
  if (tid == 0) {
    a.row_off[a.n_seq] = carry;
    *a.total = carry;
  }
}

// u_bar = RMSNorm(concatenated states) * gain for compacted rows [chunk0, chunk0 + rows).
template <typename T>
__global__ __launch_bounds__(256) void concat_norm_kernel(InjectArgs a) {
  __shared__ float red[4];
  __shared__ int s_i;
  const int j = a.chunk0 + blockIdx.x, tid = threadIdx.x;
  const int total = *a.total;
  const int lr = blockIdx.x;
  if (j >= total) {
    if (tid == 0) { a.meta_seq[lr] = -1; a.meta_pos[lr] = 0; }
    return;
  }
  if (tid == 0) {
    int i = 0;
    while (a.row_off[i + 1] <= j) ++i;
    s_i = i;
  }
  __syncthreads();
  const int i = s_i;
  const int r = j - a.row_off[i];
  if (tid == 0) { a.meta_seq[lr] = a.seq_ids[i]; a.meta_pos[lr] = a.row_start[i] + r; }
  const int W = a.concat;
  const T* src = reinterpret_cast<const T*>(a.states) + ((size_t)i * a.max_new + r + a.row_skip[i]) * W;
  float ss[1] = {0.f};
  for (int k = tid; k < W; k += 256) {
    const float v = ldv(src, k);
    ss[0] += v * v;
  }
  block_sum256<1>(ss, red);
  const float rs = rsqrtf(ss[0] / W + a.eps);
  T* dst = reinterpret_cast<T*>(a.ubar) + (size_t)lr * W;
  for (int k = tid; k < W; k += 256) stv(dst, k, ldv(src, k) * rs * ldw<T>(a.gain, k));
}

// K/V of every layer from the fused projection [rows][n_layers * 2 * kv_width]; one wave per
// (row, layer, K-or-V, kv head).  K: per-head RMSNorm * k_norm, RoPE at the row's position.
template <typename T>
__global__ __launch_bounds__(64) void kv_post_kernel(KvPostArgs a) {
  const int lr = blockIdx.x, hidx = blockIdx.y, lane = threadIdx.x;
  const int seq = a.meta_seq[lr];
  if (seq < 0) return;
  const long pos = a.meta_pos[lr];
  const int dh = a.dh, half = dh / 2;
  const int per_layer = 2 * a.nkv;
  const int layer = hidx / per_layer, kind = (hidx % per_layer) / a.nkv, kvh = hidx % a.nkv;
  const int col0 = hidx * dh;
  const bool act = lane < half;
  float x0 = 0.f, x1 = 0.f;
  if (act) {
    for (int sp = 0; sp < a.splits; ++sp) {
      const float* pr = a.part + ((size_t)sp * a.part_rows + lr) * a.N + col0;
      x0 += pr[lane];
      x1 += pr[lane + half];
    }
  }
  if (kind == 0) {
    const float ss = wave_sum(act ? x0 * x0 + x1 * x1 : 0.f);
    const float r = rsqrtf(ss / dh + a.eps);
    if (act) {
      const void* g = a.k_gain[layer];
      x0 *= r * ldw<T>(g, lane);
      x1 *= r * ldw<T>(g, lane + half);
      float c, s;
      rope_cs(pos, lane, dh, a.log_theta, c, s);
      const float y0 = x0 * c - x1 * s, y1 = x1 * c + x0 * s;
      x0 = y0;
      x1 = y1;
    }
  }
  if (act) {
    const int slot = (int)(pos % a.window);
    T* cache = reinterpret_cast<T*>(kind == 0 ? a.kcache : a.vcache);
    const size_t off = ((((size_t)layer * a.max_seqs + seq) * a.nkv + kvh) * a.window + slot) * dh;
    stv(cache, off + lane, x0);
    stv(cache, off + lane + half, x1);
  }
}

__global__ void reset_seqs_kernel(ResetArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) *a.dev_err = 0;
  if (i >= a.n) return;
  const int s = a.seq_ids[i];
  if (s < 0 || s >= a.max_seqs) { atomicOr(a.dev_err, 1); return; }
  a.seq_len[s] = 0;
  a.seq_base[s] = 0;
}

// ------------------------------------------------------------------------ top-16 merge
// One workgroup per output row: candidates are `ncand` (value, id) pairs of input row
// in_row = seq * K + slot; ids == nullptr means the id is the candidate's index.
__global__ __launch_bounds__(256) void topk_merge_kernel(MergeArgs a) {
  __shared__ float sv[256 * 4];
  __shared__ int si[256 * 4];
  const int orow = blockIdx.x, tid = threadIdx.x;
  const int b = orow / (a.K - 1), t = orow % (a.K - 1) + 1;
  const size_t in_row = (size_t)b * a.K + t;
  const float* v = a.vals + in_row * a.ncand;
  const int* id = a.ids ? a.ids + in_row * a.ncand : nullptr;
  if (!id && a.logits_out) {
    float* lo = a.logits_out + (size_t)orow * a.ncand;
    for (int c = tid; c < a.ncand; c += 256) lo[c] = v[c];
  }
  Top16 top;
  top.init();
  for (int c = tid; c < a.ncand; c += 256) top.push(v[c], id ? id[c] : c);
  // tree merge of 256 lists: 4 lists per round written to LDS
  for (int w = 1; w < 256; w <<= 1) {
    __syncthreads();
    const bool writer = (tid & (2 * w - 1)) == w;
    const int slot = tid / (2 * w);          // < 128 / w
    // LDS holds 1024 entries: 64 lists of 16; rounds with more writers go in two passes
    const int nwriters = 256 / (2 * w);
    for (int base = 0; base < nwriters; base += 64) {
      if (writer && slot >= base && slot < base + 64) {
#pragma unroll
        for (int i = 0; i < TOPK; ++i) { sv[(slot - base) * TOPK + i] = top.v[i]; si[(slot - base) * TOPK + i] = top.id[i]; }
      }
      __syncthreads();
      if ((tid & (2 * w - 1)) == 0 && slot >= base && slot < base + 64) {
#pragma unroll
        for (int i = 0; i < TOPK; ++i) top.push(sv[(slot - base) * TOPK + i], si[(slot - base) * TOPK + i]);
      }
      __syncthreads();
    }
  }
  if (tid == 0) {
#pragma unroll
    for (int i = 0; i < TOPK; ++i) {
      a.out_ids[(size_t)orow * TOPK + i] = top.id[i];
      a.out_vals[(size_t)orow * TOPK + i] = top.v[i];
    }
  }
}

// ------------------------------------------------------------------------ launchers
#define DFL_T_DISPATCH(bf, KERNEL, grid, block, st, arg)                          \
  do {                                                                           \
    if (bf) hipLaunchKernelGGL(KERNEL<bf16>, grid, block, 0, st, arg);           \
    else hipLaunchKernelGGL(KERNEL<float>, grid, block, 0, st, arg);             \
  } while (0)

hipError_t launch_draft_plan(const PlanArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(draft_plan_kernel, dim3((a.n_seq + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_embed_pre(bool bf, const RowArgs& a, int rows, hipStream_t st) {
  DFL_T_DISPATCH(bf, embed_pre_kernel, dim3(rows), dim3(256), st, a);
  return hipGetLastError();
}
hipError_t launch_post_pre(bool bf, const RowArgs& a, int rows, hipStream_t st) {
  DFL_T_DISPATCH(bf, post_pre_kernel, dim3(rows), dim3(256), st, a);
  return hipGetLastError();
}
hipError_t launch_qkv_post(bool bf, const QkvArgs& a, int rows, hipStream_t st) {
  DFL_T_DISPATCH(bf, qkv_post_kernel, dim3(rows, a.nh + 2 * a.nkv), dim3(64), st, a);
  return hipGetLastError();
}
hipError_t launch_swiglu(bool bf, const SwigluArgs& a, hipStream_t st) {
  const size_t n = (size_t)a.M * a.f;
  DFL_T_DISPATCH(bf, swiglu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st, a);
  return hipGetLastError();
}
hipError_t launch_reduce_store(bool bf, const ReduceArgs& a, hipStream_t st) {
  const size_t n = (size_t)a.M * a.N;
  DFL_T_DISPATCH(bf, reduce_store_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st, a);
  return hipGetLastError();
}
hipError_t launch_inject_plan(const InjectArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(inject_plan_kernel, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_concat_norm(bool bf, const InjectArgs& a, int rows, hipStream_t st) {
  DFL_T_DISPATCH(bf, concat_norm_kernel, dim3(rows), dim3(256), st, a);
  return hipGetLastError();
}
hipError_t launch_kv_post(bool bf, const KvPostArgs& a, int rows, int heads, hipStream_t st) {
  DFL_T_DISPATCH(bf, kv_post_kernel, dim3(rows, heads), dim3(64), st, a);
  return hipGetLastError();
}
hipError_t launch_reset(const ResetArgs& a, hipStream_t st) {
  const int n = a.n > 0 ? a.n : 1;
  hipLaunchKernelGGL(reset_seqs_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_topk_merge(const MergeArgs& a, int out_rows, hipStream_t st) {
  hipLaunchKernelGGL(topk_merge_kernel, dim3(out_rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dfl
