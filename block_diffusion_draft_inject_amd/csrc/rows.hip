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
// The sequence's attention context (ring slots of the last min(L - base, window) positions).
__device__ __forceinline__ void plan_seq(const PlanArgs& a, int* dev_err, int b) {
  int sid = a.seq_ids[b];
  if (sid < 0 || sid >= a.max_seqs) {
    atomicOr(dev_err, 1);
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
// ------------------------------------------------------------------------ post + pre
// h_out[t] = h_in[t] + Conv_post(a)_t with a = sum of `splits` partials of the sublayer output,
// then y[t] = Conv_pre(RMSNorm(h_out))_t  (or, final: y[t] = RMSNorm(h_out[t]) * final gain).
// Row t needs a_{t-2}, a_{t-1}, a_t (the taps of row t-1 read a_{t-2}) and h_{t-1}, h_t.
// 512 threads, 4 consecutive elements each per 2048-wide slice (16-byte loads); every global
// load of the row -- residuals, all partials of the three rows, conv and norm weights -- is
// issued before the first use, so the kernel pays about one memory round trip.
constexpr int PP_T = 512;
constexpr int PP_MAXS = 8;   // k-splits of the producing GEMM (the planner keeps it <= 8)

__device__ __forceinline__ f32x4 ld4f(const float* p, size_t i) { return *reinterpret_cast<const f32x4*>(p + i); }
// Four consecutive weights as raw storage (loaded now, converted later).
template <typename T>
struct Raw4;
template <>
struct Raw4<float> {
  using type = f32x4;
  __device__ static type zero() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ static type load(const void* p, size_t i) { return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + i); }
  __device__ static f32x4 cvt(type v) { return v; }
};
template <>
struct Raw4<bf16> {
  using type = uint2;
  __device__ static type zero() { return uint2{0u, 0u}; }
  __device__ static type load(const void* p, size_t i) { return *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16*>(p) + i); }
  __device__ static f32x4 cvt(type u) {
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
  }
};

template <typename T>
__device__ __forceinline__ f32x4 ld4w(const void* p, size_t i) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + i);
  } else {
    const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16*>(p) + i);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
  }
}
// Four activations at i, rounded to bf16 for a bf16 GEMM input: the hi plane holds bf16(v),
// the lo plane zeros (fp32 drafters: v itself).
template <typename T>
__device__ __forceinline__ void st4_bf16_input(void* p, size_t i, size_t plane, f32x4 v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p) + i) = v;
  } else {
    uint2 uh;
    uh.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    uh.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16*>(p) + i) = uh;
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16*>(p) + i + plane) = uint2{0u, 0u};
  }
}
// Four activations at i (16-byte aligned): fp32, or the hi and lo bf16 planes.
template <typename T>
__device__ __forceinline__ void st4_act(void* p, size_t i, size_t plane, f32x4 v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p) + i) = v;
  } else {
    bf16 h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = f2bf(v[j]);
      l[j] = f2bf(v[j] - bf2f(h[j]));
    }
    uint2 uh, ul;
    uh.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    uh.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    ul.x = (uint32_t)l[0] | ((uint32_t)l[1] << 16);
    ul.y = (uint32_t)l[2] | ((uint32_t)l[3] << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16*>(p) + i) = uh;
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16*>(p) + i + plane) = ul;
  }
}
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

// MS: the largest k-split count the launch allows for (the loads of absent splits are not
// issued at all)
template <typename T, int NV, int MS>
__global__ __launch_bounds__(PP_T) void post_pre_kernel(RowArgs a) {
  __shared__ float red[8 * 4];
  const int row = xcd_row(blockIdx.x, gridDim.x), tid = threadIdx.x;
  const int t = row % a.K;
  const int d = a.d;
  const bool conv = a.use_conv != 0;
  const bool fin = a.final_norm != 0;
  const int q0 = conv ? max(0, 2 - t) : 2;       // first of rows t-2, t-1, t that exists
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  // Every load is issued, unconditionally and before any value is used, at an address that is
  // always valid (clamped index; the gain vector stands in for absent conv weights); values
  // that do not apply are masked afterwards.  A load under a condition makes the compiler wait
  // for it inside the condition, which would serialise the loads.
  using W4 = typename Raw4<T>::type;
  f32x4 hv[2][NV], pw[2][NV], qw[2][NV], g[NV];
  W4 rpw[2][NV], rqw[2][NV], rg[NV];
  f32x4 pv[MS][3][NV];
  const bool pre = conv && !fin;
  const void* pwp = conv ? a.post_w : a.pre_gain;
  const void* qwp = pre ? a.pre_w : a.pre_gain;
  const int wd = conv ? d : 0, qd = pre ? d : 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int k = (i * PP_T + tid) * 4;
    const int kc = k < d ? k : 0;
    hv[1][i] = ld4f(a.h_in, (size_t)row * d + kc);
    hv[0][i] = ld4f(a.h_in, (size_t)(t >= 1 ? row - 1 : row) * d + kc);
    rpw[0][i] = Raw4<T>::load(pwp, kc);
    rpw[1][i] = Raw4<T>::load(pwp, wd + kc);
    rqw[0][i] = Raw4<T>::load(qwp, kc);
    rqw[1][i] = Raw4<T>::load(qwp, qd + kc);
    rg[i] = Raw4<T>::load(a.pre_gain, kc);
  }
  // conv biases: raw, in the same burst (the gain stands in when absent)
  const T* pbp = reinterpret_cast<const T*>(conv ? a.post_b : a.pre_gain);
  const T* qbp = reinterpret_cast<const T*>(pre ? a.pre_b : a.pre_gain);
  const T rpb0 = pbp[0], rpb1 = pbp[1], rqb0 = qbp[0], rqb1 = qbp[1];
  const int nsp = max(a.splits, 1);
#pragma unroll
  for (int sp = 0; sp < MS; ++sp)
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int k = (i * PP_T + tid) * 4;
        const int kc = k < d ? k : 0;
        const int spc = min(sp, nsp - 1), qc = max(q, q0);
        pv[sp][q][i] = ld4f(a.part, ((size_t)spc * a.part_rows + (row - 2 + qc)) * d + kc);
      }
  // keep the burst together: without this fence the scheduler moves some partial loads down to
  // their additions (at 8 splits, one row slice: nine serial load round trips)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const bool in = (i * PP_T + tid) * 4 < d;
    if (!(in && conv && t >= 1)) hv[0][i] = z4;
    if (!in) hv[1][i] = z4;
#pragma unroll
    for (int sp = 0; sp < MS; ++sp)
#pragma unroll
      for (int q = 0; q < 3; ++q)
        if (!(in && sp < a.splits && q >= q0)) pv[sp][q][i] = z4;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const bool in = (i * PP_T + tid) * 4 < d;
    pw[0][i] = (in && conv) ? Raw4<T>::cvt(rpw[0][i]) : z4;
    pw[1][i] = (in && conv) ? Raw4<T>::cvt(rpw[1][i]) : z4;
    qw[0][i] = (in && pre) ? Raw4<T>::cvt(rqw[0][i]) : z4;
    qw[1][i] = (in && pre) ? Raw4<T>::cvt(rqw[1][i]) : z4;
    g[i] = in ? Raw4<T>::cvt(rg[i]) : z4;
  }
  const float pb0 = conv ? ldv(&rpb0, 0) : 0.f, pb1 = conv ? ldv(&rpb1, 0) : 0.f;
  const float qb0 = pre ? ldv(&rqb0, 0) : 0.f, qb1 = pre ? ldv(&rqb1, 0) : 0.f;
  f32x4 s[3][NV];
#pragma unroll
  for (int q = 0; q < 3; ++q)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      f32x4 acc = pv[0][q][i];
#pragma unroll
      for (int sp = 1; sp < MS; ++sp) acc += pv[sp][q][i];
      s[q][i] = acc;
    }
  // post-conv taps of rows t-1 and t
  float kp00 = 1.f, kp01 = 0.f, kp10 = 1.f, kp11 = 0.f;
  if (conv) {
    float dot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      dot[0] += dot4(pw[0][i], s[1][i]);
      dot[1] += dot4(pw[1][i], s[1][i]);
      dot[2] += dot4(pw[0][i], s[2][i]);
      dot[3] += dot4(pw[1][i], s[2][i]);
    }
    block_sum<4, PP_T>(dot, red);
    kp00 = sigmoidf_(dot[0] + pb0);
    kp01 = sigmoidf_(dot[1] + pb1);
    kp10 = sigmoidf_(dot[2] + pb0);
    kp11 = sigmoidf_(dot[3] + pb1);
  }
  float ss[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int k = (i * PP_T + tid) * 4;
    if (conv) {
      hv[0][i] += kp00 * s[1][i] + kp01 * s[0][i];   // row t-1 (s[0] is row t-2, zero if absent)
      hv[1][i] += kp10 * s[2][i] + kp11 * s[1][i];
    } else {
      hv[1][i] += s[2][i];
    }
    if (k < d) *reinterpret_cast<f32x4*>(a.h_out + (size_t)row * d + k) = hv[1][i];
    ss[0] += dot4(hv[0][i], hv[0][i]);
    ss[1] += dot4(hv[1][i], hv[1][i]);
  }
  block_sum<2, PP_T>(ss, red);
  const float r0 = rsqrtf(ss[0] / d + a.eps), r1 = rsqrtf(ss[1] / d + a.eps);
  if (fin) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int k = (i * PP_T + tid) * 4;
      if (k < d) {
        const f32x4 o = hv[1][i] * r1 * g[i];
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.y) + (size_t)row * a.ldy + k) = o;
        st4_bf16_input<T>(a.y2, (size_t)row * a.ldy + k, a.y_plane, o);   // the lm_head takes bf16(h_f)
      }
    }
    return;
  }
  float dot[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    hv[0][i] = (t >= 1) ? hv[0][i] * r0 * g[i] : z4;
    hv[1][i] = hv[1][i] * r1 * g[i];
    dot[0] += dot4(qw[0][i], hv[1][i]);
    dot[1] += dot4(qw[1][i], hv[1][i]);
  }
  float k0 = 1.f, k1 = 0.f;
  if (conv) {
    block_sum<2, PP_T>(dot, red);
    k0 = sigmoidf_(dot[0] + qb0);
    k1 = sigmoidf_(dot[1] + qb1);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int k = (i * PP_T + tid) * 4;
    if (k < d) st4_act<T>(a.y, (size_t)row * a.ldy + k, a.y_plane, k0 * hv[1][i] + k1 * hv[0][i]);
  }
}

// ------------------------------------------------------------------------ per-channel conv
// The page's form of the two-tap conv ("Architecture", section "Problem 2 -- Suffix decay is
// local"): Conv(x)_t = k_t0 (.) x_t + k_t1 (.) x_{t-1} with per-channel coefficients
// k_tj[c] = sigmoid(base_j[c] + corr_tj[c / G]), a learned base kernel per channel plus a correction
// W_c x_t from the current row shared by each run of G channels.  The corrections come from a
// GEMM launched before (k-split partials, summed here in split order); a thread's 4 consecutive
// channels share one group (G % 4 == 0).

// Four activations at i: fp32, or the sum of the hi and lo bf16 planes.
template <typename T>
__device__ __forceinline__ f32x4 ld4_act(const void* p, size_t i, size_t plane) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + i);
  } else {
    const uint2 h = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16*>(p) + i);
    const uint2 l = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16*>(p) + i + plane);
    return f32x4{__uint_as_float(h.x << 16), __uint_as_float(h.x & 0xffff0000u), __uint_as_float(h.y << 16),
                 __uint_as_float(h.y & 0xffff0000u)} +
           f32x4{__uint_as_float(l.x << 16), __uint_as_float(l.x & 0xffff0000u), __uint_as_float(l.y << 16),
                 __uint_as_float(l.y & 0xffff0000u)};
  }
}

constexpr int PC_MAXS = 8;   // correction k-splits summed (the planner keeps it <= 8)

// corr_t0 and corr_t1 of the group holding channel k of row `row` (all split loads in one burst)
__device__ __forceinline__ void pc_corr(const PcArgs& a, int row, int k, float& c0, float& c1) {
  const int ng = a.d / a.G, N = 2 * ng, grp = k / a.G;
  float p0[PC_MAXS], p1[PC_MAXS];
#pragma unroll
  for (int s = 0; s < PC_MAXS; ++s) {
    const float* pr = a.part + ((size_t)min(s, a.splits - 1) * a.part_rows + row) * N;
    p0[s] = pr[grp];
    p1[s] = pr[ng + grp];
  }
  c0 = c1 = 0.f;
#pragma unroll
  for (int s = 0; s < PC_MAXS; ++s)
    if (s < a.splits) {
      c0 += p0[s];
      c1 += p1[s];
    }
}

__device__ __forceinline__ f32x4 sig4(f32x4 b, float c) {
  return f32x4{sigmoidf_(b[0] + c), sigmoidf_(b[1] + c), sigmoidf_(b[2] + c), sigmoidf_(b[3] + c)};
}

// Sublayer epilogue with the per-channel post-conv: h_out[t] = h_in[t] + k_t0 (.) a_t + k_t1 (.) a_{t-1}
// (a = x, the reduced sublayer output), then z = RMSNorm(h_out[t]) * gain -> out (activation
// planes), or, final: out = h_f (fp32) and out2 = bf16(h_f) for the lm_head.
template <typename T, int NV>
__global__ __launch_bounds__(PP_T) void post_pre_pc_kernel(PcArgs a) {
  __shared__ float red[(PP_T / 64) * 1];
  const int row = xcd_row(blockIdx.x, gridDim.x), tid = threadIdx.x, t = row % a.K, d = a.d;
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 h[NV], xt[NV], xq[NV], b0[NV], b1[NV], g[NV];
  float c0[NV], c1[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int k = (i * PP_T + tid) * 4;
    const int kc = k < d ? k : 0;
    h[i] = ld4f(a.h_in, (size_t)row * d + kc);
    xt[i] = ld4_act<T>(a.x, (size_t)row * d + kc, a.plane);
    xq[i] = ld4_act<T>(a.x, (size_t)(t >= 1 ? row - 1 : row) * d + kc, a.plane);
    b0[i] = ld4w<T>(a.base, kc);
    b1[i] = ld4w<T>(a.base, (size_t)d + kc);
    g[i] = ld4w<T>(a.gain, kc);
    pc_corr(a, row, kc, c0[i], c1[i]);
  }
  float ss[1] = {0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int k = (i * PP_T + tid) * 4;
    if (k >= d) { h[i] = z4; continue; }
    const f32x4 k0 = sig4(b0[i], c0[i]), k1 = sig4(b1[i], c1[i]);
    h[i] += k0 * xt[i] + (t >= 1 ? k1 * xq[i] : z4);
    *reinterpret_cast<f32x4*>(a.h_out + (size_t)row * d + k) = h[i];
    ss[0] += dot4(h[i], h[i]);
  }
  block_sum<1, PP_T>(ss, red);
  const float r = rsqrtf(ss[0] / d + a.eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int k = (i * PP_T + tid) * 4;
    if (k >= d) continue;
    const f32x4 o = h[i] * r * g[i];
    if (a.final_norm) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + (size_t)row * a.ldo + k) = o;
      st4_bf16_input<T>(a.out2, (size_t)row * a.ldo + k, a.plane, o);   // the lm_head takes bf16(h_f)
    } else {
      st4_act<T>(a.out, (size_t)row * a.ldo + k, a.plane, o);
    }
  }
}

// Pre-conv: y_t = k_t0 (.) z_t + k_t1 (.) z_{t-1} (z = x, the normed rows) -> out (activation planes).
template <typename T, int NV>
__global__ __launch_bounds__(PP_T) void conv_apply_kernel(PcArgs a) {
  const int row = xcd_row(blockIdx.x, gridDim.x), tid = threadIdx.x, t = row % a.K, d = a.d;
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 xt[NV], xq[NV], b0[NV], b1[NV];
  float c0[NV], c1[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int k = (i * PP_T + tid) * 4;
    const int kc = k < d ? k : 0;
    xt[i] = ld4_act<T>(a.x, (size_t)row * d + kc, a.plane);
    xq[i] = ld4_act<T>(a.x, (size_t)(t >= 1 ? row - 1 : row) * d + kc, a.plane);
    b0[i] = ld4w<T>(a.base, kc);
    b1[i] = ld4w<T>(a.base, (size_t)d + kc);
    pc_corr(a, row, kc, c0[i], c1[i]);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int k = (i * PP_T + tid) * 4;
    if (k >= d) continue;
    const f32x4 y = sig4(b0[i], c0[i]) * xt[i] + (t >= 1 ? sig4(b1[i], c1[i]) * xq[i] : z4);
    st4_act<T>(a.out, (size_t)row * a.ldo + k, a.plane, y);
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
  {
    // all split loads in one burst at valid addresses (clamped split and lane), masked after
    constexpr int QS = 8;
    const int hl = act ? lane : 0;
    float p0[QS], p1[QS];
#pragma unroll
    for (int sp = 0; sp < QS; ++sp) {
      const float* pr = a.part + ((size_t)min(sp, a.splits - 1) * a.part_rows + row) * a.N + col0;
      p0[sp] = pr[hl];
      p1[sp] = pr[hl + half];
    }
#pragma unroll
    for (int sp = 0; sp < QS; ++sp) {
      if (sp < a.splits) {
        x0 += p0[sp];
        x1 += p1[sp];
      }
    }
    if (!act) x0 = x1 = 0.f;
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
    if (gain_kind == 0) {
      st_act(dst, off + lane, a.q_plane, x0);
      st_act(dst, off + lane + half, a.q_plane, x1);
    } else {
      stv(dst, off + lane, x0);
      stv(dst, off + lane + half, x1);
    }
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
  st_act(reinterpret_cast<T*>(a.out), m * a.f + j, a.out_plane, g / (1.f + __expf(-g)) * u);
}

// Four consecutive outputs of one row per thread (f a multiple of 4).  Every split's gate and up
// vectors are requested before any is summed: the split index is clamped so that each load is
// unconditional, and absent splits are masked afterwards (a load under a condition would be
// waited for inside it).  The sums run in split order from zero, as in the one-element form, so
// the results are the same bits; each plane takes one 8-byte (bf16) or 16-byte (fp32) store.
__device__ __forceinline__ void st_act4(bf16* p, size_t i, size_t plane, const float (&v)[4]) {
  unsigned hw[2], lw[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bf16 h0 = f2bf(v[2 * h]), h1 = f2bf(v[2 * h + 1]);
    const bf16 l0 = f2bf(v[2 * h] - bf2f(h0)), l1 = f2bf(v[2 * h + 1] - bf2f(h1));
    hw[h] = (unsigned)h0 | ((unsigned)h1 << 16);
    lw[h] = (unsigned)l0 | ((unsigned)l1 << 16);
  }
  *reinterpret_cast<uint2*>(p + i) = make_uint2(hw[0], hw[1]);
  *reinterpret_cast<uint2*>(p + i + plane) = make_uint2(lw[0], lw[1]);
}
__device__ __forceinline__ void st_act4(float* p, size_t i, size_t, const float (&v)[4]) {
  *reinterpret_cast<f32x4*>(p + i) = f32x4{v[0], v[1], v[2], v[3]};
}
template <typename T, int MS>
__global__ __launch_bounds__(256) void swiglu4_kernel(SwigluArgs a) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (size_t)a.M * a.f) return;
  const size_t m = i / a.f, j = i % a.f;
  f32x4 g[MS], u[MS];
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) {
    const float* pr = a.part + ((size_t)min(sp, a.splits - 1) * a.part_rows + m) * (2 * a.f) + j;
    g[sp] = *reinterpret_cast<const f32x4*>(pr);
    u[sp] = *reinterpret_cast<const f32x4*>(pr + a.f);
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 gs = {0.f, 0.f, 0.f, 0.f}, us = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < MS; ++sp)
    if (sp < a.splits) {
      gs += g[sp];
      us += u[sp];
    }
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = gs[e] / (1.f + __expf(-gs[e])) * us[e];
  st_act4(reinterpret_cast<T*>(a.out), m * a.f + j, a.out_plane, v);
}

// ------------------------------------------------------------------------ sum partials -> T
template <typename T>
__global__ __launch_bounds__(256) void reduce_store_kernel(ReduceArgs a) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int Mv = a.m_dev ? max(0, min(a.M, *a.m_dev - a.m_off)) : a.M;
  if (i >= (size_t)Mv * a.N) return;
  float acc = 0.f;
  for (int sp = 0; sp < a.splits; ++sp) acc += a.part[(size_t)sp * a.part_rows * a.N + i];
  st_act(reinterpret_cast<T*>(a.out), i, a.out_plane, acc);
}

// Four consecutive outputs per thread (N a multiple of 4), the splits' loads unconditional and
// requested before the sums, summed in split order from zero (the same bits as above).
template <typename T, int MS>
__global__ __launch_bounds__(256) void reduce_store4_kernel(ReduceArgs a) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int Mv = a.m_dev ? max(0, min(a.M, *a.m_dev - a.m_off)) : a.M;
  if (i >= (size_t)Mv * a.N) return;
  f32x4 p[MS];
#pragma unroll
  for (int sp = 0; sp < MS; ++sp)
    p[sp] = *reinterpret_cast<const f32x4*>(a.part + (size_t)min(sp, a.splits - 1) * a.part_rows * a.N + i);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < MS; ++sp)
    if (sp < a.splits) acc += p[sp];
  const float v[4] = {acc[0], acc[1], acc[2], acc[3]};
  st_act4(reinterpret_cast<T*>(a.out), i, a.out_plane, v);
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
// ū = RMSNorm(u) * g over the concatenated tapped states of one injected row.  One workgroup
// per row: the row's sequence is found by every thread testing one sequence's row range (all
// bookkeeping loads at once), then the whole row (NVC 16-byte vectors per thread) and the gain
// are loaded in one burst and kept in registers for the scaling pass.
constexpr int CN_T = 512;
template <typename T, int NVC>
__global__ __launch_bounds__(CN_T) void concat_norm_kernel(InjectArgs a) {
  __shared__ float red[(CN_T / 64) * 1];
  __shared__ int s_i, s_r, s_skip;
  const int j = a.chunk0 + blockIdx.x, tid = threadIdx.x;
  const int lr = blockIdx.x;
  const int total = *a.total;
  for (int i = tid; i < a.n_seq; i += CN_T) {
    const int o0 = a.row_off[i], o1 = a.row_off[i + 1], sk = a.row_skip[i], st0 = a.row_start[i], sid = a.seq_ids[i];
    if (o0 <= j && j < o1) {
      s_i = i;
      s_r = j - o0;
      s_skip = sk;
      a.meta_seq[lr] = sid;
      a.meta_pos[lr] = st0 + (j - o0);
    }
  }
  if (j >= total) {
    if (tid == 0) { a.meta_seq[lr] = -1; a.meta_pos[lr] = 0; }
    return;
  }
  __syncthreads();
  const int i = s_i, r = s_r, skip = s_skip;
  const int W = a.concat;
  constexpr int VE = 16 / sizeof(T);          // elements per 16-byte vector
  const int nv = W / VE;                      // W % VE == 0 (checked on the host)
  const u32x4* sv = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.states) + ((size_t)i * a.max_new + r + skip) * W);
  const u32x4* gv = reinterpret_cast<const u32x4*>(a.gain);
  u32x4 x[NVC], g[NVC];
#pragma unroll
  for (int u = 0; u < NVC; ++u) {
    const int v = min(u * CN_T + tid, nv - 1);
    x[u] = sv[v];
    g[u] = gv[v];
  }
  float ss[1] = {0.f};
#pragma unroll
  for (int u = 0; u < NVC; ++u) {
    if (u * CN_T + tid >= nv) continue;
    const T* e = reinterpret_cast<const T*>(&x[u]);
#pragma unroll
    for (int q = 0; q < VE; ++q) {
      const float f = ldv(e, q);
      ss[0] += f * f;
    }
  }
  block_sum<1, CN_T>(ss, red);
  const float rs = rsqrtf(ss[0] / W + a.eps);
  T* dst = reinterpret_cast<T*>(a.ubar) + (size_t)lr * W;
#pragma unroll
  for (int u = 0; u < NVC; ++u) {
    const int v = u * CN_T + tid;
    if (v >= nv) continue;
    const T* e = reinterpret_cast<const T*>(&x[u]);
    const T* ge = reinterpret_cast<const T*>(&g[u]);
#pragma unroll
    for (int q = 0; q < VE; q += 4)
      st4_act<T>(dst, (size_t)v * VE + q, a.ubar_plane,
                 f32x4{ldv(e, q) * rs * ldv(ge, q), ldv(e, q + 1) * rs * ldv(ge, q + 1),
                       ldv(e, q + 2) * rs * ldv(ge, q + 2), ldv(e, q + 3) * rs * ldv(ge, q + 3)});
  }
}

// Block embed + layer 0's attention pre-norm and pre-conv: h = E[x] with x = [anchor, MASK, ...];
// z = RMSNorm(h) * g; y_t = k_t0 z_t + k_t1 z_{t-1}, k_t = sigmoid(W_c z_t + b_c) (z_{-1} = 0).
// PP_T threads, 4 elements each; all loads (two embedding rows, gain, conv weights) in one burst.
template <typename T, int NV>
__global__ __launch_bounds__(PP_T) void embed_pre_kernel(RowArgs a) {
  __shared__ float red[(PP_T / 64) * 2];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int b = row / a.K, t = row % a.K;
  const int d = a.d;
  // the call's plan (read only by later kernels of the call)
  if (t == 0 && tid == 0) plan_seq(a.plan, a.dev_err, b);
  if (row == 0 && tid < NCOUNTERS && a.plan.counters) a.plan.counters[tid] = 0;
  int anchor = a.anchor[b];
  if (anchor < 0 || anchor >= a.vocab) {   // out-of-range token: record and read row 0
    if (tid == 0 && t == 0) atomicOr(a.dev_err, 8);
    anchor = 0;
  }
  const int id_t = (t == 0) ? anchor : a.mask_id;
  const int id_p = (t <= 1) ? anchor : a.mask_id;
  const bool conv = a.use_conv != 0;
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  using W4 = typename Raw4<T>::type;
  W4 re[2][NV], rg[NV], rw[2][NV];
  const void* wp = conv ? a.pre_w : a.pre_gain;   // the gain stands in for absent conv weights
  const int wd = conv ? d : 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int k = (i * PP_T + tid) * 4;
    const int kc = k < d ? k : 0;
    re[0][i] = Raw4<T>::load(a.embed, (size_t)id_t * d + kc);
    re[1][i] = Raw4<T>::load(a.embed, (size_t)id_p * d + kc);
    rg[i] = Raw4<T>::load(a.pre_gain, kc);
    rw[0][i] = Raw4<T>::load(wp, kc);
    rw[1][i] = Raw4<T>::load(wp, wd + kc);
  }
  const float pb0 = conv ? ldw<T>(a.pre_b, 0) : 0.f, pb1 = conv ? ldw<T>(a.pre_b, 1) : 0.f;
  f32x4 e[2][NV], g[NV];
  float ss[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int k = (i * PP_T + tid) * 4;
    const bool in = k < d;
    e[0][i] = in ? Raw4<T>::cvt(re[0][i]) : z4;
    e[1][i] = (in && t > 0) ? Raw4<T>::cvt(re[1][i]) : z4;
    g[i] = in ? Raw4<T>::cvt(rg[i]) : z4;
    ss[0] += dot4(e[0][i], e[0][i]);
    ss[1] += dot4(e[1][i], e[1][i]);
    if (in) *reinterpret_cast<f32x4*>(a.h_out + (size_t)row * d + k) = e[0][i];
  }
  block_sum<2, PP_T>(ss, red);
  const float r0 = rsqrtf(ss[0] / d + a.eps), r1 = rsqrtf(ss[1] / d + a.eps);
  float dot[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int k = (i * PP_T + tid) * 4;
    const bool in = k < d;
    e[0][i] = e[0][i] * r0 * g[i];
    e[1][i] = e[1][i] * r1 * g[i];
    if (conv && in) {
      dot[0] += dot4(Raw4<T>::cvt(rw[0][i]), e[0][i]);
      dot[1] += dot4(Raw4<T>::cvt(rw[1][i]), e[0][i]);
    }
  }
  float k0 = 1.f, k1 = 0.f;
  if (conv) {
    block_sum<2, PP_T>(dot, red);
    k0 = sigmoidf_(dot[0] + pb0);
    k1 = sigmoidf_(dot[1] + pb1);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int k = (i * PP_T + tid) * 4;
    if (k < d) st4_act<T>(a.y, (size_t)row * a.ldy + k, a.y_plane, k0 * e[0][i] + k1 * e[1][i]);
  }
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
// One workgroup per output row (seq, slot >= 1).  Candidates are either sorted lists of 16
// (ids != nullptr: one list per lm_head workgroup) or raw values with id = index (fp32 path,
// first reduced to one sorted list per thread).  Lists are then reduced pairwise in LDS by
// merge-path: an entry's position in the merged list is its own index plus the number of
// entries of the other list that beat it (the order is total: ids are distinct), so 32 lanes
// merge two lists in one step.
// Number of entries of a 16-entry LDS list that beat (x, xi); the list is read with 128-bit
// LDS loads issued together (scalar reads would each wait out the LDS latency).
__device__ __forceinline__ int count_better(const float* lv, const int* li, float x, int xi) {
  f32x4 v[4];
  u32x4 d[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = reinterpret_cast<const f32x4*>(lv)[q];
    d[q] = reinterpret_cast<const u32x4*>(li)[q];
  }
  int n = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) n += cand_better(v[q][j], (int)d[q][j], x, xi) ? 1 : 0;
  return n;
}

// Best (value, id) candidate of the wave under cand_better, the same in every lane (all 64
// lanes active).  DPP steps inside each row of 16 lanes, then the four row winners are compared
// through readlane.
__device__ __forceinline__ void wave_best_dpp(float& v, int& id) {
  auto step = [&](float ov, int oi) {
    const bool take = cand_better(ov, oi, v, id);
    v = take ? ov : v;
    id = take ? oi : id;
  };
  step(dpp_f<0xB1>(v), dpp_i<0xB1>(id));
  step(dpp_f<0x4E>(v), dpp_i<0x4E>(id));
  step(dpp_f<0x141>(v), dpp_i<0x141>(id));
  step(dpp_f<0x140>(v), dpp_i<0x140>(id));
  float bv = lane_f(v, 0);
  int bi = __builtin_amdgcn_readlane(id, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const float ov = lane_f(v, r);
    const int oi = __builtin_amdgcn_readlane(id, r);
    const bool take = cand_better(ov, oi, bv, bi);
    bv = take ? ov : bv;
    bi = take ? oi : bi;
  }
  v = bv;
  id = bi;
}

// List mode with at most 256 lists: thread t holds list t (sorted).  Each wave extracts its
// own best 16 in 16 rounds of a wave-wide arg-best (the winning lane shifts its list by one),
// the four wave results go through LDS, and wave 0 places each of those 64 by its rank: lane
// (l, i) holds entry i of wave l's sorted list, and its rank is i plus the entries of the
// other three lists that beat it; ranks below 16 are the output slots.  (Ids are distinct, so
// real candidates get distinct ranks; padding entries all equal (-inf, none) and those that
// collide write the same value, covering every slot after the real ones.)
__global__ __launch_bounds__(256) void topk_merge_lists_kernel(MergeArgs a) {
  __shared__ __attribute__((aligned(16))) float wv[4][TOPK];
  __shared__ __attribute__((aligned(16))) int wi[4][TOPK];
  const int orow = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = orow / (a.K - 1), t = orow % (a.K - 1) + 1;
  if (orow == 0 && tid < NCOUNTERS && a.counters) a.counters[tid] = 0;
  const size_t in_row = (size_t)b * a.K + t;
  const int nl = a.ncand / TOPK;
  float v[TOPK];
  int id[TOPK];
  {
    const int l = min(tid, nl - 1);
    const f32x4* pv = reinterpret_cast<const f32x4*>(a.vals + in_row * a.ncand + (size_t)l * TOPK);
    const u32x4* pi = reinterpret_cast<const u32x4*>(a.ids + in_row * a.ncand + (size_t)l * TOPK);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = pv[q];
      const u32x4 y = pi[q];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[4 * q + j] = tid < nl ? x[j] : NEG_INF;
        id[4 * q + j] = tid < nl ? (int)y[j] : ID_NONE;
      }
    }
  }
#pragma unroll 1
  for (int r = 0; r < TOPK; ++r) {
    float bv = v[0];
    int bi = id[0];
    wave_best_dpp(bv, bi);
    if (lane == r) { wv[w][r] = bv; wi[w][r] = bi; }
    if (id[0] == bi && v[0] == bv) {           // the winning lane (ids are distinct)
#pragma unroll
      for (int i = 0; i + 1 < TOPK; ++i) { v[i] = v[i + 1]; id[i] = id[i + 1]; }
      v[TOPK - 1] = NEG_INF;
      id[TOPK - 1] = ID_NONE;
    }
  }
  __syncthreads();
  if (w != 0) return;
  const int l = lane >> 4, i = lane & (TOPK - 1);
  const float cv = wv[l][i];
  const int ci = wi[l][i];
  int rank = i;
#pragma unroll
  for (int o = 1; o < 4; ++o) {
    const int l2 = (l + o) & 3;
    rank += count_better(wv[l2], wi[l2], cv, ci);
  }
  if (rank < TOPK) {
    a.out_ids[(size_t)orow * TOPK + rank] = ci;
    a.out_vals[(size_t)orow * TOPK + rank] = cv;
  }
}

__global__ __launch_bounds__(256) void topk_merge_kernel(MergeArgs a) {
  __shared__ __attribute__((aligned(16))) float sv[2][256][TOPK];
  __shared__ __attribute__((aligned(16))) int si[2][256][TOPK];
  const int orow = blockIdx.x, tid = threadIdx.x;
  const int b = orow / (a.K - 1), t = orow % (a.K - 1) + 1;
  if (orow == 0 && tid < NCOUNTERS && a.counters) a.counters[tid] = 0;
  const size_t in_row = (size_t)b * a.K + t;
  const float* v = a.vals + in_row * a.ncand;
  const int* id = a.ids ? a.ids + in_row * a.ncand : nullptr;
  int have = 0;        // lists already in sv[0] (a carried partial result)
  int nl;
  if (!id) {
    if (a.logits_out) {
      float* lo = a.logits_out + (size_t)orow * a.ncand;
      for (int c = tid; c < a.ncand; c += 256) lo[c] = v[c];
    }
    Top16 top;
    top.init();
#pragma unroll 1
    for (int c = tid; c < a.ncand; c += 256) top.push(v[c], c);
#pragma unroll
    for (int j = 0; j < TOPK; ++j) { sv[0][tid][j] = top.v[j]; si[0][tid][j] = top.id[j]; }
    nl = 0;
    have = 256;
  } else {
    nl = a.ncand / TOPK;
  }
  int g0 = 0;
  do {
    const int take = min(nl - g0, 256 - have);
    if (tid < take) {
      const f32x4* pv = reinterpret_cast<const f32x4*>(v + (size_t)(g0 + tid) * TOPK);
      const u32x4* pi = reinterpret_cast<const u32x4*>(id + (size_t)(g0 + tid) * TOPK);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 x = pv[q];
        const u32x4 y = pi[q];
#pragma unroll
        for (int j = 0; j < 4; ++j) { sv[0][have + tid][4 * q + j] = x[j]; si[0][have + tid][4 * q + j] = (int)y[j]; }
      }
    }
    __syncthreads();
    int n = have + take, cur = 0;
    while (n > 1) {
      const int pairs = n / 2;
      for (int p0 = 0; p0 < pairs; p0 += 8) {
        const int pr = p0 + (tid >> 5), e = tid & 31;
        if (pr < pairs) {
          const int A = 2 * pr, Bl = 2 * pr + 1;
          const int own = e < TOPK ? A : Bl, oth = e < TOPK ? Bl : A, ei = e & (TOPK - 1);
          const float x = sv[cur][own][ei];
          const int xi = si[cur][own][ei];
          const int rank = ei + count_better(sv[cur][oth], si[cur][oth], x, xi);
          if (rank < TOPK) { sv[cur ^ 1][pr][rank] = x; si[cur ^ 1][pr][rank] = xi; }
        }
      }
      if ((n & 1) && tid < TOPK) {
        sv[cur ^ 1][pairs][tid] = sv[cur][n - 1][tid];
        si[cur ^ 1][pairs][tid] = si[cur][n - 1][tid];
      }
      __syncthreads();
      n = pairs + (n & 1);
      cur ^= 1;
    }
    if (cur == 1 && tid < TOPK) { sv[0][0][tid] = sv[1][0][tid]; si[0][0][tid] = si[1][0][tid]; }
    __syncthreads();
    have = 1;
    g0 += take;
  } while (g0 < nl);
  if (tid < TOPK) {
    a.out_ids[(size_t)orow * TOPK + tid] = si[0][0][tid];
    a.out_vals[(size_t)orow * TOPK + tid] = sv[0][0][tid];
  }
}

// ------------------------------------------------------------------------ selector context gate
// ------------------------------------------------------------------------ launchers
#define DFL_T_DISPATCH(bf, KERNEL, grid, block, st, arg)                          \
  do {                                                                           \
    if (bf) hipLaunchKernelGGL(KERNEL<bf16>, grid, block, 0, st, arg);           \
    else hipLaunchKernelGGL(KERNEL<float>, grid, block, 0, st, arg);             \
  } while (0)

hipError_t launch_embed_pre(bool bf, const RowArgs& a, int rows, hipStream_t st) {
  if (a.d % 4) return hipErrorInvalidValue;
  const int v = (a.d + 4 * PP_T - 1) / (4 * PP_T);
  if (v <= 1) {
    if (bf) hipLaunchKernelGGL((embed_pre_kernel<bf16, 1>), dim3(rows), dim3(PP_T), 0, st, a);
    else hipLaunchKernelGGL((embed_pre_kernel<float, 1>), dim3(rows), dim3(PP_T), 0, st, a);
  } else if (v <= 2) {
    if (bf) hipLaunchKernelGGL((embed_pre_kernel<bf16, 2>), dim3(rows), dim3(PP_T), 0, st, a);
    else hipLaunchKernelGGL((embed_pre_kernel<float, 2>), dim3(rows), dim3(PP_T), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <int NV, int MS>
static void launch_pp(bool bf, const RowArgs& a, int rows, hipStream_t st) {
  if (bf) hipLaunchKernelGGL((post_pre_kernel<bf16, NV, MS>), dim3(rows), dim3(PP_T), 0, st, a);
  else hipLaunchKernelGGL((post_pre_kernel<float, NV, MS>), dim3(rows), dim3(PP_T), 0, st, a);
}
template <int NV>
static void launch_pp_s(bool bf, const RowArgs& a, int rows, hipStream_t st) {
  if (a.splits <= 1) launch_pp<NV, 1>(bf, a, rows, st);
  else if (a.splits <= 2) launch_pp<NV, 2>(bf, a, rows, st);
  else if (a.splits <= 3) launch_pp<NV, 3>(bf, a, rows, st);
  else if (a.splits <= 4) launch_pp<NV, 4>(bf, a, rows, st);
  else if (a.splits <= 6) launch_pp<NV, 6>(bf, a, rows, st);
  else launch_pp<NV, PP_MAXS>(bf, a, rows, st);
}
hipError_t launch_post_pre(bool bf, const RowArgs& a, int rows, hipStream_t st) {
  if (a.splits > PP_MAXS || a.d % 4) return hipErrorInvalidValue;
  const int v = (a.d + 4 * PP_T - 1) / (4 * PP_T);
  if (v <= 1) launch_pp_s<1>(bf, a, rows, st);
  else if (v <= 2) launch_pp_s<2>(bf, a, rows, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
hipError_t launch_post_pre_pc(bool bf, const PcArgs& a, int rows, hipStream_t st) {
  if (a.d % 4 || a.G % 4 || a.d % a.G || a.splits < 1 || a.splits > PC_MAXS) return hipErrorInvalidValue;
  const int v = (a.d + 4 * PP_T - 1) / (4 * PP_T);
  if (v <= 1) {
    if (bf) hipLaunchKernelGGL((post_pre_pc_kernel<bf16, 1>), dim3(rows), dim3(PP_T), 0, st, a);
    else hipLaunchKernelGGL((post_pre_pc_kernel<float, 1>), dim3(rows), dim3(PP_T), 0, st, a);
  } else if (v <= 2) {
    if (bf) hipLaunchKernelGGL((post_pre_pc_kernel<bf16, 2>), dim3(rows), dim3(PP_T), 0, st, a);
    else hipLaunchKernelGGL((post_pre_pc_kernel<float, 2>), dim3(rows), dim3(PP_T), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
hipError_t launch_conv_apply(bool bf, const PcArgs& a, int rows, hipStream_t st) {
  if (a.d % 4 || a.G % 4 || a.d % a.G || a.splits < 1 || a.splits > PC_MAXS) return hipErrorInvalidValue;
  const int v = (a.d + 4 * PP_T - 1) / (4 * PP_T);
  if (v <= 1) {
    if (bf) hipLaunchKernelGGL((conv_apply_kernel<bf16, 1>), dim3(rows), dim3(PP_T), 0, st, a);
    else hipLaunchKernelGGL((conv_apply_kernel<float, 1>), dim3(rows), dim3(PP_T), 0, st, a);
  } else if (v <= 2) {
    if (bf) hipLaunchKernelGGL((conv_apply_kernel<bf16, 2>), dim3(rows), dim3(PP_T), 0, st, a);
    else hipLaunchKernelGGL((conv_apply_kernel<float, 2>), dim3(rows), dim3(PP_T), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
hipError_t launch_qkv_post(bool bf, const QkvArgs& a, int rows, hipStream_t st) {
  if (a.splits < 1 || a.splits > 8) return hipErrorInvalidValue;
  DFL_T_DISPATCH(bf, qkv_post_kernel, dim3(rows, a.nh + 2 * a.nkv), dim3(64), st, a);
  return hipGetLastError();
}
template <int MS>
static void launch_swiglu4(bool bf, const SwigluArgs& a, hipStream_t st) {
  const size_t n4 = (size_t)a.M * a.f / 4;
  const dim3 grid((unsigned)((n4 + 255) / 256));
  if (bf) hipLaunchKernelGGL((swiglu4_kernel<bf16, MS>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((swiglu4_kernel<float, MS>), grid, dim3(256), 0, st, a);
}
hipError_t launch_swiglu(bool bf, const SwigluArgs& a, hipStream_t st) {
  const size_t n = (size_t)a.M * a.f;
  if (a.splits < 1) return hipErrorInvalidValue;
  // the four-wide form needs whole vectors of one row and 16-byte aligned partial rows; the
  // output planes are then 8-byte aligned (plane = a multiple of f)
  const bool v4 = a.f % 4 == 0 && a.out_plane % 4 == 0 && a.splits <= 8;
  if (v4 && a.splits <= 2) launch_swiglu4<2>(bf, a, st);
  else if (v4 && a.splits <= 4) launch_swiglu4<4>(bf, a, st);
  else if (v4) launch_swiglu4<8>(bf, a, st);
  else DFL_T_DISPATCH(bf, swiglu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st, a);
  return hipGetLastError();
}
template <int MS>
static void launch_reduce_store4(bool bf, const ReduceArgs& a, hipStream_t st) {
  const size_t n4 = (size_t)a.M * a.N / 4;
  const dim3 grid((unsigned)((n4 + 255) / 256));
  if (bf) hipLaunchKernelGGL((reduce_store4_kernel<bf16, MS>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((reduce_store4_kernel<float, MS>), grid, dim3(256), 0, st, a);
}
hipError_t launch_reduce_store(bool bf, const ReduceArgs& a, hipStream_t st) {
  const size_t n = (size_t)a.M * a.N;
  if (a.splits < 1) return hipErrorInvalidValue;
  const bool v4 = a.N % 4 == 0 && a.out_plane % 4 == 0 && a.splits <= 8;
  if (v4 && a.splits <= 2) launch_reduce_store4<2>(bf, a, st);
  else if (v4 && a.splits <= 4) launch_reduce_store4<4>(bf, a, st);
  else if (v4) launch_reduce_store4<8>(bf, a, st);
  else DFL_T_DISPATCH(bf, reduce_store_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st, a);
  return hipGetLastError();
}
hipError_t launch_inject_plan(const InjectArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(inject_plan_kernel, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}
template <int NVC>
static void launch_cn(bool bf, const InjectArgs& a, int rows, hipStream_t st) {
  if (bf) hipLaunchKernelGGL((concat_norm_kernel<bf16, NVC>), dim3(rows), dim3(CN_T), 0, st, a);
  else hipLaunchKernelGGL((concat_norm_kernel<float, NVC>), dim3(rows), dim3(CN_T), 0, st, a);
}
hipError_t launch_concat_norm(bool bf, const InjectArgs& a, int rows, hipStream_t st) {
  const int nv = a.concat / (bf ? 8 : 4);
  const int per = (nv + CN_T - 1) / CN_T;
  if (per <= 1) launch_cn<1>(bf, a, rows, st);
  else if (per <= 2) launch_cn<2>(bf, a, rows, st);
  else if (per <= 4) launch_cn<4>(bf, a, rows, st);
  else if (per <= 8) launch_cn<8>(bf, a, rows, st);
  else if (per <= 16) launch_cn<16>(bf, a, rows, st);
  else return hipErrorInvalidValue;
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
  if (a.ids && a.ncand / TOPK <= 256) hipLaunchKernelGGL(topk_merge_lists_kernel, dim3(out_rows), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(topk_merge_kernel, dim3(out_rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------------ FP8 weight rows
// E4M3 codes (OCP 8-bit floating point: bias 7, 3 mantissa bits, largest finite 448,
// subnormals m * 2^-9) of a bf16 weight matrix, one power-of-two scale per row: the row's
// largest magnitude a maps into (224, 448] (scale = 2^k, k the smallest integer with
// a <= 448 * 2^k), each weight becomes the code nearest to w / 2^k (ties to even), its sign
// kept.  Rows with a below 2^-64 are stored as zero codes with scale 1.  w / 2^k is exact
// (a power-of-two scaling of a bf16 value) and every rounding step below is an exact
// operation or rintf, so the codes do not depend on the order of any arithmetic.
// One workgroup per row, 8 weights (16 bytes) per thread per step.
__device__ __forceinline__ unsigned e4m3_code(float w, int k) {
  const float x = ldexpf(fabsf(w), -k);
  unsigned code;
  if (x < 0x1p-6f) {
    const int m = (int)rintf(x * 512.f);          // subnormal steps of 2^-9; 8 -> the smallest normal
    code = (unsigned)m;                             // m == 8 is code 0x08 (exponent 1, mantissa 0)
  } else {
    int e;
    frexpf(x, &e);                                  // x = f 2^e, f in [0.5, 1): floor(log2 x) = e - 1
    int m = (int)rintf((ldexpf(x, 1 - e) - 1.f) * 8.f);   // 0..8
    int E = e - 1 + 7;
    if (m == 8) { m = 0; ++E; }
    code = ((unsigned)E << 3) | (unsigned)m;
  }
  return code | ((__float_as_uint(w) >> 31) << 7);
}

__global__ __launch_bounds__(256) void quantize_fp8_rows_kernel(const bf16* src, int cols, unsigned char* codes,
                                                                float* scales) {
  __shared__ float red[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  const bf16* row = src + (size_t)r * cols;
  float amax = 0.f;
  for (int c8 = tid; c8 < cols / 8; c8 += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + c8 * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(v[j] << 16)), fabsf(__uint_as_float(v[j] & 0xffff0000u))));
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const bool zero = !(amax >= 0x1p-64f);
  int k = 0;
  if (!zero) {
    int e;
    frexpf(amax, &e);
    k = e - 9;
    while (amax > ldexpf(448.f, k)) ++k;
    while (amax <= ldexpf(448.f, k - 1)) --k;
  }
  if (tid == 0) scales[r] = zero ? 1.f : ldexpf(1.f, k);
  unsigned char* out = codes + (size_t)r * cols;
  for (int c8 = tid; c8 < cols / 8; c8 += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + c8 * 8);
    uint2 o;
    unsigned b[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float w0 = __uint_as_float(v[j] << 16), w1 = __uint_as_float(v[j] & 0xffff0000u);
      b[2 * j] = zero ? ((__float_as_uint(w0) >> 31) << 7) : e4m3_code(w0, k);
      b[2 * j + 1] = zero ? ((__float_as_uint(w1) >> 31) << 7) : e4m3_code(w1, k);
    }
    o.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    o.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    *reinterpret_cast<uint2*>(out + c8 * 8) = o;
  }
}

// MXFP4 (OCP Microscaling): blocks of 32 consecutive weights of a row share a scale 2^s, stored as
// the byte s + 127, with s = floor(log2 a) - 2 for the block's largest magnitude a (a in [4, 8) 2^s);
// each weight is the 4-bit E2M1 code of the magnitude nearest to |w| / 2^s among 0, 0.5, 1, 1.5, 2,
// 3, 4, 6 (ties to the even code, beyond 6 saturating), with the sign of w as bit 3.  A block with
// a < 2^-64 is stored as signed zeros with scale byte 127.  Two codes per byte, element 2j in the
// low nibble.  One thread per block; |w| / 2^s is exact (a bf16 value times a power of two).
__device__ __forceinline__ unsigned e2m1_code(float w, int s) {
  const float a = fabsf(ldexpf(w, -s));
  // code = number of midpoints below a; at a midpoint the even neighbour (the lower one for
  // 0.25, 1.25, 2.5, 5; the upper one for 0.75, 1.75, 3.5)
  const unsigned c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.f);
  return c | ((__float_as_uint(w) >> 31) << 3);
}

__global__ __launch_bounds__(256) void quantize_mxfp4_rows_kernel(const bf16* src, int rows, int cols,
                                                                  unsigned char* codes, unsigned char* scales) {
  const int nb = cols / 32;
  const long blk = (long)blockIdx.x * 256 + threadIdx.x;
  if (blk >= (long)rows * nb) return;
  const long r = blk / nb;
  const int b = (int)(blk % nb);
  const u32x4* p = reinterpret_cast<const u32x4*>(src + r * cols + (long)b * 32);
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = p[i];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(v[i][j] << 16)), fabsf(__uint_as_float(v[i][j] & 0xffff0000u))));
  const bool zero = !(amax >= 0x1p-64f);
  const int s = zero ? 0 : (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127 - 2;   // floor(log2 a) - 2
  scales[blk] = (unsigned char)(s + 127);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // word i: elements 8i .. 8i + 7 of the block
    unsigned w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float w0 = __uint_as_float(v[i][j] << 16), w1 = __uint_as_float(v[i][j] & 0xffff0000u);
      w |= (e2m1_code(w0, s) | (e2m1_code(w1, s) << 4)) << (8 * j);
    }
    o[i] = w;
  }
  // 32 codes = 16 bytes: word i of o covers bytes 4i .. 4i + 3, i.e. elements 8i .. 8i + 7
  *reinterpret_cast<uint2*>(codes + r * (cols / 2) + (long)b * 16) = make_uint2(o[0], o[1]);
  *reinterpret_cast<uint2*>(codes + r * (cols / 2) + (long)b * 16 + 8) = make_uint2(o[2], o[3]);
}

hipError_t launch_quantize_mxfp4_rows(const void* src, int rows, int cols, unsigned char* codes, unsigned char* scales,
                                      hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const long n = (long)rows * (cols / 32);
  hipLaunchKernelGGL(quantize_mxfp4_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const bf16*>(src), rows, cols, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8_rows(const void* src, int rows, int cols, unsigned char* codes, float* scales,
                                    hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_fp8_rows_kernel, dim3(rows), dim3(256), 0, st, reinterpret_cast<const bf16*>(src), cols,
                     codes, scales);
  return hipGetLastError();
}

}  // namespace dfl
