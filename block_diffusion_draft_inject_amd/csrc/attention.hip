// Block + sliding-window attention of the drafter ("Architecture", kb.ekarisky.com, Component
// Breakdown rows "DFlash drafter backbone" and "Block attention mask"): every query slot of a
// block sees the last min(L - base, window) injected context positions of its sequence (ring
// slots slot0, slot0+1, ... mod window) and all K slots of its own block -- no causal mask.
// Softmax is invariant to key order, so ring order does not matter.
//
// Grouped-query attention: the G = n_heads / n_kv_heads query heads that share a KV head are
// processed together, so one workgroup owns R = G * K query rows (row r = g * K + t) and reads
// each key/value row once.  Keys are split into `chunks` per (sequence, KV head) to fill the
// chip at small batch; each chunk writes an unnormalised partial output with its running max
// and sum, and attn_combine merges them (log-sum-exp).
//
// bf16 path: K Q^T and V^T P^T on v_mfma_f32_16x16x32_bf16 (each wave owns 16 query rows); Q and
// P enter as sums of two bf16 terms (hi + lo), K and V are the bf16 cache values, running sums
// stay fp32.  fp32 path: VALU.
#include "rowops.h"

namespace dfl {

constexpr int AT_MAXR = 64;   // query rows per workgroup
constexpr int AT_MAXD = 128;  // head_dim

template <typename T>
__device__ __forceinline__ float ldt(const void* p, size_t i) {
  return ldv(reinterpret_cast<const T*>(p), i);
}

__device__ __forceinline__ bf16x8 bits_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ------------------------------------------------------------------------------ bf16 / MFMA
constexpr int MK = 64;          // keys per sub-tile
constexpr int MDH = 128;        // head_dim of the MFMA path

// Each wave computes S^T = K Q^T for its 16 query rows, i.e. the MFMA takes the keys as its A
// operand and the queries as B: lane (li, kg) then holds the scores of query row li for the keys
// 16 f + 4 kg + r of each 16-key fragment f.  A row's softmax is in-lane plus two exchanges
// across the lane groups kg, and P goes straight from registers into O^T += V^T P^T as the B
// operand (each lane's eight k-slots of a 32-key block are the keys it already holds, and the
// V^T operand is read from LDS in the same key order), so P never passes through LDS; O^T leaves
// lane (li, kg) with dims 16 n + 4 kg + r of query row li, scaled by that row's own softmax
// factor.
__global__ __launch_bounds__(256) void attn_chunk_mfma(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sk[MK][MDH + 8];
  __shared__ __attribute__((aligned(16))) bf16 svt[MDH][MK + 8];
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, li = lane & 15, kg = lane >> 4;
  const int K = a.K, G = a.nh / a.nkv, R = G * K;
  const SeqCtx ctx = a.ctx[b];
  const int n_keys = ctx.n_ctx + K;
  const int ck = (n_keys + a.chunks - 1) / a.chunks;
  const int k_begin = min(c * ck, n_keys), k_end = min(k_begin + ck, n_keys);
  const size_t pidx = ((size_t)b * a.nkv + kvh) * a.chunks + c;
  const bf16* q = reinterpret_cast<const bf16*>(a.q);
  // this (layer, sequence, KV head)'s rings, and its block keys (key n_ctx + t at row t * nkv)
  const size_t cache_base = (((size_t)a.layer * a.max_seqs + ctx.sid) * a.nkv + kvh) * (size_t)a.window * MDH;
  const bf16* kc = reinterpret_cast<const bf16*>(a.kcache) + cache_base;
  const bf16* vc = reinterpret_cast<const bf16*>(a.vcache) + cache_base;
  const size_t blk_base = ((size_t)b * K * a.nkv + kvh) * MDH;
  const bf16* kb = reinterpret_cast<const bf16*>(a.kb) + blk_base;
  const bf16* vb = reinterpret_cast<const bf16*>(a.vb) + blk_base;
  const int blk_stride = a.nkv * MDH;
  // this wave's 16 query rows as the B operand of S^T (query 16w + li, dims ks*32 + kg*8 .. +8),
  // hi and lo planes
  const int qrow = 16 * w + li;
  const bool has_rows = __builtin_amdgcn_readfirstlane(16 * w) < R;   // wave-uniform
  u32x4 qa[4], ql[4];
  {
    const int g = qrow / K, t = qrow % K;
    const bf16* qp = q + ((size_t)(b * K + t) * a.nh + (kvh * G + g)) * MDH;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qa[ks] = (qrow < R) ? *reinterpret_cast<const u32x4*>(qp + ks * 32 + kg * 8) : u32x4{0u, 0u, 0u, 0u};
      ql[ks] = (qrow < R) ? *reinterpret_cast<const u32x4*>(qp + a.q_plane + ks * 32 + kg * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  float m = NEG_INF, l = 0.f;   // query row 16w + li (the same in its four lanes)
  f32x4 acc[8];                 // O^T: acc[n][r] = O[row 16w + li][dim 16n + 4kg + r]
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // This thread's sixteen-byte pieces of the sub-tile at j0.  Keys past the chunk read the
  // chunk's last key and are used as loaded: their scores are set to -inf, so P is zero there
  // and the (finite) values drop out.  Nothing touches a loaded register before its LDS store in
  // the next iteration, so the loads stay in flight across this sub-tile's math (a select on a
  // loaded value would make the compiler wait for it right there):
  //   K: piece e = tid + 256 it is part e % 16 of key e / 16 (16 lanes read one 256-byte row);
  //   V: piece pair u = tid + 256 it (it < 2) is part u / 32 of keys 2 (u % 32) and 2 (u % 32) + 1,
  //      so that the transposed store writes (key, key + 1) pairs as 32-bit words, a wave's 64
  //      lanes on 64 distinct banks.
  // A context key j0 + key sits in ring slot s0 + key (mod window), s0 the sub-tile's first slot;
  // s0 < window and j0 + key < n_ctx <= window, so one subtraction reduces it.
  auto key_off = [&](int j0, int s0, int key, int part, bool& ctxk) {
    ctxk = j0 + key < ctx.n_ctx;
    int s = s0 + key;
    s = s >= a.window ? s - a.window : s;
    return ctxk ? s * MDH + part * 8 : (j0 + key - ctx.n_ctx) * blk_stride + part * 8;
  };
  auto load_kv = [&](int j0, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
    const int nk = min(MK, k_end - j0);
    const int s0 = (ctx.slot0 + j0) % a.window;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int e = tid + it * 256;
      const int key = e >> 4, part = e & 15;
      bool ctxk;
      const int off = key_off(j0, s0, min(key, nk - 1), part, ctxk);
      kr[it] = *reinterpret_cast<const u32x4*>((ctxk ? kc : kb) + off);
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int u = tid + it * 256;
      const int part = u >> 5, k0 = 2 * (u & 31);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bool ctxk;
        const int off = key_off(j0, s0, min(k0 + h, nk - 1), part, ctxk);
        vr[2 * it + h] = *reinterpret_cast<const u32x4*>((ctxk ? vc : vb) + off);
      }
    }
  };
  static_assert((MK * MDH / 8) / 256 == 4, "four pieces per thread");
  u32x4 kr[4], vr[4];
  if (k_begin < k_end) load_kv(k_begin, kr, vr);
  // The barriers below wait for LDS traffic only (lds_barrier), so the next sub-tile's global
  // loads, issued before this sub-tile's math, stay in flight across them.
  for (int j0 = k_begin; j0 < k_end; j0 += MK) {
    const int nk = min(MK, k_end - j0);
    lds_barrier();   // every wave is done with the previous sub-tile's K and V
    // K rows -> sk[key][dim]; V rows -> svt[dim][key] (transposed for the V^T operand)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int e = tid + it * 256;
      *reinterpret_cast<u32x4*>(&sk[e >> 4][(e & 15) * 8]) = kr[it];
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int u = tid + it * 256;
      const int part = u >> 5, k0 = 2 * (u & 31);
      const u32x4 v0 = vr[2 * it], v1 = vr[2 * it + 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // word i holds dims 2i (low half) and 2i + 1 of its key
        *reinterpret_cast<unsigned*>(&svt[part * 8 + 2 * i][k0]) = (v0[i] & 0xffffu) | (v1[i] << 16);
        *reinterpret_cast<unsigned*>(&svt[part * 8 + 2 * i + 1][k0]) = (v0[i] >> 16) | (v1[i] & 0xffff0000u);
      }
    }
    lds_barrier();
    if (j0 + MK < k_end) load_kv(j0 + MK, kr, vr);
    // a wave past the R query rows (R = 32 at block size 8) only loads and stores K and V
    if (!has_rows) continue;
    // S^T = K Q^T: s[f][r] = score of query row li and key 16f + 4kg + r
    f32x4 s[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      s[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sk[16 * f + li][ks * 32 + kg * 8]);
        s[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, bits_bf16x8(qa[ks]), s[f], 0, 0, 0);
        s[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, bits_bf16x8(ql[ks]), s[f], 0, 0, 0);
      }
    }
    // online softmax of the row: its 64 keys are 16 per lane in the lanes li + 16 kg
    float mx = NEG_INF;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = (16 * f + 4 * kg + r < nk) ? s[f][r] * a.scale : NEG_INF;
        s[f][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const float alpha = (m == NEG_INF) ? 0.f : __expf(m - mn);
    float sum = 0.f;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = (s[f][r] == NEG_INF) ? 0.f : __expf(s[f][r] - mn);
        s[f][r] = p;
        sum += p;
      }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    l = l * alpha + sum;
    m = mn;
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] *= alpha;
    // O^T += V^T P^T over two 32-key blocks: the lane's k-slots 0-3 are keys 32 k2 + 4 kg + r
    // (fragment 2 k2), slots 4-7 keys 32 k2 + 16 + 4 kg + r (fragment 2 k2 + 1).  P is split
    // into two bf16 terms, P = hi + lo with hi = bf16(P), lo = bf16(P - hi), and both are
    // multiplied with V: the product then carries ~16 mantissa bits of P instead of 8.
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      bf16x8 ph, pl;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float p = s[2 * k2 + r / 4][r % 4];
        const bf16 hi = f2bf(p);
        ph[r] = __builtin_bit_cast(__bf16, hi);
        pl[r] = __builtin_bit_cast(__bf16, f2bf(p - bf2f(hi)));
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const uint2 v0 = *reinterpret_cast<const uint2*>(&svt[16 * n + li][32 * k2 + 4 * kg]);
        const uint2 v1 = *reinterpret_cast<const uint2*>(&svt[16 * n + li][32 * k2 + 16 + 4 * kg]);
        const bf16x8 vf = bits_bf16x8(u32x4{v0.x, v0.y, v1.x, v1.y});
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, ph, acc[n], 0, 0, 0);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl, acc[n], 0, 0, 0);
      }
    }
  }
  if (qrow < R) {
    float* op = a.o_part + (pidx * R + qrow) * MDH;
#pragma unroll
    for (int n = 0; n < 8; ++n) *reinterpret_cast<f32x4*>(op + 16 * n + 4 * kg) = acc[n];
    if (kg == 0) {
      a.m_part[pidx * R + qrow] = m;
      a.l_part[pidx * R + qrow] = l;
    }
  }
}

// ------------------------------------------------------------------------------ fp32 / VALU
constexpr int VK = 32;

__global__ __launch_bounds__(256) void attn_chunk_valu(AttnArgs a) {
  __shared__ float sq[AT_MAXR][AT_MAXD + 1];
  __shared__ float sk[VK][AT_MAXD + 1];
  __shared__ float sv[VK][AT_MAXD];
  __shared__ float sp[AT_MAXR][VK + 1];
  __shared__ float s_m[AT_MAXR], s_l[AT_MAXR], s_alpha[AT_MAXR];
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int K = a.K, dh = a.dh, G = a.nh / a.nkv, R = G * K;
  const SeqCtx ctx = a.ctx[b];
  const int n_keys = ctx.n_ctx + K;
  const int ck = (n_keys + a.chunks - 1) / a.chunks;
  const int k_begin = min(c * ck, n_keys), k_end = min(k_begin + ck, n_keys);
  const size_t pidx = ((size_t)b * a.nkv + kvh) * a.chunks + c;
  const float* qg = reinterpret_cast<const float*>(a.q);
  for (int e = tid; e < R * dh; e += 256) {
    const int r = e / dh, dd = e % dh;
    const int g = r / K, t = r % K;
    sq[r][dd] = qg[((size_t)(b * K + t) * a.nh + kvh * G + g) * dh + dd];
  }
  if (tid < R) { s_m[tid] = NEG_INF; s_l[tid] = 0.f; }
  const int TPR = 256 / R;
  const int my_r = tid / TPR, my_c = tid % TPR;
  const int nd = dh / TPR;
  float o[AT_MAXD / 4];
#pragma unroll
  for (int i = 0; i < AT_MAXD / 4; ++i) o[i] = 0.f;
  const size_t cache_base = (((size_t)a.layer * a.max_seqs + ctx.sid) * a.nkv + kvh) * (size_t)a.window;
  const float* kc = reinterpret_cast<const float*>(a.kcache);
  const float* vc = reinterpret_cast<const float*>(a.vcache);
  const float* kbp = reinterpret_cast<const float*>(a.kb);
  const float* vbp = reinterpret_cast<const float*>(a.vb);
  const int kj = tid & 31, rg = tid >> 5;
  for (int j0 = k_begin; j0 < k_end; j0 += VK) {
    const int nk = min(VK, k_end - j0);
    __syncthreads();
    for (int e = tid; e < VK * dh; e += 256) {
      const int j = e / dh, dd = e % dh;
      float kv = 0.f, vv = 0.f;
      if (j < nk) {
        const int key = j0 + j;
        if (key < ctx.n_ctx) {
          const size_t off = (cache_base + (ctx.slot0 + key) % a.window) * dh + dd;
          kv = kc[off];
          vv = vc[off];
        } else {
          const size_t off = ((size_t)(b * K + key - ctx.n_ctx) * a.nkv + kvh) * dh + dd;
          kv = kbp[off];
          vv = vbp[off];
        }
      }
      sk[j][dd] = kv;
      sv[j][dd] = vv;
    }
    __syncthreads();
    for (int r = rg; r < R; r += 8) {
      float sc = NEG_INF;
      if (kj < nk) {
        float acc = 0.f;
        for (int dd = 0; dd < dh; ++dd) acc = fmaf(sq[r][dd], sk[kj][dd], acc);
        sc = acc * a.scale;
      }
      float mx = sc;
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 32));
      const float m_old = s_m[r];
      const float m_new = fmaxf(m_old, mx);
      const float pv = (kj < nk) ? __expf(sc - m_new) : 0.f;
      float sum = pv;
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 32);
      sp[r][kj] = pv;
      if (kj == 0) {
        const float alpha = (m_old == NEG_INF) ? 0.f : __expf(m_old - m_new);
        s_alpha[r] = alpha;
        s_l[r] = s_l[r] * alpha + sum;
        s_m[r] = m_new;
      }
    }
    __syncthreads();
    if (my_r < R) {
      const float alpha = s_alpha[my_r];
#pragma unroll
      for (int i = 0; i < AT_MAXD / 4; ++i) {
        if (i >= nd) break;
        const int dd = my_c + i * TPR;
        float acc = o[i] * alpha;
        for (int j = 0; j < nk; ++j) acc = fmaf(sp[my_r][j], sv[j][dd], acc);
        o[i] = acc;
      }
    }
  }
  __syncthreads();
  if (my_r < R) {
    float* op = a.o_part + (pidx * R + my_r) * dh;
#pragma unroll
    for (int i = 0; i < AT_MAXD / 4; ++i) {
      if (i >= nd) break;
      op[my_c + i * TPR] = o[i];
    }
  }
  if (tid < R) {
    a.m_part[pidx * R + tid] = s_m[tid];
    a.l_part[pidx * R + tid] = s_l[tid];
  }
}

// Merge the chunks of one query row: o = sum_c e^{m_c - M} o_c / sum_c e^{m_c - M} l_c.
// One wave per (row, KV head, sequence), blockDim / 64 rows per workgroup (four, or one when
// there are few rows, so that they spread over more CUs) and no workgroup barrier:
// lane j reads the maxima and sums of chunks j, j + 64, ... (M and the denominator are wave
// reductions), the chunk weights go through the wave's own LDS row, and lane j accumulates dims
// j and j + 64 over the chunks in order, the loads of CB chunks at a time (8 when there are at
// most 8 chunks, else 32: the 17 chunks of a batch-1 pass in one round trip, not three).
template <typename T, int CB>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int CMAX = 256;   // chunks per (sequence, KV head), at most
  __shared__ float wts[4][CMAX];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int K = a.K, dh = a.dh, G = a.nh / a.nkv, R = G * K;
  const int r = blockIdx.x * (blockDim.x >> 6) + wv;
  if (r >= R) return;   // the whole wave: the reductions below need all 64 lanes
  const size_t base = ((size_t)b * a.nkv + kvh) * a.chunks;
  const int nc = a.chunks;
  float mc[CMAX / 64], lc[CMAX / 64];
  float M = NEG_INF;
#pragma unroll
  for (int g = 0; g < CMAX / 64; ++g) {
    const int c = g * 64 + lane;
    mc[g] = c < nc ? a.m_part[(base + c) * R + r] : NEG_INF;
    lc[g] = c < nc ? a.l_part[(base + c) * R + r] : 0.f;
    M = fmaxf(M, mc[g]);
  }
  M = wave_max(M);
  float den = 0.f;
#pragma unroll
  for (int g = 0; g < CMAX / 64; ++g) {
    const float w = (mc[g] == NEG_INF) ? 0.f : __expf(mc[g] - M);
    wts[wv][g * 64 + lane] = w;
    den += w * lc[g];
  }
  den = wave_sum(den);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const size_t cstride = (size_t)R * dh;
  const float* op = a.o_part + (base * R + r) * dh;
  const int d0 = min(lane, dh - 1), d1 = min(lane + 64, dh - 1);
  float n0 = 0.f, n1 = 0.f;
  for (int c0 = 0; c0 < nc; c0 += CB) {
    float x0[CB], x1[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const size_t co = (size_t)min(c0 + u, nc - 1) * cstride;
      x0[u] = op[co + d0];
      x1[u] = op[co + d1];
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const float w = c0 + u < nc ? wts[wv][c0 + u] : 0.f;
      n0 += w * x0[u];
      n1 += w * x1[u];
    }
  }
  const int g = r / K, t = r % K, h = kvh * G + g;
  const size_t orow = ((size_t)(b * K + t) * a.nh + h) * dh;
  if (lane < dh) st_act(reinterpret_cast<T*>(a.o), orow + lane, a.o_plane, n0 / den);
  if (lane + 64 < dh) st_act(reinterpret_cast<T*>(a.o), orow + lane + 64, a.o_plane, n1 / den);
}

hipError_t launch_attention(bool bf, const AttnArgs& a, int n_seq, hipStream_t st) {
  const int R = (a.nh / a.nkv) * a.K;
  if (a.chunks > 256 || a.dh > 128) return hipErrorInvalidValue;
  const int rpw = (long)R * a.nkv * n_seq >= 1024 ? 4 : 1;   // combine: rows (waves) per workgroup
  const dim3 g1(a.chunks, a.nkv, n_seq), g2((R + rpw - 1) / rpw, a.nkv, n_seq);
  if (bf) {
    hipLaunchKernelGGL(attn_chunk_mfma, g1, dim3(256), 0, st, a);
    if (a.chunks <= 8) hipLaunchKernelGGL((attn_combine_kernel<bf16, 8>), g2, dim3(64 * rpw), 0, st, a);
    else hipLaunchKernelGGL((attn_combine_kernel<bf16, 32>), g2, dim3(64 * rpw), 0, st, a);
  } else {
    hipLaunchKernelGGL(attn_chunk_valu, g1, dim3(256), 0, st, a);
    if (a.chunks <= 8) hipLaunchKernelGGL((attn_combine_kernel<float, 8>), g2, dim3(64 * rpw), 0, st, a);
    else hipLaunchKernelGGL((attn_combine_kernel<float, 32>), g2, dim3(64 * rpw), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace dfl
