// Path selector, greedy verification, and the benchmark's stand-in target.
//
// Selector ("Architecture", kb.ekarisky.com, section "Problem 1 -- Independent picks are
// incoherent"): keep the top-16 candidates of every draft slot and score adjacent pairs,
//   S_t(a, b) = U_t(b) + < A(a) * H(h_t), B(b) >,   H(h_t) = sigmoid(W_H h_t),
// all pairs at once; only the walk over the precomputed scores is sequential.  The gates and
// pair scores are spread over one workgroup per (sequence, slot, chunk of 32 ranks); the last
// of a sequence's workgroups to finish sums the rank chunks and walks.  VITERBI: a forward and
// a backward max-plus sweep give the best path and the exact score of the second-best complete
// path (the margin); GREEDY follows the best successor.
#include "rowops.h"

namespace dfl {

constexpr int SEL_KMAX = 32;    // block size
constexpr int SEL_SR = 32;      // ranks per workgroup
constexpr int SEL_T = 512;      // threads per workgroup
constexpr int SEL_DMAX = 4096;  // hidden size (config bound)

// DPP quad permutation (lanes l ^ 1 for 0xB1, l ^ 2 for 0x4E inside each group of four)
template <int CTRL>
__device__ __forceinline__ int quad_perm_i(int v) { return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false); }
template <int CTRL>
__device__ __forceinline__ float quad_perm_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Walk state of one sequence, in LDS (the sequence's last workgroup only).
struct SelWalk {
  int cid[SEL_KMAX][TOPK];                    // candidate ids of slots 1..K-1
  float S[SEL_KMAX][TOPK][TOPK];              // S[t-1][b][a]: pair scores with the logit term
  float alpha[SEL_KMAX][TOPK];                // forward sweep, slot t at row t-1
  float beta[SEL_KMAX][TOPK];                 // backward sweep
  unsigned char bp1[SEL_KMAX][TOPK];          // best predecessor per (slot, state)
  int best[SEL_KMAX];                         // the best path's state per slot
};

// The sequential walk over the summed pair scores, in wave 0 of the last workgroup.
// Viterbi sweeps, one per wave: wave 0 the forward sweep (with predecessors), wave 1 the backward
// sweep; they read only the pair scores, so they run side by side.
__device__ void sel_sweeps(const SelectArgs& a, SelWalk& w, int role) {
  const int K = a.K, lane = threadIdx.x & 63;
  const int bi = lane >> 2, qa = lane & 3;
  if (role == 0) {
    // Viterbi as two max-plus sweeps.  Forward: alpha_t(b) = max_a alpha_{t-1}(a) + S_t(a, b),
    // alpha_1(b) = S_1(anchor, b), the predecessor kept per state (ties to the smaller a).
    // Backward: beta_t(a) = max_b S_{t+1}(a, b) + beta_{t+1}(b), beta_{K-1} = 0.  The best path
    // follows the predecessors back from the best final state (ties to the smaller state), so
    // it is the best path of the two-best list recursion with the same order.  Every other path
    // leaves the best one at some slot t in a state b != best_t, and the best path through
    // (t, b) scores alpha_t(b) + beta_t(b); so the second-best complete path scores the
    // maximum of that over the states off the best path.  Per step each lane takes four
    // predecessors (successors) of one state; the quad merges by DPP; sweep values pass
    // through LDS (one wave: its LDS accesses are ordered).
    if (lane < TOPK) w.alpha[0][lane] = w.S[0][lane][0];
    for (int t = 2; t < K; ++t) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const f32x4 av = *reinterpret_cast<const f32x4*>(&w.alpha[t - 2][4 * qa]);
      const f32x4 sv = *reinterpret_cast<const f32x4*>(&w.S[t - 1][bi][4 * qa]);
      float bv = av[0] + sv[0];
      int ba = 4 * qa;
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        const float v = av[i] + sv[i];
        ba = v > bv ? 4 * qa + i : ba;      // strictly greater: ties keep the smaller predecessor
        bv = fmaxf(v, bv);
      }
      auto merge = [&](float ov, int oa) {
        const bool take = (ov > bv) | ((ov == bv) & (oa < ba));
        bv = take ? ov : bv;
        ba = take ? oa : ba;
      };
      merge(quad_perm_f<0xB1>(bv), quad_perm_i<0xB1>(ba));
      merge(quad_perm_f<0x4E>(bv), quad_perm_i<0x4E>(ba));
      if (qa == 0) {
        w.alpha[t - 1][bi] = bv;
        w.bp1[t - 1][bi] = (unsigned char)ba;
      }
    }
  } else {
    // backward sweep: lane = 4 ai + qb holds state ai of slot t, successors 4 qb .. 4 qb + 3
    if (lane < TOPK) w.beta[K - 2][lane] = 0.f;
    for (int t = K - 2; t >= 1; --t) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const f32x4 bn = *reinterpret_cast<const f32x4*>(&w.beta[t][4 * qa]);
      float m = NEG_INF;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, w.S[t][4 * qa + i][bi] + bn[i]);   // S_{t+1}(bi, 4 qa + i)
      m = fmaxf(m, quad_perm_f<0xB1>(m));
      m = fmaxf(m, quad_perm_f<0x4E>(m));
      if (qa == 0) w.beta[t - 1][bi] = m;
    }
  }
}

__device__ void sel_walk(const SelectArgs& a, int b, SelWalk& w) {
  const int K = a.K, lane = threadIdx.x & 63;
  // ---- the walk: one wave; lane = 4 * bi + qa holds predecessors a = 4 qa .. 4 qa + 3 of state bi
  if (a.mode == 0) {
    // after sel_sweeps (both sweeps in LDS, a workgroup barrier between):
    // best final state (ties to the smaller state), then the path back through the predecessors
    float s1 = lane < TOPK ? w.alpha[K - 2][lane] : NEG_INF;
    int st = lane < TOPK ? lane : TOPK;
    for (int m = 1; m < 64; m <<= 1) {
      const float ov = __shfl_xor(s1, m, WAVE);
      const int os = __shfl_xor(st, m, WAVE);
      const bool take = (ov > s1) | ((ov == s1) & (os < st));
      s1 = take ? ov : s1;
      st = take ? os : st;
    }
    if (lane == 0) {
      for (int t = K - 1; t >= 1; --t) {
        w.best[t - 1] = st;
        a.path[(size_t)b * (K - 1) + t - 1] = w.cid[t - 1][st];
        if (t > 1) st = w.bp1[t - 1][st];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float s2 = NEG_INF;
    for (int e = lane; e < (K - 1) * TOPK; e += WAVE) {
      const int tt = e / TOPK, sb = e % TOPK;
      if (sb != w.best[tt]) s2 = fmaxf(s2, w.alpha[tt][sb] + w.beta[tt][sb]);
    }
    s2 = wave_max(s2);
    if (lane == 0) {
      if (a.score) a.score[b] = s1;
      if (a.margin) a.margin[b] = fmaxf(s1 - s2, 0.f);
    }
  } else if (a.mode == 2) {
    // sampling walk: at slot t, q(b) = softmax_b(S_t(a, b) / T) over the 16 candidates given
    // the previous pick a, cut to its top-p nucleus; the pick is the first b (candidate order)
    // whose inclusive cumulative probability exceeds u_t times the total
    int ai = 0;
    const bool in = lane < TOPK;
    const bool cut = a.top_p < 1.f;
    for (int t = 1; t < K; ++t) {
      const float z = in ? w.S[t - 1][lane][ai] * a.inv_temp : NEG_INF;
      const float mx = wave_max(z);
      const float e = in ? __expf(z - mx) : 0.f;
      float q = e / wave_sum(e);
      if (cut) {
        // mass ranked ahead of this candidate (probability descending, ties to the lower
        // index); the candidate stays while that mass is below top_p
        float before = 0.f;
#pragma unroll
        for (int j = 0; j < TOPK; ++j) {
          const float qj = __shfl(q, j, WAVE);
          if (qj > q || (qj == q && j < lane)) before += qj;
        }
        const float kept = (in && before < a.top_p) ? q : 0.f;
        q = kept / wave_sum(kept);
      }
      float c = q;
#pragma unroll
      for (int o = 1; o < TOPK; o <<= 1) {
        const float y = __shfl_up(c, o, WAVE);
        if (lane >= o) c += y;
      }
      const float total = __shfl(c, TOPK - 1, WAVE);
      const float u = a.uniforms[(size_t)b * (K - 1) + t - 1];
      const unsigned long long hit = __ballot(in && u * total < c);
      const unsigned long long pos = __ballot(in && q > 0.f);
      const int pick = hit ? __builtin_ctzll(hit) : 63 - __builtin_clzll(pos);
      const float qp = __shfl(q, pick, WAVE);
      const size_t o = (size_t)b * (K - 1) + t - 1;
      if (lane == 0) {
        a.path[o] = w.cid[t - 1][pick];
        a.q_path[o] = qp;
      }
      if (a.q_cand && in) a.q_cand[o * TOPK + lane] = q;
      ai = pick;
    }
  } else {
    // greedy: from the current candidate, the best successor (ties to the smaller index)
    int ai = 0;
    float total = 0.f, margin = __builtin_huge_valf();
    for (int t = 1; t < K; ++t) {
      const float v = lane < TOPK ? w.S[t - 1][lane][ai] : NEG_INF;
      float m1 = v;
      int i1 = lane < TOPK ? lane : 255;
      for (int m = 1; m < TOPK; m <<= 1) {
        const float ov = __shfl_xor(m1, m, WAVE);
        const int oi = __shfl_xor(i1, m, WAVE);
        const bool take = (ov > m1) | ((ov == m1) & (oi < i1));
        m1 = take ? ov : m1;
        i1 = take ? oi : i1;
      }
      m1 = __shfl(m1, 0, WAVE);
      i1 = __shfl(i1, 0, WAVE);
      float sec = (lane < TOPK && lane != i1) ? v : NEG_INF;
      for (int m = 1; m < TOPK; m <<= 1) sec = fmaxf(sec, __shfl_xor(sec, m, WAVE));
      sec = __shfl(sec, 0, WAVE);
      margin = fminf(margin, m1 - sec);
      total += m1;
      if (lane == 0) a.path[(size_t)b * (K - 1) + t - 1] = w.cid[t - 1][i1];
      ai = i1;
    }
    if (lane == 0) {
      if (a.score) a.score[b] = total;
      if (a.margin) a.margin[b] = margin;
    }
  }
}

// One workgroup per (group of up to SEL_SPW consecutive slots, chunk of 32 ranks) of sequence b
// (grid x = group * chunks + chunk, y = b; a.spw slots per group: one for small batches, the
// most parallel split, all of them for larger batches, where one workgroup per sequence needs
// no hand-off and reads each chunk of W_H once).  Phases: (1) the gates
// g_t[j] = sigmoid(W_H[j] . h_final[b][t]) of the group's slots for the chunk's ranks (bf16
// tables: MFMA with slots as rows and ranks as columns, h as hi + lo planes, the eight waves
// splitting the hidden dimension; fp32 tables: VALU dot products); (2) the chunk's share of the
// 16 x 16 pair scores of each slot, sum_j A[pred a][j] * g_t[j] * B[cand b][j] (predecessors:
// the anchor for t = 1, else the candidates of slot t - 1); (3) with several workgroups per
// sequence, the shares go to the workspace and the last workgroup to finish adds them in chunk
// order; then the logit term U_t(b) is added and the sequence's workgroup walks.
constexpr int SEL_SPW = 16;     // most slots per workgroup (one MFMA row tile)
constexpr int SEL_HROWS = 4;    // groups of at most this many slots stage their h rows in LDS

template <typename T, bool STAGE>
__global__ __launch_bounds__(SEL_T) void select_kernel(SelectArgs a) {
  // LDS pool: bf16 h planes of up to SEL_HROWS slots followed by their tables, or the tables of
  // up to SEL_SPW slots; table (slot s, side q) is [16 rows][SEL_SR + 4] floats (rows 16-byte aligned)
  constexpr int TS_ = SEL_SR + 4;
  constexpr int TABF = TOPK * TS_;
  constexpr int HHB = SEL_HROWS * 2 * SEL_DMAX * 2;
  constexpr int POOL = HHB + 2 * SEL_HROWS * TABF * 4 > 2 * SEL_SPW * TABF * 4 ? HHB + 2 * SEL_HROWS * TABF * 4
                                                                              : 2 * SEL_SPW * TABF * 4;
  __shared__ __attribute__((aligned(16))) unsigned char pool[POOL];
  __shared__ __attribute__((aligned(16))) float red[SEL_T / WAVE][SEL_SPW][SEL_SR];
  __shared__ __attribute__((aligned(16))) float gsh[SEL_SPW][SEL_SR];
  __shared__ int last_flag;
  __shared__ __attribute__((aligned(16))) SelWalk sw;
  const int K = a.K, r = a.r, d = a.d, spw = a.spw;
  const int nrc = (r + SEL_SR - 1) / SEL_SR;
  const int ngrp = (K - 1 + spw - 1) / spw;
  const int b = blockIdx.y, grp = blockIdx.x / nrc, rc = blockIdx.x % nrc;
  const int t0 = grp * spw + 1, ns = min(spw, K - t0);        // slots t0 .. t0 + ns - 1
  const int r0 = rc * SEL_SR, nr = min(SEL_SR, r - r0);       // nr: a multiple of 8
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncand = (K - 1) * TOPK;
  const int* ids = a.topk_ids + (size_t)b * ncand;
  // STAGE (bf16 tables, at most SEL_HROWS slots): h rows staged in LDS as bf16 planes
  constexpr bool stage = STAGE && sizeof(T) == 2;
  bf16 (*hh)[2][SEL_DMAX] = reinterpret_cast<bf16 (*)[2][SEL_DMAX]>(pool);
  float* tab = reinterpret_cast<float*>(pool + (stage ? HHB : 0));
  auto ta = [&](int sl, int row) { return tab + ((2 * sl) * TOPK + row) * TS_; };
  auto tb = [&](int sl, int row) { return tab + ((2 * sl + 1) * TOPK + row) * TS_; };
  // (a) table gathers, item e: slot e / (32 VPR), row (e / VPR) % 32 (0..15: A of the
  // predecessors, 16..31: B of the slot's candidates), 16 bytes v = e % VPR of ranks r0 .. r0 + nr
  constexpr int VE = 16 / sizeof(T);
  constexpr int VPR = SEL_SR / VE;
  constexpr int GPT = (2 * TOPK * SEL_SPW * VPR + SEL_T - 1) / SEL_T;
  const int ng = 2 * TOPK * ns * VPR;
  int tok[GPT];
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int e = tid + i * SEL_T, row = (e / VPR) % (2 * TOPK), t = t0 + e / (2 * TOPK * VPR);
    tok[i] = 0;
    if (e < ng) tok[i] = row < TOPK ? (t == 1 ? a.anchor[b] : ids[(t - 2) * TOPK + row]) : ids[(t - 1) * TOPK + row - TOPK];
  }
  // (b) bf16 tables: the h rows of a small group (staged in LDS below), then the W_H fragments
  // (and, for a large group, its h fragments) of the first batch, issued before the gathers
  constexpr int HPT = SEL_HROWS * SEL_DMAX / (4 * SEL_T);     // staged h pieces of 4 per thread
  f32x4 hx[HPT];
  if constexpr (stage) {
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int e = (i * SEL_T + tid) * 4, sl = min(e / d, ns - 1), k = e % d;
      hx[i] = *reinterpret_cast<const f32x4*>(a.h_final + ((size_t)b * K + t0 + sl) * d + k);
    }
  }
  constexpr int NWV = SEL_T / WAVE;
  constexpr int CB = 8;                        // 32-wide k chunks per wave and batch
  const int li = lane & 15, kg = lane >> 4;
  const int nch = d / 32;
  const int hrow = min(li, ns - 1);            // MFMA row li = slot t0 + li
  u32x4 wv[CB][2];
  f32x4 hv[CB][2];
  const bf16* w0 = reinterpret_cast<const bf16*>(a.WH) + (size_t)min(r0 + li, r - 1) * d + kg * 8;
  const bf16* w1 = reinterpret_cast<const bf16*>(a.WH) + (size_t)min(r0 + 16 + li, r - 1) * d + kg * 8;
  const float* hr = a.h_final + ((size_t)b * K + t0 + hrow) * d + kg * 8;
  auto issue = [&](int c0) {
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int c = min(c0 + NWV * u, nch - 1);
      wv[u][0] = *reinterpret_cast<const u32x4*>(w0 + c * 32);
      wv[u][1] = *reinterpret_cast<const u32x4*>(w1 + c * 32);
      if constexpr (!stage) {
        hv[u][0] = *reinterpret_cast<const f32x4*>(hr + c * 32);
        hv[u][1] = *reinterpret_cast<const f32x4*>(hr + c * 32 + 4);
      }
    }
  };
  if constexpr (sizeof(T) == 2) issue(wave);
  u32x4 xv[GPT];
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int e = tid + i * SEL_T, row = (e / VPR) % (2 * TOPK), v = e % VPR;
    const int t = t0 + e / (2 * TOPK * VPR);
    xv[i] = u32x4{0u, 0u, 0u, 0u};
    if (e < ng) {
      int k = tok[i];
      if (k < 0 || k >= a.vocab) {             // out-of-range token: record and read row 0
        atomicOr(a.dev_err, (row < TOPK && t == 1) ? 8 : 16);
        k = 0;
      }
      const T* base = reinterpret_cast<const T*>(row < TOPK ? a.A : a.B) + (size_t)k * r + r0;
      if (v * VE < nr) xv[i] = reinterpret_cast<const u32x4*>(base)[v];
    }
  }
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int e = tid + i * SEL_T, row = (e / VPR) % (2 * TOPK), v = e % VPR, sl = e / (2 * TOPK * VPR);
    if (e < ng) {
      float* dst = (row < TOPK ? ta(sl, row) : tb(sl, row - TOPK)) + v * VE;
#pragma unroll
      for (int q = 0; q < VE; ++q) dst[q] = v * VE + q < nr ? ldv(reinterpret_cast<const T*>(&xv[i]), q) : 0.f;
    }
  }
  // (1) gates
  if constexpr (sizeof(T) == 2) {
    if constexpr (stage) {
#pragma unroll
      for (int i = 0; i < HPT; ++i) {
        const int e = (i * SEL_T + tid) * 4, sl = e / d, k = e % d;
        if (sl < ns) {
          uint32_t hp[2], lp[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const bf16 h0 = f2bf(hx[i][2 * q]), h1 = f2bf(hx[i][2 * q + 1]);
            hp[q] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lp[q] = (uint32_t)f2bf(hx[i][2 * q] - bf2f(h0)) | ((uint32_t)f2bf(hx[i][2 * q + 1] - bf2f(h1)) << 16);
          }
          *reinterpret_cast<uint2*>(&hh[sl][0][k]) = make_uint2(hp[0], hp[1]);
          *reinterpret_cast<uint2*>(&hh[sl][1][k]) = make_uint2(lp[0], lp[1]);
        }
      }
    }
    lds_barrier();
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = wave; c0 < nch; c0 += NWV * CB) {
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        // a chunk past the end (its loads were clamped) adds zero: no branch, so that the
        // whole batch of loads stays ahead of the first MFMA
        const bool live = c0 + NWV * u < nch;
        const int c = min(c0 + NWV * u, nch - 1);
        u32x4 hi, lo;
        if constexpr (stage) {
          hi = *reinterpret_cast<const u32x4*>(&hh[hrow][0][c * 32 + kg * 8]);
          lo = *reinterpret_cast<const u32x4*>(&hh[hrow][1][c * 32 + kg * 8]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = e < 2 ? hv[u][0][2 * e] : hv[u][1][2 * e - 4];
            const float x1 = e < 2 ? hv[u][0][2 * e + 1] : hv[u][1][2 * e - 3];
            const bf16 h0 = f2bf(x0), h1 = f2bf(x1);
            hi[e] = (unsigned)h0 | ((unsigned)h1 << 16);
            lo[e] = (unsigned)f2bf(x0 - bf2f(h0)) | ((unsigned)f2bf(x1 - bf2f(h1)) << 16);
          }
        }
        const u32x4 z = {0u, 0u, 0u, 0u};
        const bf16x8 x0 = as_bf16x8(live ? wv[u][0] : z), x1 = as_bf16x8(live ? wv[u][1] : z);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(hi), x0, acc0, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lo), x0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(hi), x1, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lo), x1, acc1, 0, 0, 0);
      }
      if (c0 + NWV * CB < nch) issue(c0 + NWV * CB);
    }
    // D layout: lane (li, kg) holds rows (slots) 4 kg .. 4 kg + 3 of column (rank) li
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = 4 * kg + j;
      if (sl < ns) {
        red[wave][sl][li] = acc0[j];
        red[wave][sl][16 + li] = acc1[j];
      }
    }
    lds_barrier();
    if (tid < ns * SEL_SR) {
      const int sl = tid / SEL_SR, j = tid % SEL_SR;
      float g = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) g += red[w][sl][j];
      gsh[sl][j] = j < nr ? sigmoidf_(g) : 0.f;
    }
  } else {
    // fp32 tables: 16 lanes per rank, each over every 64th group of 4 k, slot by slot
    const int j = tid >> 4, p = tid & 15;
    const float* wr = reinterpret_cast<const float*>(a.WH) + (size_t)min(r0 + j, r - 1) * d;
    for (int sl = 0; sl < ns; ++sl) {
      const float* hb = a.h_final + ((size_t)b * K + t0 + sl) * d;
      float acc = 0.f;
      for (int k = p * 4; k < d; k += 64) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(wr + k);
        const f32x4 h = *reinterpret_cast<const f32x4*>(hb + k);
        acc += x[0] * h[0] + x[1] * h[1] + x[2] * h[2] + x[3] * h[3];
      }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m, WAVE);
      if (p == 0) gsh[sl][j] = j < nr ? sigmoidf_(acc) : 0.f;
    }
  }
  lds_barrier();
  // (2) this chunk's share of the pair scores, item (slot sl, b, a); with one workgroup per
  // sequence (one group, one chunk) it is the whole pair term and goes straight to the walk
  const bool single = ngrp * nrc == 1;
  // item (slot sl, state b, APT predecessors): B[b] * g_t in registers, dotted with APT A rows
  // (APT = 1 for small groups: every lane busy; 4 for large ones: fewer LDS reads per score)
  constexpr int APT = STAGE ? 1 : 4;
  for (int e = tid; e < ns * TOPK * (TOPK / APT); e += SEL_T) {
    const int sl = e / (TOPK * TOPK / APT), bi = (e / (TOPK / APT)) % TOPK, a0 = (e % (TOPK / APT)) * APT;
    const int t = t0 + sl;
    float gb[SEL_SR];
    const float* pb = tb(sl, bi);
#pragma unroll
    for (int j4 = 0; j4 < SEL_SR / 4; ++j4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(pb + 4 * j4);
      const f32x4 g = *reinterpret_cast<const f32x4*>(&gsh[sl][4 * j4]);
#pragma unroll
      for (int q = 0; q < 4; ++q) gb[4 * j4 + q] = x[q] * g[q];   // ranks >= nr are zero
    }
    float v[APT];
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const float* pa = ta(sl, a0 + i);
      float acc = 0.f;
#pragma unroll
      for (int j4 = 0; j4 < SEL_SR / 4; ++j4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(pa + 4 * j4);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc += x[q] * gb[4 * j4 + q];
      }
      v[i] = (t > 1 || a0 + i == 0) ? acc : 0.f;   // slot 1 has the anchor as its only predecessor
    }
    if (single) {
      const float u = a.topk_logits[(size_t)b * ncand + (t - 1) * TOPK + bi];
#pragma unroll
      for (int i = 0; i < APT; ++i) sw.S[t - 1][bi][a0 + i] = v[i] + u;
    } else {
      float* o = a.spart + (((size_t)b * (K - 1) + t - 1) * nrc + rc) * (TOPK * TOPK) + bi * TOPK + a0;
#pragma unroll
      for (int i = 0; i < APT; ++i) o[i] = v[i];
    }
  }
  if (single) {
    if (tid < ncand) {
      const int id = ids[tid];
      sw.cid[tid / TOPK][tid % TOPK] = (id < 0 || id >= a.vocab) ? 0 : id;   // recorded in phase (a)
    }
    __syncthreads();
    if (a.mode == 0) {
      if (wave < 2) sel_sweeps(a, sw, wave);
      __syncthreads();
    }
    if (wave != 0) return;
    sel_walk(a, b, sw);
    return;
  }
  // (3) the last workgroup of the sequence
  if (!arrive_last(a.sel_cnt + b, (unsigned)(ngrp * nrc), &last_flag)) return;
  // thread e takes pair scores e, e + SEL_T, ...: every load of a chunk is issued before any is
  // used (one memory round trip per rank chunk, not one per element)
  constexpr int EPT = ((SEL_KMAX - 1) * TOPK * TOPK + SEL_T - 1) / SEL_T;
  const int ne = (K - 1) * TOPK * TOPK;
  const float* spb = a.spart + (size_t)b * (K - 1) * nrc * (TOPK * TOPK);
  const int id = ids[min(tid, ncand - 1)];
  float sum[EPT], lg[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = min(tid + i * SEL_T, ne - 1), tt = e / (TOPK * TOPK);
    lg[i] = a.topk_logits[(size_t)b * ncand + tt * TOPK + (e % (TOPK * TOPK)) / TOPK];
    sum[i] = 0.f;
  }
  for (int q = 0; q < nrc; ++q) {
    float x[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = min(tid + i * SEL_T, ne - 1), tt = e / (TOPK * TOPK);
      x[i] = spb[((size_t)tt * nrc + q) * (TOPK * TOPK) + e % (TOPK * TOPK)];
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) sum[i] += x[i];
  }
  if (tid < ncand) sw.cid[tid / TOPK][tid % TOPK] = (id < 0 || id >= a.vocab) ? 0 : id;   // recorded in phase (a)
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid + i * SEL_T;
    if (e < ne) sw.S[e / (TOPK * TOPK)][(e % (TOPK * TOPK)) / TOPK][e % TOPK] = sum[i] + lg[i];
  }
  __syncthreads();
  if (a.mode == 0) {
    if (wave < 2) sel_sweeps(a, sw, wave);
    __syncthreads();
  }
  if (wave != 0) return;
  sel_walk(a, b, sw);
}

// Greedy longest-prefix verification: one wave per sequence, lane j on slot c0 + j of each
// 64-slot chunk.  Every chunk's draft and target ids are loaded together; the first mismatch is
// the lowest set bit of a ballot, so the accepted length costs one load round trip per chunk
// instead of one per accepted token.
__global__ __launch_bounds__(256) void verify_kernel(VerifyArgs a) {
  const int b = (int)((blockIdx.x * blockDim.x + threadIdx.x) / WAVE);
  const int lane = threadIdx.x & (WAVE - 1);
  if (b >= a.n_seq) return;   // uniform over the wave
  const int K = a.K;
  const int* dr = a.draft + (size_t)b * (K - 1);
  const int* tg = a.target + (size_t)b * K;
  int* com = a.committed + (size_t)b * K;
  int n = K - 1;              // every draft accepted unless a chunk finds a mismatch
  for (int c0 = 0; c0 < K - 1; c0 += WAVE) {
    const int i = c0 + lane;
    const bool in = i < K - 1;
    const int d = dr[in ? i : 0], g = tg[in ? i : 0];
    const unsigned long long miss = __ballot(in && d != g);
    if (miss) {
      n = c0 + __builtin_ctzll(miss);
      break;
    }
  }
  const int bonus = tg[n];
  for (int c0 = 0; c0 < K; c0 += WAVE) {
    const int i = c0 + lane;
    if (i < K) com[i] = i < n ? dr[i] : (i == n ? bonus : -1);
  }
  if (lane == 0) {
    a.n_acc[b] = n;
    if (a.n_commit) a.n_commit[b] = n + 1;
    a.next_anchor[b] = bonus;
  }
}

// Rejection-sampling verification ("Architecture", section "Speculative Decoding Context" and
// flowchart "Verification": rejection sampling keeps the scheme lossless).  One workgroup per
// sequence.  Draft i is accepted iff u_i * q_i(d_i) < p_i(d_i), in order; at the first
// rejection the committed token is drawn from r(v) = max(0, p_i(v) - q_i(v)) (q_i is zero
// outside the slot's 16 candidates, so r = p except at those), and if every draft is accepted
// from the bonus row p_K.  The draw is an inverse CDF in token order: every thread sums a
// contiguous chunk of the vocabulary, the chunk prefix sums locate the chunk holding
// u * sum(r), and its thread scans it.
__global__ __launch_bounds__(256) void verify_rejection_kernel(RejectArgs a) {
  __shared__ float part[256], pref[256];
  __shared__ int cs_id[TOPK];
  __shared__ float cs_min[TOPK];
  __shared__ int s_n, s_chunk, s_pass;
  __shared__ float s_total;
  const int b = blockIdx.x, tid = threadIdx.x, K = a.K, V = a.V;
  bool acc = false;
  if (tid < K - 1) {
    const size_t o = (size_t)b * (K - 1) + tid;
    const int d = a.draft[o];
    const bool ok = d >= 0 && d < V;
    const float pd = a.p[((size_t)b * K + tid) * V + (ok ? d : 0)];
    acc = ok && a.u_accept[o] * a.q_path[o] < pd;
  }
  if (tid < 64) {
    const unsigned long long rej = __ballot(tid < K - 1 && !acc);
    if (tid == 0) s_n = rej ? __builtin_ctzll(rej) : K - 1;
  }
  if (tid == 0) s_chunk = 256;
  __syncthreads();
  const int n = s_n;
  const float* pr = a.p + ((size_t)b * K + n) * V;      // slot n+1's row, or the bonus row
  const float ur = a.u_resample[b];
  // candidates of the rejected slot with the weight min(p, q) they lose (none for the bonus)
  if (tid < TOPK) {
    int id = 0x7fffffff;
    float m = 0.f;
    if (n < K - 1) {
      const size_t o = ((size_t)b * (K - 1) + n) * TOPK + tid;
      const int c = a.cand[o];
      if (c >= 0 && c < V) {
        id = c;
        m = fminf(pr[c], a.q_cand[o]);
      }
    }
    cs_id[tid] = id;
    cs_min[tid] = m;
  }
  __syncthreads();
  const int C = (V + 255) / 256, v0 = min(V, tid * C), v1 = min(V, v0 + C);
  // two passes at most: if the residual has no mass (rounding), draw from p itself
  for (int pass = 0; pass < 2; ++pass) {
    float sum = 0.f;
    for (int v = v0; v < v1; ++v) sum += pr[v];
    if (pass == 0)
#pragma unroll
      for (int j = 0; j < TOPK; ++j)
        if (cs_id[j] >= v0 && cs_id[j] < v1) sum -= cs_min[j];
    part[tid] = sum;
    __syncthreads();
    if (tid == 0) {
      float run = 0.f;
      for (int t = 0; t < 256; ++t) {
        pref[t] = run;
        run += part[t];
      }
      s_total = run;
      s_pass = pass;
    }
    __syncthreads();
    if (s_total > 0.f || pass == 1) break;
    __syncthreads();
  }
  const bool corrected = s_pass == 0;   // the candidates' min(p, q) was taken out
  const float target = ur * s_total;
  if (target < pref[tid] + part[tid] && part[tid] > 0.f) atomicMin(&s_chunk, tid);
  __syncthreads();
  int chunk = s_chunk;
  if (tid == 0) {
    if (chunk == 256) {   // rounding left no chunk: the last one with mass
      chunk = 0;
      for (int t = 255; t >= 0; --t)
        if (part[t] > 0.f) { chunk = t; break; }
    }
    const int c0 = min(V, chunk * C), c1 = min(V, c0 + C);
    // the chunk's candidates, ascending by id
    int lid[TOPK];
    float lmin[TOPK];
    int cnt = 0;
    if (corrected)
      for (int j = 0; j < TOPK; ++j)
        if (cs_id[j] >= c0 && cs_id[j] < c1) {
          int k = cnt++;
          while (k > 0 && lid[k - 1] > cs_id[j]) { lid[k] = lid[k - 1]; lmin[k] = lmin[k - 1]; --k; }
          lid[k] = cs_id[j];
          lmin[k] = cs_min[j];
        }
    float run = pref[chunk];
    int tok = -1, last = c0, k = 0;
    for (int v = c0; v < c1; ++v) {
      float w = pr[v];
      if (k < cnt && lid[k] == v) w -= lmin[k++];
      if (w > 0.f) last = v;
      run += w;
      if (target < run && w > 0.f) { tok = v; break; }
    }
    if (tok < 0) tok = last;
    const size_t o = (size_t)b * K;
    for (int i = 0; i < K; ++i) a.committed[o + i] = i < n ? a.draft[(size_t)b * (K - 1) + i] : (i == n ? tok : -1);
    a.n_acc[b] = n;
    if (a.n_commit) a.n_commit[b] = n + 1;
    a.next_anchor[b] = tok;
  }
}

// splitmix64 (Steele, Lea and Flood's SplitMix generator; constants as published by Vigna).
__device__ __forceinline__ unsigned long long splitmix64(unsigned long long x) {
  unsigned long long z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// One thread per (sequence b, slot j): slot j < K - 1 is target token i = j + 1, compared with
// draft i; slot K - 1 is the token after the block.  Each slot's draws depend on (seed, counter,
// b, i) alone, so the slots of a sequence are computed side by side.
__global__ __launch_bounds__(1024) void synth_target_kernel(SynthArgs a) {
  __shared__ long long ctr;
  if (threadIdx.x == 0) ctr = *a.counter;
  __syncthreads();
  if (threadIdx.x == 0) *a.counter = ctr + 1;
  const int K = a.K;
  for (long t = threadIdx.x; t < (long)a.n_seq * K; t += blockDim.x) {
    const int b = (int)(t / K), j = (int)(t - (long)b * K);
    const unsigned long long key = a.seed ^ ((unsigned long long)ctr << 24) ^ ((unsigned long long)b << 8);
    if (j == K - 1) {
      a.target[(size_t)b * K + K - 1] = (int)(splitmix64(key ^ 0xFFFFull) % (unsigned long long)a.vocab);
      continue;
    }
    const int i = j + 1;
    // p < 0: committed tokens tau uniform on {1..K} (drafts 1..tau-1 match, draft tau does not)
    const int tau = a.p < 0.f ? 1 + (int)(splitmix64(key ^ 0xABCDull) % (unsigned long long)K) : K;
    const unsigned long long h1 = splitmix64(key ^ (unsigned long long)(2 * i));
    const unsigned long long h2 = splitmix64(key ^ (unsigned long long)(2 * i + 1));
    const float u = (float)(h1 >> 40) * (1.0f / 16777216.0f);
    const int di = a.draft[(size_t)b * (K - 1) + i - 1];
    const int alt = (int)(1 + h2 % (unsigned long long)(a.vocab - 1));
    const bool match = a.p < 0.f ? i < tau : u < a.p;
    a.target[(size_t)b * K + i - 1] = match ? di : (int)(((long long)di + alt) % a.vocab);
  }
}

hipError_t launch_select(bool bf, const SelectArgs& a, int n_seq, hipStream_t st) {
  if (a.K < 2 || a.K > SEL_KMAX || a.r < 8 || a.r > 256 || a.r % 8 || a.d < 64 || a.d > SEL_DMAX || a.d % 64 ||
      !a.spart || !a.sel_cnt)
    return hipErrorInvalidValue;
  // slots per workgroup: one for small batches (the most parallel split, with a hand-off to the
  // last workgroup of each sequence), else all of them (one workgroup per sequence when the rank
  // fits one chunk: no hand-off, each chunk of W_H read once per sequence)
  SelectArgs g = a;
  const int nrc = (a.r + SEL_SR - 1) / SEL_SR;
  g.spw = (long)n_seq * (a.K - 1) * nrc <= 128 ? 1 : (a.K - 1 < SEL_SPW ? a.K - 1 : SEL_SPW);
  const dim3 grid(((a.K - 1 + g.spw - 1) / g.spw) * nrc, n_seq);
  if (bf && g.spw <= SEL_HROWS) hipLaunchKernelGGL((select_kernel<bf16, true>), grid, dim3(SEL_T), 0, st, g);
  else if (bf) hipLaunchKernelGGL((select_kernel<bf16, false>), grid, dim3(SEL_T), 0, st, g);
  else hipLaunchKernelGGL((select_kernel<float, false>), grid, dim3(SEL_T), 0, st, g);
  return hipGetLastError();
}
__global__ __launch_bounds__(256) void fill_u32_kernel(unsigned* p, int n, unsigned v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}
hipError_t launch_fill_u32(unsigned* p, int n, unsigned v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}
hipError_t launch_verify(const VerifyArgs& a, hipStream_t st) {
  if (a.n_seq <= 0) return hipSuccess;
  // four sequences (waves) per workgroup
  hipLaunchKernelGGL(verify_kernel, dim3((a.n_seq + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_verify_rejection(const RejectArgs& a, hipStream_t st) {
  if (a.K < 2 || a.K > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(verify_rejection_kernel, dim3(a.n_seq), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_synth(const SynthArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(synth_target_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace dfl
