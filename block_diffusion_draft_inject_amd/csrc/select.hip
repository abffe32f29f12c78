// Path selector, greedy verification, and the benchmark's stand-in target.
//
// Selector ("Architecture", kb.ekarisky.com, section "Problem 1 -- Independent picks are
// incoherent"): keep the top-16 candidates of every draft slot and score adjacent pairs,
//   S_t(a, b) = U_t(b) + < A(a) * H(h_t), B(b) >,   H(h_t) = sigmoid(W_H h_t),
// all pairs at once; only the walk over the precomputed scores is sequential.  One workgroup
// per sequence.  VITERBI keeps the two best partial paths per state (so the margin to the
// second-best complete path is exact); GREEDY follows the best successor.
#include "rowops.h"

namespace dfl {

constexpr int SEL_KMAX = 32;    // block size
constexpr int SEL_RMAX = 256;   // selector rank
constexpr int SEL_RC = 16;      // rank chunk of the predecessor rows staged in LDS
constexpr int SEL_NP = (SEL_KMAX - 2) * TOPK + 1;   // predecessor rows: anchor + candidates of slots 1..K-2

// order of Viterbi candidates: higher score, then smaller code (2 * predecessor + rank)
__device__ __forceinline__ bool vit_better(float s1, int c1, float s2, int c2) {
  return (s1 > s2) | ((s1 == s2) & (c1 < c2));
}

// (s1,c1) >= (s2,c2) are a sorted best-two list; insert candidate (s,c)
__device__ __forceinline__ void top2_push(float& s1, int& c1, float& s2, int& c2, float s, int c) {
  const bool b1 = vit_better(s, c, s1, c1), b2 = vit_better(s, c, s2, c2);
  s2 = b1 ? s1 : (b2 ? s : s2);
  c2 = b1 ? c1 : (b2 ? c : c2);
  s1 = b1 ? s : s1;
  c1 = b1 ? c : c1;
}

// DPP quad permutation (lanes l ^ 1 for 0xB1, l ^ 2 for 0x4E inside each group of four)
template <int CTRL>
__device__ __forceinline__ int quad_perm_i(int v) { return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false); }
template <int CTRL>
__device__ __forceinline__ float quad_perm_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// merge the best-two lists of the lanes of a quad (DPP, no LDS round trip)
template <int CTRL>
__device__ __forceinline__ void top2_quad(float& s1, int& c1, float& s2, int& c2) {
  const float o1 = quad_perm_f<CTRL>(s1), o2 = quad_perm_f<CTRL>(s2);
  const int p1 = quad_perm_i<CTRL>(c1), p2 = quad_perm_i<CTRL>(c2);
  top2_push(s1, c1, s2, c2, o1, p1);
  top2_push(s1, c1, s2, c2, o2, p2);
}

// merge the best-two lists of this lane and lane ^ m
__device__ __forceinline__ void top2_xor(float& s1, int& c1, float& s2, int& c2, int m) {
  const float o1 = __shfl_xor(s1, m, WAVE), o2 = __shfl_xor(s2, m, WAVE);
  const int p1 = __shfl_xor(c1, m, WAVE), p2 = __shfl_xor(c2, m, WAVE);
  top2_push(s1, c1, s2, c2, o1, p1);
  top2_push(s1, c1, s2, c2, o2, p2);
}

// gate[t-1][j] = sigmoid(W_H[j] . h_final[b][t]) for slots t = 1..K-1, into LDS.
// bf16 tables: one 16x16 MFMA tile per (slot tile, rank tile); the four waves split the hidden
// dimension, h enters as bf16 hi + lo planes (two MFMAs), partial tiles are summed through LDS.
template <typename T>
__device__ __forceinline__ void sel_gates(const SelectArgs& a, int b, float (*gt)[SEL_RMAX], float (*red)[64][4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, r = a.r, d = a.d;
  const float* hb = a.h_final + (size_t)b * K * d;
  if constexpr (sizeof(T) == 2) {
    const int li = lane & 15, kg = lane >> 4;
    const int nch = d / 32;                 // 32-wide k chunks; the waves take every 4th
    constexpr int BATCH = 8;               // 24 loads of 16 bytes in flight per lane
    for (int mt = 0; mt < (K + 15) / 16; ++mt)
      for (int nt = 0; nt < (r + 15) / 16; ++nt) {
        const float* hr = hb + (size_t)min(mt * 16 + li, K - 1) * d + kg * 8;
        const bf16* wr = reinterpret_cast<const bf16*>(a.WH) + (size_t)min(nt * 16 + li, r - 1) * d + kg * 8;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int c0 = wave; c0 < nch; c0 += 4 * BATCH) {
          f32x4 h0[BATCH], h1[BATCH];
          u32x4 w[BATCH];
#pragma unroll
          for (int u = 0; u < BATCH; ++u) {     // all loads of the batch first
            const int c = min(c0 + 4 * u, nch - 1);
            h0[u] = *reinterpret_cast<const f32x4*>(hr + c * 32);
            h1[u] = *reinterpret_cast<const f32x4*>(hr + c * 32 + 4);
            w[u] = *reinterpret_cast<const u32x4*>(wr + c * 32);
          }
#pragma unroll
          for (int u = 0; u < BATCH; ++u) {
            // a chunk past the end (its loads were clamped) adds zero: no branch, so that the
            // compiler keeps the whole batch of loads ahead of the first MFMA
            if (c0 + 4 * u >= nch) w[u] = u32x4{0u, 0u, 0u, 0u};
            u32x4 hi, lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x0 = e < 2 ? h0[u][2 * e] : h1[u][2 * e - 4];
              const float x1 = e < 2 ? h0[u][2 * e + 1] : h1[u][2 * e - 3];
              const bf16 a0 = f2bf(x0), a1 = f2bf(x1);
              hi[e] = (unsigned)a0 | ((unsigned)a1 << 16);
              lo[e] = (unsigned)f2bf(x0 - bf2f(a0)) | ((unsigned)f2bf(x1 - bf2f(a1)) << 16);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(hi), as_bf16x8(w[u]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lo), as_bf16x8(w[u]), acc, 0, 0, 0);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave][lane][j] = acc[j];
        __syncthreads();
        if (wave == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float g = red[0][lane][j] + red[1][lane][j] + red[2][lane][j] + red[3][lane][j];
            const int t = mt * 16 + kg * 4 + j, jj = nt * 16 + li;   // D layout: row 4 kg + j, column li
            if (t >= 1 && t < K && jj < r) gt[t - 1][jj] = sigmoidf_(g);
          }
        }
        __syncthreads();
      }
  } else {
    // fp32 tables: one wave per dot product
    const float* wh = reinterpret_cast<const float*>(a.WH);
    for (int e = wave; e < (K - 1) * r; e += 4) {
      const int t = e / r + 1, j = e % r;
      float acc = 0.f;
      for (int k = lane; k < d; k += 64) acc += hb[(size_t)t * d + k] * wh[(size_t)j * d + k];
      acc = wave_sum(acc);
      if (lane == 0) gt[t - 1][j] = sigmoidf_(acc);
    }
    __syncthreads();
  }
}

// Path selector for one sequence per workgroup.  Phases: candidates -> gates (in-kernel) ->
// pair scores S_t(a, b) for all slots at once (one thread per (slot, successor), predecessor
// rows staged in LDS by rank chunks) -> the sequential walk in one wave with shuffles only.
template <typename T>
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  __shared__ int cid[SEL_KMAX][TOPK];
  __shared__ float cu[SEL_KMAX][TOPK];
  __shared__ __attribute__((aligned(16))) float gt[SEL_KMAX][SEL_RMAX];
  __shared__ __attribute__((aligned(16))) float red[4][64][4];
  __shared__ __attribute__((aligned(16))) float ta[SEL_NP][SEL_RC + 4];
  __shared__ __attribute__((aligned(16))) float S[SEL_KMAX][TOPK][TOPK];   // S[t-1][b][a]
  __shared__ unsigned char bp1[SEL_KMAX][TOPK], bp2[SEL_KMAX][TOPK];
  __shared__ __attribute__((aligned(16))) float dv[2][TOPK];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, r = a.r;
  int anchor = a.anchor[b];
  if (anchor < 0 || anchor >= a.vocab) {   // out-of-range token: record and read row 0
    if (tid == 0) atomicOr(a.dev_err, 8);
    anchor = 0;
  }
  const int ncand = (K - 1) * TOPK, npred = (K - 2) * TOPK + 1;
  for (int e = tid; e < ncand; e += 256) {
    int id = a.topk_ids[(size_t)b * ncand + e];
    if (id < 0 || id >= a.vocab) {         // out-of-range candidate: record and read row 0
      atomicOr(a.dev_err, 16);
      id = 0;
    }
    cid[e / TOPK][e % TOPK] = id;
    cu[e / TOPK][e % TOPK] = a.topk_logits[(size_t)b * ncand + e];
  }
  __syncthreads();
  // pair scores: thread (t, bi) for t = 1..K-1 (two passes cover K up to 32), accumulated over
  // rank chunks of SEL_RC.  The first chunk's table loads are issued before the gate phase so
  // that their latency overlaps it.
  constexpr int VE = 16 / sizeof(T);
  constexpr int VPR = SEL_RC / VE;                      // 16-byte vectors per row chunk
  constexpr int XA = (SEL_NP * VPR + 255) / 256;        // predecessor vectors per thread
  float acc[2][TOPK];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int i = 0; i < TOPK; ++i) acc[q][i] = 0.f;
  u32x4 xa[XA], xb[2][VPR];
  auto issue = [&](int r0) {
    const int nv = min(SEL_RC, r - r0) / VE;           // rank is a multiple of 8
#pragma unroll
    for (int u = 0; u < XA; ++u) {
      const int e = tid + 256 * u, row = e / VPR, v = e % VPR;
      const bool ok = row < npred && v < nv;
      const int ci = max(min(row, npred - 1) - 1, 0);  // candidate index of predecessor row >= 1
      const int tok = row == 0 ? anchor : cid[ci / TOPK][ci % TOPK];
      xa[u] = ok ? reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.A) + (size_t)tok * r + r0)[v]
                 : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = min(tid + 256 * q, ncand - 1);
      const u32x4* brow = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.B) +
                                                         (size_t)cid[e / TOPK][e % TOPK] * r + r0);
#pragma unroll
      for (int v = 0; v < VPR; ++v) xb[q][v] = v < nv ? brow[v] : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto consume = [&](int r0) {
    const int rc = min(SEL_RC, r - r0);
#pragma unroll
    for (int u = 0; u < XA; ++u) {
      const int e = tid + 256 * u, row = e / VPR, v = e % VPR;
      if (row < npred) {
        const T* xe = reinterpret_cast<const T*>(&xa[u]);
#pragma unroll
        for (int j = 0; j < VE; ++j) ta[row][v * VE + j] = v * VE < rc ? ldv(xe, j) : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid + 256 * q;
      if (e >= ncand) break;
      const int t = e / TOPK + 1;
      float gb[SEL_RC];
#pragma unroll
      for (int j = 0; j < SEL_RC; ++j)
        gb[j] = j < rc ? ldv(reinterpret_cast<const T*>(&xb[q][j / VE]), j % VE) * gt[t - 1][r0 + j] : 0.f;
      const int p0 = t == 1 ? 0 : 1 + (t - 2) * TOPK;
      const int na = t == 1 ? 1 : TOPK;
#pragma unroll
      for (int ai = 0; ai < TOPK; ++ai) {
        if (ai >= na) break;
        const f32x4* pa = reinterpret_cast<const f32x4*>(ta[p0 + ai]);
        float sacc = 0.f;
#pragma unroll
        for (int j4 = 0; j4 < SEL_RC / 4; ++j4) {
          const f32x4 x = pa[j4];
          sacc += x[0] * gb[4 * j4] + x[1] * gb[4 * j4 + 1] + x[2] * gb[4 * j4 + 2] + x[3] * gb[4 * j4 + 3];
        }
        acc[q][ai] += sacc;
      }
    }
    __syncthreads();
  };
  issue(0);
  sel_gates<T>(a, b, gt, red);              // ends with a barrier: gt visible
  consume(0);
  for (int r0 = SEL_RC; r0 < r; r0 += SEL_RC) {
    issue(r0);
    consume(r0);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = tid + 256 * q;
    if (e >= ncand) break;
    const int t = e / TOPK + 1, bi = e % TOPK;
#pragma unroll
    for (int ai = 0; ai < TOPK; ++ai) S[t - 1][bi][ai] = acc[q][ai] + cu[t - 1][bi];
  }
  __syncthreads();
  if (wave != 0) return;
  // ---- the walk: one wave; lane = 4 * bi + qa holds predecessors a = 4 qa .. 4 qa + 3 of state bi
  const int bi = lane >> 2, qa = lane & 3;
  if (a.mode == 0) {
    // partial-path scores of the previous slot live in LDS (dv[0][a] = best, dv[1][a] = second);
    // each lane reads its four predecessors with two 16-byte reads, the quad merges by DPP
    if (lane < TOPK) {
      dv[0][lane] = S[0][lane][0];           // slot 1: the single path anchor -> lane
      dv[1][lane] = NEG_INF;
    }
    float d1 = 0.f, d2 = 0.f;
    for (int t = 2; t < K; ++t) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const f32x4 p1v = *reinterpret_cast<const f32x4*>(&dv[0][4 * qa]);
      const f32x4 p2v = *reinterpret_cast<const f32x4*>(&dv[1][4 * qa]);
      const f32x4 sv = *reinterpret_cast<const f32x4*>(&S[t - 1][bi][4 * qa]);
      // A predecessor's rank-1 extension always beats its rank-2 one (same pair term, better
      // or equal partial score, smaller code), so the best two of the 32 candidates are: the
      // best rank-1 extension b, and the better of the second-best rank-1 extension s and the
      // rank-2 extension w of b's predecessor.  Each lane summarises its four predecessors as
      // (b, s, w); the quad merges summaries.  An absent path enters as (-inf, 255).
      float bs = NEG_INF, ss = NEG_INF, ws = NEG_INF;
      int bc = 255, sc = 255, wc = 255;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ai = 4 * qa + i;
        const float v1 = p1v[i] + sv[i], v2 = p2v[i] + sv[i];
        const int c1 = p1v[i] != NEG_INF ? 2 * ai : 255, c2 = p2v[i] != NEG_INF ? 2 * ai + 1 : 255;
        const bool top = vit_better(v1, c1, bs, bc);
        const bool sec = !top && vit_better(v1, c1, ss, sc);
        ss = top ? bs : (sec ? v1 : ss);
        sc = top ? bc : (sec ? c1 : sc);
        ws = top ? v2 : ws;
        wc = top ? c2 : wc;
        bs = top ? v1 : bs;
        bc = top ? c1 : bc;
      }
      auto merge = [&](float obs, int obc, float oss, int osc, float ows, int owc) {
        const bool theirs = vit_better(obs, obc, bs, bc);
        // the loser's best competes with the winner's second
        const float ls = theirs ? bs : obs, ws2 = theirs ? oss : ss;
        const int lc = theirs ? bc : obc, wsc = theirs ? osc : sc;
        const bool lb = vit_better(ls, lc, ws2, wsc);
        ss = lb ? ls : ws2;
        sc = lb ? lc : wsc;
        ws = theirs ? ows : ws;
        wc = theirs ? owc : wc;
        bs = theirs ? obs : bs;
        bc = theirs ? obc : bc;
      };
      merge(quad_perm_f<0xB1>(bs), quad_perm_i<0xB1>(bc), quad_perm_f<0xB1>(ss), quad_perm_i<0xB1>(sc),
            quad_perm_f<0xB1>(ws), quad_perm_i<0xB1>(wc));
      merge(quad_perm_f<0x4E>(bs), quad_perm_i<0x4E>(bc), quad_perm_f<0x4E>(ss), quad_perm_i<0x4E>(sc),
            quad_perm_f<0x4E>(ws), quad_perm_i<0x4E>(wc));
      const bool wsec = vit_better(ws, wc, ss, sc);
      const float s1 = bs, s2 = wsec ? ws : ss;
      const int c1 = bc, c2 = wsec ? wc : sc;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (qa == 0) {
        dv[0][bi] = s1;
        dv[1][bi] = s2;
        bp1[t - 1][bi] = (unsigned char)c1;
        bp2[t - 1][bi] = (unsigned char)c2;
      }
      d1 = s1;
      d2 = s2;
    }
    if (K == 2) {
      d1 = S[0][bi][0];
      d2 = NEG_INF;
    }
    // best two complete paths over the states of slot K-1 (code 2 bi + rank)
    float s1 = NEG_INF, s2 = NEG_INF;
    int c1 = 255, c2 = 255;
    if (qa == 0) {
      if (d1 != NEG_INF) top2_push(s1, c1, s2, c2, d1, 2 * bi);
      if (d2 != NEG_INF) top2_push(s1, c1, s2, c2, d2, 2 * bi + 1);
    }
    for (int m = 4; m < 64; m <<= 1) top2_xor(s1, c1, s2, c2, m);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane == 0) {
      int st = c1 >> 1, rank = c1 & 1;
      for (int t = K - 1; t >= 1; --t) {
        a.path[(size_t)b * (K - 1) + t - 1] = cid[t - 1][st];
        if (t > 1) {
          const int code = rank == 0 ? bp1[t - 1][st] : bp2[t - 1][st];
          st = code >> 1;
          rank = code & 1;
        }
      }
      if (a.score) a.score[b] = s1;
      if (a.margin) a.margin[b] = s1 - s2;
    }
  } else if (a.mode == 2) {
    // sampling walk: at slot t, q(b) = softmax_b(S_t(a, b) / T) over the 16 candidates given
    // the previous pick a, cut to its top-p nucleus; the pick is the first b (candidate order)
    // whose inclusive cumulative probability exceeds u_t times the total
    int ai = 0;
    const bool in = lane < TOPK;
    const bool cut = a.top_p < 1.f;
    for (int t = 1; t < K; ++t) {
      const float z = in ? S[t - 1][lane][ai] * a.inv_temp : NEG_INF;
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
        a.path[o] = cid[t - 1][pick];
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
      const float v = lane < TOPK ? S[t - 1][lane][ai] : NEG_INF;
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
      if (lane == 0) a.path[(size_t)b * (K - 1) + t - 1] = cid[t - 1][i1];
      ai = i1;
    }
    if (lane == 0) {
      if (a.score) a.score[b] = total;
      if (a.margin) a.margin[b] = margin;
    }
  }
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

__global__ __launch_bounds__(1024) void synth_target_kernel(SynthArgs a) {
  __shared__ long long ctr;
  const int b = threadIdx.x;
  if (b == 0) ctr = *a.counter;
  __syncthreads();
  if (b == 0) *a.counter = ctr + 1;
  if (b >= a.n_seq) return;
  const int K = a.K;
  const unsigned long long key = a.seed ^ ((unsigned long long)ctr << 24) ^ ((unsigned long long)b << 8);
  // p < 0: committed tokens tau uniform on {1..K} (drafts 1..tau-1 match, draft tau does not)
  const int tau = a.p < 0.f ? 1 + (int)(splitmix64(key ^ 0xABCDull) % (unsigned long long)K) : K;
  for (int i = 1; i < K; ++i) {
    const unsigned long long h1 = splitmix64(key ^ (unsigned long long)(2 * i));
    const unsigned long long h2 = splitmix64(key ^ (unsigned long long)(2 * i + 1));
    const float u = (float)(h1 >> 40) * (1.0f / 16777216.0f);
    const int di = a.draft[(size_t)b * (K - 1) + i - 1];
    const int alt = (int)(1 + h2 % (unsigned long long)(a.vocab - 1));
    const bool match = a.p < 0.f ? i < tau : u < a.p;
    a.target[(size_t)b * K + i - 1] = match ? di : (int)(((long long)di + alt) % a.vocab);
  }
  a.target[(size_t)b * K + K - 1] = (int)(splitmix64(key ^ 0xFFFFull) % (unsigned long long)a.vocab);
}

hipError_t launch_select(bool bf, const SelectArgs& a, int n_seq, hipStream_t st) {
  if (bf) hipLaunchKernelGGL(select_kernel<bf16>, dim3(n_seq), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(select_kernel<float>, dim3(n_seq), dim3(256), 0, st, a);
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
