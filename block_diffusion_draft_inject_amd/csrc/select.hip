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
constexpr int SEL_RC = 16;      // selector-rank chunk staged in LDS at a time

template <typename T>
__device__ __forceinline__ float ldsel(const void* p, size_t i) {
  return ldv(reinterpret_cast<const T*>(p), i);
}

// order of Viterbi candidates: higher score, then smaller predecessor index, then rank
__device__ __forceinline__ bool vit_better(float s1, int c1, float s2, int c2) {
  return s1 > s2 || (s1 == s2 && c1 < c2);
}

template <typename T>
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  constexpr int NP = (SEL_KMAX - 2) * TOPK + 1;    // predecessor rows: anchor + candidates of slots 1..K-2
  constexpr int NC = (SEL_KMAX - 1) * TOPK;        // candidate rows of slots 1..K-1
  constexpr int VE = 16 / sizeof(T);               // table elements per 16-byte load
  __shared__ int cid[SEL_KMAX][TOPK];
  __shared__ float cu[SEL_KMAX][TOPK];
  __shared__ __attribute__((aligned(16))) float S[SEL_KMAX][TOPK][TOPK];   // S[t-1][b][a] (successor-major)
  __shared__ __attribute__((aligned(16))) float ta[NP][SEL_RC + 4];
  __shared__ __attribute__((aligned(16))) float tb[NC][SEL_RC + 4];
  __shared__ __attribute__((aligned(16))) float tg[SEL_KMAX][SEL_RC];
  __shared__ __attribute__((aligned(16))) float d1[2][TOPK];
  __shared__ __attribute__((aligned(16))) float d2[2][TOPK];
  __shared__ unsigned char bp1[SEL_KMAX][TOPK], bp2[SEL_KMAX][TOPK];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int K = a.K, r = a.r;
  int anchor = a.anchor[b];
  if (anchor < 0 || anchor >= a.vocab) {   // out-of-range token: record and read row 0
    if (tid == 0) atomicOr(a.dev_err, 8);
    anchor = 0;
  }
  const int ncand = (K - 1) * TOPK, npred = (K - 2) * TOPK + 1;
  for (int e = tid; e < ncand; e += 256) {
    cid[e / TOPK][e % TOPK] = a.topk_ids[(size_t)b * ncand + e];
    cu[e / TOPK][e % TOPK] = a.topk_logits[(size_t)b * ncand + e];
  }
  for (int e = tid; e < (K - 1) * TOPK * TOPK; e += 256) (&S[0][0][0])[e] = 0.f;
  __syncthreads();
  // pair term, accumulated over rank chunks of SEL_RC
  for (int r0 = 0; r0 < r; r0 += SEL_RC) {
    const int rc = min(SEL_RC, r - r0), nvr = rc / VE;   // r % VE == 0 (checked on the host)
    const int nload = (npred + ncand) * nvr;
    for (int e0 = tid; e0 < nload; e0 += 4 * 256) {
      u32x4 x[4];
      int rowi[4], vi[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * 256;
        const int rr = e / nvr;
        vi[u] = e % nvr;
        rowi[u] = e < nload ? rr : -1;
        int tok = 0;
        const void* tab = a.A;
        if (rr < npred) {
          tok = rr == 0 ? anchor : cid[(rr - 1) / TOPK][(rr - 1) % TOPK];
        } else if (rr < npred + ncand) {
          tok = cid[(rr - npred) / TOPK][(rr - npred) % TOPK];
          tab = a.B;
        }
        x[u] = e < nload ? reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(tab) + (size_t)tok * r + r0)[vi[u]]
                         : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (rowi[u] < 0) continue;
        const int rr = rowi[u];
        float* dst = rr < npred ? &ta[rr][vi[u] * VE] : &tb[rr - npred][vi[u] * VE];
        const T* xe = reinterpret_cast<const T*>(&x[u]);
#pragma unroll
        for (int j = 0; j < VE; ++j) dst[j] = ldv(xe, j);
      }
    }
    for (int e = tid; e < (K - 1) * rc; e += 256)
      tg[e / rc][e % rc] = a.gate[((size_t)b * (K - 1) + e / rc) * r + r0 + e % rc];
    __syncthreads();
    const int npairs = TOPK + (K - 2) * TOPK * TOPK;
    for (int e = tid; e < npairs; e += 256) {
      int t, ai, bi;
      if (e < TOPK) { t = 1; ai = 0; bi = e; }
      else { const int f = e - TOPK; t = 2 + f / (TOPK * TOPK); ai = (f / TOPK) % TOPK; bi = f % TOPK; }
      const f32x4* pa = reinterpret_cast<const f32x4*>(ta[t == 1 ? 0 : 1 + (t - 2) * TOPK + ai]);
      const f32x4* pb = reinterpret_cast<const f32x4*>(tb[(t - 1) * TOPK + bi]);
      const f32x4* pg = reinterpret_cast<const f32x4*>(tg[t - 1]);
      f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < SEL_RC / 4; ++q)
        if (4 * q < rc) acc4 += pa[q] * pg[q] * pb[q];
      S[t - 1][bi][ai] += acc4[0] + acc4[1] + acc4[2] + acc4[3];
    }
    __syncthreads();
  }
  for (int e = tid; e < (K - 1) * TOPK * TOPK; e += 256) {
    const int t1 = e / (TOPK * TOPK), bi = (e / TOPK) % TOPK;
    (&S[0][0][0])[e] += cu[t1][bi];
  }
  __syncthreads();
  // walk
  if (a.mode == 0) {
    if (tid < TOPK) {
      d1[0][tid] = S[0][tid][0];
      d2[0][tid] = NEG_INF;
    }
    __syncthreads();
    int cur = 0;
    for (int t = 2; t < K; ++t) {
      if (tid < TOPK) {
        const int bi = tid;
        float s1 = NEG_INF, s2 = NEG_INF;
        int c1 = 255, c2 = 255;
        float p1[TOPK], p2[TOPK], sa_[TOPK];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 x1 = reinterpret_cast<const f32x4*>(d1[cur])[q];
          const f32x4 x2 = reinterpret_cast<const f32x4*>(d2[cur])[q];
          const f32x4 xs = reinterpret_cast<const f32x4*>(S[t - 1][bi])[q];
#pragma unroll
          for (int j = 0; j < 4; ++j) { p1[4 * q + j] = x1[j]; p2[4 * q + j] = x2[j]; sa_[4 * q + j] = xs[j]; }
        }
#pragma unroll
        for (int ai = 0; ai < TOPK; ++ai) {
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const float prev = k == 0 ? p1[ai] : p2[ai];
            if (prev == NEG_INF) continue;
            const float sc = prev + sa_[ai];
            const int code = ai * 2 + k;
            if (vit_better(sc, code, s1, c1)) {
              s2 = s1; c2 = c1;
              s1 = sc; c1 = code;
            } else if (vit_better(sc, code, s2, c2)) {
              s2 = sc; c2 = code;
            }
          }
        }
        d1[cur ^ 1][bi] = s1;
        d2[cur ^ 1][bi] = s2;
        bp1[t - 1][bi] = (unsigned char)c1;
        bp2[t - 1][bi] = (unsigned char)c2;
      }
      __syncthreads();
      cur ^= 1;
    }
    if (tid == 0) {
      float s1 = NEG_INF, s2 = NEG_INF;
      int c1 = 255, c2 = 255;
      for (int bi = 0; bi < TOPK; ++bi)
        for (int k = 0; k < 2; ++k) {
          const float sc = k == 0 ? d1[cur][bi] : d2[cur][bi];
          if (sc == NEG_INF) continue;
          const int code = bi * 2 + k;
          if (vit_better(sc, code, s1, c1)) {
            s2 = s1; c2 = c1;
            s1 = sc; c1 = code;
          } else if (vit_better(sc, code, s2, c2)) {
            s2 = sc; c2 = code;
          }
        }
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
  } else {
    if (tid == 0) {
      int ai = 0;
      float total = 0.f, margin = __builtin_huge_valf();
      for (int t = 1; t < K; ++t) {
        float s1 = NEG_INF, s2 = NEG_INF;
        int c1 = 0;
        for (int bi = 0; bi < TOPK; ++bi) {
          const float sc = S[t - 1][bi][ai];
          if (sc > s1) { s2 = s1; s1 = sc; c1 = bi; }
          else if (sc > s2) { s2 = sc; }
        }
        margin = fminf(margin, s1 - s2);
        total += s1;
        a.path[(size_t)b * (K - 1) + t - 1] = cid[t - 1][c1];
        ai = c1;
      }
      if (a.score) a.score[b] = total;
      if (a.margin) a.margin[b] = margin;
    }
  }
}

// Greedy longest-prefix verification: one thread per sequence.
__global__ void verify_kernel(VerifyArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.n_seq) return;
  const int K = a.K;
  const int* dr = a.draft + (size_t)b * (K - 1);
  const int* tg = a.target + (size_t)b * K;
  int n = 0;
  while (n < K - 1 && dr[n] == tg[n]) ++n;
  int* com = a.committed + (size_t)b * K;
  for (int i = 0; i < K; ++i) com[i] = i < n ? dr[i] : (i == n ? tg[n] : -1);
  a.n_acc[b] = n;
  if (a.n_commit) a.n_commit[b] = n + 1;
  a.next_anchor[b] = tg[n];
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
  for (int i = 1; i < K; ++i) {
    const unsigned long long h1 = splitmix64(key ^ (unsigned long long)(2 * i));
    const unsigned long long h2 = splitmix64(key ^ (unsigned long long)(2 * i + 1));
    const float u = (float)(h1 >> 40) * (1.0f / 16777216.0f);
    const int di = a.draft[(size_t)b * (K - 1) + i - 1];
    const int alt = (int)(1 + h2 % (unsigned long long)(a.vocab - 1));
    a.target[(size_t)b * K + i - 1] = (u < a.p) ? di : (int)(((long long)di + alt) % a.vocab);
  }
  a.target[(size_t)b * K + K - 1] = (int)(splitmix64(key ^ 0xFFFFull) % (unsigned long long)a.vocab);
}

hipError_t launch_select(bool bf, const SelectArgs& a, int n_seq, hipStream_t st) {
  if (bf) hipLaunchKernelGGL(select_kernel<bf16>, dim3(n_seq), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(select_kernel<float>, dim3(n_seq), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_verify(const VerifyArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(verify_kernel, dim3((a.n_seq + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_synth(const SynthArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(synth_target_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace dfl
