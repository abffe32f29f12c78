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
  __shared__ int cid[SEL_KMAX][TOPK];
  __shared__ float cu[SEL_KMAX][TOPK];
  __shared__ float gate[SEL_RMAX];
  __shared__ float sa[TOPK][SEL_RMAX + 1];
  __shared__ float sb[TOPK][SEL_RMAX + 1];
  __shared__ float S[SEL_KMAX][TOPK][TOPK];        // S[t-1][a][b]
  __shared__ float d1[2][TOPK], d2[2][TOPK];
  __shared__ unsigned char bp1[SEL_KMAX][TOPK], bp2[SEL_KMAX][TOPK];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int K = a.K, d = a.d, r = a.r;
  int anchor = a.anchor[b];
  if (anchor < 0 || anchor >= a.vocab) {   // out-of-range token: record and read row 0
    if (tid == 0) atomicOr(a.dev_err, 8);
    anchor = 0;
  }
  for (int e = tid; e < (K - 1) * TOPK; e += 256) {
    cid[e / TOPK][e % TOPK] = a.topk_ids[(size_t)b * (K - 1) * TOPK + e];
    cu[e / TOPK][e % TOPK] = a.topk_logits[(size_t)b * (K - 1) * TOPK + e];
  }
  __syncthreads();
  for (int t = 1; t < K; ++t) {
    // context gate of slot t: one wave per output j
    for (int j = w; j < r; j += 4) {
      float acc = 0.f;
      for (int k = lane; k < d; k += 64)
        acc += ldsel<T>(a.WH, (size_t)j * d + k) * ldsel<T>(a.h_final, ((size_t)b * K + t) * d + k);
      acc = wave_sum(acc);
      if (lane == 0) gate[j] = sigmoidf_(acc);
    }
    // predecessor (A) rows and candidate (B) rows
    const int npred = (t == 1) ? 1 : TOPK;
    for (int e = tid; e < TOPK * r; e += 256) {
      const int i = e / r, j = e % r;
      sb[i][j] = ldsel<T>(a.B, (size_t)cid[t - 1][i] * r + j);
      if (i < npred) {
        const int pid = (t == 1) ? anchor : cid[t - 2][i];
        sa[i][j] = ldsel<T>(a.A, (size_t)pid * r + j);
      }
    }
    __syncthreads();
    {
      const int ai = tid / TOPK, bi = tid % TOPK;
      if (ai < npred) {
        float acc = 0.f;
        for (int j = 0; j < r; ++j) acc += sa[ai][j] * gate[j] * sb[bi][j];
        S[t - 1][ai][bi] = cu[t - 1][bi] + acc;
      }
    }
    __syncthreads();
  }
  // walk
  if (a.mode == 0) {
    if (tid < TOPK) {
      d1[0][tid] = S[0][0][tid];
      d2[0][tid] = NEG_INF;
    }
    __syncthreads();
    int cur = 0;
    for (int t = 2; t < K; ++t) {
      if (tid < TOPK) {
        const int bi = tid;
        float s1 = NEG_INF, s2 = NEG_INF;
        int c1 = 255, c2 = 255;
        for (int ai = 0; ai < TOPK; ++ai) {
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const float prev = k == 0 ? d1[cur][ai] : d2[cur][ai];
            if (prev == NEG_INF) continue;
            const float sc = prev + S[t - 1][ai][bi];
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
          const float sc = S[t - 1][ai][bi];
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
