// Shared device helpers for libdflash (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

typedef uint16_t bf16;   // bfloat16 storage (bit pattern)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf2f(bf16 b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bfloat16, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ bf16 f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16)(u >> 16);
}

// Storage-type dispatch: float storage keeps fp32, bf16 storage rounds on store.
__device__ __forceinline__ float ldv(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ldv(const bf16* p, size_t i) { return bf2f(p[i]); }
__device__ __forceinline__ void stv(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void stv(bf16* p, size_t i, float v) { p[i] = f2bf(v); }

// Activations are carried in fp32.  For bf16 drafters an activation buffer holds two bf16
// planes, hi = bf16(x) at index i and lo = bf16(x - hi) at index i + plane, so that a bf16 MFMA
// can consume it as hi*w + lo*w (about 16 mantissa bits); for fp32 drafters it is plain fp32.
__device__ __forceinline__ void st_act(bf16* p, size_t i, size_t plane, float v) {
  const bf16 hi = f2bf(v);
  p[i] = hi;
  p[i + plane] = f2bf(v - bf2f(hi));
}
__device__ __forceinline__ void st_act(float* p, size_t i, size_t, float v) { p[i] = v; }
__device__ __forceinline__ float ld_act(const bf16* p, size_t i, size_t plane) { return bf2f(p[i]) + bf2f(p[i + plane]); }
__device__ __forceinline__ float ld_act(const float* p, size_t i, size_t) { return p[i]; }

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS operations, not for its
// global loads, so prefetches stay in flight across it (__syncthreads() carries a release fence
// that waits for every outstanding global load).  The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Cross-lane data movement with DPP (no LDS round trip).  Controls used: quad_perm [1,0,3,2]
// (0xB1), quad_perm [2,3,0,1] (0x4E), row_half_mirror (0x141: lane i <- lane 7-i within 8),
// row_mirror (0x140: lane i <- lane 15-i within 16).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}

// Wave-wide sum / max, the same value in every lane.  Needs all 64 lanes active.  Within each
// row of 16 lanes the four symmetric DPP steps leave every lane with the row total (a + b is
// evaluated as b + a in the partner lane: identical rounding); the four row totals are then
// combined in lane order, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return ((lane_f(v, 0) + lane_f(v, 16)) + lane_f(v, 32)) + lane_f(v, 48);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// Block-wide sum of NV values at once for a block of NT threads; scratch holds (NT/64)*NV floats.
template <int NV, int NT = 256>
__device__ __forceinline__ void block_sum(float (&v)[NV], float* scratch) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = wave_sum(v[i]);
  lds_barrier();
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) scratch[w * NV + i] = v[i];
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) t += scratch[k * NV + i];
    v[i] = t;
  }
  lds_barrier();
}

template <int NV>
__device__ __forceinline__ void block_sum256(float (&v)[NV], float* scratch) {
  block_sum<NV, 256>(v, scratch);
}

// Candidate order for top-k: higher value first, then smaller id.
__device__ __forceinline__ bool cand_better(float va, int ia, float vb, int ib) {
  return (va > vb) | ((va == vb) & (ia < ib));   // bitwise: no short-circuit branches
}

// Wave-wide best candidate (value, id) under cand_better.
__device__ __forceinline__ void wave_best(float& v, int& id) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float v2 = __shfl_xor(v, o, WAVE);
    int i2 = __shfl_xor(id, o, WAVE);
    if (cand_better(v2, i2, v, id)) { v = v2; id = i2; }
  }
}

constexpr int NCOUNTERS = 64;   // lm_head work counters (one per 128-row tile), zeroed by the draft plan
constexpr int TOPK = 16;
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr int ID_NONE = 0x7fffffff;

// A thread-private sorted top-16 list (best first) kept in registers.
struct Top16 {
  float v[TOPK];
  int id[TOPK];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < TOPK; ++i) { v[i] = NEG_INF; id[i] = ID_NONE; }
  }
  // Insert (val, idx) if it beats the current 16th entry; keeps the list sorted.  Branch-free
  // apart from the threshold test: better[] is monotone along the sorted list, so entry i
  // takes its upper neighbour if the candidate beats that neighbour, else the candidate if it
  // beats entry i, else stays.
  __device__ __forceinline__ void push(float val, int idx) {
    if (!cand_better(val, idx, v[TOPK - 1], id[TOPK - 1])) return;
    bool b[TOPK];
#pragma unroll
    for (int i = 0; i < TOPK; ++i) b[i] = cand_better(val, idx, v[i], id[i]);
#pragma unroll
    for (int i = TOPK - 1; i >= 0; --i) {
      const bool up = i > 0 && b[i > 0 ? i - 1 : 0];
      const float vu = v[i > 0 ? i - 1 : 0];
      const int iu = id[i > 0 ? i - 1 : 0];
      v[i] = up ? vu : (b[i] ? val : v[i]);
      id[i] = up ? iu : (b[i] ? idx : id[i]);
    }
  }
  // The same for a list fed by a column stream in ascending order: idx is larger than every
  // id in the list, so on equal values the candidate ranks last and "beats" is a plain value
  // comparison (one compare per entry instead of three).
  __device__ __forceinline__ void push_asc(float val, int idx) {
    if (!(val > v[TOPK - 1])) return;
    bool b[TOPK];
#pragma unroll
    for (int i = 0; i < TOPK; ++i) b[i] = val > v[i];
#pragma unroll
    for (int i = TOPK - 1; i >= 0; --i) {
      const bool up = i > 0 && b[i > 0 ? i - 1 : 0];
      const float vu = v[i > 0 ? i - 1 : 0];
      const int iu = id[i > 0 ? i - 1 : 0];
      v[i] = up ? vu : (b[i] ? val : v[i]);
      id[i] = up ? iu : (b[i] ? idx : id[i]);
    }
  }
};

}  // namespace dfl
