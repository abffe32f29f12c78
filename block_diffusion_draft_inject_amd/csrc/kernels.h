// Internal launcher declarations for libdflash (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "common.h"

namespace dfl {

constexpr int MAX_SEG = 32;

enum GemmMode { GEMM_PARTIAL = 0, GEMM_SWIGLU = 1, GEMM_TOPK = 2 };

// C[m][n] = sum_k A[m][k] * B_n[k] where B_n is row n of a weight matrix split into
// equal row segments: row n lives at seg[n / seg_rows] + (n % seg_rows) * ldb.
struct GemmParams {
  const void* A;          // [M][lda] activations: bf16 hi plane (lo plane a_plane elements later) or fp32
  int lda;
  size_t a_plane;         // elements from the hi plane to the lo plane (bf16 drafters)
  int M;                  // rows (allocation bound)
  const int* m_dev;       // optional device row count: rows >= *m_dev - m_off are skipped
  int m_off;
  const void* seg[MAX_SEG];
  int seg_rows;
  int ldb;
  int N, K;
  int splits;             // k-splits (PARTIAL)
  // PARTIAL: part[s][m][n], row stride N
  float* part;
  // SWIGLU: out[m][j] = silu(C[m][j]) * C[m][half + j], j < half; bf16 hi plane, lo plane
  // out_plane elements later
  void* out;
  size_t out_plane;
  int half;
  // TOPK (lm_head): per (row, group) top-16 partials; rows whose slot (row % block) is 0 skipped
  float* tk_val;
  int* tk_id;
  int groups;
  int block;
  float* logits;          // optional full logits [row/block][block-1][N] for slots >= 1
  const float* row_scale; // FP8 lm_head (<= 16 rows): the weights are E4M3 codes [N][ldb bytes],
                          // weight row n stands for code * row_scale[n]
  int* counter;           // TOPK skinny (17..64 rows): per-row-tile fragment counters, zero before the launch
  const unsigned char* blk_scale;  // MXFP4 lm_head (<= 16 rows): the weights are E2M1 codes [N][K/2 bytes], with
                                   // scale byte E [N][K/32] per 32 weights standing for 2^(E - 127)
  int b_blocked;          // MFMA tiles with bf16 weights: seg[] point into 16-row-blocked copies
                          // (block_weights_kernel), not row-major matrices
};

struct GemmPlan {
  int kind;      // 0 = skinny (17..64 rows), 2 = f32 simple, 3 = stream (<= 16 rows), 4 = lm_head
                 // waves (<= 16 rows), 5 = MFMA tiles with LDS-DMA operands (more than 64 rows)
  int slc;       // stream: 64-wide chunks per wave
  int mt;        // skinny: row fragments (1,2,4); MFMA tiles: 0 = 128 x 128, 1 = 256 x 256,
                 // 2 = 256 x 128
  int splits;
  int groups;    // TOPK groups
  dim3 grid;
};

// FP8 weights (row_scale set): eight E4M3 codes (two words, lowest byte first) -> eight bf16
// values code * s, exact (an E4M3 value times a power of two fits bf16)
__device__ __forceinline__ bf16x8 fp8x8_bf16(unsigned w0, unsigned w1, float s) {
  u32x4 o;
  o[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false));
  o[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true));
  o[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false));
  o[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true));
  return as_bf16x8(o);
}

// MXFP4 weights (blk_scale set): one word of eight E2M1 codes (element 2j in the low nibble of
// byte j) -> eight bf16 values code * s, s = 2^(E - 127) of the codes' block, exact
__device__ __forceinline__ bf16x8 fp4x8_bf16(unsigned w, float s) {
  u32x4 o;
  o[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0));
  o[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1));
  o[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2));
  o[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
  return as_bf16x8(o);
}

// Row n of the segmented weight matrix.
__device__ __forceinline__ const bf16* brow_ptr(const GemmParams& p, int n) {
  const int s = n / p.seg_rows;
  return reinterpret_cast<const bf16*>(p.seg[s]) + (size_t)(n - s * p.seg_rows) * p.ldb;
}

// Rows the launch computes: M, or the device row count when one is given.
__device__ __forceinline__ int rows_valid(const GemmParams& p) {
  return p.m_dev ? max(0, min(p.M, *p.m_dev - p.m_off)) : p.M;
}

// Writes one wave-tile of logits (rows of slot >= 1 only) when full logits are requested.
__device__ __forceinline__ void store_logit(const GemmParams& p, int row, int col, float v) {
  const int slot = row % p.block;
  if (slot == 0 || col >= p.N) return;
  const size_t orow = (size_t)(row / p.block) * (p.block - 1) + (slot - 1);
  p.logits[orow * p.N + col] = v;
}

// Stores one (row, group) partial top-16 list.
__device__ __forceinline__ void store_partial(const GemmParams& p, int row, int group, const Top16& t) {
  const size_t base = ((size_t)row * p.groups + group) * TOPK;
#pragma unroll
  for (int i = 0; i < TOPK; ++i) {
    p.tk_val[base + i] = t.v[i];
    p.tk_id[base + i] = t.id[i];
  }
}

// Chooses the launch shape; deterministic in (dtype, mode, M, N, K).
GemmPlan gemm_plan(bool bf16, int mode, int M, int N, int K);
// The skinny kernels' plan for any M (row tiles of up to 64 rows).
GemmPlan gemm_plan_skinny(int mode, int M, int N, int K);
// gemm_plan for weights in format wf (0 bf16, 1 E4M3, 2 MXFP4): the same plan when its kernel
// takes that format, else the skinny plan (every format).
GemmPlan gemm_plan_wf(bool bf16, int mode, int M, int N, int K, int wf);
// Bytes of partial output the plan writes (PARTIAL) or top-k partial entries (TOPK).
size_t gemm_part_floats(const GemmPlan& pl, int mode, int M, int N);
hipError_t gemm_launch(bool bf16, const GemmPlan& pl, int mode, GemmParams p, hipStream_t st);
// Tiled MFMA kernels for more than 64 rows (pl.kind 5; pl.mt selects the tile shape).
hipError_t tile_launch(const GemmPlan& pl, int mode, const GemmParams& p, hipStream_t st);
// 16-row-blocked copy of a bf16 [rows][cols] weight matrix for the MFMA tiles (rows % 16 == 0,
// cols % 32 == 0), same size as the source
hipError_t launch_block_weights(const void* src, long rows, long cols, void* dst, hipStream_t st);
// k-steps of 32 (2048 k) whose MXFP4 block scales a tile stages in LDS at once; the MXFP4 lm_head
// tiles take at most this many (hidden <= 2048)
constexpr int TILE4_MAX_STEPS = 64;

}  // namespace dfl
