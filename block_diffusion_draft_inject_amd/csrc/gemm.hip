// Weight GEMMs of the drafter on gfx950: C = A * B^T with A = activations [M][K] and
// B = a weight matrix [N][K] (one output row per line), fp32 accumulation.
//
//  * gemm_skinny  (bf16, M <= 64): weight streaming.  Every weight byte is used by at most 4
//    row fragments, so weights go straight from HBM into VGPRs (no LDS), 32 contiguous bytes
//    per lane per load.  The k index inside a 64-wide chunk is permuted so that a lane's two
//    16-byte loads are adjacent; A and B use the same permutation, so the sum is unchanged.
//    Waves of a workgroup split K and are reduced through LDS; workgroups split K again
//    ("splits") into fp32 partials that the consumer kernel sums in a fixed order.
//  * gemm_tiled   (bf16, M > 64): 128x128x32 tiles staged through double-buffered LDS,
//    2x2 waves of 64x64, v_mfma_f32_16x16x32_bf16.
//  * Activations (A) come as two bf16 planes, hi and lo (x = hi + lo to ~16 mantissa bits);
//    every A fragment is multiplied twice, A_hi * W + A_lo * W, with bf16 weights.
//  * gemm_f32     (fp32 drafters): plain VALU dot products, for the small fp32 configuration.
//  * TOPK mode: the lm_head epilogue keeps a running top-16 per row (thread-private sorted
//    lists, merged at the end of the workgroup) over a contiguous range of column tiles and
//    writes one partial list per (row, workgroup); the full-logit matrix is never stored
//    unless requested for checking.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dfl {




__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }


// ---------------------------------------------------------------------------------------
// skinny: accumulate one wave tile of (16*MT rows) x (16*NF cols) over chunks
// c = c0, c0 + cstep, ... < c1 (chunk = 64 k values).  Software-pipelined: the loads of the
// next pair of chunks are issued before the MFMAs of the current pair, so a wave always has
// one batch of weight loads in flight while it computes.
// ---------------------------------------------------------------------------------------
template <int MT, int NF>
struct SkinnyBatch {
  u32x4 ah[2][MT][2];   // activation hi plane
  u32x4 al[2][MT][2];   // activation lo plane
  u32x4 b[2][NF][2];
  unsigned e[2][NF];    // MXFP4: the scale byte of the lane's block, kept as loaded
};

// Loads chunks c and c + cstep; both indices are clamped to clast so the loads are always
// issued (no branch around them: the compiler then keeps exact vmcnt counts and the next
// batch stays in flight while the current one is multiplied).  Weight formats WF: 0 bf16;
// 1 E4M3 codes, one 16-byte load per lane and chunk (k = 16 kg .. 16 kg + 15, the same k as the
// two bf16 halves); 2 MXFP4 codes, one 8-byte load per lane and chunk (the same 16 k, element 2j
// in the low nibble of byte j) and the scale byte of the 32-k block holding them (srow).
template <int MT, int NF, int WF = 0>
__device__ __forceinline__ void skinny_load(SkinnyBatch<MT, NF>& x, const bf16* const (&arow)[MT], size_t a_plane,
                                            const void* const (&brow)[NF], const unsigned char* const (&srow)[NF],
                                            int kg, int c, int cstep, int clast) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int k = min(c + u * cstep, clast) * 64 + kg * 16;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if constexpr (WF == 2) {
        const uint2 q = *reinterpret_cast<const uint2*>(reinterpret_cast<const unsigned char*>(brow[f]) + k / 2);
        x.b[u][f][0][0] = q.x;
        x.b[u][f][0][1] = q.y;
        x.e[u][f] = srow[f][k / 32];
      } else if constexpr (WF == 1) {
        x.b[u][f][0] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const unsigned char*>(brow[f]) + k);
      } else {
        const u32x4* q = reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16*>(brow[f]) + k);
        x.b[u][f][0] = q[0];
        x.b[u][f][1] = q[1];
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const u32x4* q = reinterpret_cast<const u32x4*>(arow[m] + k);
      const u32x4* ql = reinterpret_cast<const u32x4*>(arow[m] + a_plane + k);
      x.ah[u][m][0] = q[0];
      x.ah[u][m][1] = q[1];
      x.al[u][m][0] = ql[0];
      x.al[u][m][1] = ql[1];
    }
  }
}

template <int MT, int NF, int WF = 0>
__device__ __forceinline__ void skinny_mma(const SkinnyBatch<MT, NF>& x, bool two, const float (&bs)[NF],
                                           f32x4 (&acc)[MT][NF]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (u == 1 && !two) break;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 w;
        if constexpr (WF == 2) w = fp4x8_bf16(x.b[u][f][0][h], __uint_as_float(x.e[u][f] << 23));   // 2^(E - 127)
        else if constexpr (WF == 1) w = fp8x8_bf16(x.b[u][f][0][2 * h], x.b[u][f][0][2 * h + 1], bs[f]);
        else w = as_bf16x8(x.b[u][f][h]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x.ah[u][m][h]), w, acc[m][f], 0, 0, 0);
          acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x.al[u][m][h]), w, acc[m][f], 0, 0, 0);
        }
      }
  }
}

// bs: E4M3, the row scale of each weight row; srow: MXFP4, each weight row's scale bytes
template <int MT, int NF, int WF = 0>
__device__ __forceinline__ void skinny_acc(const bf16* const (&arow)[MT], size_t a_plane, const void* const (&brow)[NF],
                                           const unsigned char* const (&srow)[NF], const float (&bs)[NF], int kg,
                                           int c0, int c1, int cstep, f32x4 (&acc)[MT][NF]) {
  if (c0 >= c1) return;
  const int clast = c0 + (c1 - 1 - c0) / cstep * cstep;   // last chunk this wave owns
  SkinnyBatch<MT, NF> x, y;
  int c = c0;
  skinny_load<MT, NF, WF>(x, arow, a_plane, brow, srow, kg, c, cstep, clast);
  while (true) {
    const int cy = c + 2 * cstep;
    skinny_load<MT, NF, WF>(y, arow, a_plane, brow, srow, kg, cy, cstep, clast);
    skinny_mma<MT, NF, WF>(x, c + cstep < c1, bs, acc);
    if (cy >= c1) break;
    const int cx = cy + 2 * cstep;
    skinny_load<MT, NF, WF>(x, arow, a_plane, brow, srow, kg, cx, cstep, clast);
    skinny_mma<MT, NF, WF>(y, cy + cstep < c1, bs, acc);
    if (cx >= c1) break;
    c = cx;
  }
}

// weight row n (bf16 segments, or one segment of E4M3 or MXFP4 codes, ldb bytes a row) and its
// scale (E4M3) or scale bytes (MXFP4: K / 32 a row)
template <int WF>
__device__ __forceinline__ const void* wrow_ptr(const GemmParams& p, int n, float& scale, const unsigned char*& srow) {
  scale = 1.f;
  srow = nullptr;
  if constexpr (WF == 2) {
    srow = p.blk_scale + (size_t)n * (p.K / 32);
    return reinterpret_cast<const unsigned char*>(p.seg[0]) + (size_t)n * p.ldb;
  } else if constexpr (WF == 1) {
    scale = p.row_scale[n];
    return reinterpret_cast<const unsigned char*>(p.seg[0]) + (size_t)n * p.ldb;
  } else {
    return brow_ptr(p, n);
  }
}

// PARTIAL (NF=1) and SWIGLU (NF=2: gate and up fragment of the same 16 output columns).
// grid: x = column tile (16 output columns), y = row tile (16*MT rows), z = k-split.
template <int MT, int MODE, int WF = 0>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmParams p) {
  constexpr int NF = (MODE == GEMM_SWIGLU) ? 2 : 1;
  __shared__ float red[3][MT][NF][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, kg = lane >> 4;
  const int Mv = rows_valid(p);
  const int m0 = blockIdx.y * 16 * MT;
  if (m0 >= Mv) return;
  const int ncol0 = blockIdx.x * 16;
  const bf16* arow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int r = min(m0 + m * 16 + li, Mv - 1);
    arow[m] = reinterpret_cast<const bf16*>(p.A) + (size_t)r * p.lda;
  }
  const void* brow[NF];
  const unsigned char* srow[NF];
  float bs[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int n = ncol0 + li + f * p.half;     // SWIGLU: f=1 reads the up rows at offset `half`
    n = min(n, p.N - 1);
    brow[f] = wrow_ptr<WF>(p, n, bs[f], srow[f]);
  }
  const int nchunks = p.K / 64;
  const int s = blockIdx.z;
  const int c0 = (int)((long)nchunks * s / p.splits), c1 = (int)((long)nchunks * (s + 1) / p.splits);
  f32x4 acc[MT][NF];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  skinny_acc<MT, NF, WF>(arow, p.a_plane, brow, srow, bs, kg, c0 + wave, c1, 4, acc);
  // reduce the 4 waves' k-slices
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave - 1][m][f][j][lane] = acc[m][f][j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[m][f][j] += red[0][m][f][j][lane] + red[1][m][f][j][lane] + red[2][m][f][j][lane];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + m * 16 + kg * 4 + j;
      const int col = ncol0 + li;
      if (row >= Mv) continue;
      if (MODE == GEMM_PARTIAL) {
        if (col < p.N) p.part[((size_t)s * p.M + row) * p.N + col] = acc[m][0][j];
      } else {
        if (col < p.half) {
          const float v = silu_f(acc[m][0][j]) * acc[m][NF - 1][j];
          st_act(reinterpret_cast<bf16*>(p.out), (size_t)row * p.half + col, p.out_plane, v);
        }
      }
    }
}

// TOPK (lm_head) skinny, persistent with work stealing: each wave repeatedly takes the next
// 16-column fragment from a device counter (reset to 0 by the draft's plan kernel) and
// streams that fragment's weights over all of K.  Waves therefore finish together however the
// 9496 fragments of a 151936-word vocabulary divide.  Each row's candidates are kept by
// 64/(16*MT) lanes in private sorted top-16 lists, merged at the end of the workgroup; one
// partial list per (row, workgroup) is written.  grid: x = workgroups, y = row tile.
template <int MT, int WF = 0>
__global__ __launch_bounds__(256) void lmhead_topk_skinny(GemmParams p) {
  constexpr int R = 16 * MT;
  constexpr int LPR = 64 / R;          // lanes per row within a wave: 4, 2, 1
  constexpr int VPL = 16 / LPR;        // fragment values each of those lanes scans: 4, 8, 16
  constexpr int NSLOT = R * (LPR > 1 ? LPR / 2 : 1);
  __shared__ float fb[4][R][17];
  __shared__ float mv[4][NSLOT][TOPK];
  __shared__ int mi[4][NSLOT][TOPK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, kg = lane >> 4;
  const int Mv = rows_valid(p);
  const int m0 = blockIdx.y * R;
  if (m0 >= Mv) return;
  const bf16* arow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int r = min(m0 + m * 16 + li, Mv - 1);
    arow[m] = reinterpret_cast<const bf16*>(p.A) + (size_t)r * p.lda;
  }
  const int my_row = lane / LPR, my_sub = lane % LPR;
  const bool row_live = (m0 + my_row < Mv) && ((m0 + my_row) % p.block != 0);
  Top16 top;
  top.init();
  const int nfrag = (p.N + 15) / 16;
  const int nchunks = p.K / 64;
  int* ctr = p.counter + blockIdx.y;
  while (true) {
    int f = 0;
    if (lane == 0) f = atomicAdd(ctr, 1);
    f = __shfl(f, 0, WAVE);
    if (f >= nfrag) break;
    const int col = f * 16 + li;
    float bs[1];
    const unsigned char* srow[1];
    const void* brow[1] = {wrow_ptr<WF>(p, min(col, p.N - 1), bs[0], srow[0])};
    f32x4 acc[MT][1];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    skinny_acc<MT, 1, WF>(arow, p.a_plane, brow, srow, bs, kg, 0, nchunks, 1, acc);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = m * 16 + kg * 4 + j;
        fb[wave][r][li] = acc[m][0][j];
        if (p.logits && m0 + r < Mv) store_logit(p, m0 + r, col, acc[m][0][j]);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (row_live) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int c = my_sub * VPL + v;
        const int gcol = f * 16 + c;
        if (gcol < p.N) top.push(fb[wave][my_row][c], gcol);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // merge the LPR lane lists of each row inside the wave
  for (int w = 1; w < LPR; w <<= 1) {
    const int slot = my_row * (LPR / 2) + my_sub / (2 * w);
    if ((my_sub & (2 * w - 1)) == w) {
#pragma unroll
      for (int i = 0; i < TOPK; ++i) { mv[wave][slot][i] = top.v[i]; mi[wave][slot][i] = top.id[i]; }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if ((my_sub & (2 * w - 1)) == 0) {
#pragma unroll
      for (int i = 0; i < TOPK; ++i) top.push(mv[wave][slot][i], mi[wave][slot][i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // merge across the four waves (every wave has left its loop)
  __syncthreads();
  if (my_sub == 0 && wave > 0) {
#pragma unroll
    for (int i = 0; i < TOPK; ++i) { mv[wave][my_row][i] = top.v[i]; mi[wave][my_row][i] = top.id[i]; }
  }
  __syncthreads();
  if (my_sub == 0 && wave == 0) {
    for (int w = 1; w < 4; ++w)
#pragma unroll
      for (int i = 0; i < TOPK; ++i) top.push(mv[w][my_row][i], mi[w][my_row][i]);
    if (m0 + my_row < Mv) store_partial(p, m0 + my_row, blockIdx.x, top);
  }
}

// ---------------------------------------------------------------------------------------
// stream: at most 16 rows.  The SW waves of a workgroup split K: each wave keeps its K-slice
// of the activations (hi and lo planes) in registers for the whole launch and streams only
// weight rows, two 16-byte loads per lane per 64-wide chunk.  Per 16-column fragment the
// waves' 16x16 partial tiles are summed through LDS (double-buffered, one barrier per
// fragment) and waves 0..3 run the epilogue, each for the rows 4*g + wave.  The weight loads
// of the next fragment are in flight during the MFMAs, the reduction and the epilogue of the
// current one.  grid: x = fragment stride (fragments x, x + gridDim.x, ...), y = k-split.
// ---------------------------------------------------------------------------------------
constexpr int SW = 8;

template <int SLC, int NF>
struct StreamBuf {
  u32x4 b[SLC][NF][2];
};
// FP8 weights: one 16-byte load per lane per 64-k chunk, k = 16 kg .. 16 kg + 15 (the MFMA
// halves take k = 16 kg + 8 h .. +7; the activations are held in the same k order), plus the
// lane's row scale.  One weight segment (stacked copies for QKV-like and gate/up matrices).
template <int SLC, int NF>
struct StreamBuf8 {
  u32x4 q[SLC][NF];
  float s[NF];
};
// MXFP4 weights.  Slices of 2 or 4 chunks are read as 128-k super-chunks: lane (li, kg) loads 16
// bytes, the 32 codes of block k = 32 kg .. 32 kg + 31 of its row, and that block's scale byte
// (one load per row and 64 bytes per row per instruction, as for FP8).  A one-chunk slice keeps the
// FP8 order: 8 bytes per lane, k = 16 kg .. 16 kg + 15, half a block.
template <int SLC, int NF>
struct StreamBuf4 {
  static constexpr bool WIDE = SLC >= 2;
  static constexpr int NC = WIDE ? SLC / 2 : SLC;
  u32x4 q[NC][NF];   // WIDE: four words, else words 0 and 1
  unsigned e[NC][NF];   // the block's scale byte, as loaded (turned into a float only at its use,
                        // so that no wait for it lands between the loads of the ring)
};

// SWIGLU fragments interleave the two halves: lanes li < 8 take gate rows 8f .. 8f + 7, lanes
// li >= 8 the matching up rows half + 8f .. (so the epilogue pairs lane li with lane li + 8).
template <int SLC, int NF, bool GLU>
__device__ __forceinline__ void stream_load(StreamBuf<SLC, NF>& x, const GemmParams& p, int ncols, int f, int kw,
                                            int kg, int li) {
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    // the rows of a fragment (of each half for SWIGLU) lie in one weight segment (segment
    // sizes and `half` are multiples of 16, of 8 for SWIGLU): the segment index is
    // wave-uniform, so the segment pointer is a scalar load and never joins the vector-memory
    // queue that the prefetches wait in
    const bf16* row;
    if (GLU) {
      const int g0 = f * 8, u0 = p.half + f * 8;
      const int sg = __builtin_amdgcn_readfirstlane(g0 / p.seg_rows);
      const int su = __builtin_amdgcn_readfirstlane(u0 / p.seg_rows);
      const int j = min(g0 + (li & 7), ncols - 1) - g0;
      const bf16* bg = reinterpret_cast<const bf16*>(p.seg[sg]) + (size_t)(g0 - sg * p.seg_rows) * p.ldb;
      const bf16* bu = reinterpret_cast<const bf16*>(p.seg[su]) + (size_t)(u0 - su * p.seg_rows) * p.ldb;
      row = (li < 8 ? bg : bu) + (size_t)j * p.ldb;
    } else {
      const int seg = __builtin_amdgcn_readfirstlane((f * 16 + nf * p.half) / p.seg_rows);
      const int n = min(f * 16 + li, ncols - 1) + nf * p.half - seg * p.seg_rows;
      row = reinterpret_cast<const bf16*>(p.seg[seg]) + (size_t)n * p.ldb;
    }
#pragma unroll
    for (int c = 0; c < SLC; ++c) {
      // half h of the chunk: k = 32 h + 8 kg .. +7, so one load instruction covers 64
      // contiguous bytes of each of the 16 rows; chunks past K carry zero activations
      const int k = min(kw + c * 64, p.K - 64) + kg * 8;
      x.b[c][nf][0] = *reinterpret_cast<const u32x4*>(row + k);
      x.b[c][nf][1] = *reinterpret_cast<const u32x4*>(row + k + 32);
    }
  }
}

template <int SLC, int NF, bool GLU>
__device__ __forceinline__ void stream_load8(StreamBuf8<SLC, NF>& x, const GemmParams& p, int ncols, int f, int kw,
                                             int kg, int li) {
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    int n;
    if (GLU) {
      const int g0 = f * 8, j = min(g0 + (li & 7), ncols - 1) - g0;
      n = (li < 8 ? g0 : p.half + g0) + j;
    } else {
      n = min(f * 16 + li, ncols - 1) + nf * p.half;
    }
    const unsigned char* row = reinterpret_cast<const unsigned char*>(p.seg[0]) + (size_t)n * p.ldb;
#pragma unroll
    for (int c = 0; c < SLC; ++c) x.q[c][nf] = *reinterpret_cast<const u32x4*>(row + min(kw + c * 64, p.K - 64) + kg * 16);
    x.s[nf] = p.row_scale[n];
  }
}

template <int SLC, int NF, bool GLU>
__device__ __forceinline__ void stream_load4(StreamBuf4<SLC, NF>& x, const GemmParams& p, int ncols, int f, int kw,
                                             int kg, int li) {
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    int n;
    if (GLU) {
      const int g0 = f * 8, j = min(g0 + (li & 7), ncols - 1) - g0;
      n = (li < 8 ? g0 : p.half + g0) + j;
    } else {
      n = min(f * 16 + li, ncols - 1) + nf * p.half;
    }
    const unsigned char* row = reinterpret_cast<const unsigned char*>(p.seg[0]) + (size_t)n * p.ldb;
    const unsigned char* srow = p.blk_scale + (size_t)n * (p.K / 32);
    if constexpr (StreamBuf4<SLC, NF>::WIDE) {
#pragma unroll
      for (int c = 0; c < SLC / 2; ++c) {
        const int k = min(kw + c * 128, p.K - 128) + kg * 32;
        x.q[c][nf] = *reinterpret_cast<const u32x4*>(row + k / 2);
        x.e[c][nf] = srow[k / 32];
      }
    } else {
#pragma unroll
      for (int c = 0; c < SLC; ++c) {
        const int k = min(kw + c * 64, p.K - 64) + kg * 16;
        const uint2 w = *reinterpret_cast<const uint2*>(row + k / 2);
        x.q[c][nf][0] = w.x;
        x.q[c][nf][1] = w.y;
        x.e[c][nf] = srow[k / 32];
      }
    }
  }
}

template <int SLC, int NF>
__device__ __forceinline__ void stream_mma4(const StreamBuf4<SLC, NF>& x, const u32x4 (&ah)[SLC][2],
                                            const u32x4 (&al)[SLC][2], f32x4 (&acc)[NF]) {
  // activation chunk c, half h holds k = (WIDE) 128 (c / 2) + 32 kg + 16 (c % 2) + 8 h .. +7, so
  // word j of super-chunk cc (codes 8 j .. 8 j + 7 of the block) meets chunk 2 cc + j / 2, half j % 2
  constexpr bool WIDE = StreamBuf4<SLC, NF>::WIDE;
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) acc[nf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < SLC; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        const unsigned word = WIDE ? x.q[c / 2][nf][2 * (c % 2) + h] : x.q[c][nf][h];
        const float sc = __uint_as_float((WIDE ? x.e[c / 2][nf] : x.e[c][nf]) << 23);   // 2^(E - 127), E >= 1
        const bf16x8 w = fp4x8_bf16(word, sc);
        acc[nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah[c][h]), w, acc[nf], 0, 0, 0);
        acc[nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al[c][h]), w, acc[nf], 0, 0, 0);
      }
}

template <int SLC, int NF>
__device__ __forceinline__ void stream_mma8(const StreamBuf8<SLC, NF>& x, const u32x4 (&ah)[SLC][2],
                                            const u32x4 (&al)[SLC][2], f32x4 (&acc)[NF]) {
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) acc[nf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < SLC; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        const bf16x8 w = h == 0 ? fp8x8_bf16(x.q[c][nf][0], x.q[c][nf][1], x.s[nf])
                                : fp8x8_bf16(x.q[c][nf][2], x.q[c][nf][3], x.s[nf]);
        acc[nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah[c][h]), w, acc[nf], 0, 0, 0);
        acc[nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al[c][h]), w, acc[nf], 0, 0, 0);
      }
}

template <int SLC, int NF>
__device__ __forceinline__ void stream_mma(const StreamBuf<SLC, NF>& x, const u32x4 (&ah)[SLC][2],
                                           const u32x4 (&al)[SLC][2], f32x4 (&acc)[NF]) {
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) acc[nf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < SLC; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        acc[nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah[c][h]), as_bf16x8(x.b[c][nf][h]), acc[nf], 0, 0, 0);
        acc[nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al[c][h]), as_bf16x8(x.b[c][nf][h]), acc[nf], 0, 0, 0);
      }
}

// Fragments of a workgroup: x, x + G, x + 2G, ... (G = gridDim.x).  NB = 1: one fragment.
// RING = false: exactly NB fragments per workgroup (G divides the fragment count), all NB loaded
// at once and then multiplied and reduced in order.  RING = true: NB buffers in rotation, the
// loads of the next NB - 1 fragments in flight while one is multiplied and reduced.
// WF: the weight format, 0 bf16, 1 E4M3 codes with row scales, 2 MXFP4 codes with block scales.
template <int SLC, int MODE, int NB, bool RING, int WF = 0>
__global__ __launch_bounds__(SW * 64) void gemm_stream_kernel(GemmParams p) {
  constexpr int NF = 1;
  static_assert(!(WF && MODE == GEMM_TOPK), "the FP8 / MXFP4 lm_head is the wave kernel");
  using Buf = typename std::conditional<
      WF == 2, StreamBuf4<SLC, NF>,
      typename std::conditional<WF == 1, StreamBuf8<SLC, NF>, StreamBuf<SLC, NF>>::type>::type;
  constexpr bool GLU = MODE == GEMM_SWIGLU;
  constexpr int RED_FLOATS = 2 * NF * SW * 4 * 64;
  constexpr int MRG = (MODE == GEMM_TOPK) ? 4 * 64 * (TOPK + 1) : 0;   // lane lists for the final merge
  __shared__ __align__(16) float smem[RED_FLOATS + 2 * MRG];
  float (*red)[NF][SW][4][64] = reinterpret_cast<float (*)[NF][SW][4][64]>(smem);
  float (*mv)[64][TOPK + 1] = reinterpret_cast<float (*)[64][TOPK + 1]>(smem + RED_FLOATS);
  int (*mi)[64][TOPK + 1] = reinterpret_cast<int (*)[64][TOPK + 1]>(smem + RED_FLOATS + MRG);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, kg = lane >> 4;
  const int Mv = rows_valid(p);
  const int ncols = GLU ? p.half : p.N;
  const int nfrag = GLU ? (ncols + 7) / 8 : (ncols + 15) / 16;
  if (Mv <= 0 || (int)blockIdx.x >= nfrag) return;    // uniform over the workgroup
  const int s = blockIdx.y;
  const int kw = (s * SW + wave) * SLC * 64;
  // this wave's K-slice of the activations: lane (li, kg) holds row li, k = chunk + 16 kg .. +15
  u32x4 ah[SLC][2], al[SLC][2];
  {
    const bf16* arow = reinterpret_cast<const bf16*>(p.A) + (size_t)min(li, Mv - 1) * p.lda;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < SLC; ++c) {
      // bf16 weights: halves k = 32 h + 8 kg .. +7; FP8 and MXFP4 weights: k = 16 kg + 8 h .. +7;
      // MXFP4 over 2 or 4 chunks: chunk pairs form 128-k super-chunks, k = 32 kg + 16 (c % 2) + 8 h
      constexpr bool W4 = WF == 2 && SLC >= 2;
      const int c0 = W4 ? kw + (c / 2) * 128 : kw + c * 64;
      const bool ok = li < Mv && c0 < p.K;
      const int k = W4 ? min(c0, p.K - 128) + kg * 32 + (c % 2) * 16
                       : min(c0, p.K - 64) + kg * (WF ? 16 : 8);
      constexpr int HO = WF ? 8 : 32;
      const bf16* qh = arow + k;
      const bf16* ql = arow + p.a_plane + k;
      ah[c][0] = ok ? *reinterpret_cast<const u32x4*>(qh) : z;
      ah[c][1] = ok ? *reinterpret_cast<const u32x4*>(qh + HO) : z;
      al[c][0] = ok ? *reinterpret_cast<const u32x4*>(ql) : z;
      al[c][1] = ok ? *reinterpret_cast<const u32x4*>(ql + HO) : z;
    }
  }
  const int row = 4 * kg + wave;                        // epilogue row of waves 0..3
  const bool epi = wave < 4;
  const bool row_live = epi && row < Mv && (MODE != GEMM_TOPK || row % p.block != 0);
  Top16 top;
  top.init();
  auto finish = [&](const f32x4 (&acc)[NF], int buf, int f) {
#pragma unroll
    for (int nf = 0; nf < NF; ++nf)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[buf][nf][wave][j][lane] = acc[nf][j];
    lds_barrier();
    if (!epi) return;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < SW; ++w) v += red[buf][0][w][wave][lane];
    if (GLU) {
      // lane li < 8 holds gate column 8f + li, lane li + 8 the matching up column
      const float up = dpp_f<0x128>(v);   // row_ror:8 -- lane li reads lane li ^ 8 of its row
      const int col = f * 8 + li;
      if (li < 8 && row < Mv && col < ncols)
        st_act(reinterpret_cast<bf16*>(p.out), (size_t)row * p.half + col, p.out_plane, silu_f(v) * up);
      return;
    }
    const int col = f * 16 + li;
    if (row >= Mv || col >= ncols) return;
    if (MODE == GEMM_PARTIAL) {
      p.part[((size_t)s * p.M + row) * p.N + col] = v;
    } else {
      if (p.logits) store_logit(p, row, col, v);
      if (row_live) top.push(v, col);
    }
  };
  f32x4 acc[NF];
  int f = blockIdx.x;
  auto load = [&](Buf& x, int fr) {
    if constexpr (WF == 2) stream_load4<SLC, NF, GLU>(x, p, ncols, fr, kw, kg, li);
    else if constexpr (WF == 1) stream_load8<SLC, NF, GLU>(x, p, ncols, fr, kw, kg, li);
    else stream_load<SLC, NF, GLU>(x, p, ncols, fr, kw, kg, li);
  };
  auto mma = [&](const Buf& x) {
    if constexpr (WF == 2) stream_mma4(x, ah, al, acc);
    else if constexpr (WF == 1) stream_mma8(x, ah, al, acc);
    else stream_mma(x, ah, al, acc);
  };
  const int G = gridDim.x;
  if constexpr (NB == 1) {
    // one fragment for this workgroup
    Buf x;
    load(x, f);
    mma(x);
    finish(acc, 0, f);
  } else if constexpr (!RING) {
    // all NB fragments requested at once (the whole share of the weight stream in flight), then
    // multiplied and reduced in the order they were requested; the in-order wait counts let each
    // one start as soon as its own loads are in
    Buf b[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      load(b[i], min(f + i * G, nfrag - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      mma(b[i]);
      finish(acc, i & 1, f + i * G);
    }
  } else {
    // ring: the load cursor runs NB - 1 fragments ahead of the compute cursor (the scheduling
    // barrier keeps the compiler from sinking loads towards their use).  The fragment count is
    // padded to whole rounds; a padded round loads the last fragment again (cache hits) and
    // computes nothing (the test is uniform over the workgroup)
    const int nf = (nfrag - 1 - (int)blockIdx.x) / G + 1;
    const int T = (nf + NB - 1) / NB * NB;
    Buf b[NB];
    int lf = f;
#pragma unroll
    for (int i = 0; i + 1 < NB; ++i) {
      load(b[i], min(lf, nfrag - 1));
      lf += G;
      __builtin_amdgcn_sched_barrier(0);
    }
    int buf = 0;
    for (int t = 0; t < T; t += NB) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        load(b[(i + NB - 1) % NB], min(lf, nfrag - 1));
        lf += G;
        __builtin_amdgcn_sched_barrier(0);
        if (f < nfrag) {
          mma(b[i]);
          finish(acc, buf, f);
          buf ^= 1;
        }
        f += G;
      }
    }
  }
  if (MODE != GEMM_TOPK || !epi) return;
  // merge the 16 lane lists of each row (lanes li = 0..15 of one kg group) inside the wave
  for (int w = 1; w < 16; w <<= 1) {
    if ((li & (2 * w - 1)) == w) {
#pragma unroll
      for (int i = 0; i < TOPK; ++i) { mv[wave][lane][i] = top.v[i]; mi[wave][lane][i] = top.id[i]; }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if ((li & (2 * w - 1)) == 0) {
#pragma unroll
      for (int i = 0; i < TOPK; ++i) top.push(mv[wave][lane + w][i], mi[wave][lane + w][i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  if (li == 0 && row < Mv) store_partial(p, row, blockIdx.x, top);
}

// ---------------------------------------------------------------------------------------
// lm_head + top-16, at most 16 rows, K <= 2048 (K a multiple of 512): independent waves.
// The lm_head input is bf16 (the final norm writes bf16(h_f) and a zero lo plane), so only
// the hi plane is read.  The workgroup copies the activation rows into LDS once (64 KiB); then
// every wave streams whole 16-column fragments (wave w of the grid takes fragments w,
// w + waves, ...) over all of K in batches of LW_CH chunks of 64, LW_NB batches in rotation,
// the prefetch running on into the next fragment.  (Two workgroups per CU, with smaller
// batches to fit 128 VGPRs, measured 8-10% slower than one with deep batches.)  No workgroup barrier in the main loop: a wave waits only for its own
// loads.  (Handing fragments out through one device-wide counter was far slower: the ~13k
// increments of one address serialise.)  Each wave keeps, per row, 4 lane lists of the
// running top-16 (one per column quarter); at the end a row's 32 lists are merged by one
// half-wave into one partial list per (row, workgroup).
// ---------------------------------------------------------------------------------------
constexpr int LW_W = 8;             // waves per workgroup
constexpr int LW_KMAX = 2048;
constexpr int LW_LD = LW_KMAX + 8;  // LDS row stride (bf16): rows fall in distinct bank groups

constexpr int LW_GROUPS = 256;      // workgroups: one per CU (two per CU measured slower)
constexpr size_t LW_SMEM = (size_t)16 * LW_LD * 2 + (size_t)LW_W * 16 * 17 * 4;   // 73 KiB
static_assert(2 * 16 * 32 * (TOPK + 1) * 4 <= LW_SMEM, "the merge lists overlay the activation rows");

constexpr int LW_CH = 4;            // chunks of 64 k per batch
constexpr int LW_NB = 4;            // batches in rotation (LW_NB - 1 in flight; 3 measured 1.5% slower,
                                    // 5 no faster and spills in the FP8 and full-logit kernels)
struct LwBatch {
  u32x4 b[LW_CH][2];                // LW_CH chunks x (k halves 0..31 / 32..63 of the chunk)
};

__device__ __forceinline__ void lw_load(LwBatch& x, const bf16* row, int k0, int kg) {
#pragma unroll
  for (int c = 0; c < LW_CH; ++c) {
    const bf16* q = row + k0 + c * 64 + kg * 8;
    x.b[c][0] = *reinterpret_cast<const u32x4*>(q);
    x.b[c][1] = *reinterpret_cast<const u32x4*>(q + 32);
  }
}

// the two k halves of each chunk accumulate separately: two independent MFMA chains
__device__ __forceinline__ void lw_mma(const LwBatch& x, const bf16 (*sa)[LW_LD], int k0, int li, int kg,
                                       f32x4& acc0, f32x4& acc1) {
#pragma unroll
  for (int c = 0; c < LW_CH; ++c) {
    const int k = k0 + c * 64 + kg * 8;
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&sa[li][k]);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&sa[li][k + 32]);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_bf16x8(x.b[c][0]), acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, as_bf16x8(x.b[c][1]), acc1, 0, 0, 0);
  }
}

// FP8 weights (row_scale set): one byte per weight, so a batch carries 8 chunks of 64 k, each a
// single 16-byte load per lane: k = 16 kg .. 16 kg + 15 of the chunk.  The codes become bf16
// weights code * scale in registers (v_cvt_scalef32_pk_bf16_fp8, exact: an E4M3 value times a
// power of two fits bf16), and the two MFMA halves take k = 16 kg + 8 h .. +7; the activations
// are read from LDS in the same k order, so the sum is unchanged.
constexpr int LW_CH8 = 8;
struct LwBatch8 {
  u32x4 q[LW_CH8];
  float s;                          // the row's scale
};

__device__ __forceinline__ void lw_load8(LwBatch8& x, const unsigned char* row, const float* scale, int k0,
                                         int kg) {
#pragma unroll
  for (int c = 0; c < LW_CH8; ++c) x.q[c] = *reinterpret_cast<const u32x4*>(row + k0 + c * 64 + kg * 16);
  x.s = *scale;
}

__device__ __forceinline__ void lw_mma8(const LwBatch8& x, const bf16 (*sa)[LW_LD], int k0, int li, int kg,
                                        f32x4& acc0, f32x4& acc1) {
#pragma unroll
  for (int c = 0; c < LW_CH8; ++c) {
    const int k = k0 + c * 64 + kg * 16;
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&sa[li][k]);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&sa[li][k + 8]);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, fp8x8_bf16(x.q[c][0], x.q[c][1], x.s), acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, fp8x8_bf16(x.q[c][2], x.q[c][3], x.s), acc1, 0, 0, 0);
  }
}

// MXFP4 weights (blk_scale set): codes [N][K/2] bytes, element 2j in the low nibble of byte j,
// and one scale byte E per 32 weights of a row ([N][K/32]), the block's weights being
// code value * 2^(E - 127).  A batch is LW_CH4 chunks of 128 k: lane (li, kg) loads the 16 code
// bytes of k = 32 kg .. 32 kg + 31 of each chunk (one block) and the 16 scale bytes of the batch's
// blocks.  Word m of a lane's 16 bytes becomes eight bf16 weights (v_cvt_scalef32_pk_bf16_fp4,
// exact: an E2M1 value times a power of two fits bf16) and feeds the MFMA over k = 32 kg + 8 m ..
// + 7 of the chunk; the activations are read from LDS in that k order, so the sum is unchanged.
constexpr int LW_CH4 = 4;
struct LwBatch4 {
  u32x4 q[LW_CH4];
  u32x4 sc;                         // scale bytes of the batch's 16 blocks (chunk c, lane group kg: byte 4c + kg)
};

__device__ __forceinline__ void lw_load4(LwBatch4& x, const unsigned char* row, const unsigned char* srow, int k0,
                                         int kg) {
#pragma unroll
  for (int c = 0; c < LW_CH4; ++c) x.q[c] = *reinterpret_cast<const u32x4*>(row + (k0 + 128 * c) / 2 + 16 * kg);
  x.sc = *reinterpret_cast<const u32x4*>(srow + k0 / 32);
}

__device__ __forceinline__ void lw_mma4(const LwBatch4& x, const bf16 (*sa)[LW_LD], int k0, int li, int kg,
                                        f32x4& acc0, f32x4& acc1) {
#pragma unroll
  for (int c = 0; c < LW_CH4; ++c) {
    const float s = __uint_as_float(((x.sc[c] >> (8 * kg)) & 0xFFu) << 23);   // 2^(E - 127), E >= 1
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sa[li][k0 + 128 * c + 32 * kg + 8 * m]);
      const bf16x8 w = fp4x8_bf16(x.q[c][m], s);
      if (m & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w, acc1, 0, 0, 0);
      else acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w, acc0, 0, 0, 0);
    }
  }
}

// LOGITS: the full logits are written too (a global store in the fragment loop; kept out of
// the instantiation without them, where it would make the compiler's load waits coarser)
template <bool LOGITS, bool FP8 = false, bool FP4 = false>
__global__ __launch_bounds__(LW_W * 64, 2) void lmhead_topk_wave(GemmParams p) {
  using Batch = typename std::conditional<FP4, LwBatch4, typename std::conditional<FP8, LwBatch8, LwBatch>::type>::type;
  constexpr int KPB = FP4 ? 128 * LW_CH4 : 64 * (FP8 ? LW_CH8 : LW_CH);   // k per batch
  __shared__ __align__(16) unsigned char lw_smem[LW_SMEM];
  bf16 (*sa)[LW_LD] = reinterpret_cast<bf16 (*)[LW_LD]>(lw_smem);                         // [row][k]
  float (*fb)[16][17] = reinterpret_cast<float (*)[16][17]>(lw_smem + 16 * LW_LD * 2);    // [wave][row][col]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, kg = lane >> 4;
  const int Mv = rows_valid(p);
  const int K = p.K;
  if (Mv <= 0) return;   // uniform
  const int nfrag = (p.N + 15) / 16;
  const int ncb = K / KPB;                        // batches per fragment
  // fragments of wave w of workgroup g: g + G w, g + G w + G W, ... (G workgroups of W waves).
  // Each round of G W fragments covers one contiguous span, and the fragments left for the last,
  // partial round fall to the low workgroup indices one each: the workgroups' shares differ by
  // at most one fragment.  (With wave-major numbering, g W + w, the partial round fell to whole
  // workgroups: at vocabulary 151936 and hidden 2048, 163 of 256 took 40 fragments and the rest
  // 32; bf16 127.7 -> 123.2 us, E4M3 70.0 -> 69.1, MXFP4 49.5 -> 48.0.  Contiguous per-workgroup
  // spans balance as well, but read the E4M3 and MXFP4 lm_heads 3-4% slower than this.)
  const int TW = gridDim.x * LW_W;
  const int my_row = lane >> 2, my_sub = lane & 3;   // epilogue: lane handles row my_row, cols 4 sub..+3
  const bool row_live = my_row < Mv && (my_row % p.block) != 0;
  Top16 top;
  top.init();
  auto rown = [&](int frag) { return min(min(frag, nfrag - 1) * 16 + li, p.N - 1); };
  auto rowp = [&](int frag) { return reinterpret_cast<const bf16*>(p.seg[0]) + (size_t)rown(frag) * p.ldb; };
  // epilogue of one fragment: the wave's 16 x 16 tile through its own LDS slot; lane (row,
  // quarter) scans 4 columns into its list
  auto epilogue = [&](int f, const f32x4& acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      fb[wave][kg * 4 + j][li] = acc[j];
      if (LOGITS && kg * 4 + j < Mv) store_logit(p, kg * 4 + j, f * 16 + li, acc[j]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (row_live) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = f * 16 + my_sub * 4 + c;
        if (col < p.N) top.push_asc(fb[wave][my_row][my_sub * 4 + c], col);   // a lane's columns ascend
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // this wave's batches, fragment by fragment; the load cursor runs LW_NB - 1 batches ahead of the
  // compute cursor, over fragment boundaries (loads past the end read clamped, valid rows)
  const int f0 = blockIdx.x + gridDim.x * wave;
  // rounded up to whole rotations: a padded batch belongs to a fragment this wave never
  // finishes, so it changes nothing
  const int T = ((f0 < nfrag ? (nfrag - 1 - f0) / TW + 1 : 0) * ncb + LW_NB - 1) / LW_NB * LW_NB;
  int lf = f0, lcb = 0;
  auto issue = [&](Batch& b) {
    if constexpr (FP4)
      lw_load4(b, reinterpret_cast<const unsigned char*>(p.seg[0]) + (size_t)rown(lf) * p.ldb,
               p.blk_scale + (size_t)rown(lf) * (K / 32), lcb * KPB, kg);
    else if constexpr (FP8)
      lw_load8(b, reinterpret_cast<const unsigned char*>(p.seg[0]) + (size_t)rown(lf) * p.ldb, p.row_scale + rown(lf),
               lcb * KPB, kg);
    else
      lw_load(b, rowp(lf), lcb * KPB, kg);
    if (++lcb == ncb) { lcb = 0; lf += TW; }
  };
  int cf = f0, ccb = 0;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  auto step = [&](const Batch& b) {
    if constexpr (FP4)
      lw_mma4(b, sa, ccb * KPB, li, kg, acc0, acc1);
    else if constexpr (FP8)
      lw_mma8(b, sa, ccb * KPB, li, kg, acc0, acc1);
    else
      lw_mma(b, sa, ccb * KPB, li, kg, acc0, acc1);
    if (++ccb == ncb) {
      if (cf < nfrag) epilogue(cf, acc0 + acc1);   // (a padded rotation can complete a fragment past the end)
      acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
      ccb = 0;
      cf += TW;
    }
  };
  // batch i's loads strictly before batch i+1's: the compiler's in-order wait counts rely on it.
  // The activation rows are requested first, then the first LW_NB - 1 weight batches, and only
  // then are the rows written to LDS: the weight loads stay in flight across the staging (the
  // rows, requested first, are waited for first).
  // activation rows -> LDS (rows >= Mv zero), 16-byte pieces, all loads issued in one burst at
  // always-valid addresses and masked afterwards
  // thread t copies the 16-byte piece t % 256 of rows t / 256, t / 256 + 2, ... (16 rows)
  static_assert(LW_KMAX / 8 == 256 && LW_W * 64 == 512, "piece mapping assumes 256 pieces a row, 512 threads");
  const int sv = tid & 255, sq0 = tid >> 8;
  u32x4 sx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = sq0 + 2 * i;
    sx[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16*>(p.A) + (size_t)min(r, Mv - 1) * p.lda +
                                            min(sv, K / 8 - 1) * 8);
  }
  __builtin_amdgcn_sched_barrier(0);
  Batch b[LW_NB];
#pragma unroll
  for (int i = 0; i + 1 < LW_NB; ++i) {
    issue(b[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = sq0 + 2 * i;
    const u32x4 z = {0u, 0u, 0u, 0u};
    if (sv < K / 8) *reinterpret_cast<u32x4*>(&sa[r][sv * 8]) = r < Mv ? sx[i] : z;
  }
  __syncthreads();
  for (int t = 0; t < T; t += LW_NB) {
#pragma unroll
    for (int i = 0; i < LW_NB; ++i) {
      issue(b[(i + LW_NB - 1) % LW_NB]);
      __builtin_amdgcn_sched_barrier(0);
      step(b[i]);
    }
  }
  // merge: a row's 32 lane lists (4 lanes x 8 waves) go through LDS to one half-wave (wave w
  // takes rows 2w and 2w + 1), which extracts the row's best 16 in 16 rounds of a 32-lane
  // arg-best; the winning lane shifts its sorted list by one.
  float (*lv)[32][TOPK + 1] = reinterpret_cast<float (*)[32][TOPK + 1]>(lw_smem);
  int (*lid)[32][TOPK + 1] = reinterpret_cast<int (*)[32][TOPK + 1]>(lw_smem + 16 * 32 * (TOPK + 1) * 4);
  __syncthreads();   // every wave is done with the activation rows (the lists overlay them)
  {
    const int src = wave * 4 + my_sub;
#pragma unroll
    for (int i = 0; i < TOPK; ++i) { lv[my_row][src][i] = top.v[i]; lid[my_row][src][i] = top.id[i]; }
  }
  __syncthreads();
  const int hr = lane >> 5, s = lane & 31, row = wave * 2 + hr;
  float v[TOPK];
  int id[TOPK];
#pragma unroll
  for (int i = 0; i < TOPK; ++i) { v[i] = lv[row][s][i]; id[i] = lid[row][s][i]; }
  float ov = NEG_INF;
  int oi = ID_NONE;
#pragma unroll 1
  for (int r = 0; r < TOPK; ++r) {
    float bv = v[0];
    int bi = id[0];
    auto step = [&](float cv, int ci) {
      const bool take = cand_better(cv, ci, bv, bi);
      bv = take ? cv : bv;
      bi = take ? ci : bi;
    };
    // every lane ends with the best of its 16-lane row, then the two rows of each half combine
    step(dpp_f<0xB1>(bv), dpp_i<0xB1>(bi));
    step(dpp_f<0x4E>(bv), dpp_i<0x4E>(bi));
    step(dpp_f<0x141>(bv), dpp_i<0x141>(bi));
    step(dpp_f<0x140>(bv), dpp_i<0x140>(bi));
    const float u0 = lane_f(bv, 0), u1 = lane_f(bv, 16), u2 = lane_f(bv, 32), u3 = lane_f(bv, 48);
    const int j0 = __builtin_amdgcn_readlane(bi, 0), j1 = __builtin_amdgcn_readlane(bi, 16);
    const int j2 = __builtin_amdgcn_readlane(bi, 32), j3 = __builtin_amdgcn_readlane(bi, 48);
    const float x0 = hr ? u2 : u0, x1 = hr ? u3 : u1;   // (readlane takes a uniform lane index)
    const int y0 = hr ? j2 : j0, y1 = hr ? j3 : j1;
    const bool second = cand_better(x1, y1, x0, y0);
    bv = second ? x1 : x0;
    bi = second ? y1 : y0;
    if (s == r) { ov = bv; oi = bi; }
    if (id[0] == bi && v[0] == bv) {   // the winning lane (ids are distinct, unless all are empty)
#pragma unroll
      for (int i = 0; i + 1 < TOPK; ++i) { v[i] = v[i + 1]; id[i] = id[i + 1]; }
      v[TOPK - 1] = NEG_INF;
      id[TOPK - 1] = ID_NONE;
    }
  }
  if (s < TOPK && row < Mv) {
    const size_t base = ((size_t)row * p.groups + blockIdx.x) * TOPK;
    p.tk_val[base + s] = ov;
    p.tk_id[base + s] = oi;
  }
}

// ---------------------------------------------------------------------------------------
// fp32: plain dot products.  grid x = 64-column block, y = 4-row block.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  const int Mv = rows_valid(p);
  const int col = blockIdx.x * 64 + (threadIdx.x & 63);
  const int row = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (row >= Mv || col >= p.N) return;
  const float* a = reinterpret_cast<const float*>(p.A) + (size_t)row * p.lda;
  const int s = col / p.seg_rows;
  const float* b = reinterpret_cast<const float*>(p.seg[s]) + (size_t)(col - s * p.seg_rows) * p.ldb;
  float acc = 0.f;
  for (int k = 0; k < p.K; ++k) acc = fmaf(a[k], b[k], acc);
  p.part[(size_t)row * p.N + col] = acc;
}

// ---------------------------------------------------------------------------------------
// planning + launch
// ---------------------------------------------------------------------------------------
static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// The skinny kernels (weights streamed into registers, row tiles of up to 64 rows): the plan
// for 17..64 rows, and for any row count whose weight format the other kernels do not take.
GemmPlan gemm_plan_skinny(int mode, int M, int N, int K) {
  GemmPlan pl{};
  pl.splits = 1;
  pl.groups = 1;
  pl.kind = 0;
  const int nchunks = K / 64;
  pl.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  const int rt = (M + 16 * pl.mt - 1) / (16 * pl.mt);
  if (mode == GEMM_TOPK) {
    const int nfrag = (N + 15) / 16;
    pl.groups = clampi(512 / rt, 1, (nfrag + 3) / 4);   // = resident workgroups (2 per CU)
    pl.grid = dim3(pl.groups, rt, 1);
  } else {
    const int ncols = (mode == GEMM_SWIGLU) ? N / 2 : N;
    const int ct = (ncols + 15) / 16;
    if (mode == GEMM_PARTIAL) pl.splits = clampi((768 + ct * rt - 1) / (ct * rt), 1, clampi(nchunks / 4, 1, 8));
    pl.grid = dim3(ct, rt, pl.splits);
  }
  return pl;
}

GemmPlan gemm_plan_wf(bool bf16, int mode, int M, int N, int K, int wf) {
  GemmPlan pl = gemm_plan(bf16, mode, M, N, K);
  if (!bf16 || wf == 0) return pl;
  // which kernels take E4M3 (1) and MXFP4 (2) weights: the skinny, independent-wave and tile ones
  // both (the MXFP4 lm_head tiles at most TILE4_MAX_STEPS k-steps); the streaming ones both but in
  // their top-16 form
  const bool takes = pl.kind == 0 || pl.kind == 4 || (pl.kind == 3 && mode != GEMM_TOPK) ||
                     (pl.kind == 5 && (wf == 1 || mode != GEMM_TOPK || K / 32 <= TILE4_MAX_STEPS));
  return takes ? pl : gemm_plan_skinny(mode, M, N, K);
}

GemmPlan gemm_plan(bool bf16, int mode, int M, int N, int K) {
  GemmPlan pl{};
  pl.splits = 1;
  pl.groups = 1;
  if (!bf16) {
    pl.kind = 2;
    pl.grid = dim3((N + 63) / 64, (M + 3) / 4, 1);
    return pl;
  }
  if (M <= 16) {
    // stream kernel: slice = SW waves x slc chunks of 64; full K in one workgroup for the
    // nonlinear epilogues, k-splits for PARTIAL
    const int ncols = (mode == GEMM_SWIGLU) ? N / 2 : N;
    const int nfrag = (mode == GEMM_SWIGLU) ? (ncols + 7) / 8 : (ncols + 15) / 16;   // SWIGLU: 8 + 8 columns
    // workgroups loop over fragments: the fragment stride is the largest divisor of the
    // fragment count that keeps the launch at most 256 workgroups (one per CU is enough to
    // stream; every workgroup then has the same number of fragments and loads its activation
    // slice once)
    auto stride = [&](int splits) {
      if (nfrag * splits <= 256) return nfrag;
      for (int gx = 256 / splits; gx >= 1; --gx)
        if (nfrag % gx == 0 && gx * splits >= 128) return gx;
      return max(1, 256 / splits);
    };
    if (mode == GEMM_PARTIAL) {
      pl.slc = 1;
      while (pl.slc < 4 && (K + SW * 64 * pl.slc - 1) / (SW * 64 * pl.slc) > 8) pl.slc *= 2;
      pl.splits = (K + SW * 64 * pl.slc - 1) / (SW * 64 * pl.slc);
      pl.grid = dim3(stride(pl.splits), 1, 1);
      pl.kind = 3;
    } else {
      pl.slc = 1;
      while (pl.slc < 4 && SW * 64 * pl.slc < K) pl.slc *= 2;
      if (mode == GEMM_TOPK && K >= 512 && K % 512 == 0 && K <= LW_KMAX) {
        pl.kind = 4;
        pl.groups = LW_GROUPS;
        pl.grid = dim3(pl.groups, 1, 1);
        return pl;
      }
      if (SW * 64 * pl.slc >= K) {
        pl.kind = 3;
        if (mode == GEMM_TOPK) {
          pl.groups = clampi(256, 1, nfrag);
          pl.grid = dim3(pl.groups, 1, 1);
        } else {
          pl.grid = dim3(stride(1), 1, 1);
        }
      }
    }
    if (pl.kind == 3) {
      pl.grid.y = pl.splits;
      return pl;
    }
  }
  if (M <= 64) {
    return gemm_plan_skinny(mode, M, N, K);
  } else {
    // MFMA tiles with LDS-DMA operands (K is a multiple of 32 for every bf16 drafter).  TOPK:
    // 256 x 256 tiles (one workgroup per CU) once there are more than 128 rows, else 128 x 128
    // (two per CU); the workgroups resident at once split the column tiles statically.
    // PARTIAL: 128 x 128 tiles, k-splits bring the launch to about two workgroups per CU, each
    // split at least 8 k-steps of 32.  For 129..256 rows and at least 3072 columns, 256 x 128
    // tiles (the weights streamed once, not once per 128 rows), k-splits up to about one
    // workgroup per CU.  (Measured at 256 rows: QKV 16.6 -> 14.9 us, gate/up 39.6 -> 34.8 us; the
    // 2048-column GEMMs, with only 16 column tiles, ran slower on the wide tile, and so did
    // every GEMM at 512 or more rows.)
    pl.kind = 5;
    if (mode == GEMM_TOPK) {
      pl.mt = M > 128 ? 1 : 0;
      const int bt = pl.mt ? 256 : 128;
      const int rt = (M + bt - 1) / bt;
      const int ntiles = (N + bt - 1) / bt;
      pl.groups = clampi((pl.mt ? 256 : 512) / rt, 1, ntiles);
      pl.grid = dim3(pl.groups, rt, 1);
    } else {
      pl.mt = (M > 128 && M <= 256 && N >= 3072) ? 2 : 0;
      const int bm = pl.mt ? 256 : 128;
      const int rt = (M + bm - 1) / bm;
      const int ntiles = (N + 127) / 128;
      const int nk = K / 32;
      pl.splits = clampi((pl.mt ? 256 : 512) / (ntiles * rt), 1, clampi(nk / 8, 1, 8));
      pl.grid = dim3(ntiles, rt, pl.splits);
    }
  }
  return pl;
}

size_t gemm_part_floats(const GemmPlan& pl, int mode, int M, int N) {
  if (mode == GEMM_TOPK) return (size_t)M * pl.groups * TOPK;
  if (mode == GEMM_SWIGLU) return 0;
  return (size_t)pl.splits * M * N;
}

// streaming kernel with nb fragments per workgroup requested at once (nb = 0: a ring of the most
// buffers the slice's registers allow: 3 of 4 chunks, 4 of 1 or 2; nb = -2: a ring of 2)
template <int SLC, int MODE, int WF>
static void launch_stream(const GemmPlan& pl, int nb, const GemmParams& p, hipStream_t st) {
  constexpr int NBR = SLC == 4 ? 3 : 4;
  const dim3 sb(SW * 64);
  if (nb == 1) hipLaunchKernelGGL((gemm_stream_kernel<SLC, MODE, 1, false, WF>), pl.grid, sb, 0, st, p);
  else if (nb == 2) hipLaunchKernelGGL((gemm_stream_kernel<SLC, MODE, 2, false, WF>), pl.grid, sb, 0, st, p);
  else if (nb == 3) hipLaunchKernelGGL((gemm_stream_kernel<SLC, MODE, 3, false, WF>), pl.grid, sb, 0, st, p);
  else if (nb == -2) hipLaunchKernelGGL((gemm_stream_kernel<SLC, MODE, 2, true, WF>), pl.grid, sb, 0, st, p);
  else if constexpr (NBR >= 4) {
    if (nb == 4) hipLaunchKernelGGL((gemm_stream_kernel<SLC, MODE, 4, false, WF>), pl.grid, sb, 0, st, p);
    else hipLaunchKernelGGL((gemm_stream_kernel<SLC, MODE, NBR, true, WF>), pl.grid, sb, 0, st, p);
  } else {
    hipLaunchKernelGGL((gemm_stream_kernel<SLC, MODE, NBR, true, WF>), pl.grid, sb, 0, st, p);
  }
}

hipError_t gemm_launch(bool bf16, const GemmPlan& pl, int mode, GemmParams p, hipStream_t st) {
  p.splits = pl.splits;
  p.groups = pl.groups;
  const dim3 blk(256);
  if (pl.kind == 2) {
    hipLaunchKernelGGL(gemm_f32_kernel, pl.grid, blk, 0, st, p);
    return hipGetLastError();
  }
  if (pl.kind == 4) {
    if (p.seg_rows < p.N) return hipErrorInvalidValue;   // one weight segment
    if (p.blk_scale) {
      if (p.logits) hipLaunchKernelGGL((lmhead_topk_wave<true, false, true>), pl.grid, dim3(LW_W * 64), 0, st, p);
      else hipLaunchKernelGGL((lmhead_topk_wave<false, false, true>), pl.grid, dim3(LW_W * 64), 0, st, p);
    } else if (p.row_scale) {
      if (p.logits) hipLaunchKernelGGL((lmhead_topk_wave<true, true>), pl.grid, dim3(LW_W * 64), 0, st, p);
      else hipLaunchKernelGGL((lmhead_topk_wave<false, true>), pl.grid, dim3(LW_W * 64), 0, st, p);
    } else {
      if (p.logits) hipLaunchKernelGGL((lmhead_topk_wave<true, false>), pl.grid, dim3(LW_W * 64), 0, st, p);
      else hipLaunchKernelGGL((lmhead_topk_wave<false, false>), pl.grid, dim3(LW_W * 64), 0, st, p);
    }
    return hipGetLastError();
  }
  if (pl.kind == 3) {
    if ((p.seg_rows % 16 && p.seg_rows < p.N) || p.half % 8) return hipErrorInvalidValue;
    const int ncols = (mode == GEMM_SWIGLU) ? p.half : p.N;
    const int nfrag = (mode == GEMM_SWIGLU) ? (ncols + 7) / 8 : (ncols + 15) / 16;
    // fragments per workgroup: all at once when every workgroup has the same few, else a ring;
    // 4 chunks per wave leave registers for a ring of 3 (or, when 3 would pad the rounds and 2
    // does not, of 2: fc at K = 25600 has 8 fragments per workgroup, 27.7 us with 3, 25 with 2)
    const int G = (int)pl.grid.x, nf = (nfrag + G - 1) / G;
    const int nbmax = pl.slc == 4 ? 3 : 4;
    int nb = nf == 1 ? 1 : (nfrag % G == 0 && nf <= nbmax ? nf : 0);   // 0: ring of nbmax
    if (nb == 0 && pl.slc == 4 && nfrag % G == 0 && nf % 3 && nf % 2 == 0) nb = -2;   // ring of 2
    const int wf = p.blk_scale ? 2 : (p.row_scale ? 1 : 0);
    if (wf && (mode == GEMM_TOPK || p.seg_rows < (mode == GEMM_SWIGLU ? 2 * p.half : p.N)))
      return hipErrorInvalidValue;   // FP8 / MXFP4 weights: PARTIAL / SWIGLU over one weight segment
    if (wf == 2 && p.K % (pl.slc >= 2 ? 128 : 64)) return hipErrorInvalidValue;
#define DFL_STREAM(SLC)                                                                               \
  if (pl.slc == SLC) {                                                                                \
    if (mode == GEMM_TOPK) launch_stream<SLC, GEMM_TOPK, 0>(pl, nb, p, st);                           \
    else if (mode == GEMM_SWIGLU) {                                                                   \
      if (wf == 2) launch_stream<SLC, GEMM_SWIGLU, 2>(pl, nb, p, st);                                 \
      else if (wf == 1) launch_stream<SLC, GEMM_SWIGLU, 1>(pl, nb, p, st);                            \
      else launch_stream<SLC, GEMM_SWIGLU, 0>(pl, nb, p, st);                                         \
    } else {                                                                                          \
      if (wf == 2) launch_stream<SLC, GEMM_PARTIAL, 2>(pl, nb, p, st);                                \
      else if (wf == 1) launch_stream<SLC, GEMM_PARTIAL, 1>(pl, nb, p, st);                           \
      else launch_stream<SLC, GEMM_PARTIAL, 0>(pl, nb, p, st);                                        \
    }                                                                                                 \
  }
    DFL_STREAM(1)
    DFL_STREAM(2)
    DFL_STREAM(4)
#undef DFL_STREAM
    return hipGetLastError();
  }
  if (pl.kind == 0) {
    if ((p.row_scale || p.blk_scale) && p.seg_rows < (mode == GEMM_SWIGLU ? 2 * p.half : p.N))
      return hipErrorInvalidValue;                  // E4M3 / MXFP4 weights: one segment
    if (p.blk_scale && p.K % 64) return hipErrorInvalidValue;
#define DFL_SKINNY(WF)                                                                                \
    if (mode == GEMM_TOPK) {                                                                          \
      if (pl.mt == 1) hipLaunchKernelGGL((lmhead_topk_skinny<1, WF>), pl.grid, blk, 0, st, p);        \
      else if (pl.mt == 2) hipLaunchKernelGGL((lmhead_topk_skinny<2, WF>), pl.grid, blk, 0, st, p);   \
      else hipLaunchKernelGGL((lmhead_topk_skinny<4, WF>), pl.grid, blk, 0, st, p);                   \
    } else if (mode == GEMM_SWIGLU) {                                                                 \
      if (pl.mt == 1) hipLaunchKernelGGL((gemm_skinny_kernel<1, GEMM_SWIGLU, WF>), pl.grid, blk, 0, st, p);      \
      else if (pl.mt == 2) hipLaunchKernelGGL((gemm_skinny_kernel<2, GEMM_SWIGLU, WF>), pl.grid, blk, 0, st, p); \
      else hipLaunchKernelGGL((gemm_skinny_kernel<4, GEMM_SWIGLU, WF>), pl.grid, blk, 0, st, p);                 \
    } else {                                                                                          \
      if (pl.mt == 1) hipLaunchKernelGGL((gemm_skinny_kernel<1, GEMM_PARTIAL, WF>), pl.grid, blk, 0, st, p);      \
      else if (pl.mt == 2) hipLaunchKernelGGL((gemm_skinny_kernel<2, GEMM_PARTIAL, WF>), pl.grid, blk, 0, st, p); \
      else hipLaunchKernelGGL((gemm_skinny_kernel<4, GEMM_PARTIAL, WF>), pl.grid, blk, 0, st, p);                 \
    }
    if (p.blk_scale) {
      DFL_SKINNY(2)
    } else if (p.row_scale) {
      DFL_SKINNY(1)
    } else {
      DFL_SKINNY(0)
    }
#undef DFL_SKINNY
    return hipGetLastError();
  }
  if (pl.kind == 5) return tile_launch(pl, mode, p, st);
  return hipErrorInvalidValue;
}

}  // namespace dfl
