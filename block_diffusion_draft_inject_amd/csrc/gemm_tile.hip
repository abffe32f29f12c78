// Tiled MFMA GEMM for many rows (more than 64): C = A_hi W^T + A_lo W^T over bf16 operands
// (PL = 2 activation planes), or C = A_hi W^T (PL = 1: the lm_head, whose input is bf16).
//
// A workgroup of WGM x WGN waves computes a BM x BN output tile (each wave BM/WGM x BN/WGN)
// over k-steps of 32.  Operands travel global -> LDS by the LDS-DMA form of the global load
// (16 bytes per lane, one 1 KiB block of 16 rows x 32 k per wave instruction), with no VGPR
// staging; S stages rotate, so the loads of step c + S - 1 are in flight while step c is
// multiplied.  Inside a 1 KiB block the four 16-byte k-chunks of a row are stored in a
// row-dependent XOR order, so that the 16 lanes that read one chunk column of 16 rows for an
// MFMA operand fall in distinct LDS banks (for both 8- and 16-lane bank groups).
//
// Synchronisation per k-step: each wave waits for its own loads of the step (vmcnt) and
// for its LDS reads of the previous step (lgkmcnt), then all waves meet at s_barrier; after
// it the stage read one step earlier is free and is refilled.  The LDS-DMA loads are issued
// from inline assembly (the compiler does not know they write LDS; the explicit waits above
// replace its own), so the k-loop contains no other global memory access.
#include <type_traits>

#include "kernels.h"

namespace dfl {
namespace {

constexpr int MK = 32;   // k per step

// chunk order inside a row of a 16-row block: logical chunk c of row r sits in slot c ^ swz(r)
__device__ __forceinline__ int tile_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

template <int BM, int BN, int WGM, int WGN, int S, int PL = 2>
struct TileCfg {
  static constexpr int NW = WGM * WGN, NT = NW * 64; // waves, threads
  static constexpr int WM = BM / WGM, WN = BN / WGN; // wave tile
  static constexpr int FM = WM / 16, FN = WN / 16;   // MFMA fragments per wave
  static constexpr int BA = BM / 16, BB = BN / 16;   // 1 KiB blocks per stage: A hi (, A lo) (BA each), B (BB)
  static constexpr int PLc = PL;
  static_assert(PL == 1 || PL == 2, "activation planes");
  static constexpr int NBLK = PL * BA + BB;
  static constexpr int STAGE = NBLK * 1024;
  static constexpr int D = NBLK / NW;                // LDS-DMA instructions per wave per stage
  static constexpr int LDS = S * STAGE;
  static constexpr int BMc = BM, BNc = BN, Sc = S, WGNc = WGN;
  static constexpr int WF = 0;                       // bf16 weights
  static_assert(BA % NW == 0 && BB % NW == 0, "blocks per operand must split evenly over the waves");
};

// E4M3 weights (row_scale set).  One byte per weight, so a 1 KiB LDS-DMA block holds 16 weight
// rows x 64 k, two k-steps: the k-steps go in pairs.  A pair buffer holds the activation blocks of
// both steps (as for bf16 weights) and one weight block per 16 columns covering both steps; NP
// pair buffers rotate, NP - 1 pairs in flight while one is multiplied.  The four 16-byte pieces
// (16 k each) of a weight row sit in the same row-dependent XOR order as the bf16 chunks; a lane
// takes the 8 codes of its MFMA operand (k = 32 s + 8 kg .. + 7 of step s of the pair) with one
// 8-byte LDS read and widens them to bf16 (exact).  The row scale multiplies the finished
// column: the scales are powers of two, so this equals multiplying by the scaled weights.
template <int BM, int BN, int WGM, int WGN, int NP, int PL = 2>
struct Tile8Cfg {
  static constexpr int NW = WGM * WGN, NT = NW * 64;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int BA = BM / 16, BB = BN / 16;
  static constexpr int PLc = PL;
  static constexpr int NBLK = 2 * PL * BA + BB;          // blocks per pair buffer
  static constexpr int PAIR = NBLK * 1024;
  static constexpr int QA = PL * BA / NW, QB = BB / NW;   // per wave and pair: 2 QA activation, QB weight DMAs
  static constexpr int D2 = 2 * QA + QB;
  static constexpr int LDS = NP * PAIR;
  static constexpr int BMc = BM, BNc = BN, NPc = NP, WGNc = WGN;
  static constexpr int WF = 1;
  static_assert(PL == 1 || PL == 2, "activation planes");
  static_assert(NP >= 2 && NP <= 3, "pair buffers");
  static_assert(BA % NW == 0 && BB % NW == 0, "blocks per operand must split evenly over the waves");
};

// MXFP4 weights (blk_scale set).  Half a byte per weight, so a pair of k-steps (64 k) of a weight
// row is 32 bytes of codes and a 1 KiB LDS-DMA block holds 32 weight rows x 64 k (lane l: row l/2,
// one k-step of it per 16-byte half).  A pair buffer holds the activation blocks of both steps
// (as for bf16 weights) and one code block per 32 columns; where there are fewer code blocks than
// waves, only the first waves issue them (two pair buffers then, every pair waited for in full).
// The two halves of a code row are swapped on bit 3 of the row, so that the 4-byte operand reads
// of 16 rows x 4 lane groups fall in 64 distinct banks.  The block scales (one byte per row and
// k-step: a block is 32 k) of the tile's columns sit in LDS as [step][column] bytes, staged for
// up to SEG k-steps before the k-loop over them; each operand word of eight codes is widened with
// its block's scale (v_cvt_scalef32_pk_bf16_fp4, exact), so nothing is scaled after the sum.
template <int BM, int BN, int WGM, int WGN, int NP, int PL = 2>
struct Tile4Cfg {
  static constexpr int NW = WGM * WGN, NT = NW * 64;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int BA = BM / 16, BC = BN / 32;
  static constexpr int PLc = PL;
  static constexpr int NBLK = 2 * PL * BA + BC;          // blocks per pair buffer
  static constexpr int PAIR = NBLK * 1024;
  static constexpr bool CG = BC < NW;                     // code blocks issued by waves < BC only
  static constexpr int QA = PL * BA / NW, QC = CG ? 1 : BC / NW;
  static constexpr int D2 = 2 * QA + QC;
  static constexpr int SEG = TILE4_MAX_STEPS;             // k-steps of block scales staged at once
  static constexpr int SCL = SEG * BN;                    // their bytes
  static constexpr int LDS = NP * PAIR + SCL;
  static constexpr int EPB = NP * PAIR;                   // bytes an epilogue may overlay
  static constexpr int BMc = BM, BNc = BN, NPc = NP, WGNc = WGN;
  static constexpr int WF = 2;
  static_assert(PL == 1 || PL == 2, "activation planes");
  static_assert(NP >= 2 && NP <= 3 && (NP == 2 || !CG), "pair buffers");
  static_assert(BA % NW == 0 && (BC % NW == 0 || NW % BC == 0), "blocks per operand must split over the waves");
};

__device__ __forceinline__ int ctz_(unsigned x) { return __builtin_ctz(x); }
__device__ __forceinline__ int ctz_(unsigned long long x) { return __builtin_ctzll(x); }

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// one LDS-DMA load: 64 lanes x 16 bytes from base + voff[lane] to LDS [lds, lds + 1024).
// The LDS destination goes through M0, passed as an input operand bound to M0 ("{m0}"): the
// compiler loads it there itself and knows the statement reads it.  It does not look inside the
// statement for the wait state an LDS-DMA load needs after an M0 write, so the statement starts
// with one (s_nop 0).
__device__ __forceinline__ void dma16(unsigned lds, unsigned voff, const void* base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}
// the same from a per-lane 64-bit address
__device__ __forceinline__ void dma16v(unsigned lds, const void* addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "{m0}"(lds) : "memory");
}

// wait until at most N of this wave's loads are outstanding and its LDS reads are done, then
// meet the other waves
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// The per-workgroup operand streams of one tile: for DMA slot q (block NW q + wave of a stage)
// the lane's source at k-step 0 -- activation slots as a uniform base and a per-lane offset,
// weight slots as a per-lane address (a tile's weight rows may lie in different segments).
template <class T>
struct TileSrc {
  const char* base[T::D];
  unsigned voff[T::D];
  const char* addr[T::D];
  unsigned bstep;   // bytes from one k-step's weight piece to the next
};

template <class T>
__device__ __forceinline__ void tile_src(const GemmParams& p, int m0, int n0, int Mv, int ncap, int wave,
                                         int lane, TileSrc<T>& s) {
  const int r16 = lane >> 2;
  const int kc = (lane & 3) ^ tile_swz(r16);
  const char* ahi = reinterpret_cast<const char*>(p.A);
  const char* alo = reinterpret_cast<const char*>(reinterpret_cast<const bf16*>(p.A) + p.a_plane);
#pragma unroll
  for (int q = 0; q < T::D; ++q) {
    const int b = T::NW * q + wave;                // block of the stage
    if (T::NW * q < T::BA) {                       // A hi (compile-time per q: NW q < BA <=> b < BA)
      const int r = min(m0 + b * 16 + r16, Mv - 1);
      s.base[q] = ahi;
      s.voff[q] = (unsigned)(((size_t)r * p.lda + kc * 8) * 2);
    } else if (T::NW * q < T::PLc * T::BA) {       // A lo
      const int r = min(m0 + (b - T::BA) * 16 + r16, Mv - 1);
      s.base[q] = alo;
      s.voff[q] = (unsigned)(((size_t)r * p.lda + kc * 8) * 2);
    } else {                                       // weight rows
      const int n = min(n0 + (b - T::PLc * T::BA) * 16 + r16, ncap - 1);   // columns past ncap re-read the last
      if (p.b_blocked) {   // the lane's 16 bytes of its 16-row group's first block
        const int sg = n / p.seg_rows, nr = n - sg * p.seg_rows;
        s.addr[q] = reinterpret_cast<const char*>(p.seg[sg]) + (size_t)(nr >> 4) * (p.ldb / MK) * 1024 + lane * 16;
      } else {
        s.addr[q] = reinterpret_cast<const char*>(brow_ptr(p, n) + kc * 8);
      }
    }
  }
  s.bstep = p.b_blocked ? 1024u : (unsigned)(MK * 2);
}

// 16-row-blocked copy of a bf16 weight matrix [rows][cols] (rows a multiple of 16, cols of 32):
// block (g, c) -- rows 16 g .. 16 g + 15, k = 32 c .. 32 c + 31 -- is 1 KiB at
// dst + (g * cols / 32 + c) KiB, holding at byte 16 l the piece that lane l of a weight LDS-DMA
// reads in the row-major form: row 16 g + l / 4, k = 32 c + 8 ((l mod 4) XOR swz(l / 4)) .. + 7.
// A tile's weight DMA then reads one contiguous KiB per instruction, and a 16-row group's k-steps
// follow each other; LDS receives the same bytes, so results are unchanged.  One thread per
// 16-byte piece.
__global__ __launch_bounds__(256) void block_weights_kernel(const bf16* src, long rows, long cols, bf16* dst) {
  const long piece = (long)blockIdx.x * 256 + threadIdx.x;
  if (piece >= rows * cols / 8) return;
  const long blk = piece >> 6, steps = cols / MK;
  const int l = (int)(piece & 63), r16 = l >> 2;
  const long g = blk / steps, c = blk - g * steps;
  const long r = 16 * g + r16, k = MK * c + 8 * ((l & 3) ^ tile_swz(r16));
  *reinterpret_cast<u32x4*>(dst + piece * 8) = *reinterpret_cast<const u32x4*>(src + r * cols + k);
}

template <class T>
__device__ __forceinline__ void tile_issue(const TileSrc<T>& s, unsigned lds_stage, int wave, int c) {
#pragma unroll
  for (int q = 0; q < T::D; ++q) {
    const unsigned lds = lds_stage + (T::NW * q + wave) * 1024;
    if (T::NW * q < T::PLc * T::BA) dma16(lds, s.voff[q], s.base[q] + (size_t)c * MK * 2);
    else dma16v(lds, s.addr[q] + (size_t)c * s.bstep);
  }
}

template <class T>
__device__ __forceinline__ void tile_mma(const unsigned char* stage, int wm, int wn, unsigned lo,
                                         f32x4 (&acc)[T::FM][T::FN]) {
  bf16x8 b[T::FN];
#pragma unroll
  for (int j = 0; j < T::FN; ++j)
    b[j] = *reinterpret_cast<const bf16x8*>(stage + (T::PLc * T::BA + wn * T::FN + j) * 1024 + lo);
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(stage + (wm * T::FM + i) * 1024 + lo);
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b[j], acc[i][j], 0, 0, 0);
    if constexpr (T::PLc == 2) {
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(stage + (T::BA + wm * T::FM + i) * 1024 + lo);
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b[j], acc[i][j], 0, 0, 0);
    }
  }
}

// wait for stage `it` with `pend` later stages allowed to stay in flight (0 <= pend <= S - 2)
template <class T, int S>
__device__ __forceinline__ void tile_wait(int pend) {
  static_assert(S >= 2 && S <= 6, "stage count");
  if (S >= 6 && pend >= 4) wait_barrier<4 * T::D>();
  else if (S >= 5 && pend >= 3) wait_barrier<3 * T::D>();
  else if (S >= 4 && pend >= 2) wait_barrier<2 * T::D>();
  else if (S >= 3 && pend >= 1) wait_barrier<T::D>();
  else wait_barrier<0>();
}

// One output tile over k-steps [c0, c1): acc = the tile's partial products.
template <class T>
__device__ __forceinline__ void tile_run(const GemmParams& p, unsigned char* smem, int m0, int n0, int Mv, int ncap,
                                         int c0, int c1, f32x4 (&acc)[T::FM][T::FN]) {
  constexpr int S = T::Sc;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / T::WGNc, wn = wave % T::WGNc, li = lane & 15, kg = lane >> 4;
  TileSrc<T> src;
  tile_src<T>(p, m0, n0, Mv, ncap, wave, lane, src);
  const unsigned lo = li * 64 + ((kg ^ tile_swz(li)) << 4);
  const unsigned sbase = lds_addr(smem);
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int n = c1 - c0;
#pragma unroll
  for (int q = 0; q + 1 < S; ++q)
    if (q < n) tile_issue<T>(src, sbase + q * T::STAGE, wave, c0 + q);
  int st = 0;            // stage of step it
  int sl = S - 1;        // stage that step it + S - 1 goes to
  for (int it = 0; it < n; ++it) {
    tile_wait<T, S>(min(S - 2, n - 1 - it));
    if (it + S - 1 < n) tile_issue<T>(src, sbase + sl * T::STAGE, wave, c0 + it + S - 1);
    tile_mma<T>(smem + st * T::STAGE, wm, wn, lo, acc);
    st = (st + 1 == S) ? 0 : st + 1;
    sl = (sl + 1 == S) ? 0 : sl + 1;
  }
}

// The same over k-steps [c0, c0 + nk), nk even, with four stages used as two pairs: the loads
// of k-steps 2j+2 and 2j+3 go out together (each operand row's two adjacent 64-byte segments
// back to back) while steps 2j and 2j+1 are multiplied, so a workgroup meets at one barrier per
// two k-steps.  (Measured on the 256 x 256 bf16-input tile: 2540 cycles per k-step against 3050
// for the four-stage rotation, whose load rate is the same.)
template <class T>
__device__ __forceinline__ void tile_issue_pair(const TileSrc<T>& s, unsigned st_a, unsigned st_b, int wave, int c) {
#pragma unroll
  for (int q = 0; q < T::D; ++q) {
    const unsigned la = st_a + (T::NW * q + wave) * 1024, lb = st_b + (T::NW * q + wave) * 1024;
    if (T::NW * q < T::PLc * T::BA) {
      dma16(la, s.voff[q], s.base[q] + (size_t)c * MK * 2);
      dma16(lb, s.voff[q], s.base[q] + (size_t)(c + 1) * MK * 2);
    } else {
      dma16v(la, s.addr[q] + (size_t)c * s.bstep);
      dma16v(lb, s.addr[q] + (size_t)(c + 1) * s.bstep);
    }
  }
}

template <class T>
__device__ __forceinline__ void tile_run_pairs(const GemmParams& p, unsigned char* smem, int m0, int n0, int Mv,
                                               int ncap, int c0, int nk, f32x4 (&acc)[T::FM][T::FN]) {
  static_assert(T::Sc == 4, "two pairs of stages");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / T::WGNc, wn = wave % T::WGNc, li = lane & 15, kg = lane >> 4;
  TileSrc<T> src;
  tile_src<T>(p, m0, n0, Mv, ncap, wave, lane, src);
  const unsigned lo = li * 64 + ((kg ^ tile_swz(li)) << 4);
  const unsigned sbase = lds_addr(smem);
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int np = nk / 2;
  tile_issue_pair<T>(src, sbase, sbase + T::STAGE, wave, c0);
  for (int j = 0; j < np; ++j) {
    // pair j has landed for every wave, and every wave is done with pair j - 1's stages
    wait_barrier<0>();
    const int cur = (j & 1) * 2, nxt = 2 - cur;
    if (j + 1 < np) tile_issue_pair<T>(src, sbase + nxt * T::STAGE, sbase + (nxt + 1) * T::STAGE, wave, c0 + 2 * j + 2);
    tile_mma<T>(smem + cur * T::STAGE, wm, wn, lo, acc);
    tile_mma<T>(smem + (cur + 1) * T::STAGE, wm, wn, lo, acc);
  }
}

template <class T>
struct Tile8Src {
  const char* base[T::QA];
  unsigned voff[T::QA];
  const unsigned char* addr[T::QB];
};

template <class T>
__device__ __forceinline__ void tile8_src(const GemmParams& p, int m0, int n0, int Mv, int ncap, int wave, int lane,
                                          Tile8Src<T>& s) {
  const int r16 = lane >> 2;
  const int kc = (lane & 3) ^ tile_swz(r16);
  const char* ahi = reinterpret_cast<const char*>(p.A);
  const char* alo = reinterpret_cast<const char*>(reinterpret_cast<const bf16*>(p.A) + p.a_plane);
#pragma unroll
  for (int q = 0; q < T::QA; ++q) {
    const int b = T::NW * q + wave;                // activation block of a step: hi rows, then lo rows
    const bool hi = T::NW * q < T::BA;
    const int r = min(m0 + (hi ? b : b - T::BA) * 16 + r16, Mv - 1);
    s.base[q] = hi ? ahi : alo;
    s.voff[q] = (unsigned)(((size_t)r * p.lda + kc * 8) * 2);
  }
#pragma unroll
  for (int q = 0; q < T::QB; ++q) {
    const int n = min(n0 + (T::NW * q + wave) * 16 + r16, ncap - 1);   // columns past ncap re-read the last
    s.addr[q] = reinterpret_cast<const unsigned char*>(p.seg[0]) + (size_t)n * p.ldb + kc * 16;
  }
}

// the pair of k-steps c, c + 1 into the pair buffer at LDS address `pb`
template <class T>
__device__ __forceinline__ void tile8_issue(const Tile8Src<T>& s, unsigned pb, int wave, int c) {
#pragma unroll
  for (int q = 0; q < T::QA; ++q) {
    dma16(pb + (T::NW * q + wave) * 1024, s.voff[q], s.base[q] + (size_t)c * MK * 2);
    dma16(pb + (T::PLc * T::BA + T::NW * q + wave) * 1024, s.voff[q], s.base[q] + (size_t)(c + 1) * MK * 2);
  }
#pragma unroll
  for (int q = 0; q < T::QB; ++q) dma16v(pb + (2 * T::PLc * T::BA + T::NW * q + wave) * 1024, s.addr[q] + (size_t)c * MK);
}

// step st (0, 1) of the pair in `pair`: lo = the lane's activation offset in a block, lb = its
// weight offset for this step
template <class T>
__device__ __forceinline__ void tile8_mma(const unsigned char* pair, int st, int wm, int wn, unsigned lo, unsigned lb,
                                          f32x4 (&acc)[T::FM][T::FN]) {
  bf16x8 b[T::FN];
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const uint2 w = *reinterpret_cast<const uint2*>(pair + (2 * T::PLc * T::BA + wn * T::FN + j) * 1024 + lb);
    b[j] = fp8x8_bf16(w.x, w.y, 1.f);
  }
  const unsigned char* a = pair + st * T::PLc * T::BA * 1024;
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(a + (wm * T::FM + i) * 1024 + lo);
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b[j], acc[i][j], 0, 0, 0);
    if constexpr (T::PLc == 2) {
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(a + (T::BA + wm * T::FM + i) * 1024 + lo);
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b[j], acc[i][j], 0, 0, 0);
    }
  }
}

// One output tile over the k-step pairs starting at step c0 (even), np pairs: acc = the tile's
// partial products (before the row scales).
template <class T>
__device__ __forceinline__ void tile8_run(const GemmParams& p, unsigned char* smem, int m0, int n0, int Mv, int ncap,
                                          int c0, int np, f32x4 (&acc)[T::FM][T::FN]) {
  constexpr int NP = T::NPc;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / T::WGNc, wn = wave % T::WGNc, li = lane & 15, kg = lane >> 4;
  Tile8Src<T> src;
  tile8_src<T>(p, m0, n0, Mv, ncap, wave, lane, src);
  const unsigned lo = li * 64 + ((kg ^ tile_swz(li)) << 4);
  const unsigned lb0 = li * 64 + (((kg >> 1) ^ tile_swz(li)) << 4) + (kg & 1) * 8;
  const unsigned lb1 = li * 64 + (((2 + (kg >> 1)) ^ tile_swz(li)) << 4) + (kg & 1) * 8;
  const unsigned sbase = lds_addr(smem);
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q + 1 < NP; ++q)
    if (q < np) tile8_issue<T>(src, sbase + q * T::PAIR, wave, c0 + 2 * q);
  int cur = 0;   // buffer of pair j
  for (int j = 0; j < np; ++j) {
    // pair j has landed for every wave (later pairs may still be in flight), and every wave is
    // done with pair j - 1's buffer
    if (NP >= 3 && j + 1 < np) wait_barrier<T::D2>();
    else wait_barrier<0>();
    if (j + NP - 1 < np) {
      const int nb = cur == 0 ? NP - 1 : cur - 1;
      tile8_issue<T>(src, sbase + nb * T::PAIR, wave, c0 + 2 * (j + NP - 1));
    }
    tile8_mma<T>(smem + cur * T::PAIR, 0, wm, wn, lo, lb0, acc);
    tile8_mma<T>(smem + cur * T::PAIR, 1, wm, wn, lo, lb1, acc);
    cur = cur + 1 == NP ? 0 : cur + 1;
  }
}

template <class T>
struct Tile4Src {
  const char* base[T::QA];
  unsigned voff[T::QA];
  const unsigned char* addr[T::QC];
};

// half (k-step of a pair) stored at 16-byte position half ^ ((row >> 3) & 1) of a code row
__device__ __forceinline__ int tile4_swz(int row) { return (row >> 3) & 1; }

template <class T>
__device__ __forceinline__ void tile4_src(const GemmParams& p, int m0, int n0, int Mv, int ncap, int wave, int lane,
                                          Tile4Src<T>& s) {
  const int r16 = lane >> 2;
  const int kc = (lane & 3) ^ tile_swz(r16);
  const char* ahi = reinterpret_cast<const char*>(p.A);
  const char* alo = reinterpret_cast<const char*>(reinterpret_cast<const bf16*>(p.A) + p.a_plane);
#pragma unroll
  for (int q = 0; q < T::QA; ++q) {
    const int b = T::NW * q + wave;                // activation block of a step: hi rows, then lo rows
    const bool hi = T::NW * q < T::BA;
    const int r = min(m0 + (hi ? b : b - T::BA) * 16 + r16, Mv - 1);
    s.base[q] = hi ? ahi : alo;
    s.voff[q] = (unsigned)(((size_t)r * p.lda + kc * 8) * 2);
  }
  const int r32 = lane >> 1;                       // row of the lane in a code block
  const int half = (lane & 1) ^ tile4_swz(r32);   // the k-step its LDS position holds
#pragma unroll
  for (int q = 0; q < T::QC; ++q) {
    const int b = T::CG ? min(wave, T::BC - 1) : T::NW * q + wave;
    const int n = min(n0 + b * 32 + r32, ncap - 1);   // columns past ncap re-read the last
    s.addr[q] = reinterpret_cast<const unsigned char*>(p.seg[0]) + (size_t)n * p.ldb + half * 16;
  }
}

// the pair of k-steps c, c + 1 (c even) into the pair buffer at LDS address `pb`
template <class T>
__device__ __forceinline__ void tile4_issue(const Tile4Src<T>& s, unsigned pb, int wave, int c) {
#pragma unroll
  for (int q = 0; q < T::QA; ++q) {
    dma16(pb + (T::NW * q + wave) * 1024, s.voff[q], s.base[q] + (size_t)c * MK * 2);
    dma16(pb + (T::PLc * T::BA + T::NW * q + wave) * 1024, s.voff[q], s.base[q] + (size_t)(c + 1) * MK * 2);
  }
  if (!T::CG || wave < T::BC) {                    // wave-uniform
#pragma unroll
    for (int q = 0; q < T::QC; ++q) {
      const int b = T::CG ? wave : T::NW * q + wave;
      dma16v(pb + (2 * T::PLc * T::BA + b) * 1024, s.addr[q] + (size_t)c * (MK / 2));
    }
  }
}

// The block scales of columns [n0, n0 + BN) (clamped to ncap - 1) for k-steps [c, c + ns), ns <=
// SEG, into scl[step][column] (every wave is done with the previous ones: the caller's barrier).
// The compiler counts only its own loads, so its wait for these also waits for any LDS-DMA load
// issued before them; it never waits for fewer.
template <class T, int BURST>
__device__ __forceinline__ void tile4_scales(const GemmParams& p, unsigned char* scl, int n0, int ncap, int c, int ns) {
  // TPC threads per column, each SPT consecutive steps; the two scale bytes of a pair of steps are
  // one 2-byte load (c and K / 32 are even), BURST loads in flight at a time, only the bursts the
  // segment reaches, each load clamped to the segment's last pair (the bytes past ns are not
  // stored)
  constexpr int TPC = T::NT / T::BNc, SPT = T::SEG / TPC;
  static_assert(T::NT % T::BNc == 0 && SPT % 2 == 0 && (SPT / 2) % BURST == 0, "scale bytes per thread");
  const int col = threadIdx.x % T::BNc, s0 = (threadIdx.x / T::BNc) * SPT;
  const unsigned short* src = reinterpret_cast<const unsigned short*>(
      p.blk_scale + (size_t)min(n0 + col, ncap - 1) * (p.K / 32) + c);
  const int lastp = (ns - 1) / 2;
#pragma unroll 1
  for (int i0 = 0; i0 < SPT / 2 && s0 + 2 * i0 < ns; i0 += BURST) {
    unsigned short v[BURST];
#pragma unroll
    for (int i = 0; i < BURST; ++i) v[i] = src[min(s0 / 2 + i0 + i, lastp)];
#pragma unroll
    for (int i = 0; i < BURST; ++i) {
      const int st = s0 + 2 * (i0 + i);
      if (st < ns) scl[st * T::BNc + col] = (unsigned char)(v[i] & 0xFF);
      if (st + 1 < ns) scl[(st + 1) * T::BNc + col] = (unsigned char)(v[i] >> 8);
    }
  }
}

// step st (0, 1) of the pair in `pair`: lo = the lane's activation offset in a block; scl_st the
// scale row of this step
template <class T>
__device__ __forceinline__ void tile4_mma(const unsigned char* pair, int st, int wm, int wn, unsigned lo, int li, int kg,
                                          const unsigned char* scl_st, f32x4 (&acc)[T::FM][T::FN]) {
  bf16x8 b[T::FN];
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const int col = wn * T::WN + j * 16 + li;      // column of the tile
    const int r = col & 31;                        // its row in code block col / 32
    const unsigned w = *reinterpret_cast<const unsigned*>(
        pair + (2 * T::PLc * T::BA + (col >> 5)) * 1024 + r * 32 + ((st ^ tile4_swz(r)) << 4) + kg * 4);
    b[j] = fp4x8_bf16(w, __uint_as_float((unsigned)scl_st[col] << 23));   // 2^(E - 127)
  }
  const unsigned char* a = pair + st * T::PLc * T::BA * 1024;
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(a + (wm * T::FM + i) * 1024 + lo);
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b[j], acc[i][j], 0, 0, 0);
    if constexpr (T::PLc == 2) {
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(a + (T::BA + wm * T::FM + i) * 1024 + lo);
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b[j], acc[i][j], 0, 0, 0);
    }
  }
}

// One output tile over the k-step pairs starting at step c0 (even), np pairs: acc = the tile's
// sums.  The block scales of up to SEG k-steps are staged in LDS before the pairs that use them:
// once, when 2 np <= SEG (the lm_head tiles require it), else per segment of SEG k-steps (SEGS:
// the partial-sum tiles, whose registers leave room for the accumulators across the segment
// loop; in the 256 x 256 lm_head tile the same loop spilled them).
template <class T, bool SEGS>
__device__ __forceinline__ void tile4_run(const GemmParams& p, unsigned char* smem, int m0, int n0, int Mv, int ncap,
                                          int c0, int np, f32x4 (&acc)[T::FM][T::FN]) {
  constexpr int NP = T::NPc;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / T::WGNc, wn = wave % T::WGNc, li = lane & 15, kg = lane >> 4;
  unsigned char* scl = smem + NP * T::PAIR;
  const unsigned lo = li * 64 + ((kg ^ tile_swz(li)) << 4);
  const unsigned sbase = lds_addr(smem);
  // the pairs [g0, g0 + gn) of the range, their first NP - 1 already in flight and the scales of
  // their steps staged
  auto pairs = [&](const Tile4Src<T>& src, int g0, int gn) {
    const int cg = c0 + 2 * g0;
    int cur = 0;   // buffer of pair j
    for (int j = 0; j < gn; ++j) {
      // pair j has landed for every wave (later pairs may still be in flight), every wave is done
      // with pair j - 1's buffer, and (first pass) the scales are in LDS
      if (NP >= 3 && j + 1 < gn) wait_barrier<T::D2>();
      else wait_barrier<0>();
      if (j + NP - 1 < gn) {
        const int nb = cur == 0 ? NP - 1 : cur - 1;
        tile4_issue<T>(src, sbase + nb * T::PAIR, wave, cg + 2 * (j + NP - 1));
      }
      tile4_mma<T>(smem + cur * T::PAIR, 0, wm, wn, lo, li, kg, scl + (2 * j) * T::BNc, acc);
      tile4_mma<T>(smem + cur * T::PAIR, 1, wm, wn, lo, li, kg, scl + (2 * j + 1) * T::BNc, acc);
      cur = cur + 1 == NP ? 0 : cur + 1;
    }
  };
  // The first pairs' loads go out before the scales are staged, so both travel in one round trip
  // (the compiler counts only its own loads: its wait for the scale loads also waits for the pairs
  // issued before them, never for fewer).
  Tile4Src<T> src;
  tile4_src<T>(p, m0, n0, Mv, ncap, wave, lane, src);
  if constexpr (!SEGS) {
    wait_barrier<0>();                             // every wave is done with the LDS of the last tile
#pragma unroll
    for (int q = 0; q + 1 < NP; ++q)
      if (q < np) tile4_issue<T>(src, sbase + q * T::PAIR, wave, c0 + 2 * q);
    tile4_scales<T, 8>(p, scl, n0, ncap, c0, 2 * np);   // before the accumulators are live
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    pairs(src, 0, np);
  } else {
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int g0 = 0; g0 < np; g0 += T::SEG / 2) {
      const int gn = min(T::SEG / 2, np - g0);
      wait_barrier<0>();                           // every wave is done with the previous segment
#pragma unroll
      for (int q = 0; q + 1 < NP; ++q)
        if (q < gn) tile4_issue<T>(src, sbase + q * T::PAIR, wave, c0 + 2 * (g0 + q));
      tile4_scales<T, T::SEG / (2 * (T::NT / T::BNc))>(p, scl, n0, ncap, c0 + 2 * g0, 2 * gn);
      pairs(src, g0, gn);
    }
  }
}

// PARTIAL: grid x = k-split, y = column tile, z = row tile; part[split][row][col].  The split is
// the fastest grid index: workgroups go to the eight XCDs round-robin by linear index, so with
// eight splits each XCD takes one k-range and its L2 fetches only that slice of the activation
// rows (every column tile of a split reads the same slice), instead of all of them.
template <class T, int OCC>
__global__ __launch_bounds__(T::NT, OCC) void gemm_tile_partial(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[T::LDS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / T::WGNc, wn = wave % T::WGNc, li = lane & 15, kg = lane >> 4;
  const int Mv = rows_valid(p);
  const int m0 = blockIdx.z * T::BMc, n0 = blockIdx.y * T::BNc;
  if (m0 >= Mv) return;
  const int nk = p.K / MK, s = blockIdx.x;
  f32x4 acc[T::FM][T::FN];
  float sc[T::FN];   // E4M3: the row scale of each of the lane's columns
  if constexpr (T::WF == 1) {
    // whole pairs of k-steps per split (K is a multiple of 64)
    const int np = nk / 2;
    const int p0 = (int)((long)np * s / p.splits), p1 = (int)((long)np * (s + 1) / p.splits);
#pragma unroll
    for (int j = 0; j < T::FN; ++j) sc[j] = p.row_scale[min(n0 + wn * T::WN + j * 16 + li, p.N - 1)];
    tile8_run<T>(p, smem, m0, n0, Mv, p.N, 2 * p0, p1 - p0, acc);
  } else if constexpr (T::WF == 2) {
    // MXFP4: whole pairs of k-steps per split, the block scales applied inside
    const int np = nk / 2;
    const int p0 = (int)((long)np * s / p.splits), p1 = (int)((long)np * (s + 1) / p.splits);
#pragma unroll
    for (int j = 0; j < T::FN; ++j) sc[j] = 1.f;
    tile4_run<T, true>(p, smem, m0, n0, Mv, p.N, 2 * p0, p1 - p0, acc);
  } else {
    const int c0 = (int)((long)nk * s / p.splits), c1 = (int)((long)nk * (s + 1) / p.splits);
#pragma unroll
    for (int j = 0; j < T::FN; ++j) sc[j] = 1.f;
    if constexpr (T::Sc == 4) {
      if ((c1 - c0) % 2 == 0) tile_run_pairs<T>(p, smem, m0, n0, Mv, p.N, c0, c1 - c0, acc);
      else tile_run<T>(p, smem, m0, n0, Mv, p.N, c0, c1, acc);
    } else {
      tile_run<T>(p, smem, m0, n0, Mv, p.N, c0, c1, acc);
    }
  }
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * T::WM + i * 16 + kg * 4 + r;
        const int col = n0 + wn * T::WN + j * 16 + li;
        if (row < Mv && col < p.N) p.part[((size_t)s * p.M + row) * p.N + col] = acc[i][j][r] * sc[j];
      }
}

// TOPK (lm_head): grid x = workgroups per row tile (static tile split: tiles x, x + gridDim.x,
// ...), y = row tile.  After each tile its logits pass through LDS 64 columns at a time; TPR
// threads share a row (64 / TPR columns each) and keep running top-16 lists: a thread first
// marks the columns that beat its list's 16th entry, then inserts only those.  The lists of a
// row are merged at the end into one partial list per (row, workgroup).  The 256-row tile keeps
// one list per row, on its first 256 threads (one wave per SIMD): a list of n random columns
// takes about 16 + 16 ln(n / 16) insertions, so splitting a row over two lists adds insertions
// that the SIMDs, not the waves, pay for (224 rows: 282 -> 269 us; 960 rows: 711 -> 668 us).
template <class T, int OCC, bool LOGITS>
__global__ __launch_bounds__(T::NT, OCC) void lmhead_topk_tile(GemmParams p) {
  constexpr int BM = T::BMc, BN = T::BNc;
  constexpr int TPR = BM >= 256 ? 1 : T::NT / BM;   // threads per row in the epilogue
  constexpr int EPT = BM * TPR;                   // epilogue threads (the first EPT of the workgroup)
  constexpr int CPT = 64 / TPR;                   // columns per thread in a 64-column pass
  using MaskT = typename std::conditional<(CPT > 32), unsigned long long, unsigned>::type;   // one bit per column
  static_assert(T::NT % BM == 0 && EPT <= T::NT && CPT % 4 == 0, "row split");
  static_assert(T::LDS >= BM * 68 * 4, "epilogue buffer must fit in the stages");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[T::LDS];
  float (*ep)[68] = reinterpret_cast<float (*)[68]>(smem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WGNc, wn = wave % T::WGNc, li = lane & 15, kg = lane >> 4;
  const int Mv = rows_valid(p);
  const int m0 = blockIdx.y * BM;
  if (m0 >= Mv) return;
  // a contiguous range of columns per workgroup, in 16-column blocks, walked in tiles of BN: the
  // last tile of a range is partial, its columns past the range re-read the range's last weight
  // row (cache hits) and are skipped by the epilogue.  (Against whole tiles handed out
  // round-robin: 960 rows, 64 workgroups per row tile, 708 -> 673 us; 224 rows unchanged, where
  // each workgroup's partial third tile costs about as much as the whole third tile that 82 of
  // the 256 workgroups ran before: the k-step cost there does not follow the weight bytes.)
  const int nblk = (p.N + 15) / 16;
  const int cbeg = (int)((long)nblk * blockIdx.x / gridDim.x) * 16;
  const int cend = min((int)((long)nblk * (blockIdx.x + 1) / gridDim.x) * 16, p.N);
  const int nk = p.K / MK;
  const bool ep_thr = tid < EPT;
  const int lrow = ep_thr ? tid / TPR : 0, part = tid % TPR;
  const int my_row = m0 + lrow;
  const bool row_live = ep_thr && my_row < Mv && (my_row % p.block) != 0;
  Top16 top;
  top.init();
  for (int n0 = cbeg; n0 < cend; n0 += BN) {
    f32x4 acc[T::FM][T::FN];
    if constexpr (T::WF == 1) {
      // E4M3: the row scales of the lane's columns (read after the k-loop: held across it, they
      // pushed the 256 x 256 tile past its registers)
      tile8_run<T>(p, smem, m0, n0, Mv, cend, 0, nk / 2, acc);
      float sc[T::FN];
#pragma unroll
      for (int j = 0; j < T::FN; ++j) sc[j] = p.row_scale[min(n0 + wn * T::WN + j * 16 + li, p.N - 1)];
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) acc[i][j] *= sc[j];
    } else if constexpr (T::WF == 2) {
      tile4_run<T, false>(p, smem, m0, n0, Mv, cend, 0, nk / 2, acc);
    } else if constexpr (T::Sc == 4) {
      if (nk % 2 == 0) tile_run_pairs<T>(p, smem, m0, n0, Mv, cend, 0, nk, acc);
      else tile_run<T>(p, smem, m0, n0, Mv, cend, 0, nk, acc);
    } else {
      tile_run<T>(p, smem, m0, n0, Mv, cend, 0, nk, acc);
    }
    wait_barrier<0>();   // every wave is done reading the stages; the epilogue buffer overlays them
#pragma unroll
    for (int q = 0; q < BN / 64; ++q) {
      const int owner = (q * 64) / T::WN;        // wave column holding these 64 columns
      const int j0 = ((q * 64) % T::WN) / 16;
      static_assert(T::WN % 64 == 0, "a 64-column pass lies in one wave column");
      if (wn == owner) {
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r) ep[wm * T::WM + i * 16 + kg * 4 + r][jj * 16 + li] = acc[i][j0 + jj][r];
      }
      wait_barrier<0>();
      const int cb = part * CPT;
      if (LOGITS && ep_thr && my_row < Mv) {
        for (int c = 0; c < CPT; ++c)
          if (n0 + q * 64 + cb + c < cend) store_logit(p, my_row, n0 + q * 64 + cb + c, ep[lrow][cb + c]);
      }
      // threshold: the better of the 16th entries of the row's lists (a value below another
      // list's 16th entry has 16 better values in that list and cannot reach the row's top 16).
      // Every id in either list comes from an earlier pass, so it is smaller than the columns
      // of this pass: a column beats an entry exactly when its value is larger.
      float tv = top.v[TOPK - 1];
      if (TPR == 2) tv = fmaxf(tv, dpp_f<0xB1>(tv));   // the partner thread of the row is lane ^ 1
      if (row_live) {
        // which of the thread's columns beat the threshold; then one push per such column, so
        // a wave runs as many pushes as its busiest lane needs (not one per column that any
        // lane needs)
        const int cg = n0 + q * 64 + cb;         // global column of the thread's first value
        MaskT mask = 0;
#pragma unroll
        for (int c4 = 0; c4 < CPT / 4; ++c4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&ep[lrow][cb + c4 * 4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int col = cg + c4 * 4 + e;
            mask |= (MaskT)(col < cend && v[e] > tv) << (c4 * 4 + e);
          }
        }
        // the next marked value is read from LDS before the current one is inserted, so the
        // read's latency overlaps the insertion (b32 lm_head 269 -> 267 us)
        if (mask) {
          int c = ctz_(mask);
          mask &= mask - 1;
          float val = ep[lrow][cb + c];
          while (true) {
            const int cn = mask ? ctz_(mask) : c;
            const float vn = ep[lrow][cb + cn];
            top.push_asc(val, cg + c);   // a thread's columns ascend
            if (!mask) break;
            mask &= mask - 1;
            c = cn;
            val = vn;
          }
        }
      }
      wait_barrier<0>();
    }
  }
  // merge the TPR lists of each row through LDS (pairwise halving)
  float (*mv)[TOPK + 1] = reinterpret_cast<float (*)[TOPK + 1]>(smem);
  int (*mi)[TOPK + 1] = reinterpret_cast<int (*)[TOPK + 1]>(smem + T::NT * (TOPK + 1) * 4);
#pragma unroll
  for (int w = 1; w < TPR; w <<= 1) {
    if ((part & (2 * w - 1)) == w) {
#pragma unroll
      for (int i = 0; i < TOPK; ++i) { mv[tid][i] = top.v[i]; mi[tid][i] = top.id[i]; }
    }
    wait_barrier<0>();
    if ((part & (2 * w - 1)) == 0) {
#pragma unroll
      for (int i = 0; i < TOPK; ++i) top.push(mv[tid + w][i], mi[tid + w][i]);
    }
    wait_barrier<0>();
  }
  if (ep_thr && part == 0 && my_row < Mv) store_partial(p, my_row, blockIdx.x, top);
}

}  // namespace

// Tile configurations: 0 = 128 x 128 (2 x 2 waves, 3 stages, two workgroups per CU),
// 1 = 256 x 256 (4 x 2 waves of 64 x 128, two waves per SIMD, 3 stages, one workgroup per CU),
// 2 = 256 x 128 (4 x 2 waves of 64 x 64, one workgroup per CU, 160 KiB of LDS: four stages used
// as two pairs): all rows of a batch of up to 256 in one tile, so each weight tile is streamed
// once.
// The lm_head variants read the hi plane only; with half the bytes per stage the big tile
// keeps four stages in flight.
using TileSmall = TileCfg<128, 128, 2, 2, 3>;
using TileBig = TileCfg<256, 256, 4, 2, 3>;
using TileTall = TileCfg<256, 128, 4, 2, 4>;
using TileSmallHi = TileCfg<128, 128, 2, 2, 3, 1>;
using TileBigHi = TileCfg<256, 256, 4, 2, 4, 1>;
// E4M3 weights: pair buffers of 40 / 72 KiB (layer GEMMs, two each) and 24 / 48 KiB (lm_head,
// three each)
using TileSmall8 = Tile8Cfg<128, 128, 2, 2, 2>;
using TileTall8 = Tile8Cfg<256, 128, 4, 2, 2>;
using TileSmallHi8 = Tile8Cfg<128, 128, 2, 2, 3, 1>;
using TileBigHi8 = Tile8Cfg<256, 256, 4, 2, 3, 1>;
// MXFP4 weights: pair buffers of 36 / 68 KiB (layer GEMMs, two each; the 256 x 128 tile's four
// code blocks issued by waves 0-3) and 20 / 40 KiB (lm_head, three each), plus 8 / 16 KiB of
// staged block scales
using TileSmall4 = Tile4Cfg<128, 128, 2, 2, 2>;
using TileTall4 = Tile4Cfg<256, 128, 4, 2, 2>;
using TileSmallHi4 = Tile4Cfg<128, 128, 2, 2, 3, 1>;
using TileBigHi4 = Tile4Cfg<256, 256, 4, 2, 3, 1>;

hipError_t launch_block_weights(const void* src, long rows, long cols, void* dst, hipStream_t st) {
  if (!src || !dst || rows <= 0 || cols <= 0 || rows % 16 || cols % MK) return hipErrorInvalidValue;
  const long grid = (rows * cols / 8 + 255) / 256;
  if (grid > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(block_weights_kernel, dim3((unsigned)grid), dim3(256), 0, st, reinterpret_cast<const bf16*>(src),
                     rows, cols, reinterpret_cast<bf16*>(dst));
  return hipGetLastError();
}

hipError_t tile_launch(const GemmPlan& pl, int mode, const GemmParams& p, hipStream_t st) {
  if (p.K % MK) return hipErrorInvalidValue;
  // blocked bf16 weights: whole 16-row groups per segment and whole k-steps per row
  if (p.b_blocked && (p.row_scale || p.blk_scale || p.seg_rows % 16 || p.ldb % MK)) return hipErrorInvalidValue;
  if (p.blk_scale) {   // MXFP4 weights: one segment, whole pairs of k-steps, at most SEG k-steps a workgroup
    if (p.K % (2 * MK) || p.seg_rows < p.N || p.row_scale) return hipErrorInvalidValue;
    if (mode == GEMM_TOPK && p.K / MK > TILE4_MAX_STEPS) return hipErrorInvalidValue;
    if (mode == GEMM_TOPK) {
      if (pl.mt) {
        if (p.logits) hipLaunchKernelGGL((lmhead_topk_tile<TileBigHi4, 1, true>), pl.grid, dim3(TileBigHi4::NT), 0, st, p);
        else hipLaunchKernelGGL((lmhead_topk_tile<TileBigHi4, 1, false>), pl.grid, dim3(TileBigHi4::NT), 0, st, p);
      } else {
        if (p.logits) hipLaunchKernelGGL((lmhead_topk_tile<TileSmallHi4, 2, true>), pl.grid, dim3(TileSmallHi4::NT), 0, st, p);
        else hipLaunchKernelGGL((lmhead_topk_tile<TileSmallHi4, 2, false>), pl.grid, dim3(TileSmallHi4::NT), 0, st, p);
      }
    } else if (mode == GEMM_PARTIAL) {
      const dim3 g(pl.grid.z, pl.grid.x, pl.grid.y);
      if (pl.mt == 2) hipLaunchKernelGGL((gemm_tile_partial<TileTall4, 1>), g, dim3(TileTall4::NT), 0, st, p);
      else if (pl.mt == 0) hipLaunchKernelGGL((gemm_tile_partial<TileSmall4, 2>), g, dim3(TileSmall4::NT), 0, st, p);
      else return hipErrorInvalidValue;
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (p.row_scale) {   // E4M3 weights: one segment, whole pairs of k-steps
    if (p.K % (2 * MK) || p.seg_rows < p.N || p.blk_scale) return hipErrorInvalidValue;
    if (mode == GEMM_TOPK) {
      if (pl.mt) {
        if (p.logits) hipLaunchKernelGGL((lmhead_topk_tile<TileBigHi8, 1, true>), pl.grid, dim3(TileBigHi8::NT), 0, st, p);
        else hipLaunchKernelGGL((lmhead_topk_tile<TileBigHi8, 1, false>), pl.grid, dim3(TileBigHi8::NT), 0, st, p);
      } else {
        if (p.logits) hipLaunchKernelGGL((lmhead_topk_tile<TileSmallHi8, 2, true>), pl.grid, dim3(TileSmallHi8::NT), 0, st, p);
        else hipLaunchKernelGGL((lmhead_topk_tile<TileSmallHi8, 2, false>), pl.grid, dim3(TileSmallHi8::NT), 0, st, p);
      }
    } else if (mode == GEMM_PARTIAL) {
      const dim3 g(pl.grid.z, pl.grid.x, pl.grid.y);
      if (pl.mt == 2) hipLaunchKernelGGL((gemm_tile_partial<TileTall8, 1>), g, dim3(TileTall8::NT), 0, st, p);
      else if (pl.mt == 0) hipLaunchKernelGGL((gemm_tile_partial<TileSmall8, 2>), g, dim3(TileSmall8::NT), 0, st, p);
      else return hipErrorInvalidValue;
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (mode == GEMM_TOPK) {
    if (pl.mt) {
      const dim3 blk(TileBigHi::NT);
      if (p.logits) hipLaunchKernelGGL((lmhead_topk_tile<TileBigHi, 1, true>), pl.grid, blk, 0, st, p);
      else hipLaunchKernelGGL((lmhead_topk_tile<TileBigHi, 1, false>), pl.grid, blk, 0, st, p);
    } else {
      const dim3 blk(TileSmallHi::NT);
      if (p.logits) hipLaunchKernelGGL((lmhead_topk_tile<TileSmallHi, 2, true>), pl.grid, blk, 0, st, p);
      else hipLaunchKernelGGL((lmhead_topk_tile<TileSmallHi, 2, false>), pl.grid, blk, 0, st, p);
    }
  } else if (mode == GEMM_PARTIAL) {
    const dim3 g(pl.grid.z, pl.grid.x, pl.grid.y);   // (split, column tile, row tile)
    if (pl.mt == 2) hipLaunchKernelGGL((gemm_tile_partial<TileTall, 1>), g, dim3(TileTall::NT), 0, st, p);
    else if (pl.mt) hipLaunchKernelGGL((gemm_tile_partial<TileBig, 1>), g, dim3(TileBig::NT), 0, st, p);
    else hipLaunchKernelGGL((gemm_tile_partial<TileSmall, 2>), g, dim3(TileSmall::NT), 0, st, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dfl
