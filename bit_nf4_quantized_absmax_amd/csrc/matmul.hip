// Fused NF4-dequant matmuls on gfx950 bf16 MFMA.
//
// Forward (automatone.win, "QLoRA paper explained", How it works: the frozen
// 4-bit weights are dequantized to BFloat16 on the fly for the math):
//     Y [M, N] = [X | T] [deq(W) | B]^T,            T = s X A^T (given)
// the K loop over packed NF4 tiles plus one (r <= 64) or two (r <= 128)
// extra contraction steps that fold in the LoRA up-projection T B^T.
//
// dX (same page: gradients flow through the frozen 4-bit base; gptget.net,
// "QLoRA: Efficient Finetuning of Quantized LLMs", Deep Analysis /
// Methodology: the backward matmul dequantizes to 16-bit):
//     dX [M, K] = [dY | G] [deq(W) ; A],           G = s dY B (given)
// contraction over N: the dequantized tile is written transposed into LDS.
//
// Design (both kernels):
//  * 256 x 256 output tile, contraction step 64, 512 threads = 8 waves in two
//    groups of 4.  Group g owns output rows 128 g .. +127; wave (g, q) owns a
//    128 x 64 block computed with 4 x 2 MFMA 32x32x16 bf16 (fp32 accumulate).
//  * Ping-pong: each step has two phases separated by barriers.  In phase 0
//    group 0 runs its MFMAs on stage `cur` while group 1 dequantizes its half
//    of the next weight tile into stage `cur ^ 1`; in phase 1 the roles swap.
//    One wave per SIMD issues MFMAs while the other does the VALU/LDS work of
//    the dequantization, so the matrix cores never wait for the expansion.
//  * The left operand (X or dY) goes global -> LDS with 16-byte DMA loads
//    (global_load_lds_dwordx4), rows XOR-swizzled by 16-byte chunk so that
//    both the DMA writes and the MFMA operand reads are bank-conflict free.
//    The two stages are separate LDS arrays so the compiler does not wait for
//    the DMA before reading the other stage.
//  * Packed weight bytes, block codes and group scales are prefetched two
//    steps ahead in registers.
//  * Tiles are mapped so that consecutive tiles (sharing left-operand rows)
//    run on the same XCD and its L2.
//  * Epilogue: accumulators -> bf16 (round to nearest even) -> per-wave LDS
//    staging -> 16-byte global stores.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace qlora {

#define QLORA_LDS(p) ((__attribute__((address_space(3))) void *)(p))

__constant__ uint32_t cMMNF4Level[16] = {QLORA_NF4_LEVEL_BITS};
__constant__ uint32_t cMMT8Level[256] = {QLORA_T8_LEVEL_BITS};

constexpr int kBM = 256;               // output rows per tile
constexpr int kBN = 256;               // output columns per tile
constexpr int kBK = 64;                // contraction step
constexpr int kThreadsMM = 512;
constexpr int kXBytes = kBM * kBK * 2;         // left stage: 256 rows x 128 B (swizzled)
constexpr int kWLd = kBK + 8;                  // right stage row stride in bf16 (144 B, padded)
constexpr int kWBytes = kBN * kWLd * 2;        // right stage bytes

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; a field at its maximum does not wait).
constexpr int kWaitLgkm0 = 0xC07F;          // lgkmcnt(0)
constexpr int kWaitVm0Lgkm0 = 0x0070;       // vmcnt(0) lgkmcnt(0)
constexpr int kWaitVm3Lgkm0 = 0x0073;       // all but the 3 refill loads of a forward step
constexpr int kWaitVm6Lgkm0 = 0x0076;       // all but the 6 refill loads of a dX step

// Wave roles.  The two wave groups must share every SIMD (one wave of each per
// SIMD) so that one group's MFMAs overlap the other group's expansion; waves of
// a workgroup are placed on the 4 SIMDs round-robin (wave w on SIMD w % 4), so
// waves 0-3 form group 0 and waves 4-7 group 1.
#ifndef QLORA_GROUP_OF_WAVE
#define QLORA_GROUP_OF_WAVE(w) ((w) >> 2)
#define QLORA_INDEX_IN_GROUP(w) ((w) & 3)
#endif
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ int wave_group() { return QLORA_GROUP_OF_WAVE(wave_id()); }
__device__ __forceinline__ int wave_in_group() { return QLORA_INDEX_IN_GROUP(wave_id()); }
// thread index 0..255 within its group
__device__ __forceinline__ int thread_in_group() { return wave_in_group() * 64 + (threadIdx.x & 63); }

// Byte offset of 16-byte chunk `chunk` (0..7) of row `row` in a swizzled stage.
__device__ __forceinline__ int xswz(int row, int chunk) {
  return row * 128 + 16 * (chunk ^ ((row & 7) ^ ((row >> 3) & 1)));
}

// Left operand tile: rows m0 .. m0+255 of a row-major bf16 matrix (row
// stride ld elements, `cols` columns, cols % 8 == 0), columns c0 .. c0+63,
// DMA'd into a swizzled stage by the 4 waves of one group (`gw` = wave index
// within the group).  Each wave issues blocks u = 8 gw .. 8 gw + 7 of 8 rows
// (1 KB, one DMA instruction each); lane i of a block lands in slot i, i.e.
// row 8 u + i / 8 at position i % 8, which holds logical chunk
// (i % 8) ^ swizzle(row).  Rows past `rows` are clamped to the last row
// (their results are never stored); chunks past `cols` are clamped to the
// row's last chunk (finite data that meets zero weights in the contraction
// tail).
__device__ __forceinline__ void dma_left(uint8_t *stage, const uint16_t *src, int64_t ld, int m0, int rows,
                                         int c0, int cols, int gw) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int u = gw * 8 + j;
    const int row = u * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row & 7) ^ ((row >> 3) & 1));
    const int grow = min(m0 + row, rows - 1);
    const int gcol = min(c0 + chunk * 8, cols - 8);
    const uint16_t *g = src + static_cast<int64_t>(grow) * ld + gcol;
    const int off = __builtin_amdgcn_readfirstlane(u * 1024);
    __builtin_amdgcn_global_load_lds(g, QLORA_LDS(stage + off), 16, 0, 0);
  }
}

// Workgroup barrier without a memory-model fence: waits for this wave's LDS
// operations (and, with kWaitVm*, for its DMA loads) and then s_barrier.  A
// fence would also wait for every outstanding DMA and prefetch load.  The
// signal fences stop the compiler from moving memory accesses across it, and
// the scheduling barriers keep each phase its own scheduling region (no
// instruction of one phase is moved into another).
template <int kWait>
__device__ __forceinline__ void raw_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWait);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

// One 64-wide contraction step of this wave's 128 x 64 block.
// MFMA 32x32x16: lane l supplies row (l & 31) of A and column (l & 31) of B,
// with contraction elements 8 (l >> 5) .. +7 of each 16-wide sub-step.
__device__ __forceinline__ void mfma_step(const uint8_t *xs, const uint8_t *ws, f32x16_t (&acc)[4][2]) {
  const int lane = threadIdx.x & 63;
  const int wm = wave_group(), wn = wave_in_group();
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int chunk = 2 * s + lh;
    bf16x8_t a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8_t *>(xs + xswz(wm * 128 + 32 * i + lr, chunk));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = *reinterpret_cast<const bf16x8_t *>(ws + (wn * 64 + 32 * j + lr) * (kWLd * 2) + chunk * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Narrow [rows, r] bf16 matrix (T, G or B) as one 64-wide contraction step:
// columns j0 .. j0+63, zero past r.  Stored swizzled (left) or padded (right).
template <bool kLeft>
__device__ __forceinline__ void load_narrow(uint8_t *stage, const uint16_t *src, int r, int row0, int rows, int j0) {
  if ((r & 7) == 0) {
    for (int idx = threadIdx.x; idx < kBM * 8; idx += kThreadsMM) {
      const int row = idx >> 3, c = idx & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row0 + row < rows && j0 + 8 * c < r)
        v = *reinterpret_cast<const uint4 *>(src + static_cast<int64_t>(row0 + row) * r + j0 + 8 * c);
      const int off = kLeft ? xswz(row, c) : row * (kWLd * 2) + 16 * c;
      *reinterpret_cast<uint4 *>(stage + off) = v;
    }
  } else {
    for (int idx = threadIdx.x; idx < kBM * 64; idx += kThreadsMM) {
      const int row = idx >> 6, j = idx & 63;
      uint16_t v = 0;
      if (row0 + row < rows && j0 + j < r) v = src[static_cast<int64_t>(row0 + row) * r + j0 + j];
      const int off = kLeft ? xswz(row, j >> 3) + 2 * (j & 7) : row * (kWLd * 2) + 2 * j;
      *reinterpret_cast<uint16_t *>(stage + off) = v;
    }
  }
}

// Epilogue: each wave writes its 128 x 64 block as bf16 into its own 16 KB LDS
// region (16-byte chunks XOR-swizzled by row), then streams it out with
// 16-byte stores guarded by the matrix bounds (ncols % 8 == 0).
// MFMA 32x32 output layout: lane l holds column l & 31; element e holds row
// 8 (e / 4) + 4 (l >> 5) + (e % 4).
__device__ __forceinline__ void store_tile(const f32x16_t (&acc)[4][2], uint8_t *region, uint16_t *out, int64_t ld,
                                           int row0, int col0, int nrows, int ncols) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int c = 32 * j + (lane & 31);
        const int off = r * 128 + 16 * ((c >> 3) ^ (r & 7)) + 2 * (c & 7);
        *reinterpret_cast<uint16_t *>(region + off) = f32_to_bf16(acc[i][j][e]);
      }
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int idx = t * 64 + lane;
    const int r = idx >> 3, c = idx & 7;
    const uint4 v = *reinterpret_cast<const uint4 *>(region + r * 128 + 16 * (c ^ (r & 7)));
    const int gr = row0 + r, gc = col0 + 8 * c;
    if (gr < nrows && gc < ncols) *reinterpret_cast<uint4 *>(out + static_cast<int64_t>(gr) * ld + gc) = v;
  }
}

__device__ __forceinline__ void init_tables(float2 *lut2, float *t8) {
  for (int i = threadIdx.x; i < 256; i += kThreadsMM) {
    lut2[i] = make_float2(u2f(cMMNF4Level[i & 15]), u2f(cMMNF4Level[i >> 4]));
    t8[i] = u2f(cMMT8Level[i]);
  }
}

// Tile index -> (tile_row, tile_col).  Hardware spreads consecutive workgroups
// over the 8 XCDs; remap so consecutive logical tiles (which share rows of the
// left operand) run on the same XCD.
__device__ __forceinline__ void tile_coords(int tiles_cols, int &tr, int &tc) {
  int lid = blockIdx.x;
  const int nt = gridDim.x;
  if ((nt & 7) == 0) lid = (blockIdx.x & 7) * (nt >> 3) + (blockIdx.x >> 3);
  tr = lid / tiles_cols;
  tc = lid % tiles_cols;
}

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

// ===========================================================================
// Forward
// ===========================================================================

// Packed weight bytes of one thread's share of a tile: group g expands weight
// rows 128 g .. +127 of the tile; thread (tg = tid % 256) takes row tg / 2 and
// 32 codes (16 bytes) of half tg % 2 of the row's 64-element block.
struct FwdPack {
  uint4 p;
  uint32_t code;
  float c2;
  __device__ __forceinline__ void load(const NF4View &w, int n0, int k0) {
    const int tg = thread_in_group(), grp = wave_group();
    const int n = min(n0 + 128 * grp + (tg >> 1), w.N - 1);
    const int64_t blk = (static_cast<int64_t>(n) * w.K + k0) >> 6;
    p = *reinterpret_cast<const uint4 *>(w.packed + (blk << 5) + (tg & 1) * 16);
    code = w.code8[blk];
    c2 = w.c2[blk >> 8];
  }
  __device__ __forceinline__ void expand(uint8_t *ws, const float2 *lut2, const float *t8, float mean) const {
    const int tg = thread_in_group(), grp = wave_group();
    const int row = 128 * grp + (tg >> 1), half = tg & 1;
    const float chat = decode_absmax(t8[code], c2, mean);
    const uint32_t words[4] = {p.x, p.y, p.z, p.w};
    uint32_t o[16];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float2 l = lut2[(words[wd] >> (8 * b)) & 0xffu];
        o[wd * 4 + b] = pack_bf16x2(l.x * chat, l.y * chat);
      }
    uint4 *d = reinterpret_cast<uint4 *>(ws + row * (kWLd * 2) + half * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
};

// ===========================================================================
// dX
// ===========================================================================

// Group g expands tile columns (K) 128 g .. +127 for all 64 contraction rows
// (N).  Thread tg: weight rows 2 (tg % 32), +1 and 16 columns 16 (tg / 32) ..
// +15 (8 packed bytes per row, one block constant per row).  Written
// transposed: LDS row = K column, two adjacent N values per 32-bit word.
struct DxPack {
  uint2 p0, p1;
  uint32_t code0, code1;
  float c20, c21;
  __device__ __forceinline__ void load(const NF4View &w, int n0, int k0) {
    const int tg = thread_in_group(), grp = wave_group();
    const int n = n0 + 2 * (tg & 31);
    const int na = min(n, w.N - 1), nb = min(n + 1, w.N - 1);
    const int k = min(k0 + 128 * grp + 16 * (tg >> 5), w.K - 16);
    const int64_t e0 = static_cast<int64_t>(na) * w.K + k, e1 = static_cast<int64_t>(nb) * w.K + k;
    p0 = *reinterpret_cast<const uint2 *>(w.packed + (e0 >> 1));
    p1 = *reinterpret_cast<const uint2 *>(w.packed + (e1 >> 1));
    code0 = w.code8[e0 >> 6];
    code1 = w.code8[e1 >> 6];
    c20 = w.c2[e0 >> 14];
    c21 = w.c2[e1 >> 14];
  }
  // Rows past N must contribute zero: they multiply dY columns that are zero
  // only if the weight rows are zero too (dY past N is never loaded as data).
  __device__ __forceinline__ void expand(uint8_t *ws, const float2 *lut2, const float *t8, float mean, int n0,
                                         int N) const {
    const int tg = thread_in_group(), grp = wave_group();
    const int np = tg & 31;
    const int kl = 128 * grp + 16 * (tg >> 5);
    const float ch0 = (n0 + 2 * np < N) ? decode_absmax(t8[code0], c20, mean) : 0.f;
    const float ch1 = (n0 + 2 * np + 1 < N) ? decode_absmax(t8[code1], c21, mean) : 0.f;
    const uint32_t w0[2] = {p0.x, p0.y}, w1[2] = {p1.x, p1.y};
#pragma unroll
    for (int wd = 0; wd < 2; ++wd)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float2 la = lut2[(w0[wd] >> (8 * b)) & 0xffu];
        const float2 lb = lut2[(w1[wd] >> (8 * b)) & 0xffu];
        const uint32_t pa = pack_bf16x2(la.x * ch0, la.y * ch0);   // row n:   k, k+1
        const uint32_t pb = pack_bf16x2(lb.x * ch1, lb.y * ch1);   // row n+1: k, k+1
        const int k = kl + wd * 8 + b * 2;
        *reinterpret_cast<uint32_t *>(ws + k * (kWLd * 2) + 4 * np) = __builtin_amdgcn_perm(pb, pa, 0x05040100u);
        *reinterpret_cast<uint32_t *>(ws + (k + 1) * (kWLd * 2) + 4 * np) =
            __builtin_amdgcn_perm(pb, pa, 0x07060302u);
      }
  }
};

// A [r, K] rows j0 .. j0+63 (zero past r), columns k0 .. k0+255, transposed
// into a padded right stage as [k][j].
__device__ __forceinline__ void load_a_transposed(uint8_t *ws, const uint16_t *A, int r, int K, int j0, int k0) {
  for (int idx = threadIdx.x; idx < kBK * kBN; idx += kThreadsMM) {
    const int j = idx >> 8, k = idx & 255;
    uint16_t v = 0;
    if (j0 + j < r && k0 + k < K) v = A[static_cast<int64_t>(j0 + j) * K + k0 + k];
    *reinterpret_cast<uint16_t *>(ws + k * (kWLd * 2) + 2 * j) = v;
  }
}

// ===========================================================================
// The ping-pong main loop, shared by both kernels.
//   kDx = false: left = X [M, K] (contraction K), right = deq(W) rows.
//   kDx = true:  left = dY [M, N] (contraction N), right = deq(W)^T.
// ===========================================================================
template <bool kDx>
struct Pack;
template <>
struct Pack<false> {
  using T = FwdPack;
};
template <>
struct Pack<true> {
  using T = DxPack;
};

template <bool kDx>
__global__ __launch_bounds__(kThreadsMM) void k_matmul(const uint16_t *__restrict__ L, int M, NF4View w,
                                                       const uint16_t *__restrict__ Ln,
                                                       const uint16_t *__restrict__ Rn, int r,
                                                       uint16_t *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t sX0[kXBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sX1[kXBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sW0[kWBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sW1[kWBytes];
  __shared__ float2 sLut[256];
  __shared__ float sT8[256];
  using P = typename Pack<kDx>::T;

  const int K = w.K, N = w.N;
  const int ncols = kDx ? K : N;           // output columns
  const int Kc = kDx ? N : K;              // contraction length (multiple of 8; of 64 for the forward)
  const int ldl = kDx ? N : K;             // row stride of the left operand
  int tr, tc;
  tile_coords((ncols + kBN - 1) / kBN, tr, tc);
  const int m0 = tr * kBM, c0 = tc * kBN;
  // wave-uniform group index in an SGPR, so the group branches are scalar
  const int grp = __builtin_amdgcn_readfirstlane(wave_group());
  const float mean = w.mean[0];
  const int KT = (Kc + kBK - 1) / kBK;

  // right-operand tile origin: forward (n0 = c0, k = step), dX (n = step, k0 = c0)
  auto pack_load = [&](P &pk, int kt) {
    if (kDx)
      pk.load(w, kt * kBK, c0);
    else
      pk.load(w, c0, kt * kBK);
  };
  auto pack_expand = [&](const P &pk, uint8_t *ws, int kt) {
    if constexpr (kDx)
      pk.expand(ws, sLut, sT8, mean, kt * kBK, N);
    else
      pk.expand(ws, sLut, sT8, mean);
  };
  // In a contraction tail (dX with N % 64 != 0) the DMA cannot zero the dY
  // columns past N; their chunks are clamped to valid data and the weight rows
  // past N are expanded as exact zeros, so they contribute nothing.
  const int gw = __builtin_amdgcn_readfirstlane(wave_in_group());

  f32x16_t acc[4][2];
  zero_acc(acc);
  init_tables(sLut, sT8);

  P pk0, pk1;
  pack_load(pk0, 0);
  if (KT > 1) pack_load(pk1, 1);
  if (grp == 1) dma_left(sX0, L, ldl, m0, M, 0, Kc, gw);
  __syncthreads();                 // tables ready
  pack_expand(pk0, sW0, 0);
  if (KT > 2) pack_load(pk0, 2);
  __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
  __syncthreads();

  // Pipeline steps: multiply stage CUR, fill stage CUR ^ 1 with step kt + 1.
  // Group 1 expands its half of the next weight tile in phase 0, then issues
  // the DMA of the next left tile and its refill loads; group 0 expands its
  // half in phase 1.  The DMA has a whole phase (the other group's MFMAs) to
  // land before the end-of-step barrier.  Each group runs its own loop (the
  // barrier sequence is identical), so no register state merges across groups.
  // Refill loads always go out (clamped to the last step) to keep the register
  // flow branch-free; the extra loads near the end are never used.
  constexpr int kEndWait = kDx ? kWaitVm6Lgkm0 : kWaitVm3Lgkm0;
  // `more` (a next step exists) is a compile-time flag: the unrolled loop body
  // is branch-free, so the compiler's load-wait bookkeeping stays exact and it
  // never drains the prefetches it does not need.
  auto step0 = [&](auto cur_tag, auto more_tag, int kt, P &pk) __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_tag)::value;
    constexpr bool kMore = decltype(more_tag)::value;
    mfma_step(CUR ? sX1 : sX0, CUR ? sW1 : sW0, acc);
    raw_barrier<kWaitLgkm0>();
    if constexpr (kMore) {
      pack_expand(pk, CUR ? sW0 : sW1, min(kt + 1, KT - 1));
      pack_load(pk, min(kt + 3, KT - 1));
    }
    raw_barrier<kEndWait>();
  };
  auto step1 = [&](auto cur_tag, auto more_tag, int kt, P &pk) __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_tag)::value;
    constexpr bool kMore = decltype(more_tag)::value;
    if constexpr (kMore) {
      pack_expand(pk, CUR ? sW0 : sW1, min(kt + 1, KT - 1));
      dma_left(CUR ? sX0 : sX1, L, ldl, m0, M, min(kt + 1, KT - 1) * kBK, Kc, gw);
      // The end-of-step wait counts on the refill loads being the newest
      // memory operations of this wave: nothing may move across this point.
      __builtin_amdgcn_sched_barrier(0);
      pack_load(pk, min(kt + 3, KT - 1));
    }
    raw_barrier<kWaitLgkm0>();
    mfma_step(CUR ? sX1 : sX0, CUR ? sW1 : sW0, acc);
    raw_barrier<kEndWait>();   // this group's DMA has landed
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  // Every step of the loop prepares a next one (the step past the end expands
  // and loads a clamped, never-used tile), so the loop body has no branches.
  // An odd number of steps ends with one single step.
  const int KT2 = KT & ~1;
  if (grp == 0) {
    for (int kt = 0; kt < KT2; kt += 2) {
      step0(C0(), T_(), kt, pk1);
      step0(C1(), T_(), kt + 1, pk0);
    }
    if (KT & 1) step0(C0(), F_(), KT - 1, pk1);
  } else {
    for (int kt = 0; kt < KT2; kt += 2) {
      step1(C0(), T_(), kt, pk1);
      step1(C1(), T_(), kt + 1, pk0);
    }
    if (KT & 1) step1(C0(), F_(), KT - 1, pk1);
  }

  // LoRA steps: left = Ln [M, r] (T or G), right = B [N, r] or A^T.
  for (int j0 = 0; j0 < r; j0 += kBK) {
    load_narrow<true>(sX0, Ln, r, m0, M, j0);
    if (kDx)
      load_a_transposed(sW0, Rn, r, K, j0, c0);
    else
      load_narrow<false>(sW0, Rn, r, c0, N, j0);
    __syncthreads();
    mfma_step(sX0, sW0, acc);
    __syncthreads();
  }

  const int wave = wave_id();
  uint8_t *region = (wave < 2 ? sX0 : wave < 4 ? sX1 : wave < 6 ? sW0 : sW1) + (wave & 1) * 16384;
  store_tile(acc, region, out, ncols, m0 + wave_group() * 128, c0 + wave_in_group() * 64, M, ncols);
}

// ---------------------------------------------------------------------------
hipError_t launch_matmul_fwd(const uint16_t *X, int M, const NF4View &w, const uint16_t *T,
                             const uint16_t *B, int r, uint16_t *Y, hipStream_t s) {
  if (small_m_ok(M, r)) return launch_small_m_fwd(X, M, w, T, B, r, Y, s);
  const int tiles = ((M + kBM - 1) / kBM) * ((w.N + kBN - 1) / kBN);
  hipLaunchKernelGGL(k_matmul<false>, dim3(tiles), dim3(kThreadsMM), 0, s, X, M, w, T, B, r, Y);
  return hipGetLastError();
}

hipError_t launch_matmul_dx(const uint16_t *dY, int M, const NF4View &w, const uint16_t *G,
                            const uint16_t *A, int r, uint16_t *dX, hipStream_t s) {
  const int tiles = ((M + kBM - 1) / kBM) * ((w.K + kBN - 1) / kBN);
  hipLaunchKernelGGL(k_matmul<true>, dim3(tiles), dim3(kThreadsMM), 0, s, dY, M, w, G, A, r, dX);
  return hipGetLastError();
}

}  // namespace qlora
