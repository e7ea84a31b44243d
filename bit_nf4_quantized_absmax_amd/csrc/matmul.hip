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
// contraction over N.
//
// Design (both kernels):
//  * 256 x 256 output tile, contraction step 64, 512 threads = 8 waves, two
//    per SIMD.  Wave (wm, wn) owns the 128 x 64 block (rows 128 wm, columns
//    64 wn) as 4 x 2 MFMA 32x32x16 bf16 accumulators (fp32).
//  * Every wave multiplies and dequantizes: during step t it runs the 32
//    MFMAs of stage t while its threads expand the weight tile of step t + 1
//    into the other stage (each thread half a 64-code block: one absmax
//    constant, 32 table lookups, 4 16-byte LDS writes).  The two waves of a
//    SIMD overlap one's expansion with the other's MFMAs.  One barrier per
//    step.
//  * Expansion: each of the 16 fp32 NF4 levels sits in its own LDS bank, so the
//    64 lanes' lookups never conflict; each weight is fl32(level * c_hat)
//    rounded to bf16, as in the dequantizer.
//  * The left operand (X or dY) goes global -> LDS with 16-byte DMA loads
//    (global_load_lds_dwordx4) one step ahead; packed weight bytes, block codes
//    and group scales are prefetched two steps ahead in registers.
//  * LDS tiles are 16-byte-chunk XOR-swizzled by row so that DMA writes,
//    expansion writes and MFMA operand reads are bank-conflict free.  The
//    forward weight tile is [256 n][64 k] (read like the left operand); the
//    dX tile is [64 n][256 k], written row-wise by the expansion and read
//    column-wise with ds_read_b64_tr_b16 (within a group of 16 lanes, lane i
//    gets element i % 4 of the 8-byte reads of lanes i / 4 + 4 e, e = 0..3),
//    which yields the 8-consecutive-n operands without a transposed store.
//  * Operands of MFMA sub-step s + 1 are read while sub-step s multiplies,
//    and the last four MFMAs of a step run after its barrier, covering the
//    first operand reads of the next step.  The left-operand DMA is issued
//    from inline asm so that the compiler's LDS wait counts stay exact.
//  * Tiles are mapped so that consecutive tiles (sharing left-operand rows)
//    run on the same XCD and its L2.
//  * Epilogue: accumulators -> bf16 (round to nearest even) -> per-wave LDS
//    staging -> 16-byte global stores.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace qlora {

#define QLORA_LDS(p) ((__attribute__((address_space(3))) void *)(p))

__constant__ uint32_t cMMQ4Level[3 * 16] = {QLORA_Q4_LEVEL_BITS};
__constant__ uint32_t cMMT8Level[256] = {QLORA_T8_LEVEL_BITS};

// Operands of up to kMmGroupMax products in one launch (a single call is a
// group of one): left operand, LoRA pair, dropout mask and output per member.
constexpr int kMmGroupMax = 4;
struct MatmulArgs {
  const uint16_t *L[kMmGroupMax];
  const uint16_t *Ln[kMmGroupMax];
  const uint16_t *Rn[kMmGroupMax];
  const uint32_t *keep[kMmGroupMax];
  uint16_t *out[kMmGroupMax];
  NF4View w[kMmGroupMax];
  const uint16_t *wd[kMmGroupMax];   // dequantized bf16 weight [N, K] (k_matmul_pre; N and K from w)
  int M[kMmGroupMax];
  int r[kMmGroupMax];
  int tcols[kMmGroupMax];
  int t0[kMmGroupMax + 1];
  int n;
};

namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;                  // output rows per tile
constexpr int kBN = 256;                  // output columns per tile
constexpr int kBK = 64;                   // contraction step
constexpr int kThreadsMM = 512;
constexpr int kStageBytes = 256 * 64 * 2; // every stage holds 256 x 64 bf16

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8); vm = 63 / lgkm = 15 do not wait.
constexpr int wait_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | 0x70 | ((lgkm & 15) << 8); }

// 128-byte rows (64 bf16): chunk c of row r at 16-byte position c ^ f(r).
__device__ __forceinline__ int swz128(int row, int chunk) {
  return row * 128 + 16 * (chunk ^ ((row & 7) ^ ((row >> 3) & 1)));
}
// 512-byte rows (256 bf16): chunk c (0..31) of row r at c ^ g(r),
// g(r) = 4 (r % 4) + (r / 4) % 4 (within the chunk's half row).
__device__ __forceinline__ int swz512(int row, int chunk) {
  return row * 512 + 16 * (chunk ^ (((row & 3) << 2) | ((row >> 2) & 3)));
}

// Workgroup barrier without a memory-model fence (a fence would also wait for
// every outstanding DMA and prefetch): waits per kWait, then s_barrier.  The
// signal fences stop the compiler from moving memory accesses across it and
// the scheduling barriers keep each side its own scheduling region.
template <int kWait>
__device__ __forceinline__ void raw_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWait);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

// Left operand tile: rows m0 .. m0+255 (clamped to rows - 1: never stored)
// and columns c0 .. c0+63 (16-byte chunks clamped to the row's last chunk,
// cols % 8 == 0: finite data that meets zero weights in a contraction tail)
// of a row-major bf16 matrix with row pitch ld, DMA'd into a swizzled stage.
// Wave w issues the four 1 KB instructions of rows 32 w .. 32 w + 31; lane i
// of an instruction lands in slot i (row 8 u + i / 8, position i % 8).
__device__ __forceinline__ void dma_left(uint8_t *stage, const uint16_t *src, int64_t ld, int m0, int rows, int c0,
                                         int cols, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int u = wave * 4 + j;
    const int row = u * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row & 7) ^ ((row >> 3) & 1));
    const int grow = min(m0 + row, rows - 1);
    const int gcol = min(c0 + chunk * 8, cols - 8);
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(stage) + u * 1024);
    dma16(src + static_cast<int64_t>(grow) * ld + gcol, dst);
  }
}

// Half of a 64-code weight block: 32 packed nibbles (low nibble first), the
// block's first-level constant code and its group's second-level scale.
struct WBlock {
  uint4 p;
  uint32_t code;
  float c2;
};

// Codes 32 half .. +31 of the block W[n][k .. k+63] (n < N, k % 64 == 0, k < K).
__device__ __forceinline__ void load_block(WBlock &b, const NF4View &w, int n, int k, int half) {
  const int64_t blk = (static_cast<int64_t>(n) * w.K + k) >> 6;
  b.p = *reinterpret_cast<const uint4 *>(w.packed + (blk << 5) + 16 * half);
  b.code = w.code8[blk];
  b.c2 = w.c2[blk >> 8];
}

// NF4 level lookups from the 16-entry fp32 table: for a packed word w (8
// codes) lo4 / hi4 hold 4 x (low / high) nibble of every byte, i.e. the byte
// offsets of the levels of codes 2 b and 2 b + 1.
__device__ __forceinline__ uint32_t nf4_lo4(uint32_t w) { return (w << 2) & 0x3C3C3C3Cu; }
__device__ __forceinline__ uint32_t nf4_hi4(uint32_t w) { return (w >> 2) & 0x3C3C3C3Cu; }
__device__ __forceinline__ float nf4_level(const float *nf4, uint32_t off4, int b) {
  return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(nf4) + __builtin_amdgcn_ubfe(off4, 8 * b, 8));
}

// Chunk c (codes 8 c .. 8 c + 7 of the half block): the 8 fp32 levels, then
// 8 bf16 = fl32(level * chat).  Split so that the table reads can be issued a
// while before their products are needed.
__device__ __forceinline__ void chunk_levels(float (&lv)[8], const WBlock &b, int c, const float *nf4) {
  const uint32_t words[4] = {b.p.x, b.p.y, b.p.z, b.p.w};
  uint32_t lo4 = nf4_lo4(words[c]), hi4 = nf4_hi4(words[c]);
  asm volatile("" : "+v"(lo4), "+v"(hi4));   // keep the byte offsets: one extract per code
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    lv[2 * q] = nf4_level(nf4, lo4, q);
    lv[2 * q + 1] = nf4_level(nf4, hi4, q);
  }
}
__device__ __forceinline__ uint4 scale_chunk(const float (&lv)[8], float chat) {
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(lv[2 * q] * chat, lv[2 * q + 1] * chat);
  return make_uint4(o[0], o[1], o[2], o[3]);
}
__device__ __forceinline__ uint4 expand_chunk(const WBlock &b, int c, float chat, const float *nf4) {
  float lv[8];
  chunk_levels(lv, b, c, nf4);
  return scale_chunk(lv, chat);
}

__device__ __forceinline__ bf16x4_t ds_tr16(const uint8_t *p) {
  typedef __attribute__((address_space(3))) bf16x4_t lds_t;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_t *)((__attribute__((address_space(3))) uint8_t *)(p)));
}

// MFMA operands of one 16-wide sub-step: lane l supplies rows 32 i + l % 32
// of the wave's left block and columns 32 j + l % 32 of its right block, with
// contraction elements 8 (l / 32) .. +7 of the sub-step.
struct Frag {
  bf16x8_t a[4], b[2];
};

// Per-thread byte offsets of the operand reads (fixed for the whole kernel):
//   xo[s]     left block, sub-step s; fragment i adds 4096 i (32 rows), since
//             the row swizzle repeats every 16 rows;
//   wo[s]     forward weight block, likewise;
//   to[j][h]  dX weight tile (transposed reads), half h of fragment j;
//             sub-step s adds 8192 s (16 rows), the swizzle repeating every 16.
struct OpOffsets {
  uint32_t xo[4], wo[4], to[2][2];
};

template <bool kDx>
__device__ __forceinline__ OpOffsets op_offsets() {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int lr = lane & 31, lh = lane >> 5;
  OpOffsets o;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    o.xo[s] = static_cast<uint32_t>(swz128(128 * wm + lr, 2 * s + lh));
    o.wo[s] = static_cast<uint32_t>(swz128(64 * wn + lr, 2 * s + lh));
  }
  // [64 n][256 k] tile: group G = lane / 16 reads columns
  // 64 wn + 32 j + 16 (G % 2) .. +15, rows 8 (G / 2) + 4 h .. +3 (+ 16 s);
  // source lane t points at row t / 4, columns 4 (t % 4) .. +3.
  const int t = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      o.to[j][h] = static_cast<uint32_t>(
          swz512(8 * (g >> 1) + 4 * h + (t >> 2), 8 * wn + 4 * j + 2 * (g & 1) + ((t & 3) >> 1)) + 8 * (t & 1));
  return o;
}

template <bool kDx>
__device__ __forceinline__ void load_frag(Frag &f, const uint8_t *xs, const uint8_t *ws, const OpOffsets &o, int s) {
  // in the order the MFMAs (i major, j minor) first need them: a0 b0 b1 a1 a2 a3
  auto ld_a = [&](int i) { f.a[i] = *reinterpret_cast<const bf16x8_t *>(xs + o.xo[s] + 4096 * i); };
  auto ld_b = [&](int j) {
    if (!kDx) {
      f.b[j] = *reinterpret_cast<const bf16x8_t *>(ws + o.wo[s] + 4096 * j);
    } else {
      const bf16x4_t lo = ds_tr16(ws + o.to[j][0] + 8192 * s);
      const bf16x4_t hi = ds_tr16(ws + o.to[j][1] + 8192 * s);
      f.b[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  ld_a(0);
  ld_b(0);
  ld_b(1);
  ld_a(1);
  ld_a(2);
  ld_a(3);
}

// MFMAs of left fragments i0 .. i1 - 1 (all right fragments).
template <int i0, int i1>
__device__ __forceinline__ void mfma_rows(const Frag &f, f32x16_t (&acc)[4][2]) {
#pragma unroll
  for (int i = i0; i < i1; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}
__device__ __forceinline__ void mfma_frag(const Frag &f, f32x16_t (&acc)[4][2]) { mfma_rows<0, 4>(f, acc); }

// A whole 64-wide step without expansion (the LoRA steps).
template <bool kDx>
__device__ __forceinline__ void mfma_stage(const uint8_t *xs, const uint8_t *ws, const OpOffsets &o,
                                           f32x16_t (&acc)[4][2]) {
  Frag f[2];
  load_frag<kDx>(f[0], xs, ws, o, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < 3) load_frag<kDx>(f[(s + 1) & 1], xs, ws, o, s + 1);
    mfma_frag(f[s & 1], acc);
  }
}

// Narrow [rows, r] bf16 matrix (T, G or B), columns j0 .. j0+63 (zero past r)
// of rows row0 .. row0+255 (zero past `rows`), into a 128-byte-row stage.
__device__ __forceinline__ void load_narrow(uint8_t *stage, const uint16_t *src, int r, int row0, int rows, int j0) {
  if ((r & 7) == 0) {
    for (int idx = threadIdx.x; idx < 256 * 8; idx += kThreadsMM) {
      const int row = idx >> 3, c = idx & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row0 + row < rows && j0 + 8 * c < r)
        v = *reinterpret_cast<const uint4 *>(src + static_cast<int64_t>(row0 + row) * r + j0 + 8 * c);
      *reinterpret_cast<uint4 *>(stage + swz128(row, c)) = v;
    }
  } else {
    for (int idx = threadIdx.x; idx < 256 * 64; idx += kThreadsMM) {
      const int row = idx >> 6, j = idx & 63;
      uint16_t v = 0;
      if (row0 + row < rows && j0 + j < r) v = src[static_cast<int64_t>(row0 + row) * r + j0 + j];
      *reinterpret_cast<uint16_t *>(stage + swz128(row, j >> 3) + 2 * (j & 7)) = v;
    }
  }
}

// A [r, K] rows j0 .. j0+63 (zero past r) and columns k0 .. k0+255 (zero past
// K) into a [64 j][256 k] stage (the dX weight layout).
__device__ __forceinline__ void load_a_tile(uint8_t *stage, const uint16_t *A, int r, int K, int j0, int k0) {
  for (int idx = threadIdx.x; idx < 64 * 32; idx += kThreadsMM) {
    const int j = idx >> 5, c = idx & 31;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j0 + j < r && k0 + 8 * c < K)
      v = *reinterpret_cast<const uint4 *>(A + static_cast<int64_t>(j0 + j) * K + k0 + 8 * c);
    *reinterpret_cast<uint4 *>(stage + swz512(j, c)) = v;
  }
}

// Dequantized dX weight tile: rows n0 .. n0+63 (clamped to N - 1) and
// columns k0 .. k0+255 (16-byte chunks clamped to the row's last) of a
// row-major bf16 [N, K] matrix, DMA'd into the [64 n][256 k] swz512 layout.
// Wave w issues the 1 KB instructions 4 w .. 4 w + 3 (two 512-byte rows
// each); lane i of an instruction lands in slot i (row 2 u + i / 32,
// position i % 32).
__device__ __forceinline__ void dma_wdx(uint8_t *stage, const uint16_t *W, int N, int K, int n0, int k0, int wave,
                                        int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int u = wave * 4 + j;
    const int row = 2 * u + (lane >> 5);
    const int chunk = (lane & 31) ^ (((row & 3) << 2) | ((row >> 2) & 3));
    const int grow = min(n0 + row, N - 1);
    const int gcol = min(k0 + chunk * 8, K - 8);
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(stage) + u * 1024);
    dma16(W + static_cast<int64_t>(grow) * K + gcol, dst);
  }
}

// The LoRA contraction steps of a tile: left = Ln [M, r] (T or G), right =
// B [N, r] (forward) or A [r, K] (dX), 64 adapter columns per step.
template <bool kDx>
__device__ __forceinline__ void lora_tile_steps(uint8_t *xs, uint8_t *ws, const uint16_t *Ln, const uint16_t *Rn,
                                                int r, int M, int N, int K, int m0, int c0, const OpOffsets &ops,
                                                f32x16_t (&acc)[4][2]) {
  for (int j0 = 0; j0 < r; j0 += kBK) {
    load_narrow(xs, Ln, r, m0, M, j0);
    if (kDx)
      load_a_tile(ws, Rn, r, K, j0, c0);
    else
      load_narrow(ws, Rn, r, c0, N, j0);
    __syncthreads();
    mfma_stage<kDx>(xs, ws, ops, acc);
    __syncthreads();
  }
}

// Epilogue: the wave's 128 x 64 block as bf16 into its own 16 KB region of
// the stages (16-byte chunks XOR-swizzled by row), then 16-byte stores
// guarded by the matrix bounds (ncols % 8 == 0).  MFMA 32x32 output layout:
// lane l holds column l % 32; element e holds row 8 (e / 4) + 4 (l / 32) + e % 4.
__device__ __forceinline__ void store_tile(const f32x16_t (&acc)[4][2], uint8_t *region, uint16_t *out, int M,
                                           int ncols, int m0, int c0, int wave, int lane) {
  const int wm = wave >> 2, wnn = wave & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int cc = 32 * j + (lane & 31);
        *reinterpret_cast<uint16_t *>(region + rr * 128 + 16 * ((cc >> 3) ^ (rr & 7)) + 2 * (cc & 7)) =
            f32_to_bf16(acc[i][j][e]);
      }
  __builtin_amdgcn_s_waitcnt(wait_imm(63, 0));
#pragma unroll 4
  for (int t = 0; t < 16; ++t) {
    const int idx = t * 64 + lane;
    const int rr = idx >> 3, c = idx & 7;
    const uint4 v = *reinterpret_cast<const uint4 *>(region + rr * 128 + 16 * (c ^ (rr & 7)));
    const int gr = m0 + 128 * wm + rr, gc = c0 + 64 * wnn + 8 * c;
    if (gr < M && gc < ncols) *reinterpret_cast<uint4 *>(out + static_cast<int64_t>(gr) * ncols + gc) = v;
  }
}

// Workgroup -> (member, tile_row, tile_col).  Hardware spreads consecutive
// workgroups over the 8 XCDs; remap so consecutive logical tiles (which share
// rows of the left operand) run on the same XCD.  Member j of a grouped launch
// owns logical tiles [t0[j], t0[j + 1]), row-major over its own tile grid.
// kBand > 1: within a member, tiles go in bands of kBand tile rows, each band
// column by column, so that the ~32 consecutive tiles one XCD runs at a time
// form a kBand x (32 / kBand) block that shares left-operand rows and weight
// columns in that XCD's L2 (the last band may be shorter).
template <int kBand = 1>
__device__ __forceinline__ int tile_coords(const MatmulArgs &a, int &tr, int &tc) {
  int lid = blockIdx.x;
  const int nt = gridDim.x;
  if ((nt & 7) == 0) lid = (blockIdx.x & 7) * (nt >> 3) + (blockIdx.x >> 3);
  int m = 0;
#pragma unroll
  for (int j = 1; j < kMmGroupMax; ++j) m = (j < a.n && lid >= a.t0[j]) ? j : m;
  const int local = lid - a.t0[m];
  const int tcols = a.tcols[m];
  if (kBand == 1) {
    tr = local / tcols;
    tc = local % tcols;
  } else {
    const int trows = (a.t0[m + 1] - a.t0[m]) / tcols;
    const int band = local / (kBand * tcols);
    const int h = min(kBand, trows - band * kBand);   // rows in this band
    const int j = local - band * kBand * tcols;
    tc = j / h;
    tr = band * kBand + j % h;
  }
  return m;
}

}  // namespace

// kDx = false: left = X [M, K] (contraction K), weight tile [256 n][64 k].
// kDx = true:  left = dY [M, N] (contraction N), weight tile [64 n][256 k].
// kDrop (dX only): the LoRA term is gated by the dropout keep mask of the
// LoRA input, dX = dY deq(W) + (G A) * keep (keep: bit k % 32 of word
// [m][k / 32]); the LoRA steps then run first, the mask zeroes their dropped
// elements in the accumulators, and the base contraction follows.
template <bool kDx, bool kDrop>
__global__ __launch_bounds__(kThreadsMM) void k_matmul(const MatmulArgs args) {
  __shared__ __attribute__((aligned(16))) uint8_t sX0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sX1[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sW0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sW1[kStageBytes];
  __shared__ __attribute__((aligned(64))) float sNf4[16];
  __shared__ float sT8[256];

  int tr, tc;
  const int mem = tile_coords(args, tr, tc);
  const uint16_t *__restrict__ L = args.L[mem];
  const uint16_t *__restrict__ Ln = args.Ln[mem];
  const uint16_t *__restrict__ Rn = args.Rn[mem];
  const uint32_t *__restrict__ keep = args.keep[mem];
  uint16_t *__restrict__ out = args.out[mem];
  const NF4View w = args.w[mem];
  const int M = args.M[mem], r = args.r[mem];
  const int K = w.K, N = w.N;
  const int ncols = kDx ? K : N;           // output columns
  const int Kc = kDx ? N : K;              // contraction length (multiple of 8; of 64 for the forward)
  const int m0 = tr * kBM, c0 = tc * kBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float mean = w.mean[0];
  const int KT = (Kc + kBK - 1) / kBK;

  // This thread's half block in contraction step kt (half = tid % 2):
  //   forward: row n = c0 + tid / 2 (an output column), k = 64 kt
  //   dX:      row n = 64 kt + trow (a contraction index), k = c0 + 64 tkb,
  //            lane bits (half, tkb % 2, row / 4 % 4, row % 4) and wave bits
  //            (row / 16, tkb / 2): each 16-lane cycle of an expansion write
  //            covers rows r, r + 4, r + 8, r + 12 and the four (tkb % 2,
  //            half) pairs, which the [64][256] swizzle maps to 16 distinct
  //            4-bank groups (no bank conflicts).
  // Neighbouring lanes read neighbouring bytes of a row (the two halves of a
  // block, and in dX two neighbouring blocks: 64 contiguous bytes), so a load
  // instruction touches few cache lines.  Rows past N (dX contraction tail)
  // expand to exact zeros; columns past the matrix are clamped (never stored).
  const int half = tid & 1;
  const int trow = kDx ? (((lane >> 4) & 3) + 4 * ((lane >> 2) & 3) + 16 * (wave & 3)) : (tid >> 1);
  const int tkb = kDx ? (((lane >> 1) & 1) + 2 * ((wave >> 2) & 1)) : 0;   // block within the tile row (dX)
  auto block_load = [&](WBlock &b, int kt) __attribute__((always_inline)) {
    if (kDx)
      load_block(b, w, min(kBK * kt + trow, N - 1), min(c0 + 64 * tkb, K - 64), half);
    else
      load_block(b, w, min(c0 + trow, N - 1), kBK * kt, half);
  };
  auto block_chat = [&](const WBlock &b, int kt) __attribute__((always_inline)) {
    const float c = decode_absmax(sT8[b.code], b.c2, mean);
    return (kDx && kBK * kt + trow >= N) ? 0.f : c;
  };
  auto put_chunk = [&](uint8_t *ws, int c, uint4 v) __attribute__((always_inline)) {
    if (kDx)
      *reinterpret_cast<uint4 *>(ws + swz512(trow, 8 * tkb + 4 * half + c)) = v;
    else
      *reinterpret_cast<uint4 *>(ws + swz128(trow, 4 * half + c)) = v;
  };

  const OpOffsets ops = op_offsets<kDx>();
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto lora_steps = [&]() __attribute__((always_inline)) {
    lora_tile_steps<kDx>(sX0, sW0, Ln, Rn, r, M, N, K, m0, c0, ops, acc);
  };
  if constexpr (kDrop) {
    lora_steps();
    // Accumulator (i, j, e) of this lane: row 128 wm + 32 i + 8 (e / 4) +
    // 4 (lane / 32) + e % 4, column 64 wn + 32 j + lane % 32 of the tile; the
    // two column blocks' mask words are adjacent (K % 64 == 0).
    const int wm = wave >> 2, wnn = wave & 3;
    const int kw = K >> 5;
    const int cw = (c0 + 64 * wnn) >> 5;
    if (cw < kw) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + 128 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          const uint2 kb = row < M ? *reinterpret_cast<const uint2 *>(keep + static_cast<int64_t>(row) * kw + cw)
                                   : make_uint2(0u, 0u);
          if (!((kb.x >> (lane & 31)) & 1u)) acc[i][0][e] = 0.f;
          if (!((kb.y >> (lane & 31)) & 1u)) acc[i][1][e] = 0.f;
        }
    }
  }

  for (int i = tid; i < 256; i += kThreadsMM) {
    if (i < 16) sNf4[i] = u2f(cMMQ4Level[16 * w.qtype + i]);
    sT8[i] = u2f(cMMT8Level[i]);
  }

  // Prologue: block of step 0 expanded into stage 0, left tile 0 DMA'd, the
  // block of step 1 in flight.
  WBlock b0, b1;
  block_load(b0, 0);
  block_load(b1, min(1, KT - 1));
  dma_left(sX0, L, Kc, m0, M, 0, Kc, wave, lane);
  __syncthreads();   // tables
  {
    const float chat = block_chat(b0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) put_chunk(sW0, c, expand_chunk(b0, c, chat, sNf4));
  }
  raw_barrier<wait_imm(0, 0)>();

  // Step kt multiplies stage CUR while expanding the block of kt + 1 (loaded a
  // step ago) into the other weight stage, DMAs the left tile of kt + 1 into
  // the other left stage and loads the block of kt + 2 into the registers
  // freed by step kt - 1.  The end-of-step barrier waits for all of this
  // wave's memory operations: the vector-memory counter is only relied on to
  // retire LDS DMAs in order among themselves, not against the register
  // loads issued after them (a partial count there let a DMA still be in
  // flight at the barrier).  Software
  // pipelined so that every wave always has MFMAs ready to issue:
  //  * head: operands of sub-step 0, the block's absmax code and the levels
  //    of chunk 0 are read while the last four MFMAs of the previous step
  //    (held back from before the barrier, their operands in registers) run;
  //  * sub-step s: two MFMAs, then the levels of chunk s + 1 (one sub-step
  //    ahead, so their LDS latency is hidden) and the operands of sub-step
  //    s + 1 are read, two more MFMAs, then chunk s is scaled and written
  //    while the last four MFMAs run.
  Frag fa, fb;   // operands of the even / odd sub-steps
#pragma unroll
  for (int i = 0; i < 4; ++i) fb.a[i] = bf16x8_t{};
#pragma unroll
  for (int j = 0; j < 2; ++j) fb.b[j] = bf16x8_t{};
  auto step = [&](auto cur_tag, int kt, WBlock &bn, WBlock &bl) __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_tag)::value;
    const uint8_t *xs = CUR ? sX1 : sX0;
    const uint8_t *wr = CUR ? sW1 : sW0;
    uint8_t *xn = CUR ? sX0 : sX1;
    uint8_t *wn = CUR ? sW0 : sW1;
    float lv[2][8];   // levels of chunk s in lv[s & 1], read one sub-step ahead
    load_frag<kDx>(fa, xs, wr, ops, 0);
    const float t8 = sT8[bn.code];
    chunk_levels(lv[0], bn, 0, sNf4);
    // First use of the whole block of kt + 1 before any newer load is issued:
    // the wait for it then covers only loads issued a step ago.
    asm volatile("" ::"v"(bn.p.x), "v"(bn.p.y), "v"(bn.p.z), "v"(bn.p.w), "v"(bn.c2));
    __builtin_amdgcn_sched_barrier(0);
    mfma_rows<2, 3>(fb, acc);
    dma_left(xn, L, Kc, m0, M, min(kt + 1, KT - 1) * kBK, Kc, wave, lane);
    __builtin_amdgcn_sched_barrier(0);
    mfma_rows<3, 4>(fb, acc);
    block_load(bl, min(kt + 2, KT - 1));
    __builtin_amdgcn_sched_barrier(0);
    const float c = decode_absmax(t8, bn.c2, mean);
    const float chat = (kDx && kBK * (kt + 1) + trow >= N) ? 0.f : c;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      Frag &cur = (s & 1) ? fb : fa;
      Frag &nxt = (s & 1) ? fa : fb;
      mfma_rows<0, 1>(cur, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (s < 3) chunk_levels(lv[(s + 1) & 1], bn, s + 1, sNf4);
      if (s < 3) load_frag<kDx>(nxt, xs, wr, ops, s + 1);
      mfma_rows<1, 2>(cur, acc);
      __builtin_amdgcn_sched_barrier(0);
      put_chunk(wn, s, scale_chunk(lv[s & 1], chat));
      if (s < 3) mfma_rows<2, 4>(cur, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    raw_barrier<wait_imm(0, 0)>();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  int kt = 0;
  for (; kt + 2 <= KT; kt += 2) {
    step(C0(), kt, b1, b0);
    step(C1(), kt + 1, b0, b1);
  }
  if (kt < KT) step(C0(), kt, b1, b0);
  mfma_rows<2, 4>(fb, acc);   // held back by the last step

  if constexpr (!kDrop) lora_steps();

  uint8_t *region = (wave < 2 ? sX0 : wave < 4 ? sX1 : wave < 6 ? sW0 : sW1) + (wave & 1) * 16384;
  store_tile(acc, region, out, M, ncols, m0, c0, wave, lane);
}

// Tile rows per band of the pre-dequantized kernels' tile order.  Their bf16
// weight tiles are 4x the packed bytes, so an XCD's concurrent tiles should
// share weight columns as well as left-operand rows: bands of 4 rows (4 x 8
// tiles at a time) measured 1-2 % faster than row-major order on the 7B
// layer (2 and 8: in between).
constexpr int kPreBand = 4;

// ---------------------------------------------------------------------------
// The same products with the weight already dequantized: wd is the bf16
// [N, K] matrix that the codec's dequantizer writes, bit for bit the values
// the fused kernel expands, so the outputs are identical to k_matmul's.  The
// weight tile is DMA'd like the left operand (the forward tile [256 n][64 k]
// in the left operand's layout, the dX tile [64 n][256 k] in the layout the
// transposed operand reads expect) one step ahead, and every wave only
// multiplies: no table reads, scaling or expansion writes in the loop.  The
// dX contraction (over N) has no zero-padded tail here: N % 64 == 0.
template <bool kDx, bool kPipe>
__global__ __launch_bounds__(kThreadsMM) void k_matmul_pre(const MatmulArgs args) {
  __shared__ __attribute__((aligned(16))) uint8_t sX0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sX1[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sW0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sW1[kStageBytes];

  int tr, tc;
  const int mem = tile_coords<kPreBand>(args, tr, tc);
  const uint16_t *__restrict__ L = args.L[mem];
  const uint16_t *__restrict__ Ln = args.Ln[mem];
  const uint16_t *__restrict__ Rn = args.Rn[mem];
  uint16_t *__restrict__ out = args.out[mem];
  const uint16_t *__restrict__ Wd = args.wd[mem];
  const int M = args.M[mem], r = args.r[mem];
  const int K = args.w[mem].K, N = args.w[mem].N;
  const int ncols = kDx ? K : N;
  const int Kc = kDx ? N : K;
  const int m0 = tr * kBM, c0 = tc * kBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KT = Kc / kBK;
  // kPipe (every member has r == 64 and an even step count): the LoRA step
  // is one more step of the same pipeline.  T or G [M, 64] and B [N, 64]
  // have the left operand's 128-byte row layout and A [64, K] the dX weight
  // tile's, so the last contraction step DMAs them like the next tile (no
  // zero padding: j < r throughout).  Otherwise the LoRA tiles are staged
  // after the loop.
  auto dma_x = [&](uint8_t *xs, int kt) __attribute__((always_inline)) {
    dma_left(xs, L, Kc, m0, M, kBK * kt, Kc, wave, lane);
  };
  auto dma_w = [&](uint8_t *ws, int kt) __attribute__((always_inline)) {
    if (kDx)
      dma_wdx(ws, Wd, N, K, kBK * kt, c0, wave, lane);
    else
      dma_left(ws, Wd, K, c0, N, kBK * kt, K, wave, lane);
  };
  auto dma_lora = [&](uint8_t *xs, uint8_t *ws) __attribute__((always_inline)) {
    dma_left(xs, Ln, r, m0, M, 0, r, wave, lane);
    if (kDx)
      dma_wdx(ws, Rn, r, K, 0, c0, wave, lane);
    else
      dma_left(ws, Rn, r, c0, N, 0, r, wave, lane);
  };

  const OpOffsets ops = op_offsets<kDx>();
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  dma_x(sX0, 0);
  dma_w(sW0, 0);
  raw_barrier<wait_imm(0, 0)>();

  // Step kt multiplies stage CUR while both tiles of kt + 1 are DMA'd into
  // the other stages; the end-of-step barrier waits for them.  As in the
  // fused kernel, the operands of sub-step s + 1 are read while sub-step s
  // multiplies and the last four MFMAs of a step run after its barrier.
  Frag fa, fb;
#pragma unroll
  for (int i = 0; i < 4; ++i) fb.a[i] = bf16x8_t{};
#pragma unroll
  for (int j = 0; j < 2; ++j) fb.b[j] = bf16x8_t{};
  // kMode 0: DMA step kt + 1 (clamped to the last step); 1: DMA the LoRA
  // tiles (the last contraction step of kPipe); 2: no DMA.
  auto step = [&](auto cur_tag, auto mode_tag, int kt) __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_tag)::value;
    constexpr int kMode = decltype(mode_tag)::value;
    const uint8_t *xs = CUR ? sX1 : sX0;
    const uint8_t *wr = CUR ? sW1 : sW0;
    uint8_t *xn = CUR ? sX0 : sX1;
    uint8_t *wn = CUR ? sW0 : sW1;
    load_frag<kDx>(fa, xs, wr, ops, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_rows<2, 3>(fb, acc);
    if (kMode == 0) dma_x(xn, min(kt + 1, KT - 1));
    if (kMode == 1) dma_lora(xn, wn);
    __builtin_amdgcn_sched_barrier(0);
    mfma_rows<3, 4>(fb, acc);
    if (kMode == 0) dma_w(wn, min(kt + 1, KT - 1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      Frag &cur = (s & 1) ? fb : fa;
      Frag &nxt = (s & 1) ? fa : fb;
      mfma_rows<0, 1>(cur, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (s < 3) load_frag<kDx>(nxt, xs, wr, ops, s + 1);
      mfma_rows<1, 2>(cur, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (s < 3) mfma_rows<2, 4>(cur, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    raw_barrier<wait_imm(0, 0)>();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  int kt = 0;
  if constexpr (kPipe) {
    for (; kt + 2 < KT; kt += 2) {
      step(C0(), C0(), kt);
      step(C1(), C0(), kt + 1);
    }
    step(C0(), C0(), KT - 2);
    step(C1(), C1(), KT - 1);
    step(C0(), C2(), KT);
    mfma_rows<2, 4>(fb, acc);   // held back by the last step
  } else {
    for (; kt + 2 <= KT; kt += 2) {
      step(C0(), C0(), kt);
      step(C1(), C0(), kt + 1);
    }
    if (kt < KT) step(C0(), C0(), kt);
    mfma_rows<2, 4>(fb, acc);   // held back by the last step
    lora_tile_steps<kDx>(sX0, sW0, Ln, Rn, r, M, N, K, m0, c0, ops, acc);
  }
  uint8_t *region = (wave < 2 ? sX0 : wave < 4 ? sX1 : wave < 6 ? sW0 : sW1) + (wave & 1) * 16384;
  store_tile(acc, region, out, M, ncols, m0, c0, wave, lane);
}

// ---------------------------------------------------------------------------
// A group of products of one kind (forward or dX, with or without the mask):
// one launch over the concatenated tile grids.
template <bool kDx, bool kDrop>
static hipError_t launch_mm_group(int count, const MatmulJob *jobs, hipStream_t s) {
  if (count < 1 || count > kMmGroupMax) return hipErrorInvalidValue;
  MatmulArgs a{};
  a.n = count;
  int tiles = 0;
  for (int j = 0; j < count; ++j) {
    const MatmulJob &jb = jobs[j];
    const int ncols = kDx ? jb.w.K : jb.w.N;
    a.L[j] = jb.L;
    a.Ln[j] = jb.Ln;
    a.Rn[j] = jb.Rn;
    a.keep[j] = jb.keep;
    a.out[j] = jb.out;
    a.w[j] = jb.w;
    a.M[j] = jb.M;
    a.r[j] = jb.r;
    a.tcols[j] = (ncols + kBN - 1) / kBN;
    a.t0[j] = tiles;
    tiles += ((jb.M + kBM - 1) / kBM) * a.tcols[j];
  }
  a.t0[count] = tiles;
  hipLaunchKernelGGL((k_matmul<kDx, kDrop>), dim3(tiles), dim3(kThreadsMM), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_matmul_fwd_group(int count, const MatmulJob *jobs, hipStream_t s) {
  return launch_mm_group<false, false>(count, jobs, s);
}

// Products with dequantized weights (MatmulJob::wd set, w.N / w.K the shape).
template <bool kDx>
static hipError_t launch_pre_group(int count, const MatmulJob *jobs, hipStream_t s) {
  if (count < 1 || count > kMmGroupMax) return hipErrorInvalidValue;
  MatmulArgs a{};
  a.n = count;
  int tiles = 0;
  for (int j = 0; j < count; ++j) {
    const MatmulJob &jb = jobs[j];
    const int ncols = kDx ? jb.w.K : jb.w.N;
    a.L[j] = jb.L;
    a.Ln[j] = jb.Ln;
    a.Rn[j] = jb.Rn;
    a.out[j] = jb.out;
    a.w[j] = jb.w;
    a.wd[j] = jb.wd;
    a.M[j] = jb.M;
    a.r[j] = jb.r;
    a.tcols[j] = (ncols + kBN - 1) / kBN;
    a.t0[j] = tiles;
    tiles += ((jb.M + kBM - 1) / kBM) * a.tcols[j];
  }
  a.t0[count] = tiles;
  if (tiles == 0) return hipSuccess;
  bool pipe = true;
  for (int j = 0; j < count; ++j) pipe = pipe && jobs[j].r == kBK && ((kDx ? jobs[j].w.N : jobs[j].w.K) / kBK) % 2 == 0;
  if (pipe)
    hipLaunchKernelGGL((k_matmul_pre<kDx, true>), dim3(tiles), dim3(kThreadsMM), 0, s, a);
  else
    hipLaunchKernelGGL((k_matmul_pre<kDx, false>), dim3(tiles), dim3(kThreadsMM), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pre_matmul_fwd_group(int count, const MatmulJob *jobs, hipStream_t s) {
  return launch_pre_group<false>(count, jobs, s);
}

hipError_t launch_pre_matmul_dx(const MatmulJob &job, hipStream_t s) { return launch_pre_group<true>(1, &job, s); }

hipError_t launch_matmul_fwd(const uint16_t *X, int M, const NF4View &w, const uint16_t *T,
                             const uint16_t *B, int r, uint16_t *Y, hipStream_t s) {
  if (small_m_ok(M, r)) return launch_small_m_fwd(X, M, w, T, B, r, Y, s);
  const MatmulJob job{X, T, B, nullptr, Y, w, M, r};
  return launch_mm_group<false, false>(1, &job, s);
}

hipError_t launch_matmul_dx(const uint16_t *dY, int M, const NF4View &w, const uint16_t *G,
                            const uint16_t *A, int r, uint16_t *dX, hipStream_t s) {
  const MatmulJob job{dY, G, A, nullptr, dX, w, M, r};
  return launch_mm_group<true, false>(1, &job, s);
}

hipError_t launch_matmul_dx_drop(const uint16_t *dY, int M, const NF4View &w, const uint16_t *G,
                                 const uint16_t *A, int r, const uint32_t *keep, uint16_t *dX, hipStream_t s) {
  const MatmulJob job{dY, G, A, keep, dX, w, M, r};
  return launch_mm_group<true, true>(1, &job, s);
}

}  // namespace qlora
