// LoRA branch products on gfx950 bf16 MFMA (fp32 accumulation).
//
// The adapters are "a pair of small low-rank matrices per layer" trained in
// 16-bit while the base stays frozen (automatone.win, "QLoRA paper
// explained", The problem and How it works; creativeworksofknowledge.com,
// "QLoRA: Fine-Tune 70B on One GPU", Code: r, lora_alpha).  With A [r, K],
// B [N, r] and s = alpha / r:
//   k_lora_nt   T = s X A^T  [M, r]   contraction over K (A rows read as is)
//               G = s dY B   [M, r]   contraction over N (B read transposed)
//   k_lora_tn   dA = G^T X   [r, K]   contraction over M (both read transposed)
//               dB = dY^T T  [N, r]
//   k_sum_partials   fixed-order sum of the M-split partials of k_lora_tn
//   k_lora_nt_shared, k_lora_tn_shared   T and dA of several linears that
//               read the same X (q / k / v, gate / up), one launch each; the
//               tiles are those of k_lora_nt / k_lora_tn, so the results are
//               bit-identical
// G and T carry the scale, which is applied once, in fp32, before T and G are
// rounded to bf16.  These are streaming products: each reads its wide operand
// (X or dY) once from HBM.
//
// Common design (both products):
//  * Operand tiles go global -> LDS with 16-byte DMA loads
//    (global_load_lds_dwordx4), eight 128-byte rows (1 KB) per instruction,
//    16-byte chunks XOR-swizzled by row.  Every wave owns a private ring of
//    stages in LDS and keeps several stages in flight; waves take interleaved
//    stages of the contraction and are summed in LDS in wave order at the end
//    (deterministic).  There is no barrier in the main loop.
//  * MFMA operands are read from LDS by inline-asm blocks that also wait for
//    their own data: the compiler then sees no LDS read of DMA-written memory,
//    which it would otherwise guard with conservative vmcnt(0) waits; the
//    waits on the DMA stream (vmcnt, in issue order) are explicit.
//  * A contraction-major operand (B [N, r], X, dY, G, T with the contraction
//    over rows) is read with ds_read_b64_tr_b16: within each group of 16
//    lanes, lane i receives element i % 4 of the 8-byte reads of lanes
//    i / 4 + 4 e (e = 0..3).  Pointing source lane t at row t / 4 and columns
//    4 (t % 4) .. +3 of a 4 x 16 block hands lane i column i of that block, 4
//    consecutive rows: two such reads make one MFMA operand of 8 consecutive
//    contraction indices, with no transpose pass through memory.
//  * Each workgroup starts its walk over the contraction at a different
//    stage, so that concurrent workgroups do not all read the same column band
//    of row-major operands whose row pitch is a power of two (which
//    concentrates the traffic on a few HBM channels).
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace qlora {

#define QLORA_LORA_LDS(p) ((__attribute__((address_space(3))) void *)(p))

namespace {

constexpr int kLoWaves = 4;     // waves per workgroup, one per SIMD
constexpr int kLoThreads = kLoWaves * 64;

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// s_waitcnt immediate (gfx9 encoding) for vmcnt(n), other counters not waited.
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// Tiles have 128-byte rows (64 bf16); chunk c of row `row` is stored at
// 16-byte position c ^ swz_f(row).
__device__ __forceinline__ int swz_f(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + 16 * (chunk ^ swz_f(row)); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t *)(p)));
}

// DMA rows row0 .. row0 + kRows - 1 and columns col0 .. col0 + 63 of a bf16
// matrix (row pitch ld elements, 16-byte aligned rows) into a swizzled tile.
// Rows past nrows are clamped to row nrows - 1 and chunks past ncols to the
// row's last chunk (ncols % 8 == 0): finite data that the kernels mask or
// never store.  Lane i of instruction u lands in slot i: row 8 u + i / 8,
// position i % 8, i.e. logical chunk (i % 8) ^ swz_f(row).
template <int kRows>
__device__ __forceinline__ void dma_tile(uint8_t *dst, const uint16_t *src, int64_t ld, int row0, int nrows,
                                         int col0, int ncols, int lane) {
#pragma unroll
  for (int u = 0; u < kRows / 8; ++u) {
    const int row = 8 * u + (lane >> 3);
    const int chunk = (lane & 7) ^ swz_f(row);
    const int grow = min(row0 + row, nrows - 1);
    const int gcol = min(col0 + 8 * chunk, ncols - 8);
    __builtin_amdgcn_global_load_lds(src + static_cast<int64_t>(grow) * ld + gcol, QLORA_LORA_LDS(dst + u * 1024),
                                     16, 0, 0);
  }
}

// Byte offset, within a swizzled tile, of this lane's transposed-read source
// for column block cb (32 columns) and half h of a 16-row sub-step (the
// sub-step adds 2048 bytes): group G = lane / 16 covers columns
// 32 cb + 16 (G % 2) .. +15 and rows 8 (G / 2) + 4 h .. +3; source lane
// t = lane % 16 points at row t / 4 of those and columns 4 (t % 4) .. +3.
__device__ __forceinline__ uint32_t tr_offset(int lane, int cb, int h) {
  const int t = lane & 15, g = lane >> 4;
  const int row = 8 * (g >> 1) + 4 * h + (t >> 2);
  const int chunk = 4 * cb + 2 * (g & 1) + ((t & 3) >> 1);
  return static_cast<uint32_t>(swz(row, chunk) + 8 * (t & 1));
}

__device__ __forceinline__ bf16x8_t join_tr(u32x2_t lo, u32x2_t hi) {
  uint4 v = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return __builtin_bit_cast(bf16x8_t, v);
}

// Zero the elements of an 8-element operand whose contraction index
// (first + q, q = 0..7) is >= limit.
__device__ __forceinline__ bf16x8_t mask_tail(bf16x8_t v, int first, int limit) {
  uint4 u = __builtin_bit_cast(uint4, v);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo = (first + 2 * q < limit) ? 0x0000FFFFu : 0u;
    const uint32_t hi = (first + 2 * q + 1 < limit) ? 0xFFFF0000u : 0u;
    w[q] &= lo | hi;
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
}

// ===========================================================================
// k_lora_nt: out[m][j0 + j] = scale sum_k L[m][k] R(j, k), j < 64.
//   kRT = false: R(j, k) = R[j][k]  (A [r, K]: 16-byte operand reads)
//   kRT = true:  R(j, k) = R[k][j]  (B [N, r]: transposed reads)
// Workgroup: 32 rows of L; wave w takes the 64-wide contraction stages
// w, w + 4, ... (rotated per workgroup).  Stage = L tile [32 m][64 k] (4 KB)
// + R tile (8 KB: [64 j][64 k] or [64 k][64 j]).  MFMA 32x32x16: lane l
// supplies row l % 32 of the L tile and column l % 32 (+ 32 jb) of the R side
// with contraction elements 8 (l / 32) .. +7 of each 16-wide sub-step.
// ===========================================================================
constexpr int kNtRows = 32;
constexpr int kNtSlots = 3;
constexpr int kNtLB = kNtRows * 128;          // L tile bytes
constexpr int kNtRB = 64 * 128;               // R tile bytes
constexpr int kNtStage = kNtLB + kNtRB;
constexpr int kNtDma = kNtRows / 8 + 8;       // DMA instructions per stage

template <bool kRT>
struct NtStage {
  bf16x8_t a[4], b0[4], b1[4];
};

// Operand reads of one stage at byte offset kOff of the wave's ring.
// vo[s]: this lane's offset of sub-step s in an L tile (rows l % 32);
// vt[jb][h]: transposed-read offsets in an R tile.
template <int kOff>
__device__ __forceinline__ void nt_read(const uint32_t (&vo)[4], const uint32_t (&vt)[2][2], NtStage<false> &st) {
  asm volatile(
      "ds_read_b128 %0, %12 offset:%16\n\t"
      "ds_read_b128 %1, %12 offset:%17\n\t"
      "ds_read_b128 %2, %12 offset:%18\n\t"
      "ds_read_b128 %3, %13 offset:%16\n\t"
      "ds_read_b128 %4, %13 offset:%17\n\t"
      "ds_read_b128 %5, %13 offset:%18\n\t"
      "ds_read_b128 %6, %14 offset:%16\n\t"
      "ds_read_b128 %7, %14 offset:%17\n\t"
      "ds_read_b128 %8, %14 offset:%18\n\t"
      "ds_read_b128 %9, %15 offset:%16\n\t"
      "ds_read_b128 %10, %15 offset:%17\n\t"
      "ds_read_b128 %11, %15 offset:%18\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(st.a[0]), "=&v"(st.b0[0]), "=&v"(st.b1[0]), "=&v"(st.a[1]), "=&v"(st.b0[1]), "=&v"(st.b1[1]),
        "=&v"(st.a[2]), "=&v"(st.b0[2]), "=&v"(st.b1[2]), "=&v"(st.a[3]), "=&v"(st.b0[3]), "=&v"(st.b1[3])
      : "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "n"(kOff), "n"(kOff + kNtLB), "n"(kOff + kNtLB + 4096)
      : "memory");
  (void)vt;
}

template <int kOff, int kS0>
__device__ __forceinline__ void nt_read_tr_half(const uint32_t (&vo)[4], const uint32_t (&vt)[2][2],
                                                NtStage<true> &st) {
  u32x2_t t[2][2][2];   // [sub-step][jb][h]
  asm volatile(
      "ds_read_b128 %0, %10 offset:%16\n\t"
      "ds_read_b128 %1, %11 offset:%16\n\t"
      "ds_read_b64_tr_b16 %2, %12 offset:%17\n\t"
      "ds_read_b64_tr_b16 %3, %13 offset:%17\n\t"
      "ds_read_b64_tr_b16 %4, %14 offset:%17\n\t"
      "ds_read_b64_tr_b16 %5, %15 offset:%17\n\t"
      "ds_read_b64_tr_b16 %6, %12 offset:%18\n\t"
      "ds_read_b64_tr_b16 %7, %13 offset:%18\n\t"
      "ds_read_b64_tr_b16 %8, %14 offset:%18\n\t"
      "ds_read_b64_tr_b16 %9, %15 offset:%18\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(st.a[kS0]), "=&v"(st.a[kS0 + 1]), "=&v"(t[0][0][0]), "=&v"(t[0][0][1]), "=&v"(t[0][1][0]),
        "=&v"(t[0][1][1]), "=&v"(t[1][0][0]), "=&v"(t[1][0][1]), "=&v"(t[1][1][0]), "=&v"(t[1][1][1])
      : "v"(vo[kS0]), "v"(vo[kS0 + 1]), "v"(vt[0][0]), "v"(vt[0][1]), "v"(vt[1][0]), "v"(vt[1][1]), "n"(kOff),
        "n"(kOff + kNtLB + 2048 * kS0), "n"(kOff + kNtLB + 2048 * (kS0 + 1))
      : "memory");
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    st.b0[kS0 + s] = join_tr(t[s][0][0], t[s][0][1]);
    st.b1[kS0 + s] = join_tr(t[s][1][0], t[s][1][1]);
  }
}

template <int kOff>
__device__ __forceinline__ void nt_read(const uint32_t (&vo)[4], const uint32_t (&vt)[2][2], NtStage<true> &st) {
  nt_read_tr_half<kOff, 0>(vo, vt, st);
  nt_read_tr_half<kOff, 2>(vo, vt, st);
}

// One workgroup's tile: rows 32 mt .. +31 of L, output columns j0 .. j0 + 63.
// The walk over the contraction starts at stage mt % (stages), so a tile's
// summation order depends only on mt.
template <bool kRT>
__device__ __forceinline__ void lora_nt_tile(uint8_t (&smem)[kLoWaves][kNtSlots][kNtStage],
                                             const uint16_t *__restrict__ L, int M, int Kc,
                                             const uint16_t *__restrict__ R, int rcols, int r, float scale,
                                             uint16_t *__restrict__ out, int mt, int j0) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = mt * kNtRows;
  const int nst = (Kc + 63) / 64;
  const int n_i = nst > wave ? (nst - wave + kLoWaves - 1) / kLoWaves : 0;
  const int rot = static_cast<int>(static_cast<unsigned>(mt) % static_cast<unsigned>(nst));
  // contraction offset of this wave's i-th stage (rotated, always < Kc for i < n_i)
  auto kof = [&](int i) {
    int t = wave + kLoWaves * i + rot;
    if (t >= nst) t -= nst;
    return t * 64;
  };
  uint8_t *ring = smem[wave][0];
  auto issue = [&](int i, int slot) {
    uint8_t *st = ring + slot * kNtStage;
    const int k0 = kof(i);
    dma_tile<kNtRows>(st, L, Kc, m0, M, k0, Kc, lane);
    if (kRT)
      dma_tile<64>(st + kNtLB, R, rcols, k0, Kc, j0, rcols, lane);   // rows k, columns j
    else
      dma_tile<64>(st + kNtLB, R, Kc, j0, rcols, k0, Kc, lane);      // rows j (rcols = rows of A), columns k
  };

  const uint32_t base = lds_addr(ring);
  const int lr = lane & 31, lh = lane >> 5;
  uint32_t vo[4], vt[2][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) vo[s] = base + static_cast<uint32_t>(swz(lr, 2 * s + lh));
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int h = 0; h < 2; ++h) vt[jb][h] = base + tr_offset(lane, jb, h);

  f32x16_t acc[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    acc[0][e] = 0.f;
    acc[1][e] = 0.f;
  }
  auto compute = [&](int k0, const NtStage<kRT> &st) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8_t x = (k0 + 8 * (2 * s + lh) < Kc) ? st.a[s] : bf16x8_t{};
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, st.b0[s], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, st.b1[s], acc[1], 0, 0, 0);
    }
  };
  // Stage i: issue stage i + 2 (if any), wait until stage i has landed (the
  // younger stages, issued after it, may still be in flight), read, multiply.
  auto wait_for = [&](int i) {
    const int younger = min(n_i - 1 - i, 2);
    if (younger >= 2)
      __builtin_amdgcn_s_waitcnt(vm_wait(2 * kNtDma));
    else if (younger == 1)
      __builtin_amdgcn_s_waitcnt(vm_wait(kNtDma));
    else
      __builtin_amdgcn_s_waitcnt(vm_wait(0));
  };
  if (n_i > 0) issue(0, 0);
  if (n_i > 1) issue(1, 1);
  int i = 0;
  for (; i + 3 <= n_i; i += 3) {
    NtStage<kRT> st;
    if (i + 2 < n_i) issue(i + 2, 2);
    wait_for(i);
    nt_read<0>(vo, vt, st);
    compute(kof(i), st);
    if (i + 3 < n_i) issue(i + 3, 0);
    wait_for(i + 1);
    nt_read<kNtStage>(vo, vt, st);
    compute(kof(i + 1), st);
    if (i + 4 < n_i) issue(i + 4, 1);
    wait_for(i + 2);
    nt_read<2 * kNtStage>(vo, vt, st);
    compute(kof(i + 2), st);
  }
  if (i < n_i) {   // tail: stages i (slot 0) and possibly i + 1 (slot 1), both already issued
    NtStage<kRT> st;
    wait_for(i);
    nt_read<0>(vo, vt, st);
    compute(kof(i), st);
    if (i + 1 < n_i) {
      wait_for(i + 1);
      nt_read<kNtStage>(vo, vt, st);
      compute(kof(i + 1), st);
    }
  }
  __builtin_amdgcn_s_waitcnt(vm_wait(0));

  // Wave partials (32 x 64 fp32) into the wave's own first slot, then the
  // sum over waves in wave order.  MFMA 32x32 output: lane l holds column
  // l % 32 of block jb; element e holds row 8 (e / 4) + 4 (l / 32) + e % 4.
  float *red = reinterpret_cast<float *>(ring);
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[(8 * (e >> 2) + 4 * lh + (e & 3)) * 64 + 32 * jb + lr] = acc[jb][e];
  __syncthreads();
  const int row = threadIdx.x >> 3, c = threadIdx.x & 7;
  float sm[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) sm[q] = reinterpret_cast<const float *>(smem[0][0])[row * 64 + 8 * c + q];
#pragma unroll
  for (int w = 1; w < kLoWaves; ++w)
#pragma unroll
    for (int q = 0; q < 8; ++q) sm[q] += reinterpret_cast<const float *>(smem[w][0])[row * 64 + 8 * c + q];
  const int gm = m0 + row;
  const int jl = j0 + 8 * c;
  if (gm < M) {
    uint16_t *o = out + static_cast<int64_t>(gm) * r + jl;
    if (jl + 8 <= r && (r & 7) == 0) {
      *reinterpret_cast<uint4 *>(o) =
          make_uint4(pack_bf16x2(sm[0] * scale, sm[1] * scale), pack_bf16x2(sm[2] * scale, sm[3] * scale),
                     pack_bf16x2(sm[4] * scale, sm[5] * scale), pack_bf16x2(sm[6] * scale, sm[7] * scale));
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (jl + q < r) o[q] = f32_to_bf16(sm[q] * scale);
    }
  }
}

// Grid (row tiles, 64-column chunks of r).
template <bool kRT>
__global__ __launch_bounds__(kLoThreads) void k_lora_nt(const uint16_t *__restrict__ L, int M, int Kc,
                                                        const uint16_t *__restrict__ R, int rcols, int r,
                                                        float scale, uint16_t *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLoWaves][kNtSlots][kNtStage];
  lora_nt_tile<kRT>(smem, L, M, Kc, R, rcols, r, scale, out, blockIdx.x, blockIdx.y * 64);
}

// Members sharing the left operand (e.g. q, k and v, or gate and up, all
// reading the same X): member i has its own R (A_i [r_i, K]), r_i, scale and
// output.  1-D grid over (row tile, member chunk), member chunks fastest and
// mapped so that the chunks of one row tile run back to back on one XCD:
// the X rows come from HBM once and from that XCD's L2 for the other chunks.
// Each output tile is computed exactly as by k_lora_nt.
template <bool kRT>
__global__ __launch_bounds__(kLoThreads) void k_lora_nt_shared(const uint16_t *__restrict__ L, int M, int Kc,
                                                               LoraShared sh) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLoWaves][kNtSlots][kNtStage];
  const unsigned nb = gridDim.x;
  unsigned lid = blockIdx.x;
  if ((nb & 7u) == 0) lid = (blockIdx.x & 7u) * (nb >> 3) + (blockIdx.x >> 3);
  const int Y = sh.y0[sh.n];
  const int mt = static_cast<int>(lid / static_cast<unsigned>(Y));
  const int y = static_cast<int>(lid % static_cast<unsigned>(Y));
  int i = 0;
  while (i + 1 < sh.n && y >= sh.y0[i + 1]) ++i;
  lora_nt_tile<kRT>(smem, L, M, Kc, sh.R[i], sh.rcols[i], sh.r[i], sh.scale[i], sh.out[i], mt,
                    (y - sh.y0[i]) * 64);
}

// ===========================================================================
// k_lora_tn: acc[j][d] = sum_m Q[m][j0 + j] P[m][d0 + d] over an M-split,
// j, d < 64.  Workgroup (d-tile of 64, split): wave w takes the 32-row
// stages w, w + 4, ... of the split (rotated per d-tile).  Stage = P tile
// [32 m][64 d] + Q tile [32 m][64 j] (4 KB each); both MFMA operands come
// from transposed reads (contraction over rows).  Output: bf16 directly
// (one split) as [j][d] (dA) or [d][j] (dB), else fp32 partials of the same
// orientation, summed by k_sum_partials.
// ===========================================================================
constexpr int kTnRows = 32;
constexpr int kTnSlots = 4;
constexpr int kTnTile = kTnRows * 128;      // 4 KB
constexpr int kTnStage = 2 * kTnTile;       // P then Q
constexpr int kTnDma = 2 * kTnRows / 8;     // DMA instructions per stage
constexpr int kTnRedPitch = 65;             // floats per row of a wave's 64 x 64 partial
constexpr int kTnGroupMax = 16;             // products per grouped launch

struct TnStage {
  bf16x8_t q[2][2], p[2][2];   // [sub-step][column block]
};

template <int kOff>
__device__ __forceinline__ void tn_read(const uint32_t (&vt)[2][2], TnStage &st) {
  u32x2_t t[2][2][2][2];   // [tile: Q, P][sub-step][cb][h]
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%20\n\t"
      "ds_read_b64_tr_b16 %1, %17 offset:%20\n\t"
      "ds_read_b64_tr_b16 %2, %18 offset:%20\n\t"
      "ds_read_b64_tr_b16 %3, %19 offset:%20\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:%21\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:%21\n\t"
      "ds_read_b64_tr_b16 %6, %18 offset:%21\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:%21\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:%22\n\t"
      "ds_read_b64_tr_b16 %9, %17 offset:%22\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:%22\n\t"
      "ds_read_b64_tr_b16 %11, %19 offset:%22\n\t"
      "ds_read_b64_tr_b16 %12, %16 offset:%23\n\t"
      "ds_read_b64_tr_b16 %13, %17 offset:%23\n\t"
      "ds_read_b64_tr_b16 %14, %18 offset:%23\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:%23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t[0][0][0][0]), "=&v"(t[0][0][0][1]), "=&v"(t[0][0][1][0]), "=&v"(t[0][0][1][1]),
        "=&v"(t[0][1][0][0]), "=&v"(t[0][1][0][1]), "=&v"(t[0][1][1][0]), "=&v"(t[0][1][1][1]),
        "=&v"(t[1][0][0][0]), "=&v"(t[1][0][0][1]), "=&v"(t[1][0][1][0]), "=&v"(t[1][0][1][1]),
        "=&v"(t[1][1][0][0]), "=&v"(t[1][1][0][1]), "=&v"(t[1][1][1][0]), "=&v"(t[1][1][1][1])
      : "v"(vt[0][0]), "v"(vt[0][1]), "v"(vt[1][0]), "v"(vt[1][1]), "n"(kOff + kTnTile),
        "n"(kOff + kTnTile + 2048), "n"(kOff), "n"(kOff + 2048)
      : "memory");
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      st.q[s][cb] = join_tr(t[0][s][cb][0], t[0][s][cb][1]);
      st.p[s][cb] = join_tr(t[1][s][cb][0], t[1][s][cb][1]);
    }
}

// One workgroup's tile: d-tile dt (columns 64 dt .. +63 of P), M-split sp,
// columns j0 .. j0 + 63 of Q.  The walk over the split starts at stage
// dt % (stages), so a tile's summation order depends only on (dt, sp).
__device__ __forceinline__ void lora_tn_tile(uint8_t (&smem)[kLoWaves][kTnSlots][kTnStage],
                                             const uint16_t *__restrict__ P, int M, int D,
                                             const uint16_t *__restrict__ Q, int qcols, int r,
                                             int stages_per_split, bool out_j_major, uint16_t *__restrict__ out,
                                             float *__restrict__ part, int64_t part_plane, int part_pitch, int dt,
                                             int sp, int j0) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int d0 = dt * 64;
  const int nms = (M + kTnRows - 1) / kTnRows;
  const int sbeg = sp * stages_per_split;
  const int count = max(0, min(nms, sbeg + stages_per_split) - sbeg);
  const int mend = min(M, (sbeg + count) * kTnRows);
  const int n_i = count > wave ? (count - wave + kLoWaves - 1) / kLoWaves : 0;
  const int rot = count > 0 ? static_cast<int>(static_cast<unsigned>(dt) % static_cast<unsigned>(count)) : 0;
  auto mof = [&](int i) {
    int t = wave + kLoWaves * i + rot;
    if (t >= count) t -= count;
    return (sbeg + t) * kTnRows;
  };
  uint8_t *ring = smem[wave][0];
  auto issue = [&](int i, int slot) {
    uint8_t *st = ring + slot * kTnStage;
    const int m0 = mof(i);
    dma_tile<kTnRows>(st, P, D, m0, M, d0, D, lane);
    dma_tile<kTnRows>(st + kTnTile, Q, qcols, m0, M, j0, qcols, lane);
  };
  const uint32_t base = lds_addr(ring);
  const int lr = lane & 31, lh = lane >> 5;
  uint32_t vt[2][2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int h = 0; h < 2; ++h) vt[cb][h] = base + tr_offset(lane, cb, h);

  f32x16_t acc[2][2];   // [jb][db]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
  auto compute = [&](int m0, TnStage &st) {
    if (m0 + kTnRows > mend) {   // rows past the split (or M) contribute zero
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) st.q[s][cb] = mask_tail(st.q[s][cb], m0 + 16 * s + 8 * lh, mend);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int db = 0; db < 2; ++db)
          acc[jb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.q[s][jb], st.p[s][db], acc[jb][db], 0, 0, 0);
  };
  auto wait_for = [&](int i) {
    const int younger = min(n_i - 1 - i, 3);
    if (younger >= 3)
      __builtin_amdgcn_s_waitcnt(vm_wait(3 * kTnDma));
    else if (younger == 2)
      __builtin_amdgcn_s_waitcnt(vm_wait(2 * kTnDma));
    else if (younger == 1)
      __builtin_amdgcn_s_waitcnt(vm_wait(kTnDma));
    else
      __builtin_amdgcn_s_waitcnt(vm_wait(0));
  };
  if (n_i > 0) issue(0, 0);
  if (n_i > 1) issue(1, 1);
  if (n_i > 2) issue(2, 2);
  int i = 0;
  for (; i + 4 <= n_i; i += 4) {
    TnStage st;
    if (i + 3 < n_i) issue(i + 3, 3);
    wait_for(i);
    tn_read<0>(vt, st);
    compute(mof(i), st);
    if (i + 4 < n_i) issue(i + 4, 0);
    wait_for(i + 1);
    tn_read<kTnStage>(vt, st);
    compute(mof(i + 1), st);
    if (i + 5 < n_i) issue(i + 5, 1);
    wait_for(i + 2);
    tn_read<2 * kTnStage>(vt, st);
    compute(mof(i + 2), st);
    if (i + 6 < n_i) issue(i + 6, 2);
    wait_for(i + 3);
    tn_read<3 * kTnStage>(vt, st);
    compute(mof(i + 3), st);
  }
  if (i < n_i) {   // tail: up to three stages, already issued into slots 0, 1, 2
    TnStage st;
    wait_for(i);
    tn_read<0>(vt, st);
    compute(mof(i), st);
    if (i + 1 < n_i) {
      wait_for(i + 1);
      tn_read<kTnStage>(vt, st);
      compute(mof(i + 1), st);
    }
    if (i + 2 < n_i) {
      wait_for(i + 2);
      tn_read<2 * kTnStage>(vt, st);
      compute(mof(i + 2), st);
    }
  }
  __builtin_amdgcn_s_waitcnt(vm_wait(0));

  // Wave partials: acc[jb][db][e] at lane l is (j, d) =
  // (32 jb + 8 (e / 4) + 4 (l / 32) + e % 4, 32 db + l % 32); stored as
  // red[j * 65 + d] in the wave's own ring, then summed in wave order.
  float *red = reinterpret_cast<float *>(ring);
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        red[(32 * jb + 8 * (e >> 2) + 4 * lh + (e & 3)) * kTnRedPitch + 32 * db + lr] = acc[jb][db][e];
  __syncthreads();
  // thread t: output row t / 4 of the orientation, 16 consecutive columns
  const int orow = threadIdx.x >> 2, oc0 = 16 * (threadIdx.x & 3);
  float sm[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int j = out_j_major ? orow : oc0 + q;
    const int d = out_j_major ? oc0 + q : orow;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kLoWaves; ++w) v += reinterpret_cast<const float *>(smem[w][0])[j * kTnRedPitch + d];
    sm[q] = v;
  }
  // global (row, column) of this thread's first element, and the bounds
  const int grow = out_j_major ? j0 + orow : d0 + orow;
  const int gcol = out_j_major ? d0 + oc0 : j0 + oc0;
  const int nrow = out_j_major ? r : D;
  const int ncol = out_j_major ? D : r;
  if (grow >= nrow) return;
  if (part) {
    float *dst = part + sp * part_plane + static_cast<int64_t>(grow) * part_pitch + gcol;
#pragma unroll
    for (int q = 0; q < 16; q += 4)
      *reinterpret_cast<float4 *>(dst + q) = make_float4(sm[q], sm[q + 1], sm[q + 2], sm[q + 3]);
  } else {
    uint16_t *dst = out + static_cast<int64_t>(grow) * ncol + gcol;
    if (gcol + 16 <= ncol && (ncol & 7) == 0) {
#pragma unroll
      for (int q = 0; q < 16; q += 8)
        *reinterpret_cast<uint4 *>(dst + q) =
            make_uint4(pack_bf16x2(sm[q], sm[q + 1]), pack_bf16x2(sm[q + 2], sm[q + 3]),
                       pack_bf16x2(sm[q + 4], sm[q + 5]), pack_bf16x2(sm[q + 6], sm[q + 7]));
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (gcol + q < ncol) dst[q] = f32_to_bf16(sm[q]);
    }
  }
}

// Grid (d-tiles, M-splits, 64-column chunks of r).
__global__ __launch_bounds__(kLoThreads) void k_lora_tn(const uint16_t *__restrict__ P, int M, int D,
                                                        const uint16_t *__restrict__ Q, int qcols, int r,
                                                        int stages_per_split, bool out_j_major,
                                                        uint16_t *__restrict__ out, float *__restrict__ part,
                                                        int64_t part_plane, int part_pitch) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLoWaves][kTnSlots][kTnStage];
  lora_tn_tile(smem, P, M, D, Q, qcols, r, stages_per_split, out_j_major, out, part, part_plane, part_pitch,
               blockIdx.x, blockIdx.y, blockIdx.z * 64);
}

// dA of members sharing P = X (q, k, v or gate, up): member i has its own
// Q = G_i, r_i, output and partial planes.  1-D grid over (d-tile, split,
// member chunk), member chunks fastest and XCD-mapped as in k_lora_nt_shared,
// so that the tiles reading one block of X run back to back on one XCD.
// Each tile is computed exactly as by k_lora_tn.
__global__ __launch_bounds__(kLoThreads) void k_lora_tn_shared(const uint16_t *__restrict__ P, int M, int D,
                                                               int splits, int stages_per_split, bool out_j_major,
                                                               int part_pitch, LoraShared sh) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLoWaves][kTnSlots][kTnStage];
  const unsigned nb = gridDim.x;
  unsigned lid = blockIdx.x;
  if ((nb & 7u) == 0) lid = (blockIdx.x & 7u) * (nb >> 3) + (blockIdx.x >> 3);
  const unsigned Y = static_cast<unsigned>(sh.y0[sh.n]);
  const int y = static_cast<int>(lid % Y);
  const int sp = static_cast<int>((lid / Y) % static_cast<unsigned>(splits));
  const int dt = static_cast<int>(lid / Y / static_cast<unsigned>(splits));
  int i = 0;
  while (i + 1 < sh.n && y >= sh.y0[i + 1]) ++i;
  lora_tn_tile(smem, P, M, D, sh.R[i], sh.rcols[i], sh.r[i], stages_per_split, out_j_major,
               sh.part[i] ? nullptr : sh.out[i], sh.part[i], sh.plane[i], part_pitch, dt, sp, (y - sh.y0[i]) * 64);
}

// out[row][col] = bf16(sum_sp part[sp][row][col]) (splits in order).
__global__ __launch_bounds__(256) void k_sum_partials(const float *__restrict__ part, int splits,
                                                      int64_t plane, int pitch, int nrow, int ncol,
                                                      uint16_t *__restrict__ out) {
  const int64_t total = static_cast<int64_t>(nrow) * ncol;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    const int row = static_cast<int>(idx / ncol), col = static_cast<int>(idx % ncol);
    const float *p = part + static_cast<int64_t>(row) * pitch + col;
    float s = p[0];
    for (int sp = 1; sp < splits; ++sp) s += p[sp * plane];
    out[idx] = f32_to_bf16(s);
  }
}

// Several k_lora_tn products in one launch (for example dA and dB of the
// linears of a layer): problem i owns workgroups [wg0[i], wg0[i + 1]) and
// decodes (d-tile, split, column chunk) from its local index; every tile is
// computed exactly as by k_lora_tn, so results do not depend on the grouping.
struct TnGroup {
  const uint16_t *P[kTnGroupMax];
  const uint16_t *Q[kTnGroupMax];
  uint16_t *out[kTnGroupMax];
  float *part[kTnGroupMax];
  int64_t plane[kTnGroupMax];
  int M[kTnGroupMax];
  int D[kTnGroupMax];
  int qcols[kTnGroupMax];
  int r[kTnGroupMax];
  int per[kTnGroupMax];
  int pitch[kTnGroupMax];
  int dt[kTnGroupMax];
  int sp[kTnGroupMax];
  int jmaj[kTnGroupMax];
  int wg0[kTnGroupMax + 1];
  int n;
};

__device__ __forceinline__ int tn_problem(const int *wg0, int n) {
  int i = 0;
#pragma unroll
  for (int j = 1; j < kTnGroupMax; ++j) i = (j < n && static_cast<int>(blockIdx.x) >= wg0[j]) ? j : i;
  return i;
}

__global__ __launch_bounds__(kLoThreads) void k_lora_tn_group(const TnGroup g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLoWaves][kTnSlots][kTnStage];
  const int i = tn_problem(g.wg0, g.n);
  const int local = static_cast<int>(blockIdx.x) - g.wg0[i];
  const int dt = local % g.dt[i];
  const int sp = (local / g.dt[i]) % g.sp[i];
  const int jc = local / (g.dt[i] * g.sp[i]);
  lora_tn_tile(smem, g.P[i], g.M[i], g.D[i], g.Q[i], g.qcols[i], g.r[i], g.per[i], g.jmaj[i] != 0,
               g.sp[i] == 1 ? g.out[i] : nullptr, g.part[i], g.plane[i], g.pitch[i], dt, sp, 64 * jc);
}

// The k_sum_partials of several products in one launch: problem i covers
// elements [e0[i], e0[i + 1]) of the concatenated outputs.
struct SumGroup {
  const float *part[kTnGroupMax];
  uint16_t *out[kTnGroupMax];
  int64_t plane[kTnGroupMax];
  int64_t e0[kTnGroupMax + 1];
  int splits[kTnGroupMax];
  int pitch[kTnGroupMax];
  int ncol[kTnGroupMax];
  int n;
};

__global__ __launch_bounds__(256) void k_sum_partials_group(const SumGroup g) {
  const int64_t total = g.e0[g.n];
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    int i = 0;
    for (int j = 1; j < g.n; ++j) i = idx >= g.e0[j] ? j : i;
    const int64_t li = idx - g.e0[i];
    const int row = static_cast<int>(li / g.ncol[i]), col = static_cast<int>(li % g.ncol[i]);
    const float *p = g.part[i] + static_cast<int64_t>(row) * g.pitch[i] + col;
    float sum = p[0];
    for (int sp = 1; sp < g.splits[i]; ++sp) sum += p[sp * g.plane[i]];
    g.out[i][li] = f32_to_bf16(sum);
  }
}

// dst [rows, rq] = src [rows, r] with zero columns r .. rq - 1 (rq = r rounded
// up to 8): 16-byte aligned rows for the DMA tiles.
__global__ __launch_bounds__(256) void k_pad_cols(const uint16_t *__restrict__ src, int rows, int r, int rq,
                                                  uint16_t *__restrict__ dst) {
  const int64_t total = static_cast<int64_t>(rows) * rq;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = idx / rq;
    const int col = static_cast<int>(idx % rq);
    dst[idx] = col < r ? src[row * r + col] : static_cast<uint16_t>(0);
  }
}

int round8(int r) { return (r + 7) & ~7; }
size_t align256(size_t b) { return (b + 255) / 256 * 256; }
unsigned grid_for(int64_t total) { return static_cast<unsigned>(std::min<int64_t>((total + 255) / 256, 4096)); }

// Pads an r-column matrix into ws when r % 8 != 0; returns the matrix to use
// and its column count.
const uint16_t *padded(const uint16_t *src, int rows, int r, void *ws, int &cols, hipStream_t s) {
  if ((r & 7) == 0) {
    cols = r;
    return src;
  }
  cols = round8(r);
  uint16_t *dst = static_cast<uint16_t *>(ws);
  hipLaunchKernelGGL(k_pad_cols, dim3(grid_for(static_cast<int64_t>(rows) * cols)), dim3(256), 0, s, src, rows, r,
                     cols, dst);
  return dst;
}

// M-splits of k_lora_tn: enough workgroups to cover the 256 compute units in
// whole rounds (one workgroup per CU: the LDS ring is 128 KB), at least 8
// stages per split, a small penalty per extra split for the partial traffic.
// Splits of one launch whose products together have `tiles` d-tile x column
// chunk tiles (the same split for all of them).
int tn_splits_tiles(int M, int tiles) {
  const int nms = (M + kTnRows - 1) / kTnRows;
  int best = 1;
  double best_score = -1.0;
  for (int sp = 1; sp <= 8; ++sp) {
    if (sp > 1 && nms / sp < 8) break;
    const int wg = tiles * sp;
    const int rounds = (wg + 255) / 256;
    const double score = static_cast<double>(wg) / (256.0 * rounds) - 0.03 * (sp - 1);
    if (score > best_score + 1e-9) {
      best = sp;
      best_score = score;
    }
  }
  return best;
}

int tn_splits(int M, int D) {
  const int dt = (D + 63) / 64;
  const int nms = (M + kTnRows - 1) / kTnRows;
  int best = 1;
  double best_score = -1.0;
  for (int sp = 1; sp <= 8; ++sp) {
    if (sp > 1 && nms / sp < 8) break;
    const int wg = dt * sp;
    const int rounds = (wg + 255) / 256;
    const double score = static_cast<double>(wg) / (256.0 * rounds) - 0.03 * (sp - 1);
    if (score > best_score + 1e-9) {
      best = sp;
      best_score = score;
    }
  }
  return best;
}

}  // namespace

hipError_t launch_lora_down(const uint16_t *X, int M, int K, const uint16_t *A, int r, float scale, uint16_t *T,
                            hipStream_t s) {
  const dim3 grid((M + kNtRows - 1) / kNtRows, (r + 63) / 64);
  hipLaunchKernelGGL((k_lora_nt<false>), grid, dim3(kLoThreads), 0, s, X, M, K, A, r, r, scale, T);
  return hipGetLastError();
}

size_t lora_grad_in_ws_bytes(int N, int r) {
  return (r & 7) ? align256(static_cast<size_t>(N) * round8(r) * 2) : 256;
}

hipError_t launch_lora_grad_in(const uint16_t *dY, int M, int N, const uint16_t *B, int r, float scale,
                               uint16_t *G, void *ws, hipStream_t s) {
  int cols = 0;
  const uint16_t *Bp = padded(B, N, r, ws, cols, s);
  const dim3 grid((M + kNtRows - 1) / kNtRows, (r + 63) / 64);
  hipLaunchKernelGGL((k_lora_nt<true>), grid, dim3(kLoThreads), 0, s, dY, M, N, Bp, cols, r, scale, G);
  return hipGetLastError();
}

// workspace: [padded Q (r % 8 != 0)] | [fp32 partials (more than one split)]
size_t lora_grad_ws_bytes(int M, int D, int r, int sp) {
  const size_t pad = (r & 7) ? align256(static_cast<size_t>(M) * round8(r) * 2) : 0;
  if (sp <= 0) sp = tn_splits(M, D);
  const int jc = (r + 63) / 64;
  const size_t part = sp > 1 ? align256(static_cast<size_t>(sp) * (64 * jc) * (((D + 63) / 64) * 64) * 4) : 0;
  return std::max<size_t>(pad + part, 256);
}

hipError_t launch_lora_down_shared(const uint16_t *X, int M, int K, int n, const uint16_t *const *A, const int *r,
                                   const float *scale, uint16_t *const *T, hipStream_t s) {
  LoraShared sh{};
  sh.n = n;
  sh.y0[0] = 0;
  for (int i = 0; i < n; ++i) {
    sh.R[i] = A[i];
    sh.out[i] = T[i];
    sh.scale[i] = scale[i];
    sh.rcols[i] = r[i];
    sh.r[i] = r[i];
    sh.y0[i + 1] = sh.y0[i] + (r[i] + 63) / 64;
  }
  const unsigned blocks = static_cast<unsigned>((M + kNtRows - 1) / kNtRows) * static_cast<unsigned>(sh.y0[n]);
  hipLaunchKernelGGL((k_lora_nt_shared<false>), dim3(blocks), dim3(kLoThreads), 0, s, X, M, K, sh);
  return hipGetLastError();
}

// Per member: [padded G (r % 8 != 0)] | [fp32 partials (more than one split)],
// the layout of lora_grad_ws_bytes, one region after the other.
size_t lora_dA_shared_ws_bytes(int M, int K, int n, const int *r) {
  size_t total = 0;
  for (int i = 0; i < n; ++i) total += lora_grad_ws_bytes(M, K, r[i], 0);
  return total;
}

hipError_t launch_lora_dA_shared(const uint16_t *X, int M, int K, int n, const uint16_t *const *G, const int *r,
                                 uint16_t *const *dA, void *ws, hipStream_t s) {
  const int sp = tn_splits(M, K);
  const int dt = (K + 63) / 64;
  const int nms = (M + kTnRows - 1) / kTnRows;
  const int per = (nms + sp - 1) / sp;
  const int pcol = dt * 64;                    // partial planes [64 jc_i, dt * 64], as in launch_lora_grad_w
  LoraShared sh{};
  sh.n = n;
  sh.y0[0] = 0;
  char *base = static_cast<char *>(ws);
  for (int i = 0; i < n; ++i) {
    const size_t pad = (r[i] & 7) ? align256(static_cast<size_t>(M) * round8(r[i]) * 2) : 0;
    int qcols = 0;
    sh.R[i] = padded(G[i], M, r[i], base, qcols, s);
    sh.rcols[i] = qcols;
    sh.r[i] = r[i];
    sh.out[i] = dA[i];
    const int jc = (r[i] + 63) / 64;
    sh.part[i] = sp > 1 ? reinterpret_cast<float *>(base + pad) : nullptr;
    sh.plane[i] = static_cast<int64_t>(64 * jc) * pcol;
    sh.y0[i + 1] = sh.y0[i] + jc;
    base += lora_grad_ws_bytes(M, K, r[i], 0);
  }
  const unsigned blocks = static_cast<unsigned>(dt) * static_cast<unsigned>(sp) * static_cast<unsigned>(sh.y0[n]);
  hipLaunchKernelGGL(k_lora_tn_shared, dim3(blocks), dim3(kLoThreads), 0, s, X, M, K, sp, per, true, pcol, sh);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp == 1) return e;
  for (int i = 0; i < n; ++i) {
    hipLaunchKernelGGL(k_sum_partials, dim3(grid_for(static_cast<int64_t>(r[i]) * K)), dim3(256), 0, s, sh.part[i],
                       sp, sh.plane[i], pcol, r[i], K, dA[i]);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_lora_grad_w_group(int count, const GradWJob *jobs, hipStream_t s) {
  if (count < 1 || count > kTnGroupMax) return hipErrorInvalidValue;
  TnGroup g{};
  SumGroup sg{};
  g.n = count;
  int64_t wg = 0, el = 0;
  for (int i = 0; i < count; ++i) {
    const GradWJob &jb = jobs[i];
    const size_t pad = (jb.r & 7) ? align256(static_cast<size_t>(jb.M) * round8(jb.r) * 2) : 0;
    int qcols = 0;
    const uint16_t *Qp = padded(jb.Q, jb.M, jb.r, jb.ws, qcols, s);
    const int sp = jb.splits > 0 ? jb.splits : tn_splits(jb.M, jb.D);
    const int jc = (jb.r + 63) / 64;
    const int dt = (jb.D + 63) / 64;
    const int nms = (jb.M + kTnRows - 1) / kTnRows;
    // partial planes in the output orientation: [64 jc, dt * 64] or [dt * 64, 64 jc]
    const int prow = jb.out_r_major ? 64 * jc : dt * 64;
    const int pcol = jb.out_r_major ? dt * 64 : 64 * jc;
    g.P[i] = jb.P;
    g.Q[i] = Qp;
    g.out[i] = jb.out;
    g.part[i] = sp > 1 ? reinterpret_cast<float *>(static_cast<char *>(jb.ws) + pad) : nullptr;
    g.plane[i] = static_cast<int64_t>(prow) * pcol;
    g.M[i] = jb.M;
    g.D[i] = jb.D;
    g.qcols[i] = qcols;
    g.r[i] = jb.r;
    g.per[i] = (nms + sp - 1) / sp;
    g.pitch[i] = pcol;
    g.dt[i] = dt;
    g.sp[i] = sp;
    g.jmaj[i] = jb.out_r_major ? 1 : 0;
    g.wg0[i] = static_cast<int>(wg);
    wg += static_cast<int64_t>(dt) * sp * jc;
    if (sp > 1) {
      const int k = sg.n++;
      sg.part[k] = g.part[i];
      sg.out[k] = jb.out;
      sg.plane[k] = g.plane[i];
      sg.e0[k] = el;
      sg.splits[k] = sp;
      sg.pitch[k] = pcol;
      sg.ncol[k] = jb.out_r_major ? jb.D : jb.r;
      el += static_cast<int64_t>(jb.out_r_major ? jb.r : jb.D) * sg.ncol[k];
    }
  }
  g.wg0[count] = static_cast<int>(wg);
  sg.e0[sg.n] = el;
  hipLaunchKernelGGL(k_lora_tn_group, dim3(static_cast<unsigned>(wg)), dim3(kLoThreads), 0, s, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sg.n == 0) return e;
  hipLaunchKernelGGL(k_sum_partials_group, dim3(grid_for(el)), dim3(256), 0, s, sg);
  return hipGetLastError();
}

int lora_grad_pair_splits(int M, int K, int N, int r) {
  const int jc = (r + 63) / 64;
  return tn_splits_tiles(M, jc * ((K + 63) / 64 + (N + 63) / 64));
}

int lora_grad_splits(int M, int K, int N, int r, bool dA, bool dB) {
  if (dA && dB) return lora_grad_pair_splits(M, K, N, r);
  return dA ? tn_splits(M, K) : tn_splits(M, N);
}

size_t lora_grad_pair_ws_bytes(int M, int D, int K, int N, int r) {
  return lora_grad_ws_bytes(M, D, r, std::max(tn_splits(M, D), lora_grad_pair_splits(M, K, N, r)));
}

hipError_t launch_lora_grad_w(const uint16_t *P, const uint16_t *Q, int M, int D, int r, bool out_r_major,
                              uint16_t *out, void *ws, hipStream_t s) {
  const GradWJob job{P, Q, M, D, r, out_r_major, out, ws, 0};
  return launch_lora_grad_w_group(1, &job, s);
}

}  // namespace qlora
