// Decode-regime forward for 4 < M <= 64 tokens (one linear or a group of
// linears sharing M), K % 256 == 0:
//     Y [M, N] = X deq(W)^T + T B^T,   T = bf16(s X A^T) or given
// (automatone.win, "QLoRA paper explained", How it works: the 4-bit weights
// are dequantized on the fly for the math and never stored in 16-bit.)
//
// The work is bound by the packed-weight stream from HBM; three kernels:
//  * k_ss_down: partial down-projections X[:, c] A[:, c]^T per 256-column
//    chunk c (fp32), one workgroup per (linear, chunk, 64 adapter rows);
//  * k_ss_stream: one workgroup per CU, persistent.  It first forms its
//    share of T = bf16(s * sum of the partials in chunk order) (also to the
//    caller's T_out), beside its first weight DMAs.  Work unit = (linear, 64
//    weight rows, 256 columns); units are ordered by linear, row tile and
//    column and every workgroup takes an equal contiguous range, so each CU
//    streams the same number of bytes.  A unit's packed bytes (64 rows x 128
//    bytes: whole cache lines), block codes, group scales and X columns
//    (16 kMB token rows x 512 bytes) are DMA'd global -> LDS two units ahead
//    into three-stage rings.  Only LDS DMAs touch global memory in the loop,
//    so the end-of-unit wait can count them in issue order and leave the
//    newest unit's DMAs in flight; no wait ever drains the DMA stream.  Wave (rh, kq) multiplies rows 32 rh .. +31
//    by block kq of the unit: lane (n = l % 16, g = l / 16) takes codes
//    16 g .. 16 g + 15 of its row's block, expands them through a
//    byte -> bf16x2 table of the NF4 levels (32 copies, one per lane of a half
//    wave) into MFMA 16x16x32 operands and scales each block's partial
//    product by its c_hat in fp32, so the dequantized weight is
//    bf16(NF4[q]) * c_hat (the reading of the other decode-regime kernels,
//    within the matmul tolerance).  At the end of a row tile (or of the
//    range) the four k-quarter sums are added in LDS in a fixed order and
//    the 64-row sum is stored (fp32) to the segment's slot;
//  * k_ss_epi: one workgroup per row tile sums its segments in workgroup
//    order, adds T B^T (one more MFMA chain per 16 x 16 output tile) and
//    stores Y in bf16.  (Finishing the tiles inside the stream kernel would
//    need device-scope fences between workgroups, which write back and
//    invalidate the L2 under the other workgroups' streams.)
// Results are deterministic for a given call and device (the segment split
// depends on the linears of the call and on the CU count).
// LDS tiles are 16-byte-chunk XOR-swizzled by row so that the DMA writes and
// the operand reads are bank-conflict free.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace qlora {

__constant__ uint32_t cSsQ4Level[3 * 16] = {QLORA_Q4_LEVEL_BITS};
__constant__ uint32_t cSsT8Level[256] = {QLORA_T8_LEVEL_BITS};

namespace {

constexpr int kSsRows = 64;                       // weight rows per tile
constexpr int kSsWaves = 8;
constexpr int kSsThreads = kSsWaves * 64;
constexpr int kSsStepK = 256;                     // columns per unit
constexpr int kSsWPacked = kSsRows * 128;         // packed bytes per unit
constexpr int kSsWStage = kSsWPacked + 512;       // + 64 x 4 code bytes + 64 group scales
constexpr int kSsLutCopies = 32;
constexpr int kSsMaxGrid = 256;                   // workgroups of the stream kernel (at most)
constexpr int kSsDownThreads = 256;
constexpr int kSsMaxKT = 64;                      // K <= 16384 on this path

// s_waitcnt immediate (vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int ss_wait(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | 0x70 | ((lgkm & 15) << 8); }

template <int kWait>
__device__ __forceinline__ void ss_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWait);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

// 4-byte-per-lane global -> LDS DMA (lane i lands at dst + 4 i).
__device__ __forceinline__ void dma4(const void *src, uint32_t dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(dst) : "memory");
}

// Swizzled positions: weight rows (128 bytes, 8 chunks) and X token rows
// (512 bytes, 32 chunks).
__device__ __forceinline__ int ss_wpos(int row, int chunk) { return row * 128 + 16 * (chunk ^ ((row >> 1) & 7)); }
__device__ __forceinline__ int ss_xpos(int row, int chunk) { return row * 512 + 16 * (chunk ^ (row & 15)); }

// First unit of workgroup w of G over U units.
__device__ __forceinline__ int64_t ss_ub(int w, int G, int64_t U) { return (static_cast<int64_t>(w) * U) / G; }
// Workgroup whose range holds unit u.
__device__ __forceinline__ int ss_wg_of(int64_t u, int G, int64_t U) {
  int w = static_cast<int>((u * G) / U);
  while (w + 1 < G && ss_ub(w + 1, G, U) <= u) ++w;
  while (w > 0 && ss_ub(w, G, U) > u) --w;
  return w;
}

}  // namespace

// ---------------------------------------------------------------------------
// Down-projection partials: workgroup (linear, chunk c, adapter block jb);
// wave w: adapter rows 64 jb + 16 w + l % 16, all token tiles.
// P [chunk][M][r] fp32.
template <int kMB>
__global__ __launch_bounds__(kSsDownThreads) void k_ss_down(SmGroup grp) {
  int li = 0;
  while (li + 1 < grp.n && static_cast<int>(blockIdx.x) >= grp.down_start[li + 1]) ++li;
  const SmLinear &L = grp.lin[li];
  const int M = grp.M, K = L.w.K, r = L.r;
  const int local = blockIdx.x - grp.down_start[li];
  const int KT = K / kSsStepK;
  const int c = local % KT, jb = local / KT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 15, g = lane >> 4;
  const int j = 64 * jb + 16 * wave + nl;
  const uint16_t *arow = L.A + static_cast<int64_t>(min(j, r - 1)) * K;
  f32x4_t acc[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bf16x8_t av[8];
  bf16x8_t xv[8][kMB];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int k = kSsStepK * c + 32 * s + 8 * g;
    av[s] = *reinterpret_cast<const bf16x8_t *>(arow + k);
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
      xv[s][mb] = *reinterpret_cast<const bf16x8_t *>(L.X + static_cast<int64_t>(min(16 * mb + nl, M - 1)) * K + k);
  }
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[s][mb], av[s], acc[mb], 0, 0, 0);
  // D layout: lane holds column (adapter row) j, tokens 4 g + e.
  float *P = L.Pd + static_cast<int64_t>(c) * M * r;
  if (j < r) {
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mb + 4 * g + e;
        if (m < M) P[static_cast<int64_t>(m) * r + j] = acc[mb][e];
      }
  }
}

// ---------------------------------------------------------------------------
// Row tiles per work unit: one unit = kPT tiles x 256 columns, sharing one X
// chunk.  Each wait-and-barrier round then moves kPT x 8 KB of weights (the
// per-round cost of the LDS DMA stream is fixed, so larger rounds stream
// faster), within the 160 KB of LDS.
// From three token tiles up, X takes two stages (prefetched one unit ahead)
// instead of three, which leaves room for more weight tiles per unit: each X
// chunk then serves 2-3 row tiles instead of 1-2.
template <int kMB>
constexpr int ss_pt() {
  return kMB == 1 ? 4 : (kMB == 2 ? 3 : (kMB == 3 ? 3 : 2));
}
int ss_pt_of(int kmb) { return kmb == 1 ? 4 : (kmb == 2 ? 3 : (kmb == 3 ? 3 : 2)); }

// Per-linear values the DMA iterators need, reloaded when they cross into the
// next linear.
struct SsLin {
  const uint16_t *X;
  const uint8_t *packed;
  const uint8_t *code8;
  const float *c2;
  int K, N, KT, groups;
};
template <int kPT>
__device__ __forceinline__ SsLin ss_lin(const SmGroup &grp, int li) {
  const SmLinear &L = grp.lin[li];
  SsLin c;
  c.X = L.X;
  c.packed = L.w.packed;
  c.code8 = L.w.code8;
  c.c2 = L.w.c2;
  c.K = L.w.K;
  c.N = L.w.N;
  c.KT = L.w.K / kSsStepK;
  c.groups = (grp.item0[li + 1] - grp.item0[li] + kPT - 1) / kPT;
  return c;
}
struct SsPos {
  int li, group, kt;
  SsLin c;
};
template <int kPT>
__device__ __forceinline__ SsPos ss_locate(const SmGroup &grp, int64_t u) {
  SsPos p;
  p.li = 0;
  while (p.li + 1 < grp.n && u >= grp.cost0[p.li + 1]) ++p.li;
  p.c = ss_lin<kPT>(grp, p.li);
  const int64_t rel = u - grp.cost0[p.li];
  p.group = static_cast<int>(rel / p.c.KT);
  p.kt = static_cast<int>(rel % p.c.KT);
  return p;
}
template <int kPT>
__device__ __forceinline__ void ss_advance(const SmGroup &grp, SsPos &p) {
  if (++p.kt == p.c.KT) {
    p.kt = 0;
    if (++p.group == p.c.groups) {
      p.group = 0;
      if (p.li + 1 < grp.n) {
        ++p.li;
        p.c = ss_lin<kPT>(grp, p.li);
      }
    }
  }
}

// Segment slots: linear li's slot area holds (groups + workgroups) x kPT
// pieces; tile t of group g summed by workgroup w is piece
// (g + w - first workgroup of li) kPT + t.
template <int kMB>
__device__ __forceinline__ float *ss_slot(const SmLinear &L, int group, int t, int w, int wfirst) {
  constexpr int kPiece = 2 * 2 * kMB * 4 * 64;
  constexpr int kPT = ss_pt<kMB>();
  return L.P + (static_cast<int64_t>(group + w - wfirst) * kPT + t) * kPiece;
}

// Finishes rows 32 rh .. +31 of tile t of group `group` of linear L (one
// wave): the segments of workgroups wf .. wl in workgroup order, then the LoRA
// term and the bf16 store.  Every load (segments, B rows, T) is issued
// before its first use.
template <int kMB>
__device__ __forceinline__ void ss_finish_rows(const SmLinear &L, int M, int group, int t, int rh, int lane, int wf,
                                               int wl, int wfirst) {
  constexpr int kPT = ss_pt<kMB>();
  constexpr int kMaxSeg = 3;                    // segments summed per pass
  constexpr int kMaxJ = 4;                      // 32-column adapter chunks per pass
  const int nl = lane & 15, g = lane >> 4;
  const int N = L.w.N, r = L.r;
  const int tile = kPT * group + t;
  const int n0 = kSsRows * tile + 32 * rh;
  const uint16_t *T = L.Tin;
  f32x4_t v[2][kMB];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) v[rg][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int w0 = wf; w0 <= wl; w0 += kMaxSeg) {
    f32x4_t seg[kMaxSeg][2][kMB];
#pragma unroll
    for (int i = 0; i < kMaxSeg; ++i) {
      const float *src = ss_slot<kMB>(L, group, t, min(w0 + i, wl), wfirst);
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) seg[i][rg][mb][e] = src[(((rh * 2 + rg) * kMB + mb) * 4 + e) * 64 + lane];
    }
#pragma unroll
    for (int i = 0; i < kMaxSeg; ++i)
      if (w0 + i <= wl)
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[rg][mb][e] += seg[i][rg][mb][e];
  }
  // LoRA: A operand T[16 mb + nl, j + 8 g ..], B operand B[n, j + 8 g ..].
  for (int j00 = 0; j00 < r; j00 += 32 * kMaxJ) {
    bf16x8_t bop[kMaxJ][2], top[kMaxJ][kMB];
#pragma unroll
    for (int jj = 0; jj < kMaxJ; ++jj) {
      const int j = j00 + 32 * jj + 8 * g;
      const int jc = j < r ? j : 0;             // r % 8 == 0
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
        bop[jj][rg] =
            *reinterpret_cast<const bf16x8_t *>(L.B + static_cast<int64_t>(min(n0 + 16 * rg + nl, N - 1)) * r + jc);
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
        top[jj][mb] = *reinterpret_cast<const bf16x8_t *>(T + static_cast<int64_t>(min(16 * mb + nl, M - 1)) * r + jc);
    }
#pragma unroll
    for (int jj = 0; jj < kMaxJ; ++jj) {
      const bool jok = j00 + 32 * jj + 8 * g < r;
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        const bf16x8_t a = (jok && 16 * mb + nl < M) ? top[jj][mb] : bf16x8_t{};
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
          v[rg][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, jok ? bop[jj][rg] : bf16x8_t{}, v[rg][mb], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int n = n0 + 16 * rg + nl;
    if (n < N) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int mm = 16 * mb + 4 * g + e;
          if (mm < M) L.Y[static_cast<int64_t>(mm) * N + n] = f32_to_bf16(v[rg][mb][e]);
        }
    }
  }
}

template <int kMB>
__global__ __launch_bounds__(kSsThreads) void k_ss_stream(SmGroup grp) {
  constexpr int kPT = ss_pt<kMB>();
  constexpr int kXS = kMB >= 3 ? 2 : 3;         // X stages: X one or two units ahead
  constexpr int kWS = 3;                        // weight stages: two units ahead
  constexpr int kXStage = kMB * 16 * 512;
  constexpr int kWStage = kPT * kSsWStage;
  constexpr int kPiece = 2 * 2 * kMB * 4 * 64;  // floats: [rh][rg][mb][e][lane]
  // DMA instructions per wave and unit: kPT (packed weights), waves
  // 0 .. 2 kPT - 1 one gather (codes of tile w, or group scales of tile
  // w - kPT), and kMB (X).  At the end of unit q everything up to unit q + 1
  // must have landed.  Three X stages: unit q issues the weights, then the X,
  // of q + 2, and both may stay in flight.  Two X stages: unit q issues the X
  // of q + 1, then the weights of q + 2; only those weights may stay in
  // flight (the counter retires DMAs in issue order).
  constexpr int kAfter = kXS == 3 ? kPT + kMB : kPT;
  constexpr int kAfterG = kAfter + 1;
  static_assert(2 * kPiece * 4 <= kXStage, "tile sums fit in an X stage");
  __shared__ __attribute__((aligned(16))) uint8_t sX[kXS * kXStage];
  __shared__ __attribute__((aligned(16))) uint8_t sW[kWS * kWStage];
  __shared__ uint32_t sLut[256 * kSsLutCopies];
  __shared__ float sT8[256];
  __shared__ float sMean[kSmMaxGroup];

  const int G = gridDim.x, w = blockIdx.x;
  const int64_t U = grp.cost0[grp.n];
  const int64_t u0 = ss_ub(w, G, U), u1 = ss_ub(w + 1, G, U);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rh = wave & 1, kq = wave >> 1;
  const int nl = lane & 15, g = lane >> 4;
  const int M = grp.M;
  const bool gather = wave < 2 * kPT;
  if (u0 >= u1) return;                         // (the grid never exceeds the unit count)

  const int qt = grp.lin[0].w.qtype;            // the linears of a group share one 4-bit type
  for (int i = tid; i < 256 * kSsLutCopies; i += kSsThreads) {
    const int byte = i / kSsLutCopies;
    sLut[i] = pack_bf16x2(u2f(cSsQ4Level[16 * qt + (byte & 15)]), u2f(cSsQ4Level[16 * qt + (byte >> 4)]));
  }
  if (tid < 256) sT8[tid] = u2f(cSsT8Level[tid]);
  if (tid < grp.n) sMean[tid] = grp.lin[tid].w.mean[0];

  // DMA of unit number q (counted from u0; units past the range repeat the
  // last one).  Weights of tile t: wave w fills rows 8 w .. 8 w + 7 of the
  // tile's packed part; lane i lands at position i % 8 of row 8 w + i / 8 and
  // fetches chunk (i % 8) ^ f(row).  X: wave w fills token rows 2 (kMB w + j)
  // and + 1; lane i lands at position i % 32 and fetches chunk
  // (i % 32) ^ (row % 16); rows past M repeat row M - 1 (never stored).
  const uint32_t xbase = lds_addr(sX), wbase = lds_addr(sW);
  const int wrow = 8 * wave + (lane >> 3);
  const int wchunk = (lane & 7) ^ ((wrow >> 1) & 7);
  int xoff[kMB];                                // element offset of this lane's X chunk in its row
#pragma unroll
  for (int j = 0; j < kMB; ++j) {
    const int row = 2 * (kMB * wave + j) + (lane >> 5);
    xoff[j] = 8 * ((lane & 31) ^ (row & 15));
  }
  auto dma_x = [&](int q, const SsPos &p) __attribute__((always_inline)) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(xbase + (q % kXS) * kXStage + kMB * wave * 1024);
#pragma unroll
    for (int j = 0; j < kMB; ++j) {
      const int row = 2 * (kMB * wave + j) + (lane >> 5);
      dma16(p.c.X + static_cast<int64_t>(min(row, M - 1)) * p.c.K + kSsStepK * p.kt + xoff[j], dst + j * 1024);
    }
  };
  auto dma_w = [&](int q, const SsPos &p) __attribute__((always_inline)) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(wbase + (q % kWS) * kWStage);
    const int64_t rb = p.c.K >> 1;
#pragma unroll
    for (int t = 0; t < kPT; ++t) {
      const int n0 = kSsRows * (kPT * p.group + t);
      dma16(p.c.packed + static_cast<int64_t>(min(n0 + wrow, p.c.N - 1)) * rb + 128 * p.kt + 16 * wchunk,
            dst + t * kSsWStage + wave * 1024);
    }
    if (gather) {
      const int t = wave < kPT ? wave : wave - kPT;
      const int n0 = kSsRows * (kPT * p.group + t);
      const int64_t cb = static_cast<int64_t>(min(n0 + lane, p.c.N - 1)) * (p.c.K >> 6) + 4 * p.kt;  // 4-aligned
      if (wave < kPT)
        dma4(p.c.code8 + cb, dst + t * kSsWStage + kSsWPacked);
      else
        dma4(p.c.c2 + (cb >> 8), dst + t * kSsWStage + kSsWPacked + 256);
    }
  };
  auto round_end = [&]() __attribute__((always_inline)) {
    if (gather)
      ss_barrier<ss_wait(kAfterG, 0)>();
    else
      ss_barrier<ss_wait(kAfter, 0)>();
  };

  const int nq = static_cast<int>(u1 - u0);
  SsPos pc = ss_locate<kPT>(grp, u0);          // compute position
  SsPos px = pc, pw = pc;                     // DMA positions (X, weights)
  int qx = 0, qw = 0;
  auto issue_w = [&]() __attribute__((always_inline)) {
    dma_w(qw, pw);
    if (qw + 1 < nq) ss_advance<kPT>(grp, pw);
    ++qw;
  };
  auto issue_x = [&]() __attribute__((always_inline)) {
    dma_x(qx, px);
    if (qx + 1 < nq) ss_advance<kPT>(grp, px);
    ++qx;
  };
  auto issue_next = [&]() __attribute__((always_inline)) {
    if constexpr (kXS == 3) {
      issue_w();
      issue_x();
    } else {
      issue_x();
      issue_w();
    }
  };
  // Prologue in the steady-state order: W(0) X(0) W(1) X(1) with three X
  // stages, X(0) W(0) W(1) with two.
  if constexpr (kXS == 3) {
    issue_next();
    issue_next();
  } else {
    issue_x();
    issue_w();
    issue_w();
  }
  // T for the epilogue kernel while those DMAs fly: this workgroup's equal
  // share of the M r elements of every linear (main_start: prefix sums),
  // each the sum of its chunk partials in chunk order.  The partial loads
  // are younger than the DMAs, so their waits also cover the DMAs, which the
  // first round needs anyway.
  {
    const int E = grp.main_start[grp.n];
    const int e0 = static_cast<int>((static_cast<int64_t>(w) * E) / G);
    const int e1 = static_cast<int>((static_cast<int64_t>(w + 1) * E) / G);
    for (int li = 0; li < grp.n; ++li) {          // uniform: the share's part in each linear
      const int lo = max(e0, grp.main_start[li]) - grp.main_start[li];
      const int hi = min(e1, grp.main_start[li + 1]) - grp.main_start[li];
      if (lo >= hi) continue;
      const SmLinear &L = grp.lin[li];
      const int KT = L.w.K / kSsStepK;             // <= kSsMaxKT
      for (int i = lo + tid; i < hi; i += kSsThreads) {
        // addresses formed in vector registers (the stream loop needs the
        // scalar ones), 16 chunk loads in flight, summed in chunk order
        int stride = M * L.r;
        asm volatile("" : "+v"(stride));
        const float *pp = L.Pd + i;
        float t = 0.f;
        for (int c0 = 0; c0 < KT; c0 += 16) {
          float pv[16];
#pragma unroll
          for (int c = 0; c < 16; ++c) pv[c] = c0 + c < KT ? pp[c * stride] : 0.f;
#pragma unroll
          for (int c = 0; c < 16; ++c)
            if (c0 + c < KT) t += pv[c];
          pp += 16 * stride;
        }
        const uint16_t v = f32_to_bf16(L.scale * t);
        const_cast<uint16_t *>(L.Tin)[i] = v;
        if (L.Tout) L.Tout[i] = v;
      }
    }
  }
  round_end();

  f32x4_t acc[kPT][2][kMB];
#pragma unroll
  for (int t = 0; t < kPT; ++t)
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) acc[t][rg][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint32_t lutl = static_cast<uint32_t>(lane & 31);
  float mean = sMean[pc.li];
  int wfirst = ss_wg_of(grp.cost0[pc.li], G, U);

  for (int q = 0; q < nq; ++q) {
    issue_next();                               // weights of unit q + 2, X of q + 2 or q + 1

    const uint8_t *xs = sX + (q % kXS) * kXStage;
    const uint8_t *ws0 = sW + (q % kWS) * kWStage;
    bf16x8_t xa[kMB][2];
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        xa[mb][tt] = *reinterpret_cast<const bf16x8_t *>(xs + ss_xpos(16 * mb + nl, 8 * kq + 2 * g + tt));
#pragma unroll
    for (int t = 0; t < kPT; ++t) {
      const uint8_t *ws = ws0 + t * kSsWStage;
      const float *c2s = reinterpret_cast<const float *>(ws + kSsWPacked + 256);
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const int row = 32 * rh + 16 * rg + nl;
        const uint2 pk = *reinterpret_cast<const uint2 *>(ws + ss_wpos(row, 2 * kq + (g >> 1)) + 8 * (g & 1));
        const int code = ws[kSsWPacked + 4 * row + kq];
        const float chat = decode_absmax(sT8[code], c2s[row], mean);
        const uint32_t words[2] = {pk.x, pk.y};
        bf16x8_t wop[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          uint32_t o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = sLut[((words[tt] >> (8 * i)) & 0xffu) * kSsLutCopies + lutl];
          wop[tt] = __builtin_bit_cast(bf16x8_t, o);
        }
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
          f32x4_t part =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mb][0], wop[0], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mb][1], wop[1], part, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][rg][mb][e] = __builtin_fmaf(chat, part[e], acc[t][rg][mb][e]);
        }
      }
    }

    const bool group_end = pc.kt == pc.c.KT - 1 || q == nq - 1;
    round_end();

    if (group_end) {
      // Per tile: k-quarter sums ((q0 + q2) + (q1 + q3)) per row half, in LDS,
      // then the 64-row sum to its slot.  The sums use this unit's X stage:
      // consumed, and refilled only by the next unit's DMA.
      float *sRed = reinterpret_cast<float *>(sX + (q % kXS) * kXStage);
      auto red_at = [&](int slot, int rg, int mb, int e) -> float & {
        return sRed[((((slot * 2 + rh) * 2 + rg) * kMB + mb) * 4 + e) * 64 + lane];
      };
#pragma unroll
      for (int t = 0; t < kPT; ++t) {
        if (kq >= 2) {
#pragma unroll
          for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
              for (int e = 0; e < 4; ++e) red_at(kq - 2, rg, mb, e) = acc[t][rg][mb][e];
        }
        ss_barrier<ss_wait(63, 0)>();
        if (kq < 2) {
#pragma unroll
          for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[t][rg][mb][e] += red_at(kq, rg, mb, e);
        }
        if (kq == 1) {
#pragma unroll
          for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
              for (int e = 0; e < 4; ++e) red_at(1, rg, mb, e) = acc[t][rg][mb][e];
        }
        ss_barrier<ss_wait(63, 0)>();
        if (kq == 0) {
          float *dst = ss_slot<kMB>(grp.lin[pc.li], pc.group, t, w, wfirst);
#pragma unroll
          for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                dst[(((rh * 2 + rg) * kMB + mb) * 4 + e) * 64 + lane] = acc[t][rg][mb][e] + red_at(1, rg, mb, e);
        }
        ss_barrier<ss_wait(63, 0)>();            // sRed is reused by the next tile
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb) acc[t][rg][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (q + 1 < nq) {
      const int li0 = pc.li;
      ss_advance<kPT>(grp, pc);
      if (pc.li != li0) {
        mean = sMean[pc.li];
        wfirst = ss_wg_of(grp.cost0[pc.li], G, U);
      }
    }
  }
  ss_barrier<ss_wait(0, 0)>();                  // the clamped DMAs past the range

}

// One workgroup (2 waves: row halves) per row tile.
template <int kMB>
__global__ __launch_bounds__(128) void k_ss_epi(SmGroup grp, int G) {
  constexpr int kPT = ss_pt<kMB>();
  const int tg = blockIdx.x;
  int li = 0;
  while (li + 1 < grp.n && tg >= grp.item0[li + 1]) ++li;
  const SmLinear &L = grp.lin[li];
  const int tile = tg - grp.item0[li];
  const int group = tile / kPT, t = tile % kPT;
  const int64_t U = grp.cost0[grp.n];
  const int KT = L.w.K / kSsStepK;
  const int64_t gs = grp.cost0[li] + static_cast<int64_t>(group) * KT;
  ss_finish_rows<kMB>(L, grp.M, group, t, threadIdx.x >> 6, threadIdx.x & 63, ss_wg_of(gs, G, U),
                      ss_wg_of(gs + KT - 1, G, U), ss_wg_of(grp.cost0[li], G, U));
}

// ---------------------------------------------------------------------------
namespace {
int ss_grid() {
  static int grid[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (grid[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
    grid[dev] = std::min(cus, kSsMaxGrid);
  }
  return grid[dev];
}
}  // namespace

bool small_m_stream_ok(int64_t M, int K, int r) {
  return M > 4 && M <= 64 && r % 8 == 0 && K >= kSsStepK && K % kSsStepK == 0 && K / kSsStepK <= kSsMaxKT;
}

// Per linear: the segment slots ((groups + workgroups) x kPT pieces of 64
// rows x 16 kMB tokens, fp32), the down-projection partials [K / 256][M][r]
// fp32 (read by the stream kernel while other workgroups already write
// slots, hence their own region) and T [M][r] bf16.
static size_t ss_slot_bytes(int M, int N, int K, int r) {
  const int kmb = (M + 15) / 16, pt = ss_pt_of(kmb);
  const int tiles = (N + kSsRows - 1) / kSsRows;
  const size_t groups = static_cast<size_t>((tiles + pt - 1) / pt);
  const size_t slots = (groups + kSsMaxGrid) * pt * (2 * 2 * kmb * 4 * 64) * 4;
  return (slots + 255) / 256 * 256;
}
static size_t ss_part_bytes(int M, int K, int r) {
  return (static_cast<size_t>(K / kSsStepK) * M * r * 4 + 255) / 256 * 256;
}
size_t small_m_stream_ws_bytes(int M, int N, int K, int r) {
  return ss_slot_bytes(M, N, K, r) + ss_part_bytes(M, K, r) + (static_cast<size_t>(M) * r * 2 + 255) / 256 * 256;
}

bool small_m_stream_group_ok(const SmGroup &grp) {
  for (int i = 0; i < grp.n; ++i) {
    const SmLinear &L = grp.lin[i];
    if (L.P == nullptr || !small_m_stream_ok(grp.M, L.w.K, L.r)) return false;
  }
  return grp.n >= 1;
}

template <int kMB>
static hipError_t ss_launch(SmGroup &grp, hipStream_t s) {
  constexpr int kPT = ss_pt<kMB>();
  int64_t units = 0;
  for (int i = 0; i < grp.n; ++i) {
    const SmLinear &L = grp.lin[i];
    const int groups = (grp.item0[i + 1] - grp.item0[i] + kPT - 1) / kPT;
    grp.cost0[i] = static_cast<int>(units);
    units += static_cast<int64_t>(groups) * (L.w.K / kSsStepK);
  }
  grp.cost0[grp.n] = static_cast<int>(units);
  const int grid = static_cast<int>(std::min<int64_t>(ss_grid(), units));
  hipLaunchKernelGGL(k_ss_down<kMB>, dim3(grp.down_start[grp.n]), dim3(kSsDownThreads), 0, s, grp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_ss_stream<kMB>, dim3(grid), dim3(kSsThreads), 0, s, grp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_ss_epi<kMB>, dim3(grp.item0[grp.n]), dim3(128), 0, s, grp, grid);
  return hipGetLastError();
}

// Each linear's L.P is the start of its workspace region
// (small_m_stream_ws_bytes).  Plans tiles (item0), down-projection blocks
// (down_start) and each linear's first T element (main_start); ss_launch
// plans the units.
hipError_t launch_small_m_stream(SmGroup &grp, hipStream_t s) {
  int tiles = 0, down = 0, fin = 0;
  for (int i = 0; i < grp.n; ++i) {
    SmLinear &L = grp.lin[i];
    const int M = grp.M, N = L.w.N, K = L.w.K, r = L.r;
    char *base = reinterpret_cast<char *>(L.P);
    L.Pd = reinterpret_cast<float *>(base + ss_slot_bytes(M, N, K, r));
    L.Tin = reinterpret_cast<const uint16_t *>(base + ss_slot_bytes(M, N, K, r) + ss_part_bytes(M, K, r));
    grp.item0[i] = tiles;
    grp.down_start[i] = down;
    grp.main_start[i] = fin;
    tiles += (N + kSsRows - 1) / kSsRows;
    down += (K / kSsStepK) * ((r + 63) / 64);
    fin += M * r;
  }
  grp.item0[grp.n] = tiles;
  grp.down_start[grp.n] = down;
  grp.main_start[grp.n] = fin;
  switch ((grp.M + 15) / 16) {
    case 1: return ss_launch<1>(grp, s);
    case 2: return ss_launch<2>(grp, s);
    case 3: return ss_launch<3>(grp, s);
    default: return ss_launch<4>(grp, s);
  }
}

}  // namespace qlora
