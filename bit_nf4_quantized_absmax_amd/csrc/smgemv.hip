// Decode-regime forward for M <= 4 tokens (dequant-GEMV), one linear or a
// group of linears:
//     Y [M, N] = X deq(W)^T + T B^T
// (automatone.win, "QLoRA paper explained", How it works: the 4-bit weights
// are dequantized on the fly for the math and never stored in 16-bit.)
//
// Work item = 4 weight rows x the whole K of one linear.  The items are dealt
// round robin to the workgroups of a persistent grid, and the waves of a
// workgroup claim its items one at a time; every wave runs each of its items
// alone, so there is no cross-wave reduction and no barrier after the
// set-up.  Per chunk of 2048
// columns, lane l takes columns 32 l .. 32 l + 31: one 16-byte load per row
// (a whole row segment per instruction, full cache lines), the block code and
// group scale of its half-block, and the matching 32 bf16 of each token row
// of X.  Codes expand through a byte -> bf16x2 table of the NF4 levels (one
// copy per lane: conflict-free) and meet X in v_dot2_f32_bf16 (fp32
// accumulation); each half-block's sum is scaled by its c_hat in fp32.  The
// dequantized weight is therefore bf16(NF4[q]) * c_hat, the same reading as
// the other decode-regime kernels (within the matmul tolerance).
//
// Each wave keeps the loads of its next step (item, chunk) in flight while it
// computes the current one.  When the X rows of the whole group fit next to
// the table (kXL), they are copied into LDS once per workgroup (16 waves):
// the per-step loads are then the weight stream alone and registers allow 16
// waves per CU; T is formed there once too.  The one-token kernel issues the
// loads of X and T in the set-up before its first weight batch.  Otherwise (more
// tokens, or X too large) X and the partials are loaded with each step
// (8-wave workgroups).
// The LoRA term T B^T (T = bf16(s * sum of the down-projection partials) or
// as given) is a dot2 over lane pairs of adapter columns; wave sums use
// butterfly shuffles in a fixed order, so results are deterministic.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace qlora {

__constant__ uint32_t cGvQ4Level[3 * 16] = {QLORA_Q4_LEVEL_BITS};

constexpr int kGvRows = 4;             // rows per item
constexpr int kGvChunk = 2048;         // columns per chunk: 64 lanes x 32
constexpr int kGvMaxM = 4;
constexpr int kGvPS = 4;               // down-projection partial slices (at most)
constexpr int kGvLutBytes = 256 * 64 * 4;
constexpr int kGvXGroup = 80;          // LDS bytes per 32 bf16 of X (64 + 16 pad: conflict-free 16-byte reads)
constexpr int kGvXBytes = 163840 - kGvLutBytes - 1024 - 1024;   // LDS left for X and T
constexpr int kGvXJ = 6;               // X copy slots (64 x 16 bytes) per wave in the set-up (16 waves)
constexpr int kGvPSX = 12;             // partial slices of the one-token path (one per 2048 columns)

int small_m_gemv_max() { return kGvMaxM; }

// 8-bit constant table entry i, computed as the table is defined: E4M3-shaped
// magnitude (bias 7, subnormals at exponent 0) over 480 with IEEE division,
// negative half mirrored (creativeworksofknowledge.com, "QLoRA: Fine-Tune 70B
// on One GPU", The three innovations: constants quantized to 8 bits).  No
// memory load, so the set-up's first wait covers the X copy as well.
__device__ __forceinline__ float gv_t8_level(int i) {
  const int k = i >= 128 ? i - 128 : 127 - i;
  const int e = k >> 3, f = k & 7;
  const float mag = e == 0 ? ldexpf(static_cast<float>(f), -9) : ldexpf(static_cast<float>(8 + f), e - 10);
  const float v = __fdiv_rn(mag, 480.0f);
  return i >= 128 ? v : -v;
}

// Work plan in the kernel arguments (item0 / nch of SmGroup): the linears
// are ordered by chunks per item, most first; workgroup b of G takes items
// b, b + G, b + 2 G, ..., so every workgroup gets the same mix of linears
// and item lengths.  Its waves start on its first items and claim the next
// one from an LDS counter when they start an item, so they finish within
// about one item of each other (a fixed split over waves left some waves
// with two 6-chunk items where others had one).  Every item is still
// computed by one wave in chunk order: the results do not depend on which
// wave takes it.
__device__ __forceinline__ int gv_linear_of(const SmGroup &grp, int item) {
  int li = 0;
  while (li + 1 < grp.n && item >= grp.item0[li + 1]) ++li;
  return li;
}

// Claims the next item of the workgroup (all lanes get the same value).
__device__ __forceinline__ int gv_claim(int *counter, int lane) {
  int v = 0;
  if (lane == 0) v = atomicAdd(counter, 1);
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Everything one step (item, chunk) consumes from global memory, loaded as one
// batch.  Every batch issues the same loads (clamped addresses, masks applied
// where the values are used), so waiting for batch s while batch s + 1 is in
// flight is an exact count.
template <int kM, bool kP, bool kXL>
struct GvBatch {
  uint4 pk[kGvRows];                       // packed codes, columns 32 lane .. +31 of each row
  uint32_t code[kGvRows];                  // 8-bit block code of the lane's half-block
  float c2[kGvRows];                       // group scale
  uint4 xv[kXL ? 1 : kM][kXL ? 1 : 4];     // X[m, 32 lane .. +31] (kXL: from LDS instead)
  uint32_t bpair[kGvRows];                 // B[n, 2 lane .. 2 lane + 1]
  uint32_t tw[kXL ? 1 : kM][kXL ? 1 : (kP ? kGvPS * 2 : 1)];   // partials (fp32 bits) or T pair (bf16x2); kXL: LDS
};

struct GvStep {
  int item, c, li;
};

template <int kM, bool kP, bool kXL>
__device__ __forceinline__ void gv_load(const SmGroup &grp, const GvStep &st, int lane,
                                        GvBatch<kM, kP, kXL> &b) {
  const SmLinear &L = grp.lin[st.li];
  const int N = L.w.N, K = L.w.K, KB = K >> 6, r = L.r, M = grp.M;
  const int n0 = (st.item - grp.item0[st.li]) * kGvRows;
  const int k0 = st.c * kGvChunk + 32 * lane;
  const int kc = k0 < K ? k0 : K - 32;
#pragma unroll
  for (int i = 0; i < kGvRows; ++i) {
    const int64_t n = min(n0 + i, N - 1);
    const int64_t blk = n * KB + (kc >> 6);
    b.pk[i] = *reinterpret_cast<const uint4 *>(L.w.packed + ((n * K + kc) >> 1));
    b.code[i] = L.w.code8[blk];
    b.c2[i] = L.w.c2[blk >> 8];
  }
  if constexpr (!kXL) {
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const uint4 *xp = reinterpret_cast<const uint4 *>(L.X + static_cast<int64_t>(min(m, M - 1)) * K + kc);
#pragma unroll
      for (int q = 0; q < 4; ++q) b.xv[m][q] = xp[q];
    }
  }
  const int jc = 2 * lane < r ? 2 * lane : 0;
#pragma unroll
  for (int i = 0; i < kGvRows; ++i)
    b.bpair[i] = *reinterpret_cast<const uint32_t *>(L.B + static_cast<int64_t>(min(n0 + i, N - 1)) * r + jc);
  if constexpr (!kXL) {
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const int mc = min(m, M - 1);
      if constexpr (kP) {
#pragma unroll
        for (int s = 0; s < kGvPS; ++s) {
          const int sc = min(s, L.S - 1);
          const uint2 pv = *reinterpret_cast<const uint2 *>(L.P + (static_cast<int64_t>(sc) * M + mc) * r + jc);
          b.tw[m][2 * s] = pv.x;
          b.tw[m][2 * s + 1] = pv.y;
        }
      } else {
        b.tw[m][0] = *reinterpret_cast<const uint32_t *>(L.Tin + static_cast<int64_t>(mc) * r + jc);
      }
    }
  }
}

// T pair (bf16x2 of T[m, j], T[m, j + 1]) of linear L from the partials or as
// given; 0 past the token count.
template <bool kP>
__device__ __forceinline__ uint32_t gv_t_pair(const SmLinear &L, int M, int m, int j) {
  if (m >= M) return 0u;
  if constexpr (kP) {
    float t0 = 0.f, t1 = 0.f;
    for (int s = 0; s < L.S; ++s) {
      const float2 pv = *reinterpret_cast<const float2 *>(L.P + (static_cast<int64_t>(s) * M + m) * L.r + j);
      t0 += pv.x;
      t1 += pv.y;
    }
    return pack_bf16x2(L.scale * t0, L.scale * t1);
  } else {
    return *reinterpret_cast<const uint32_t *>(L.Tin + static_cast<int64_t>(m) * L.r + j);
  }
}

template <int kM, bool kP, bool kXL>
__global__ __launch_bounds__(kXL ? 1024 : 512) void k_sm_gemv(SmGroup grp) {
  constexpr int kWaves = kXL ? 16 : 8;
  __shared__ uint32_t sLut[256 * 64];   // word 64 * byte + lane: bf16x2 (NF4[lo], NF4[hi])
  __shared__ float sT8[256];
  __shared__ __attribute__((aligned(16))) uint8_t sX[kXL ? kGvXBytes : 16];
  __shared__ int sNext;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Items b, b + G, ... of the group for workgroup b, claimed by its waves
  // as in k_sm_gemv1.
  const int G = gridDim.x;
  const int nitems = grp.item0[grp.n];
  const int bid = blockIdx.x;
  const int cnt = nitems > bid ? (nitems - 1 - bid) / G + 1 : 0;   // items of this workgroup
  if (cnt == 0) return;                                // uniform per workgroup
  const bool active = wave < cnt;                      // uniform per wave

  // Next step of this wave, or `st` itself at the end (a harmless repeat
  // load).  nxt: the index claimed when the current item started.
  int nxt = cnt;
  auto advance = [&](const GvStep &st) __attribute__((always_inline)) {
    GvStep nx = st;
    if (st.c + 1 < grp.nch[st.li]) {
      ++nx.c;
    } else if (nxt < cnt) {
      nx.item = bid + G * nxt;
      nx.c = 0;
      nx.li = gv_linear_of(grp, nx.item);
    }
    return nx;
  };

  const int first = active ? bid + G * wave : bid;
  GvStep cur{first, 0, gv_linear_of(grp, first)};
  GvBatch<kM, kP, kXL> ba, bb;
  if (active) gv_load(grp, cur, lane, ba);            // first batch before the set-up below

  // Tables (and X) into LDS.
  {
    const uint32_t *lvt = cGvQ4Level + 16 * grp.lin[0].w.qtype;   // one 4-bit type per group
    for (int e = wave; e < 16; e += kWaves) {
      const float lo = u2f(lvt[e]);
#pragma unroll
      for (int j = 0; j < 16; ++j) sLut[64 * (e + 16 * j) + lane] = pack_bf16x2(lo, u2f(lvt[j]));
    }
    if (threadIdx.x < 256) sT8[threadIdx.x] = gv_t8_level(threadIdx.x);
    if (threadIdx.x == 0) sNext = kWaves;
    if constexpr (kXL) {
      // X (one token row: 80-byte groups of 32 bf16) and T of every linear.
      // X is copied in slots of 64 units of 16 bytes (one load instruction),
      // slot j of the group going to wave j % 16; all loads are issued before
      // the LDS stores, so the set-up costs one memory latency, overlapping
      // the first weight batch.  Wave w < n forms T of linear w.
      uint4 xr[kGvXJ];
      int xdst[kGvXJ];
#pragma unroll
      for (int j = 0; j < kGvXJ; ++j) {
        const int slot = wave + kWaves * j;
        xdst[j] = -1;
        xr[j] = make_uint4(0, 0, 0, 0);
        if (slot < grp.xs0[grp.n]) {
          int li = 0;
          while (li + 1 < grp.n && slot >= grp.xs0[li + 1]) ++li;
          const SmLinear &L = grp.lin[li];
          const int units = L.w.K >> 3;
          const int unit = (slot - grp.xs0[li]) * 64 + lane;
          xr[j] = reinterpret_cast<const uint4 *>(L.X)[min(unit, units - 1)];
          if (unit < units) xdst[j] = grp.xoff[li] + (unit >> 2) * kGvXGroup + (unit & 3) * 16;
        }
      }
      uint32_t tv = 0u;
      int tdst = -1, tj = 0;
      uint16_t *tout = nullptr;
      if (wave < grp.n) {
        const SmLinear &L = grp.lin[wave];
        tj = 2 * lane;
        if (tj < L.r) {
          if constexpr (kP) {
            float2 pv[kGvPS];
#pragma unroll
            for (int s2 = 0; s2 < kGvPS; ++s2)
              pv[s2] = *reinterpret_cast<const float2 *>(L.P + static_cast<int64_t>(min(s2, L.S - 1)) * L.r + tj);
            float t0 = 0.f, t1 = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < kGvPS; ++s2) {
              const bool on = s2 < L.S;
              t0 += on ? pv[s2].x : 0.f;
              t1 += on ? pv[s2].y : 0.f;
            }
            tv = pack_bf16x2(L.scale * t0, L.scale * t1);
          } else {
            tv = *reinterpret_cast<const uint32_t *>(L.Tin + tj);
          }
          tdst = grp.toff[wave] + 2 * tj;
          if (blockIdx.x == 0) tout = L.Tout;
        }
      }
#pragma unroll
      for (int j = 0; j < kGvXJ; ++j)
        if (xdst[j] >= 0) *reinterpret_cast<uint4 *>(sX + xdst[j]) = xr[j];
      if (tdst >= 0) {
        *reinterpret_cast<uint32_t *>(sX + tdst) = tv;
        if (tout) *reinterpret_cast<uint32_t *>(tout + tj) = tv;
      }
    }
  }
  __syncthreads();
  if (!active) return;                                  // no barrier follows

  float acc[kGvRows][kM];
#pragma unroll
  for (int i = 0; i < kGvRows; ++i)
#pragma unroll
    for (int m = 0; m < kM; ++m) acc[i][m] = 0.f;

  // Consume batch `b` of step `st` (its loads issued one step earlier).
  auto compute = [&](const GvStep &st, const GvBatch<kM, kP, kXL> &b) __attribute__((always_inline)) {
    const SmLinear &L = grp.lin[st.li];
    const int N = L.w.N, K = L.w.K, r = L.r, M = grp.M;
    const int k0 = st.c * kGvChunk + 32 * lane;
    const bool kin = k0 < K;                            // K % 64 == 0: all 32 columns or none
    const float mean = L.w.mean[0];
    uint4 xl[kM][4];
    if constexpr (kXL) {
      const int kc = kin ? k0 : K - 32;
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const uint8_t *xp = sX + grp.xoff[st.li] + (min(m, M - 1) * (K >> 5) + (kc >> 5)) * kGvXGroup;
#pragma unroll
        for (int q = 0; q < 4; ++q) xl[m][q] = *reinterpret_cast<const uint4 *>(xp + 16 * q);
      }
    }
#pragma unroll
    for (int i = 0; i < kGvRows; ++i) {
      const float chat = kin ? decode_absmax(sT8[b.code[i]], b.c2[i], mean) : 0.f;
      const uint32_t words[4] = {b.pk[i].x, b.pk[i].y, b.pk[i].z, b.pk[i].w};
      float part[kM];
#pragma unroll
      for (int m = 0; m < kM; ++m) part[m] = 0.f;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t wpair = sLut[64 * ((words[wd] >> (8 * q)) & 0xffu) + lane];
#pragma unroll
          for (int m = 0; m < kM; ++m) {
            const uint4 &x4 = kXL ? xl[m][wd] : b.xv[kXL ? 0 : m][kXL ? 0 : wd];
            const uint32_t xpair = q == 0 ? x4.x : q == 1 ? x4.y : q == 2 ? x4.z : x4.w;
            part[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wpair),
                                                      __builtin_bit_cast(bf16x2_t, xpair), part[m], false);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < kM; ++m) acc[i][m] = __builtin_fmaf(chat, part[m], acc[i][m]);
    }
    if (st.c + 1 < grp.nch[st.li]) return;
    // Last chunk of the item: LoRA term, wave sums, stores.
    const int n0 = (st.item - grp.item0[st.li]) * kGvRows;
    const bool jok = 2 * lane < r;
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      uint32_t tpair;
      if constexpr (kXL) {
        tpair = jok && m < M ? reinterpret_cast<const uint32_t *>(sX + grp.toff[st.li])[m * (r >> 1) + lane] : 0u;
      } else {
        if constexpr (kP) {
          float t0 = 0.f, t1 = 0.f;
#pragma unroll
          for (int s = 0; s < kGvPS; ++s)
            if (s < L.S) {
              t0 += u2f(b.tw[m][2 * s]);
              t1 += u2f(b.tw[m][2 * s + 1]);
            }
          tpair = pack_bf16x2(L.scale * t0, L.scale * t1);
        } else {
          tpair = b.tw[m][0];
        }
        if (!jok || m >= M) tpair = 0u;
        if (L.Tout && n0 == 0 && jok && m < M)
          *reinterpret_cast<uint32_t *>(L.Tout + static_cast<int64_t>(m) * r + 2 * lane) = tpair;
      }
#pragma unroll
      for (int i = 0; i < kGvRows; ++i) {
        const float v = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, tpair),
                                                        __builtin_bit_cast(bf16x2_t, b.bpair[i]), acc[i][m], false);
        const float sum = wave_sum(v);
        acc[i][m] = 0.f;
        const int n = n0 + i;
        if (lane == 0 && m < M && n < N) L.Y[static_cast<int64_t>(m) * N + n] = f32_to_bf16(sum);
      }
    }
  };

  // Two batches alternate: loads of step s + 1 are issued before step s is
  // consumed (a register copy would wait for them).
  auto step = [&](GvBatch<kM, kP, kXL> &now, GvBatch<kM, kP, kXL> &next) __attribute__((always_inline)) -> bool {
    if (cur.c == 0) nxt = gv_claim(&sNext, lane);
    const GvStep nx = advance(cur);
    const bool more = nx.item != cur.item || nx.c != cur.c;
    gv_load(grp, nx, lane, next);
    compute(cur, now);
    cur = nx;
    return more;
  };
  while (step(ba, bb) && step(bb, ba)) {
  }
}

// ---------------------------------------------------------------------------
// M = 1 with X and T of the whole group in LDS: the per-step loads are the
// weight stream plus three narrow loads shared by the 4 rows of an item
// (block codes, group scales, B rows), redistributed with lane permutes, so a
// step issues 8 vector memory instructions for 4 KB of packed weights.
struct Gv1Batch {
  uint4 pk[kGvRows];   // packed codes of row i, columns 32 lane .. +31
  uint32_t cw0, cw1;   // codes of row (lane >> 4), blocks 2 (lane & 15) and +1 of the chunk
  float c2v;           // group scale: row (lane >> 1) & 3, first group of the chunk + (lane & 1)
  uint4 bq;            // B[row (lane >> 4), 8 (lane & 15) .. +7]
};

__device__ __forceinline__ void gv1_load(const SmGroup &grp, const GvStep &st, int lane, Gv1Batch &b) {
  const SmLinear &L = grp.lin[st.li];
  const int N = L.w.N, K = L.w.K, KB = K >> 6, r = L.r;
  const int64_t nb2 = (static_cast<int64_t>(N) * KB + 255) >> 8;
  const int n0 = (st.item - grp.item0[st.li]) * kGvRows;
  const int k0 = st.c * kGvChunk + 32 * lane;
  const int kc = k0 < K ? k0 : K - 32;
  // B first: it is used only on an item's last chunk, so on other steps its
  // registers are free for the compiler to reuse, which waits for the load
  // that writes them; as the oldest load of the batch that wait is short.
  {
    const int64_t n = min(n0 + (lane >> 4), N - 1);
    const int j = 8 * (lane & 15);
    b.bq = *reinterpret_cast<const uint4 *>(L.B + n * r + (j < r ? j : 0));
  }
#pragma unroll
  for (int i = 0; i < kGvRows; ++i) {
    const int64_t n = min(n0 + i, N - 1);
    b.pk[i] = *reinterpret_cast<const uint4 *>(L.w.packed + ((n * K + kc) >> 1));
  }
  {
    const int64_t n = min(n0 + (lane >> 4), N - 1);
    const int blk = st.c * kGvChunk / 64 + 2 * (lane & 15);
    b.cw0 = L.w.code8[n * KB + min(blk, KB - 1)];
    b.cw1 = L.w.code8[n * KB + min(blk + 1, KB - 1)];
  }
  {
    const int64_t n = min(n0 + ((lane >> 1) & 3), N - 1);
    const int64_t g = ((n * KB + st.c * kGvChunk / 64) >> 8) + (lane & 1);
    b.c2v = L.w.c2[min(g, nb2 - 1)];
  }
}

template <bool kP>
__global__ __launch_bounds__(1024) void k_sm_gemv1(SmGroup grp) {
  constexpr int kWaves = 16;
  // One LDS block so that the table sits at address 0: a table read is then a
  // single v_perm address with no base add.
  __shared__ struct __attribute__((aligned(16))) {
    uint32_t lut[256 * 64];   // word 64 * byte + lane: bf16x2 (NF4[lo], NF4[hi])
    float t8[256];
    uint8_t x[kGvXBytes];
    float mean[kSmMaxGroup];  // each linear's constant mean
    int next;                 // the workgroup's next unclaimed item
  } sm;
  uint32_t *const sLut = sm.lut;
  float *const sT8 = sm.t8;
  uint8_t *const sX = sm.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Workgroup b takes items b, b + G, b + 2 G, ... (G workgroups): every
  // workgroup gets the same mix of linears and of item lengths.  Its waves
  // start on its first 16 items and claim the next one from an LDS counter
  // whenever they start an item (the linears are ordered longest item first,
  // so the long items go first).
  const int G = gridDim.x;
  const int nitems = grp.item0[grp.n];
  const int bid = blockIdx.x;
  const int cnt = nitems > bid ? (nitems - 1 - bid) / G + 1 : 0;   // items of this workgroup
  if (cnt == 0) return;                                // uniform per workgroup
  const bool active = wave < cnt;                      // uniform per wave

  int nxt = cnt;                                       // index claimed when the current item started
  auto advance = [&](const GvStep &st) __attribute__((always_inline)) {
    GvStep nx = st;
    if (st.c + 1 < grp.nch[st.li]) {
      ++nx.c;
    } else if (nxt < cnt) {
      nx.item = bid + G * nxt;
      nx.c = 0;
      nx.li = gv_linear_of(grp, nx.item);
    }
    return nx;
  };

  const int first = active ? bid + G * wave : bid;
  GvStep cur{first, 0, gv_linear_of(grp, first)};
  Gv1Batch ba, bb;

  // Set-up: the first weight batch, then the X and T loads, go out before
  // anything waits (storing X and T then waits for the batch too: loads
  // complete in order).  The X copy's slot bounds are read once, so that
  // finding a slot's linear needs no memory round trip.
  {
    if (active) gv1_load(grp, cur, lane, ba);
    int xs[kSmMaxGroup + 1];                           // slot bounds of the linears' X copies
#pragma unroll
    for (int i = 0; i <= kSmMaxGroup; ++i) xs[i] = grp.xs0[i];
    uint4 xr[kGvXJ];
    int xdst[kGvXJ];
#pragma unroll
    for (int j = 0; j < kGvXJ; ++j) {
      const int slot = wave + kWaves * j;
      xdst[j] = -1;
      xr[j] = make_uint4(0, 0, 0, 0);
      if (slot < xs[grp.n]) {
        int li = 0;
#pragma unroll
        for (int i = 1; i < kSmMaxGroup; ++i) li += (i < grp.n && slot >= xs[i]) ? 1 : 0;
        const SmLinear &L = grp.lin[li];
        const int units = L.w.K >> 3;
        const int unit = (slot - xs[li]) * 64 + lane;
        xr[j] = reinterpret_cast<const uint4 *>(L.X)[min(unit, units - 1)];
        if (unit < units) xdst[j] = grp.xoff[li] + (unit >> 2) * kGvXGroup + (unit & 3) * 16;
      }
    }
    // T of linear w from wave w: its partial slices (or T as given).
    const int tj = 2 * lane;
    const bool tact = wave < grp.n && tj < grp.lin[wave < grp.n ? wave : 0].r;
    float2 pv[kP ? kGvPSX : 1];
    uint32_t tin = 0u;
    if (tact) {
      const SmLinear &L = grp.lin[wave];
      if constexpr (kP) {
#pragma unroll
        for (int s2 = 0; s2 < kGvPSX; ++s2)
          pv[s2] = *reinterpret_cast<const float2 *>(L.P + static_cast<int64_t>(min(s2, L.S - 1)) * L.r + tj);
      } else {
        tin = *reinterpret_cast<const uint32_t *>(L.Tin + tj);
      }
    }

    const uint32_t *lvt = cGvQ4Level + 16 * grp.lin[0].w.qtype;   // one 4-bit type per group
    for (int e = wave; e < 16; e += kWaves) {
      const float lo = u2f(lvt[e]);
#pragma unroll
      for (int j = 0; j < 16; ++j) sLut[64 * (e + 16 * j) + lane] = pack_bf16x2(lo, u2f(lvt[j]));
    }
    if (threadIdx.x < 256) sT8[threadIdx.x] = gv_t8_level(threadIdx.x);
    if (threadIdx.x == 0) sm.next = kWaves;
    // The means come from LDS in the step loop: a global load there would be
    // the youngest load when the step waits, and waiting for it would also
    // wait for the next batch.
    if (threadIdx.x < grp.n) sm.mean[threadIdx.x] = grp.lin[threadIdx.x].w.mean[0];
    if (tact) {
      const SmLinear &L = grp.lin[wave];
      uint32_t tv = tin;
      if constexpr (kP) {
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < kGvPSX; ++s2) {
          const bool on = s2 < L.S;
          t0 += on ? pv[s2].x : 0.f;
          t1 += on ? pv[s2].y : 0.f;
        }
        tv = pack_bf16x2(L.scale * t0, L.scale * t1);
      }
      *reinterpret_cast<uint32_t *>(sX + grp.toff[wave] + 2 * tj) = tv;
      if (bid == 0 && L.Tout) *reinterpret_cast<uint32_t *>(L.Tout + tj) = tv;
    }
#pragma unroll
    for (int j = 0; j < kGvXJ; ++j)
      if (xdst[j] >= 0) *reinterpret_cast<uint4 *>(sX + xdst[j]) = xr[j];
  }
  // Storing X waited for the first batch already (loads complete in order);
  // saying so here leaves no load of the set-up outstanding at the loop, so
  // that the compiler's waits in the loop count only the loop's own batches.
  __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0)
  __syncthreads();
  if (!active) return;                                  // no barrier follows

  float acc[kGvRows];
#pragma unroll
  for (int i = 0; i < kGvRows; ++i) acc[i] = 0.f;

  auto compute = [&](const GvStep &st, const Gv1Batch &b) __attribute__((always_inline)) {
    const SmLinear &L = grp.lin[st.li];
    const int N = L.w.N, K = L.w.K, KB = K >> 6, r = L.r;
    const int k0 = st.c * kGvChunk + 32 * lane;
    const bool kin = k0 < K;                            // K % 64 == 0: all 32 columns or none
    const int kc = kin ? k0 : K - 32;
    const float mean = sm.mean[st.li];
    const int n0 = (st.item - grp.item0[st.li]) * kGvRows;
    uint4 xl[4];
    const uint8_t *xp = sX + grp.xoff[st.li] + (kc >> 5) * kGvXGroup;
#pragma unroll
    for (int q = 0; q < 4; ++q) xl[q] = *reinterpret_cast<const uint4 *>(xp + 16 * q);
    const uint32_t cwp = (b.cw0 & 0xffu) | ((b.cw1 & 0xffu) << 8);
    const uint32_t lane4 = 4u * lane;
#pragma unroll
    for (int i = 0; i < kGvRows; ++i) {
      // Code of (row i, block of this lane) from lane 16 i + lane / 4; group
      // scale from lane 2 i + (its group - the chunk's first group of row i).
      const uint32_t cv = __builtin_amdgcn_ds_bpermute(4 * (16 * i + (lane >> 2)), cwp);
      const uint32_t code = (cv >> (8 * ((lane >> 1) & 1))) & 0xffu;
      const int64_t n = min(n0 + i, N - 1);
      const int64_t b0 = n * KB + st.c * kGvChunk / 64;
      const int sel = static_cast<int>(((b0 + (lane >> 1)) >> 8) - (b0 >> 8));
      const float c2 = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (2 * i + sel), __float_as_int(b.c2v)));
      const float chat = kin ? decode_absmax(sT8[code], c2, mean) : 0.f;
      const uint32_t words[4] = {b.pk[i].x, b.pk[i].y, b.pk[i].z, b.pk[i].w};
      float part = 0.f;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // Table byte address 256 * byte + 4 * lane in one v_perm: byte 0 of
          // the result is 4 * lane, byte 1 is code byte q of the word.
          const uint32_t addr = __builtin_amdgcn_perm(words[wd], lane4, 0x0C0C0000u | ((4u + q) << 8));
          const uint32_t wpair = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(sLut) + addr);
          const uint32_t xpair = q == 0 ? xl[wd].x : q == 1 ? xl[wd].y : q == 2 ? xl[wd].z : xl[wd].w;
          part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wpair),
                                                 __builtin_bit_cast(bf16x2_t, xpair), part, false);
        }
      }
      acc[i] = __builtin_fmaf(chat, part, acc[i]);
    }
    if (st.c + 1 < grp.nch[st.li]) return;
    // Last chunk of the item: LoRA term (lane: row lane / 16, adapter columns
    // 8 (lane % 16) .. +7), wave sums, stores.  The lane index goes through an
    // empty asm so that its T address is formed here: hoisted out of the step
    // loop it would be spilled, and reloading a spill waits for every load in
    // flight, the next batch included.
    int lj = lane;
    asm volatile("" : "+v"(lj));
    const int j = 8 * (lj & 15);
    float lp = 0.f;
    if (j < r) {
      const uint4 tq = *reinterpret_cast<const uint4 *>(sX + grp.toff[st.li] + 2 * j);
      const uint32_t tw[4] = {tq.x, tq.y, tq.z, tq.w};
      const uint32_t bw[4] = {b.bq.x, b.bq.y, b.bq.z, b.bq.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        lp = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, tw[e]), __builtin_bit_cast(bf16x2_t, bw[e]),
                                             lp, false);
    }
#pragma unroll
    for (int i = 0; i < kGvRows; ++i) {
      const float sum = wave_sum(acc[i] + ((lane >> 4) == i ? lp : 0.f));
      acc[i] = 0.f;
      if (lane == 0 && n0 + i < N) L.Y[n0 + i] = f32_to_bf16(sum);
    }
  };

  auto step = [&](Gv1Batch &now, Gv1Batch &next) __attribute__((always_inline)) -> bool {
    if (cur.c == 0) nxt = gv_claim(&sm.next, lane);
    const GvStep nx = advance(cur);
    const bool more = nx.item != cur.item || nx.c != cur.c;
    gv1_load(grp, nx, lane, next);
    // All of the next batch is issued before this one is consumed: moving
    // the consumption up would wait for this batch before the next is out.
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, now);
    cur = nx;
    return more;
  };
  while (step(ba, bb) && step(bb, ba)) {
  }
}

// ---------------------------------------------------------------------------
// One-token down-projection partials: P[c][j] = X[chunk c] . A[j, chunk c]
// (fp32, unscaled), one wave per (linear, adapter row j, 2048-column chunk c):
// a 1 KB load of the A row segment and of X, 16 dot2 per lane and a wave sum
// in a fixed order.  Slices are summed (in slice order) by the GEMV set-up.
__global__ __launch_bounds__(256) void k_sm_down_gemv(SmGroup grp) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gw >= grp.dg0[grp.n]) return;
  int li = 0;
  while (li + 1 < grp.n && gw >= grp.dg0[li + 1]) ++li;
  const SmLinear &L = grp.lin[li];
  if (!L.P) return;
  const int K = L.w.K, r = L.r;
  const int rem = gw - grp.dg0[li];
  const int j = rem % r, c = rem / r;
  const int k0 = c * kGvChunk + 32 * lane;
  const bool kin = k0 < K;
  const int kc = kin ? k0 : K - 32;
  const uint4 *ap = reinterpret_cast<const uint4 *>(L.A + static_cast<int64_t>(j) * K + kc);
  const uint4 *xp = reinterpret_cast<const uint4 *>(L.X + kc);
  uint4 a[4], x[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    a[q] = ap[q];
    x[q] = xp[q];
  }
  float part = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t aw[4] = {a[q].x, a[q].y, a[q].z, a[q].w};
    const uint32_t xw[4] = {x[q].x, x[q].y, x[q].z, x[q].w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, aw[e]), __builtin_bit_cast(bf16x2_t, xw[e]),
                                             part, false);
  }
  const float sum = wave_sum(kin ? part : 0.f);
  if (lane == 0) L.P[static_cast<int64_t>(c) * r + j] = sum;
}

int small_m_gemv_slices(int K) { return (K + kGvChunk - 1) / kGvChunk; }

bool small_m_gemv_xl(const SmGroup &grp) {
  if (grp.M != 1) return false;
  int64_t xbytes = 0, tbytes = 0;
  int slots = 0;
  for (int i = 0; i < grp.n; ++i) {
    const SmLinear &L = grp.lin[i];
    if (small_m_gemv_slices(L.w.K) > kGvPSX) return false;
    xbytes += static_cast<int64_t>(L.w.K >> 5) * kGvXGroup;
    tbytes += static_cast<int64_t>(L.r) * 2;
    slots += ((L.w.K >> 3) + 63) / 64;
  }
  return xbytes + tbytes <= kGvXBytes && slots <= kGvXJ * 16;
}

hipError_t launch_small_m_down_gemv(SmGroup &grp, hipStream_t s) {
  int items = 0;
  for (int i = 0; i < grp.n; ++i) {
    grp.dg0[i] = items;
    items += grp.lin[i].r * small_m_gemv_slices(grp.lin[i].w.K);
  }
  grp.dg0[grp.n] = items;
  hipLaunchKernelGGL(k_sm_down_gemv, dim3((items + 3) / 4), dim3(256), 0, s, grp);
  return hipGetLastError();
}

static int gv_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

template <int kM, bool kXL>
static void gv_launch(bool p, int grid, const SmGroup &grp, hipStream_t s) {
  constexpr int threads = kXL ? 1024 : 512;
  if (p)
    hipLaunchKernelGGL((k_sm_gemv<kM, true, kXL>), dim3(grid), dim3(threads), 0, s, grp);
  else
    hipLaunchKernelGGL((k_sm_gemv<kM, false, kXL>), dim3(grid), dim3(threads), 0, s, grp);
}

hipError_t launch_small_m_gemv(SmGroup &grp, hipStream_t s) {
  // Linears with more chunks per item first (stable), so that a workgroup
  // whose range spans two linears starts on the longer items.
  auto chunks = [](const SmLinear &L) { return (L.w.K + kGvChunk - 1) / kGvChunk; };
  for (int i = 1; i < grp.n; ++i)
    for (int j = i; j > 0 && chunks(grp.lin[j]) > chunks(grp.lin[j - 1]); --j) std::swap(grp.lin[j], grp.lin[j - 1]);
  int items = 0;
  int64_t xbytes = 0;
  for (int i = 0; i < grp.n; ++i) {
    const int tiles = (grp.lin[i].w.N + kGvRows - 1) / kGvRows;
    grp.item0[i] = items;
    grp.nch[i] = (grp.lin[i].w.K + kGvChunk - 1) / kGvChunk;
    grp.xoff[i] = static_cast<int>(xbytes);
    items += tiles;
    xbytes += static_cast<int64_t>(grp.M) * (grp.lin[i].w.K >> 5) * kGvXGroup;
  }
  {
    int64_t t = xbytes;
    int xs = 0;
    for (int i = 0; i < grp.n; ++i) {
      grp.toff[i] = static_cast<int>(t);
      t += static_cast<int64_t>(grp.M) * grp.lin[i].r * 2;
      grp.xs0[i] = xs;
      xs += ((grp.lin[i].w.K >> 3) + 63) / 64;
    }
    grp.xs0[grp.n] = xs;
  }
  grp.item0[grp.n] = items;
  const bool xl = small_m_gemv_xl(grp);
  const int cus = gv_cu_count();
  // kXL: one 16-wave workgroup per CU; else two 8-wave workgroups per CU.
  const int waves = xl ? 16 : 8;
  const int grid = std::max(1, std::min(xl ? cus : 2 * cus, (items + waves - 1) / waves));
  const bool p = grp.lin[0].P != nullptr;
  if (xl) {
    if (p)
      hipLaunchKernelGGL(k_sm_gemv1<true>, dim3(grid), dim3(1024), 0, s, grp);
    else
      hipLaunchKernelGGL(k_sm_gemv1<false>, dim3(grid), dim3(1024), 0, s, grp);
    return hipGetLastError();
  }
  switch (grp.M) {
    case 1: gv_launch<1, false>(p, grid, grp, s); break;
    case 2: gv_launch<2, false>(p, grid, grp, s); break;
    case 3: gv_launch<3, false>(p, grid, grp, s); break;
    default: gv_launch<4, false>(p, grid, grp, s); break;
  }
  return hipGetLastError();
}

}  // namespace qlora
