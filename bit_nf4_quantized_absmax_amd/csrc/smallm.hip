// Small-M forward (M <= 64 tokens, the decode regime), for one linear or a
// group of independent linears sharing M:
//     Y [M, N] = X deq(W)^T + T B^T,   T = s X A^T [M, r]
// The frozen weight is read once, as packed NF4, and dequantized in registers
// on its way into the product (automatone.win, "QLoRA paper explained", How
// it works: dequantize on the fly, compute, discard the 16-bit copy).  The
// work is bound by HBM bandwidth and by load latency, so both kernels issue
// every load a wave needs before the first use.
//
// k_sm_down: partial LoRA down-projections P[s] = X[:, chunk s] A[:, chunk s]^T
//   (fp32, unscaled; at most 4 column chunks), one workgroup per (chunk, 16
//   adapter rows); the 16 waves split the chunk and are summed in LDS in wave
//   order.
// k_sm_main: one workgroup per 16 weight rows x the whole K.  Wave w takes the
//   blocks b = w, w + 16, ...; lane (n = l % 16, g = l / 16) loads 8 packed
//   bytes (codes 16 g .. 16 g + 15 of block b of row n), expands them through
//   a byte -> bf16x2 table of the NF4 levels into MFMA 16x16x32 operands (rows =
//   tokens, padded to 16) and scales each block's partial product by its
//   c_hat in fp32.  The dequantized weight is therefore bf16(NF4[q]) * c_hat
//   rather than bf16(NF4[q] * c_hat): the constant is applied after the
//   bf16 rounding of the level, an exact scaling per block up to fp32
//   rounding of the sums, within the matmul tolerance.  Waves 0 .. 3 add
//   T B^T, T = bf16(s * sum of the partials) (or T as given).  The 16 wave
//   accumulators are summed in LDS in wave order: results are deterministic.
#include <algorithm>
#include <cstdlib>

#include "common.h"
#include "launch.h"

namespace qlora {

__constant__ uint32_t cSmQ4Level[3 * 16] = {QLORA_Q4_LEVEL_BITS};
__constant__ uint32_t cSmT8Level[256] = {QLORA_T8_LEVEL_BITS};

constexpr int kSmMaxM = 64;
constexpr int kSmRows = 16;           // weight rows per main workgroup
constexpr int kSmWaves = 16;
constexpr int kSmThreads = kSmWaves * 64;
constexpr int kSmDownSteps = 8;       // 32-column MFMA steps per load batch in k_sm_down
constexpr int kSmMaxSplits = 2;       // column chunks of the down-projection (partials)
constexpr int kSmWait0 = 0xC07F;      // s_waitcnt lgkmcnt(0)

// The decode-regime threshold: kSmMaxM, or the environment variable
// QLORA_SMALL_M_MAX (a decimal integer, clamped to [0, kSmMaxM]; read once per
// process), so that the tile kernels can be timed at small M.  0 sends every
// M to the tile kernels.
int small_m_max() {
  static const int v = [] {
    const char *e = getenv("QLORA_SMALL_M_MAX");
    if (!e || !*e) return kSmMaxM;
    char *end = nullptr;
    const long x = strtol(e, &end, 10);
    if (!end || *end != '\0' || x < 0) return kSmMaxM;
    return static_cast<int>(std::min<long>(x, kSmMaxM));
  }();
  return v;
}

__device__ __forceinline__ void sm_barrier_lds_only() {
  // Barrier after LDS writes that leaves this wave's global loads in flight
  // (__syncthreads would also wait for them).
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kSmWait0);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ int sm_find(const int *start, int n) {
  int i = 0;
  while (i + 1 < n && static_cast<int>(blockIdx.x) >= start[i + 1]) ++i;
  return i;
}

// 8 consecutive bf16 of a row (zero past `len`); vector load when the row
// start and j are 16-byte aligned.
__device__ __forceinline__ bf16x8_t load8_bf16(const uint16_t *row, int j, int len, bool vec) {
  if (vec) {
    if (j < len) return *reinterpret_cast<const bf16x8_t *>(row + j);
    return bf16x8_t{};
  }
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (j + e < len) ? row[j + e] : static_cast<uint16_t>(0);
  return __builtin_bit_cast(bf16x8_t, v);
}

// 8 bf16 of X at (m, k), address clamped into X: rows m >= M repeat row M - 1
// (their results are never stored) and columns k >= K are only read for
// blocks whose products are skipped or multiplied by zero.  No branch, so the
// compiler's wait counts stay exact.
__device__ __forceinline__ bf16x8_t load_x(const uint16_t *X, int m, int M, int K, int k) {
  return *reinterpret_cast<const bf16x8_t *>(X + static_cast<int64_t>(min(m, M - 1)) * K + min(k, K - 8));
}

// ---------------------------------------------------------------------------
template <int kMB>
__global__ __launch_bounds__(kSmThreads) void k_sm_down(SmGroup grp) {
  __shared__ float red[kSmWaves][kMB * 16][17];
  const int li = sm_find(grp.down_start, grp.n);
  const SmLinear &L = grp.lin[li];
  const int M = grp.M, K = L.w.K, r = L.r;
  const int local = blockIdx.x - grp.down_start[li];
  const int jt = local % L.jtiles, s = local / L.jtiles;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar loads and branches
  const int nl = lane & 15, g = lane >> 4;
  const int j = 16 * jt + nl;
  const int kw = L.kw;                                  // columns per wave, multiple of 32
  const int kbeg = (s * kSmWaves + wave) * kw;
  const int kend = min(kbeg + kw, K);
  const uint16_t *arow = L.A + static_cast<int64_t>(min(j, r - 1)) * K;

  f32x4_t acc[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = kbeg; k0 < kend; k0 += 32 * kSmDownSteps) {
    bf16x8_t av[kSmDownSteps];
#pragma unroll
    for (int t = 0; t < kSmDownSteps; ++t) {
      const int k = k0 + 32 * t + 8 * g;
      // Clamped, branch-free: steps past kend are skipped below and adapter
      // rows j >= r (arow clamped) are never stored.
      av[t] = *reinterpret_cast<const bf16x8_t *>(arow + min(k, K - 8));
    }
#pragma unroll
    for (int t = 0; t < kSmDownSteps; ++t) {
      const int k = k0 + 32 * t + 8 * g;
      if (k0 + 32 * t >= kend) break;                   // uniform per wave
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(load_x(L.X, 16 * mb + nl, M, K, k), av[t], acc[mb], 0, 0,
                                                         0);
    }
  }
  // D layout of MFMA 16x16: lane holds column (adapter row) nl, rows 4 g + e.
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][16 * mb + 4 * g + e][nl] = acc[mb][e];
  __syncthreads();
  float *P = L.P + static_cast<int64_t>(s) * M * r;
  for (int idx = threadIdx.x; idx < kMB * 16 * 16; idx += kSmThreads) {
    const int m = idx >> 4, c = idx & 15, jj = 16 * jt + c;
    if (m < M && jj < r) {
      float v = red[0][m][c];
#pragma unroll
      for (int w = 1; w < kSmWaves; ++w) v += red[w][m][c];
      P[static_cast<int64_t>(m) * r + jj] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// LoRA term of k_sm_main: acc[mb] += T B^T for this wave's 32 adapter columns
// (lane holds T[16 mb + nl, j0 .. j0+7] and B[n, j0 .. j0+7]); T is formed from
// the partials (bf16 of s times their fp32 sum in slice order) or taken as given.
template <int kMB, int kPS, bool kP>
struct SmLora {
  bf16x8_t bop;
  bf16x8_t top[kMB];
  f32x4_t pv[kMB][kPS][2];

  // Loads use clamped addresses so that every wave issues the same number;
  // masks are applied where the values are consumed.
  __device__ __forceinline__ void load(const SmLinear &L, int M, int n, int nl, int jc) {
    const int r = L.r;
    bop = *reinterpret_cast<const bf16x8_t *>(L.B + static_cast<int64_t>(n) * r + jc);
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const int mc = min(16 * mb + nl, M - 1);
      if constexpr (kP) {
#pragma unroll
        for (int s = 0; s < kPS; ++s) {
          const int sc = min(s, L.S - 1);
          const f32x4_t *pp = reinterpret_cast<const f32x4_t *>(L.P + (static_cast<int64_t>(sc) * M + mc) * r + jc);
          pv[mb][s][0] = pp[0];
          pv[mb][s][1] = pp[1];
        }
      } else {
        top[mb] = *reinterpret_cast<const bf16x8_t *>(L.Tin + static_cast<int64_t>(mc) * r + jc);
      }
    }
  }

  __device__ __forceinline__ void apply(const SmLinear &L, int M, int nl, int j0, bool jok, bool write_t,
                                        f32x4_t (&acc)[kMB]) {
    const int r = L.r;
    const bf16x8_t b = jok ? bop : bf16x8_t{};
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const int m = 16 * mb + nl;
      const bool ok = jok && m < M;
      bf16x8_t t8 = top[mb];
      if constexpr (kP) {
        float t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = 0.f;
#pragma unroll
        for (int s = 0; s < kPS; ++s)
          if (s < L.S)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              t[e] += pv[mb][s][0][e];
              t[4 + e] += pv[mb][s][1][e];
            }
        uint32_t tw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) tw[e] = pack_bf16x2(L.scale * t[2 * e], L.scale * t[2 * e + 1]);
        t8 = __builtin_bit_cast(bf16x8_t, tw);
      }
      if (!ok) t8 = bf16x8_t{};
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t8, b, acc[mb], 0, 0, 0);
      if (write_t && ok) {
        uint16_t tv[8];
        __builtin_memcpy(tv, &t8, sizeof(tv));
#pragma unroll
        for (int e = 0; e < 8; ++e) L.Tout[static_cast<int64_t>(m) * r + j0 + e] = tv[e];
      }
    }
  }
};

template <int kMB, bool kP>
__global__ __launch_bounds__(kSmThreads) void k_sm_main(SmGroup grp) {
  // Blocks per load batch and wave: the batch's weight and X loads are all in
  // registers at once (X: 8 kMB VGPRs per block).  With kLoraFirst the LoRA
  // operands are loaded with the first batch and applied before it; larger
  // token counts apply them after the main loop to leave room for X.
  constexpr bool kLoraFirst = kMB <= 2;
  constexpr int kBlk = kMB == 1 ? 6 : (kMB == 2 ? 3 : (kMB == 3 ? 2 : 1));
  constexpr int kPS = kSmMaxSplits;
  // Byte -> bf16x2 (NF4[lo nibble], NF4[hi nibble]), one copy per lane so that
  // the 64 lanes of a lookup hit 64 distinct banks: word 64 * byte + lane.
  __shared__ uint32_t sLut[256 * 64];
  __shared__ float sT8[256];
  __shared__ float red[kSmWaves][kMB * 16][kSmRows + 1];
  const int li = sm_find(grp.main_start, grp.n);
  const SmLinear &L = grp.lin[li];
  const int M = grp.M, N = L.w.N, K = L.w.K, r = L.r;
  const int tile = blockIdx.x - grp.main_start[li];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar loads and branches
  const int nl = lane & 15, g = lane >> 4;
  const int n0 = tile * kSmRows;
  const int n = min(n0 + nl, N - 1);            // rows past N are computed, never stored
  const int KB = K >> 6;
  const int j0 = 32 * (wave & 3) + 8 * g;       // LoRA columns of waves 0 .. 3
  const bool lora_wave = 32 * wave < r;
  const bool jok = lora_wave && j0 < r;
  const int jc = jok ? j0 : 0;                  // r % 8 == 0: 16-byte aligned rows

  // Issue order: table, LoRA operands, weights, X; every later wait then
  // leaves the loads behind it in flight.
  const float mean = L.w.mean[0];
  const float t8v = u2f(cSmT8Level[threadIdx.x & 255]);
  __builtin_amdgcn_sched_barrier(0);

  SmLora<kLoraFirst ? kMB : 1, kPS, kP> lora;
  if constexpr (kLoraFirst) lora.load(L, M, n, nl, jc);
  __builtin_amdgcn_sched_barrier(0);

  uint2 pk[kBlk];
  uint32_t code[kBlk];
  float c2v[kBlk];
  bf16x8_t xb[kBlk][kMB][2];
  const uint8_t *prow = L.w.packed + static_cast<int64_t>(n) * (K >> 1);
  const int64_t rowblk = static_cast<int64_t>(n) * KB;
  // Block b of this wave's batch: lane (nl, g) holds codes 16 g .. 16 g + 15 of
  // row n (bytes 8 g ..), MFMA t contracts elements 16 g + 8 t .. +7 of every
  // lane group, so each MFMA stays inside one block and c_hat scales its sum.
  auto load_batch = [&](int b0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kBlk; ++u) {
      const int b = min(b0 + u * kSmWaves, KB - 1);
      pk[u] = *reinterpret_cast<const uint2 *>(prow + 32 * b + 8 * g);
      code[u] = L.w.code8[rowblk + b];
      c2v[u] = L.w.c2[(rowblk + b) >> 8];
    }
#pragma unroll
    for (int u = 0; u < kBlk; ++u) {
      const int k = 64 * (b0 + u * kSmWaves) + 16 * g;
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int t = 0; t < 2; ++t) xb[u][mb][t] = load_x(L.X, 16 * mb + nl, M, K, k + 8 * t);
    }
  };
  load_batch(wave);

  // LUT: thread (wave, lane) writes entries byte = wave + 16 j, j = 0 .. 15,
  // whose low nibble is `wave` and high nibble j (uniform scalar loads).  The
  // linears of a group share one 4-bit type.
  {
    const uint32_t *lvt = cSmQ4Level + 16 * grp.lin[0].w.qtype;
    const float lo = u2f(lvt[wave]);
#pragma unroll
    for (int j = 0; j < 16; ++j) sLut[64 * (wave + 16 * j) + lane] = pack_bf16x2(lo, u2f(lvt[j]));
  }
  sT8[threadIdx.x & 255] = t8v;                 // four threads write each entry, same value
  sm_barrier_lds_only();

  f32x4_t acc[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (kLoraFirst)
    if (lora_wave) lora.apply(L, M, nl, j0, jok, L.Tout && tile == 0, acc);

  for (int b0 = wave; b0 < KB; b0 += kSmWaves * kBlk) {
    if (b0 != wave) load_batch(b0);
#pragma unroll
    for (int u = 0; u < kBlk; ++u) {
      const int b = b0 + u * kSmWaves;
      if (b >= KB) break;                         // uniform per wave
      const float chat = decode_absmax(sT8[code[u]], c2v[u], mean);
      const uint32_t words[2] = {pk[u].x, pk[u].y};
      bf16x8_t wop[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = sLut[64 * ((words[t] >> (8 * i)) & 0xffu) + lane];
        wop[t] = __builtin_bit_cast(bf16x8_t, o);
      }
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        f32x4_t part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[u][mb][0], wop[0], f32x4_t{0.f, 0.f, 0.f, 0.f},
                                                               0, 0, 0);
        part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[u][mb][1], wop[1], part, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mb][e] = __builtin_fmaf(chat, part[e], acc[mb][e]);
      }
    }
  }

  if constexpr (!kLoraFirst) {
    // One token tile at a time: fewer registers than loading all of them.
    if (lora_wave) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        SmLora<1, kPS, kP> one;
        f32x4_t (&a1)[1] = *reinterpret_cast<f32x4_t(*)[1]>(&acc[mb]);
        one.load(L, M, n, nl + 16 * mb, jc);
        one.apply(L, M, nl + 16 * mb, j0, jok, L.Tout && tile == 0, a1);
      }
    }
  }

  // Cross-wave sum in wave order; D layout: lane holds column nl, rows 4 g + e.
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][16 * mb + 4 * g + e][nl] = acc[mb][e];
  __syncthreads();
  for (int idx = threadIdx.x; idx < kMB * 16 * kSmRows; idx += kSmThreads) {
    const int m = idx / kSmRows, c = idx % kSmRows;
    if (m < M && n0 + c < N) {
      float v = red[0][m][c];
#pragma unroll
      for (int w = 1; w < kSmWaves; ++w) v += red[w][m][c];
      L.Y[static_cast<int64_t>(m) * N + n0 + c] = f32_to_bf16(v);
    }
  }
}

// ---------------------------------------------------------------------------
// Column split of the down-projection into partial slices; kw columns per
// wave, a multiple of 32.
static int sm_splits(int M, int K, int *kw_out) {
  // GEMV regime: up to 4 slices, aiming at 256 columns per wave (one load
  // batch).  Wider token tiles: at most 2 slices (their registers hold them).
  const int target = M <= small_m_gemv_max() ? std::min(4, (K + kSmWaves * 256 - 1) / (kSmWaves * 256))
                                             : kSmMaxSplits;
  const int per = kSmWaves * 32 * target;
  const int kw = 32 * ((K + per - 1) / per);
  if (kw_out) *kw_out = kw;
  return (K + kSmWaves * kw - 1) / (kSmWaves * kw);
}

bool small_m_ok(int64_t M, int r) { return M >= 1 && M <= small_m_max() && r % 8 == 0; }

size_t small_m_ws_bytes(int M, int K, int r) {
  int S = sm_splits(M, K, nullptr);
  if (M == 1) S = std::max(S, small_m_gemv_slices(K));
  return (static_cast<size_t>(S) * M * r * sizeof(float) + 255) / 256 * 256;
}

template <int kMB>
static void sm_launch_main(bool p, int grid, const SmGroup &grp, hipStream_t s) {
  if (p)
    hipLaunchKernelGGL((k_sm_main<kMB, true>), dim3(grid), dim3(kSmThreads), 0, s, grp);
  else
    hipLaunchKernelGGL((k_sm_main<kMB, false>), dim3(grid), dim3(kSmThreads), 0, s, grp);
}

hipError_t launch_small_m(SmGroup &grp, hipStream_t s) {
  // The streaming path takes four launches; a single linear at M <= 16 is
  // launch-bound and takes the two-launch path below instead.
  if (small_m_stream_group_ok(grp) && (grp.n > 1 || grp.M > 16)) return launch_small_m_stream(grp, s);
  if (grp.M <= small_m_gemv_max() && small_m_gemv_xl(grp)) {
    bool any_p = false;
    for (int i = 0; i < grp.n; ++i) {
      SmLinear &L = grp.lin[i];
      L.S = small_m_gemv_slices(L.w.K);
      any_p = any_p || L.P != nullptr;
    }
    if (any_p) {
      hipError_t e = launch_small_m_down_gemv(grp, s);
      if (e != hipSuccess) return e;
    }
    return launch_small_m_gemv(grp, s);
  }
  int down = 0, main = 0;
  bool any_down = false;
  for (int i = 0; i < grp.n; ++i) {
    SmLinear &L = grp.lin[i];
    L.S = sm_splits(grp.M, L.w.K, &L.kw);
    L.jtiles = (L.r + 15) / 16;
    grp.down_start[i] = down;
    grp.main_start[i] = main;
    if (L.P) {
      down += L.S * L.jtiles;
      any_down = true;
    }
    main += (L.w.N + kSmRows - 1) / kSmRows;
  }
  grp.down_start[grp.n] = down;
  grp.main_start[grp.n] = main;
  const int mb = (grp.M + 15) / 16;
  if (any_down) {
    switch (mb) {
      case 1: hipLaunchKernelGGL(k_sm_down<1>, dim3(down), dim3(kSmThreads), 0, s, grp); break;
      case 2: hipLaunchKernelGGL(k_sm_down<2>, dim3(down), dim3(kSmThreads), 0, s, grp); break;
      case 3: hipLaunchKernelGGL(k_sm_down<3>, dim3(down), dim3(kSmThreads), 0, s, grp); break;
      default: hipLaunchKernelGGL(k_sm_down<4>, dim3(down), dim3(kSmThreads), 0, s, grp); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (grp.M <= small_m_gemv_max()) return launch_small_m_gemv(grp, s);
  const bool p = grp.lin[0].P != nullptr;       // all linears of a group alike
  switch (mb) {
    case 1: sm_launch_main<1>(p, main, grp, s); break;
    case 2: sm_launch_main<2>(p, main, grp, s); break;
    case 3: sm_launch_main<3>(p, main, grp, s); break;
    default: sm_launch_main<4>(p, main, grp, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_small_m_fwd(const uint16_t *X, int M, const NF4View &w, const uint16_t *T, const uint16_t *B,
                              int r, uint16_t *Y, hipStream_t s) {
  SmGroup grp{};
  grp.n = 1;
  grp.M = M;
  SmLinear &L = grp.lin[0];
  L.X = X;
  L.w = w;
  L.B = B;
  L.Tin = T;
  L.r = r;
  L.scale = 1.f;
  L.Y = Y;
  return launch_small_m(grp, s);
}

}  // namespace qlora
