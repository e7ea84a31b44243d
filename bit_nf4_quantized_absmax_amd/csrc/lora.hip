// LoRA branch products on gfx950 bf16 MFMA (fp32 accumulation).
//
// The adapters are "a pair of small low-rank matrices per layer" trained in
// 16-bit while the base stays frozen (automatone.win, "QLoRA paper
// explained", The problem and How it works; creativeworksofknowledge.com,
// "QLoRA: Fine-Tune 70B on One GPU", Code: r, lora_alpha).  With A [r, K],
// B [N, r]:
//   k_skinny_nt<false>   T = s X A^T   (contraction over K, both K-contiguous)
//   k_skinny_nt<true>    G = s dY B    (contraction over N; B read transposed)
//   k_grad_partial       P^T Q over an M-slice -> fp32 partials
//   k_grad_reduce        fixed-order sum of the partials, bf16 out
// with (P, Q) = (X, G) for dA = s G0^T X [r, K] and (dY, T) for
// dB = s dY^T T0 [N, r], where T0, G0 are the unscaled products: the scale
// s = alpha / r is applied once, in fp32, before T and G are rounded to bf16.
// These are streaming products: each reads its wide operand (X or dY) once.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace qlora {

constexpr int kSkThreads = 512;   // 8 waves, each a slice of the contraction
constexpr int kSkRows = 32;       // output rows per workgroup

// out[m][j] = scale * sum_k L[m][k] R(j, k) for m in a 32-row tile, j < r, where
// R(j, k) = Rm[j * ldr + k] (kTransR = false, Rm = A [r, K]) or
// R(j, k) = Rm[k * r + j] (kTransR = true, Rm = B [N, r]).
// Wave w takes contraction steps of 32 with index w, w + 8, ...; the 8 wave
// partials are summed in LDS in wave order (deterministic).
template <bool kTransR, int kRP>
__global__ __launch_bounds__(kSkThreads) void k_skinny_nt(const uint16_t *__restrict__ L, int M, int Kc,
                                                          const uint16_t *__restrict__ Rm, int r, float scale,
                                                          uint16_t *__restrict__ out) {
  constexpr int kJB = kRP / 16;
  __shared__ float red[8][kSkRows][kRP + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lrow = lane & 15, lk = (lane >> 4) * 8;
  const int m0 = blockIdx.x * kSkRows;

  f32x4_t acc[2][kJB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < kJB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Kc % 8 == 0: an 8-element chunk is wholly inside or wholly past Kc.
  const int steps = (Kc + 31) / 32;
  for (int st = wave; st < steps; st += 8) {
    const int k = st * 32 + lk;
    const bool kin = k < Kc;
    bf16x8_t av[2], bv[kJB];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = m0 + i * 16 + lrow;
      if (m < M && kin)
        av[i] = *reinterpret_cast<const bf16x8_t *>(L + static_cast<int64_t>(m) * Kc + k);
      else
        av[i] = bf16x8_t{};
    }
#pragma unroll
    for (int j = 0; j < kJB; ++j) {
      const int jr = j * 16 + lrow;
      if (jr < r && kin) {
        if (!kTransR) {
          bv[j] = *reinterpret_cast<const bf16x8_t *>(Rm + static_cast<int64_t>(jr) * Kc + k);
        } else {
          uint16_t t[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = Rm[static_cast<int64_t>(k + e) * r + jr];
          bv[j] = __builtin_bit_cast(bf16x8_t, t);
        }
      } else {
        bv[j] = bf16x8_t{};
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < kJB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < kJB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][i * 16 + (lane >> 4) * 4 + v][j * 16 + (lane & 15)] = acc[i][j][v];
  __syncthreads();
  for (int idx = threadIdx.x; idx < kSkRows * kRP; idx += kSkThreads) {
    const int row = idx / kRP, j = idx % kRP;
    float s = red[0][row][j];
#pragma unroll
    for (int w = 1; w < 8; ++w) s += red[w][row][j];
    if (m0 + row < M && j < r) out[static_cast<int64_t>(m0 + row) * r + j] = f32_to_bf16(s * scale);
  }
}

template <bool kTransR>
static hipError_t launch_skinny(const uint16_t *L, int M, int Kc, const uint16_t *R, int r, float scale,
                                uint16_t *out, hipStream_t s) {
  const dim3 grid((M + kSkRows - 1) / kSkRows);
  if (r <= 64)
    hipLaunchKernelGGL((k_skinny_nt<kTransR, 64>), grid, dim3(kSkThreads), 0, s, L, M, Kc, R, r, scale, out);
  else
    hipLaunchKernelGGL((k_skinny_nt<kTransR, 128>), grid, dim3(kSkThreads), 0, s, L, M, Kc, R, r, scale, out);
  return hipGetLastError();
}

hipError_t launch_lora_down(const uint16_t *X, int M, int K, const uint16_t *A, int r, float scale, uint16_t *T,
                            hipStream_t s) {
  return launch_skinny<false>(X, M, K, A, r, scale, T, s);
}

hipError_t launch_lora_grad_in(const uint16_t *dY, int M, int N, const uint16_t *B, int r, float scale,
                               uint16_t *G, hipStream_t s) {
  return launch_skinny<true>(dY, M, N, B, r, scale, G, s);
}

// ---------------------------------------------------------------------------
// dA / dB: out = P^T Q, P [M, D], Q [M, r] (Q already carries the scale).
// Workgroup (tile d0 .. d0+63, split sp) sums m in its slice of M in steps
// of 64 rows: P and Q tiles go to LDS row-major and are read transposed into
// the MFMA operands (8 consecutive m per lane).  4 waves, wave w owns
// d0 + 16 w .. +15 and all r columns.
// ---------------------------------------------------------------------------
constexpr int kGrThreads = 256;
constexpr int kGrD = 64;      // D per workgroup
constexpr int kGrM = 64;      // M rows per step

static int grad_splits(int M, int D) {
  const int dt = (D + kGrD - 1) / kGrD;
  int sp = (1024 + dt - 1) / dt;
  const int msteps = (M + kGrM - 1) / kGrM;
  if (sp > msteps) sp = msteps;
  if (sp < 1) sp = 1;
  return sp;
}

template <int kRP>
__global__ __launch_bounds__(kGrThreads) void k_grad_partial(const uint16_t *__restrict__ P,
                                                             const uint16_t *__restrict__ Q, int M, int D,
                                                             int r, int rows_per_split,
                                                             float *__restrict__ part) {
  constexpr int kJB = kRP / 16;
  __shared__ uint16_t sP[kGrM][kGrD + 2];
  __shared__ uint16_t sQ[kGrM][kRP + 2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d0 = blockIdx.x * kGrD;
  const int sp = blockIdx.y;
  const int mbeg = sp * rows_per_split;
  const int mend = min(M, mbeg + rows_per_split);

  f32x4_t acc[kJB];
#pragma unroll
  for (int j = 0; j < kJB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int m0 = mbeg; m0 < mend; m0 += kGrM) {
    for (int idx = threadIdx.x; idx < kGrM * kGrD; idx += kGrThreads) {
      const int mm = idx / kGrD, dd = idx % kGrD;
      const int m = m0 + mm, d = d0 + dd;
      sP[mm][dd] = (m < mend && d < D) ? P[static_cast<int64_t>(m) * D + d] : 0;
    }
    for (int idx = threadIdx.x; idx < kGrM * kRP; idx += kGrThreads) {
      const int mm = idx / kRP, j = idx % kRP;
      const int m = m0 + mm;
      sQ[mm][j] = (m < mend && j < r) ? Q[static_cast<int64_t>(m) * r + j] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGrM; kk += 32) {
      const int mb = kk + (lane >> 4) * 8;
      uint16_t t[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = sP[mb + e][wave * 16 + (lane & 15)];
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, t);
#pragma unroll
      for (int j = 0; j < kJB; ++j) {
        uint16_t u[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = sQ[mb + e][j * 16 + (lane & 15)];
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, u), acc[j], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // part[sp][d][j], d < D_pad = tiles * 64, j < kRP
  const int dpad = gridDim.x * kGrD;
  float *dst = part + static_cast<int64_t>(sp) * dpad * kRP;
#pragma unroll
  for (int j = 0; j < kJB; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int d = d0 + wave * 16 + (lane >> 4) * 4 + v;
      dst[static_cast<int64_t>(d) * kRP + j * 16 + (lane & 15)] = acc[j][v];
    }
}

template <int kRP>
__global__ __launch_bounds__(256) void k_grad_reduce(const float *__restrict__ part, int splits, int D, int dpad,
                                                     int r, bool out_r_major, uint16_t *__restrict__ out) {
  const int64_t total = static_cast<int64_t>(D) * r;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    const int d = static_cast<int>(idx / r), j = static_cast<int>(idx % r);
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) s += part[(static_cast<int64_t>(sp) * dpad + d) * kRP + j];
    const uint16_t v = f32_to_bf16(s);
    if (out_r_major)
      out[static_cast<int64_t>(j) * D + d] = v;
    else
      out[static_cast<int64_t>(d) * r + j] = v;
  }
}

size_t lora_grad_ws_bytes(int M, int D, int r) {
  const int rp = r <= 64 ? 64 : 128;
  const int dt = (D + kGrD - 1) / kGrD;
  return static_cast<size_t>(grad_splits(M, D)) * dt * kGrD * rp * sizeof(float);
}

hipError_t launch_lora_grad_w(const uint16_t *P, const uint16_t *Q, int M, int D, int r, bool out_r_major,
                              uint16_t *out, void *ws, hipStream_t s) {
  const int sp = grad_splits(M, D);
  const int dt = (D + kGrD - 1) / kGrD;
  const int msteps = (M + kGrM - 1) / kGrM;
  const int rows_per_split = ((msteps + sp - 1) / sp) * kGrM;
  float *part = static_cast<float *>(ws);
  const int64_t total = static_cast<int64_t>(D) * r;
  const unsigned rgrid = static_cast<unsigned>(std::min<int64_t>((total + 255) / 256, 4096));
  if (r <= 64) {
    hipLaunchKernelGGL(k_grad_partial<64>, dim3(dt, sp), dim3(kGrThreads), 0, s, P, Q, M, D, r, rows_per_split,
                       part);
    hipLaunchKernelGGL(k_grad_reduce<64>, dim3(rgrid), dim3(256), 0, s, part, sp, D, dt * kGrD, r,
                       out_r_major, out);
  } else {
    hipLaunchKernelGGL(k_grad_partial<128>, dim3(dt, sp), dim3(kGrThreads), 0, s, P, Q, M, D, r,
                       rows_per_split, part);
    hipLaunchKernelGGL(k_grad_reduce<128>, dim3(rgrid), dim3(256), 0, s, part, sp, D, dt * kGrD, r,
                       out_r_major, out);
  }
  return hipGetLastError();
}

}  // namespace qlora
