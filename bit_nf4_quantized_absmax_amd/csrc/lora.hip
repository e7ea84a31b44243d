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
// dA / dB: out = P^T Q over M, P [M, D] (X or dY), Q [M, r] (G or T, already
// carrying the scale).  The contraction runs over M, which is the slow index
// of both operands, so:
//  * Q is first transposed into Qt [r, Mp] (k_transpose_narrow, Mp = M
//    rounded up to 8) so that 8 consecutive m of one column are one 16-byte
//    load;
//  * each lane loads an 8 (m) x 8 (d) block of P with eight 16-byte loads
//    and transposes it in registers (32 v_perm), giving eight MFMA operands
//    of 8 consecutive m for 8 different d.
// Workgroup (d-tile of 128, M-split sp): 4 waves take interleaved 32-row
// sub-steps of the split; MFMA 16x16x32 with A-row i of fragment f holding
// d = d0 + 8 i + f.  The 4 wave partials are summed in LDS in wave order and
// the split partials by k_grad_reduce in split order (deterministic).
// ---------------------------------------------------------------------------
constexpr int kGrThreads = 256;
constexpr int kGrD = 128;     // d per workgroup (16 lanes x 8)
constexpr int kGrSub = 32;    // m per MFMA sub-step

static int grad_splits(int M, int D) {
  const int dt = (D + kGrD - 1) / kGrD;
  int sp = (512 + dt - 1) / dt;
  const int msteps = (M + 4 * kGrSub - 1) / (4 * kGrSub);
  if (sp > msteps) sp = msteps;
  if (sp < 1) sp = 1;
  return sp;
}

static int padded_m(int M) { return (M + 7) & ~7; }

// Qt [rp, Mp] from Q [M, r] (rows j >= r and columns m >= M are zero).
__global__ __launch_bounds__(256) void k_transpose_narrow(const uint16_t *__restrict__ Q, int M, int r, int rp,
                                                          int Mp, uint16_t *__restrict__ Qt) {
  __shared__ uint16_t tile[64][129];
  const int m0 = blockIdx.x * 128;
  for (int idx = threadIdx.x; idx < 128 * 64; idx += 256) {
    const int mm = idx >> 6, j = idx & 63;
    const int m = m0 + mm;
    tile[j][mm] = (m < M && j < r) ? Q[static_cast<int64_t>(m) * r + j] : static_cast<uint16_t>(0);
  }
  __syncthreads();
  for (int jb = 0; jb < rp; jb += 64) {
    if (jb > 0) {
      __syncthreads();
      for (int idx = threadIdx.x; idx < 128 * 64; idx += 256) {
        const int mm = idx >> 6, j = idx & 63;
        const int m = m0 + mm;
        tile[j][mm] = (m < M && jb + j < r) ? Q[static_cast<int64_t>(m) * r + jb + j] : static_cast<uint16_t>(0);
      }
      __syncthreads();
    }
    for (int idx = threadIdx.x; idx < 64 * 128; idx += 256) {
      const int j = idx >> 7, mm = idx & 127;
      const int m = m0 + mm;
      if (m < Mp) Qt[static_cast<int64_t>(jb + j) * Mp + m] = tile[j][mm];
    }
  }
}

template <int kRP>
__global__ __launch_bounds__(kGrThreads) void k_grad_partial(const uint16_t *__restrict__ P,
                                                             const uint16_t *__restrict__ Qt, int M, int Mp,
                                                             int D, int rows_per_split, float *__restrict__ part) {
  constexpr int kJB = kRP / 16;
  __shared__ float red[kGrD][kRP + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d0 = blockIdx.x * kGrD;
  const int sp = blockIdx.y;
  const int mbeg = sp * rows_per_split;
  const int mend = min(M, mbeg + rows_per_split);
  const int dl = d0 + 8 * (lane & 15);     // this lane's 8 d columns
  const int mg = 8 * (lane >> 4);          // this lane's 8-row group within the sub-step

  f32x4_t acc[8][kJB];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int j = 0; j < kJB; ++j) acc[f][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int m0 = mbeg + wave * kGrSub; m0 < mend; m0 += 4 * kGrSub) {
    // P block: rows m0 + mg .. +7, columns dl .. dl+7 (zero outside)
    uint32_t v[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + mg + i;
      uint4 t = make_uint4(0, 0, 0, 0);
      if (m < mend && dl < D) t = *reinterpret_cast<const uint4 *>(P + static_cast<int64_t>(m) * D + dl);
      v[i][0] = t.x; v[i][1] = t.y; v[i][2] = t.z; v[i][3] = t.w;
    }
    // 8 x 8 transpose of 16-bit elements: a[f] dword p = (P[2p][f], P[2p+1][f])
    uint32_t a[8][4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        a[2 * c][p] = __builtin_amdgcn_perm(v[2 * p + 1][c], v[2 * p][c], 0x05040100u);
        a[2 * c + 1][p] = __builtin_amdgcn_perm(v[2 * p + 1][c], v[2 * p][c], 0x07060302u);
      }
    // Qt fragments: column j = 16 jb + lane % 16, the lane's 8 rows of m
    bf16x8_t b[kJB];
#pragma unroll
    for (int jb = 0; jb < kJB; ++jb) {
      const int m = m0 + mg;
      uint4 t = make_uint4(0, 0, 0, 0);
      if (m < Mp) t = *reinterpret_cast<const uint4 *>(Qt + static_cast<int64_t>(16 * jb + (lane & 15)) * Mp + m);
      b[jb] = __builtin_bit_cast(bf16x8_t, t);
    }
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const bf16x8_t af = __builtin_bit_cast(bf16x8_t, a[f]);
#pragma unroll
      for (int jb = 0; jb < kJB; ++jb)
        acc[f][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b[jb], acc[f][jb], 0, 0, 0);
    }
  }
  // acc[f][jb][e] at lane l: d = d0 + 8 (4 (l / 16) + e) + f, j = 16 jb + l % 16.
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int jb = 0; jb < kJB; ++jb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int dd = 8 * (4 * (lane >> 4) + e) + f, j = 16 * jb + (lane & 15);
            if (w == 0)
              red[dd][j] = acc[f][jb][e];
            else
              red[dd][j] += acc[f][jb][e];
          }
    }
    __syncthreads();
  }
  const int dpad = gridDim.x * kGrD;
  float *dst = part + static_cast<int64_t>(sp) * dpad * kRP;
  for (int idx = threadIdx.x; idx < kGrD * kRP; idx += kGrThreads) {
    const int dd = idx / kRP, j = idx % kRP;
    dst[static_cast<int64_t>(d0 + dd) * kRP + j] = red[dd][j];
  }
}

template <int kRP>
__global__ __launch_bounds__(256) void k_grad_reduce(const float *__restrict__ part, int splits, int D, int dpad,
                                                     int r, bool out_r_major, uint16_t *__restrict__ out) {
  const int64_t total = static_cast<int64_t>(D) * r;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    int d, j;
    if (out_r_major) {   // consecutive threads write consecutive d of one j row
      j = static_cast<int>(idx / D);
      d = static_cast<int>(idx % D);
    } else {
      d = static_cast<int>(idx / r);
      j = static_cast<int>(idx % r);
    }
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) s += part[(static_cast<int64_t>(sp) * dpad + d) * kRP + j];
    const uint16_t v = f32_to_bf16(s);
    if (out_r_major)
      out[static_cast<int64_t>(j) * D + d] = v;
    else
      out[static_cast<int64_t>(d) * r + j] = v;
  }
}

// workspace: Qt [rp, Mp] bf16 (256-byte aligned) | partials [splits, dpad, rp] fp32
size_t lora_grad_ws_bytes(int M, int D, int r) {
  const int rp = r <= 64 ? 64 : 128;
  const int dt = (D + kGrD - 1) / kGrD;
  const size_t qt = ((static_cast<size_t>(rp) * padded_m(M) * 2 + 255) / 256) * 256;
  return qt + static_cast<size_t>(grad_splits(M, D)) * dt * kGrD * rp * sizeof(float);
}

hipError_t launch_lora_grad_w(const uint16_t *P, const uint16_t *Q, int M, int D, int r, bool out_r_major,
                              uint16_t *out, void *ws, hipStream_t s) {
  const int rp = r <= 64 ? 64 : 128;
  const int Mp = padded_m(M);
  const int sp = grad_splits(M, D);
  const int dt = (D + kGrD - 1) / kGrD;
  const int msteps = (M + kGrSub - 1) / kGrSub;
  const int rows_per_split = ((msteps + sp - 1) / sp) * kGrSub;
  uint16_t *Qt = static_cast<uint16_t *>(ws);
  const size_t qt = ((static_cast<size_t>(rp) * Mp * 2 + 255) / 256) * 256;
  float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + qt);
  hipLaunchKernelGGL(k_transpose_narrow, dim3((Mp + 127) / 128), dim3(256), 0, s, Q, M, r, rp, Mp, Qt);
  const int64_t total = static_cast<int64_t>(D) * r;
  const unsigned rgrid = static_cast<unsigned>(std::min<int64_t>((total + 255) / 256, 4096));
  if (rp == 64) {
    hipLaunchKernelGGL(k_grad_partial<64>, dim3(dt, sp), dim3(kGrThreads), 0, s, P, Qt, M, Mp, D, rows_per_split,
                       part);
    hipLaunchKernelGGL(k_grad_reduce<64>, dim3(rgrid), dim3(256), 0, s, part, sp, D, dt * kGrD, r, out_r_major, out);
  } else {
    hipLaunchKernelGGL(k_grad_partial<128>, dim3(dt, sp), dim3(kGrThreads), 0, s, P, Qt, M, Mp, D, rows_per_split,
                       part);
    hipLaunchKernelGGL(k_grad_reduce<128>, dim3(rgrid), dim3(256), 0, s, part, sp, D, dt * kGrD, r, out_r_major,
                       out);
  }
  return hipGetLastError();
}

}  // namespace qlora
