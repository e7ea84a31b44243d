// LoRA dropout on the adapter input (creativeworksofknowledge.com, "QLoRA:
// Fine-Tune 70B on One GPU", Code: lora_dropout on the adapters).
//
// The keep mask is counter-based: element e = m K + k of X [M, K] is kept iff
// word e % 4 of Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011) at counter (e / 4 as a 64-bit
// value in words 0 and 1, words 2 and 3 zero) under key (seed low, seed high)
// is >= t = floor(p 2^32).  The mask is stored as bits (bit k % 32 of word
// [m][k / 32]); the dropped input X_d = X where kept, +0 elsewhere (exact in
// bf16).  The 1 / (1 - p) scaling is folded into the LoRA scale by the host.
//
//  k_dropout_mask   X -> (X_d, mask bits): one thread per 32 elements of a
//                   row (K % 32 == 0), 8 Philox blocks, 4 16-byte loads and
//                   stores of bf16, one mask word.
//  k_dropout_apply  (X, mask bits) -> X_d (the backward pass rebuilds X_d
//                   from the forward pass's bits).
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace qlora {
namespace {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;   // round multipliers
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;   // key increments
constexpr int kDropThreads = 256;

struct U4 {
  uint32_t x, y, z, w;
};

// Philox4x32-10 of counter (c0, c1, 0, 0) under key (k0, k1).
__device__ __forceinline__ U4 philox(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1) {
  uint32_t x = c0, y = c1, z = 0, w = 0;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * x;
    const uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * z;
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    x = hi1 ^ y ^ k0;
    y = lo1;
    z = hi0 ^ w ^ k1;
    w = lo0;
  }
  return U4{x, y, z, w};
}

// 32 bf16 of X (4 x 16 bytes), zeroed where bit i of `bits` is clear.
__device__ __forceinline__ void masked_copy(const uint16_t *src, uint16_t *dst, uint32_t bits) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint4 v = reinterpret_cast<const uint4 *>(src)[q];
    uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int i = 8 * q + 2 * h;
      const uint32_t lo = ((bits >> i) & 1u) ? 0x0000FFFFu : 0u;
      const uint32_t hi = ((bits >> (i + 1)) & 1u) ? 0xFFFF0000u : 0u;
      u[h] &= lo | hi;
    }
    reinterpret_cast<uint4 *>(dst)[q] = make_uint4(u[0], u[1], u[2], u[3]);
  }
}

__global__ __launch_bounds__(kDropThreads) void k_dropout_mask(const uint16_t *__restrict__ X, int64_t chunks,
                                                               uint32_t k0, uint32_t k1, uint32_t thresh,
                                                               uint16_t *__restrict__ Xd,
                                                               uint32_t *__restrict__ keep) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kDropThreads;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * kDropThreads + threadIdx.x; c < chunks; c += stride) {
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t b = static_cast<uint64_t>(c) * 8 + j;   // Philox block of elements 4 b .. 4 b + 3
      const U4 r = philox(static_cast<uint32_t>(b), static_cast<uint32_t>(b >> 32), k0, k1);
      bits |= (r.x >= thresh ? 1u : 0u) << (4 * j);
      bits |= (r.y >= thresh ? 1u : 0u) << (4 * j + 1);
      bits |= (r.z >= thresh ? 1u : 0u) << (4 * j + 2);
      bits |= (r.w >= thresh ? 1u : 0u) << (4 * j + 3);
    }
    keep[c] = bits;
    masked_copy(X + c * 32, Xd + c * 32, bits);
  }
}

__global__ __launch_bounds__(kDropThreads) void k_dropout_apply(const uint16_t *__restrict__ X, int64_t chunks,
                                                                const uint32_t *__restrict__ keep,
                                                                uint16_t *__restrict__ Xd) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kDropThreads;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * kDropThreads + threadIdx.x; c < chunks; c += stride)
    masked_copy(X + c * 32, Xd + c * 32, keep[c]);
}

unsigned drop_grid(int64_t chunks) {
  return static_cast<unsigned>(std::min<int64_t>((chunks + kDropThreads - 1) / kDropThreads, 8192));
}

}  // namespace

hipError_t launch_dropout_mask(const uint16_t *X, int64_t n, uint64_t seed, uint32_t thresh, uint16_t *Xd,
                               uint32_t *keep, hipStream_t s) {
  const int64_t chunks = n / 32;
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dropout_mask, dim3(drop_grid(chunks)), dim3(kDropThreads), 0, s, X, chunks,
                     static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), thresh, Xd, keep);
  return hipGetLastError();
}

hipError_t launch_dropout_apply(const uint16_t *X, int64_t n, const uint32_t *keep, uint16_t *Xd, hipStream_t s) {
  const int64_t chunks = n / 32;
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dropout_apply, dim3(drop_grid(chunks)), dim3(kDropThreads), 0, s, X, chunks, keep, Xd);
  return hipGetLastError();
}

}  // namespace qlora
