// NF4 + double-quantization codec kernels for gfx950.
//
// Quantize (automatone.win, "QLoRA paper explained", How it works / 4-bit
// NormalFloat and Double Quantization; creativeworksofknowledge.com, "QLoRA:
// Fine-Tune 70B on One GPU", The three innovations / 1-2):
//   pass 1  k_quant_blocks   one read of W: per-64 absmax, NF4 codes, nibbles
//   pass 2  k_tree_sum       fp64 pairwise tree of the absmax values (fixed
//                            order, levels of aligned 2048-chunks until at
//                            most 2048 partials remain)
//   pass 3  k_quant_consts   last tree level, mean, per-256 scale c2, 8-bit
//                            constant codes
// Dequantize: k_dequant     packed codes -> bf16, one read, one write.
//
// Bit-exactness rules: fp32 division is IEEE correctly rounded (hipcc's
// default), no fused multiply-add (-ffp-contract=off), bf16 conversion is
// round-to-nearest-even, the tree order is fixed.
#include "common.h"
#include "launch.h"

namespace qlora {

__constant__ uint32_t cQ4Level[3 * 16] = {QLORA_Q4_LEVEL_BITS};
__constant__ uint32_t cQ4Thresh[3 * 15] = {QLORA_Q4_THRESH_BITS};
__constant__ uint32_t cT8Level[256] = {QLORA_T8_LEVEL_BITS};
__constant__ uint32_t cT8Thresh[255] = {QLORA_T8_THRESH_BITS};

constexpr int kTreeChunk = 2048;   // elements reduced by one workgroup of k_tree_sum
constexpr int kThreads = 256;

// Nearest level of a 4-bit table, ties to the lower code: the number of its 15
// ascending thresholds (th, in LDS) strictly below x, by a 4-step binary
// search (equal thresholds, as FP4's two zero levels give, are counted alike).
__device__ __forceinline__ uint32_t q4_code(float x, const float *th) {
  uint32_t q = (x > th[7]) ? 8u : 0u;
  q += (x > th[q + 3]) ? 4u : 0u;
  q += (x > th[q + 1]) ? 2u : 0u;
  q += (x > th[q]) ? 1u : 0u;
  return q;
}

// ---------------------------------------------------------------------------
// Pass 1.  Each lane owns 4 consecutive elements; 16 lanes form one block of
// 64.  The lane group reduces |w| with cross-lane max, every lane divides its
// elements by the block absmax and codes them, and writes its 2 packed bytes.
// Elements past n do not exist: they do not enter the max and pack as 0.
// The input is fp32 (kIn = 0) or 16-bit bit patterns, bf16 (1) or fp16 (2),
// which widen to fp32 exactly, so every input type codes its fp32 value.
// ---------------------------------------------------------------------------
template <int kIn>
__device__ __forceinline__ float widen(const void *W, int64_t i) {
  if (kIn == 0) return static_cast<const float *>(W)[i];
  const uint16_t h = static_cast<const uint16_t *>(W)[i];
  if (kIn == 1) return u2f(static_cast<uint32_t>(h) << 16);
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

constexpr int kQU = 2;   // 4-element chunks per thread per pass of k_quant_blocks

template <int kIn>
__device__ __forceinline__ void load_chunk(const void *W, int64_t e, int64_t n, float w[4]) {
  if (e + 3 < n && kIn == 0) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(static_cast<const float *>(W) + e));
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if (e + 3 < n) {
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(static_cast<const uint16_t *>(W) + e));
    const uint32_t hs[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = kIn == 1 ? u2f(hs[i] << 16)
                      : static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(hs[i])));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (e + i < n) ? widen<kIn>(W, e + i) : 0.0f;
  }
}

// A thread takes kQU chunks kThreads apart (a 16-lane block group stays
// within one block) and loads all of them before coding the first; W is read
// once, through streaming loads.
template <int kIn>
__global__ __launch_bounds__(kThreads) void k_quant_blocks(const void *__restrict__ W, int64_t n,
                                                           int qtype, uint8_t *__restrict__ packed,
                                                           float *__restrict__ absmax) {
  const uint32_t zero = static_cast<uint32_t>(q4_zero_code(qtype));
  __shared__ float sTh[16];
  if (threadIdx.x < 15) sTh[threadIdx.x] = u2f(cQ4Thresh[15 * qtype + threadIdx.x]);
  __syncthreads();
  const int64_t nchunks = ((n + kBlock - 1) / kBlock) * 16;  // 4-element chunks, whole blocks
  const int64_t span = static_cast<int64_t>(kThreads) * kQU;
  for (int64_t c0 = static_cast<int64_t>(blockIdx.x) * span + threadIdx.x; c0 < nchunks;
       c0 += static_cast<int64_t>(gridDim.x) * span) {
    float w[kQU][4];
#pragma unroll
    for (int u = 0; u < kQU; ++u) {
      const int64_t c = c0 + u * kThreads;
      if (c < nchunks) {
        load_chunk<kIn>(W, c * 4, n, w[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[u][i] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kQU; ++u) {
      // nchunks is a multiple of 16 and a block's 16 lanes share c >> 4, so
      // a block group is wholly in range or wholly out.
      const int64_t c = c0 + u * kThreads;
      if (c >= nchunks) break;
      const int64_t e = c * 4;
      const bool full = (e + 3 < n);
      float a = fmaxf(fmaxf(fabsf(w[u][0]), fabsf(w[u][1])), fmaxf(fabsf(w[u][2]), fabsf(w[u][3])));
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 16));

      uint32_t q[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        q[i] = (a > 0.0f) ? q4_code(w[u][i] / a, sTh) : zero;
        if (e + i >= n) q[i] = 0u;
      }
      const uint32_t b0 = q[0] | (q[1] << 4), b1 = q[2] | (q[3] << 4);
      uint8_t *dst = packed + (e >> 1);
      if (full) {
        *reinterpret_cast<uint16_t *>(dst) = static_cast<uint16_t>(b0 | (b1 << 8));
      } else {
        if (e < n) dst[0] = static_cast<uint8_t>(b0);
        if (e + 2 < n) dst[1] = static_cast<uint8_t>(b1);
      }
      if ((threadIdx.x & 15) == 0) absmax[c >> 4] = a;
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 2.  Workgroup g reduces in[2048 g, 2048 g + 2048) (zero beyond len) to
// one fp64 value with the neighbour-pairing tree: 8 values per thread
// ((v0+v1)+(v2+v3))+((v4+v5)+(v6+v7)), then level by level in LDS,
// s'[t] = s[2t] + s[2t+1].  Because chunks are aligned powers of two,
// applying this again to the partials reproduces the global tree exactly.
// The last level (at most 2048 partials) runs at the start of pass 3.
// ---------------------------------------------------------------------------
// Tree sum of chunk `chunk`, called by every thread of the workgroup; the
// result is in s[0] on return (after a barrier).
template <typename Tin>
__device__ __forceinline__ void tree_chunk(const Tin *__restrict__ in, int64_t len, int64_t chunk, double *s) {
  const int t = threadIdx.x;
  const int64_t base = chunk * kTreeChunk + t * 8;
  double v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (base + i < len) ? static_cast<double>(in[base + i]) : 0.0;
  s[t] = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
  __syncthreads();
  for (int width = kThreads / 2; width >= 1; width >>= 1) {
    double tmp = 0.0;
    if (t < width) tmp = s[2 * t] + s[2 * t + 1];
    __syncthreads();
    if (t < width) s[t] = tmp;
    __syncthreads();
  }
}

template <typename Tin>
__global__ __launch_bounds__(kThreads) void k_tree_sum(const Tin *__restrict__ in, int64_t len,
                                                       double *__restrict__ out) {
  __shared__ double s[kThreads];
  tree_chunk(in, len, blockIdx.x, s);
  if (threadIdx.x == 0) out[blockIdx.x] = s[0];
}

// ---------------------------------------------------------------------------
// Pass 3.  Every workgroup first sums the last tree level (plen <= 2048
// partials, the same tree as pass 2), then mean = fl32(sum / nb).  One wave
// per group of 256 constants, 4 per
// lane: d = fl32(c - mean), c2 = max |d| over the group, code = number of T8
// thresholds below fl32(d / c2) (binary search over the 255 thresholds, with
// +inf as a 256th sentinel).  c2 = 0 -> code 127.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_quant_consts(const float *__restrict__ absmax, int64_t nb,
                                                           const double *__restrict__ partials, int64_t plen,
                                                           uint8_t *__restrict__ code8,
                                                           float *__restrict__ c2,
                                                           float *__restrict__ mean_out) {
  __shared__ float thr[256];
  __shared__ double s[kThreads];
  for (int i = threadIdx.x; i < 256; i += kThreads) thr[i] = (i < 255) ? u2f(cT8Thresh[i]) : INFINITY;
  tree_chunk(partials, plen, 0, s);                    // ends with a barrier: thr is ready too
  const float mean = static_cast<float>(s[0] / static_cast<double>(nb));
  if (blockIdx.x == 0 && threadIdx.x == 0) mean_out[0] = mean;

  const int lane = threadIdx.x & 63;
  const int64_t nb2 = (nb + kGroup - 1) / kGroup;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6); g < nb2;
       g += waves) {
    const int64_t idx = g * kGroup + lane * 4;
    float d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = (idx + i < nb) ? (absmax[idx + i] - mean) : 0.0f;
    float m = fmaxf(fmaxf(fabsf(d[0]), fabsf(d[1])), fmaxf(fabsf(d[2]), fabsf(d[3])));
    m = wave_max(m);
    uint32_t codes = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = 127;
      if (m > 0.0f) {
        const float x = d[i] / m;
        lo = 0;
#pragma unroll
        for (int step = 128; step >= 1; step >>= 1)
          if (thr[lo + step - 1] < x) lo += step;
      }
      codes |= lo << (8 * i);
    }
    if (idx + 3 < nb) {
      *reinterpret_cast<uint32_t *>(code8 + idx) = codes;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (idx + i < nb) code8[idx + i] = static_cast<uint8_t>(codes >> (8 * i));
    }
    if (lane == 0) c2[g] = m;
  }
}

// ---------------------------------------------------------------------------
// Dequantize: a thread expands kDqU chunks of 8 consecutive elements (4
// packed bytes -> one 16-byte store of bf16; the 8 share one block constant,
// 8 | 64).  Chunk u of a thread lies kThreads chunks after chunk u - 1, so
// each load and store instruction is contiguous across the workgroup; all
// loads of the kDqU chunks are issued before the first is used.  Levels are
// read in pairs, one LDS entry per packed byte.  Codes are read once and the
// output is written once: both go through non-temporal (streaming) accesses.
// ---------------------------------------------------------------------------
constexpr int kDqU = 8;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t *__restrict__ packed,
                                                      const uint8_t *__restrict__ code8,
                                                      const float *__restrict__ c2,
                                                      const float *__restrict__ mean_p, int64_t n, int qtype,
                                                      uint16_t *__restrict__ out) {
  __shared__ float2 pairs[256];   // byte -> (level of its low nibble, level of its high nibble)
  __shared__ float t8[256];
  for (int i = threadIdx.x; i < 256; i += kThreads) {
    pairs[i] = make_float2(u2f(cQ4Level[16 * qtype + (i & 15)]), u2f(cQ4Level[16 * qtype + (i >> 4)]));
    t8[i] = u2f(cT8Level[i]);
  }
  __syncthreads();
  const float mean = mean_p[0];
  const int64_t nchunks = (n + 7) / 8;
  const int64_t span = static_cast<int64_t>(kThreads) * kDqU;
  for (int64_t c0 = static_cast<int64_t>(blockIdx.x) * span + threadIdx.x; c0 < nchunks;
       c0 += static_cast<int64_t>(gridDim.x) * span) {
    uint32_t p[kDqU], cc[kDqU];
    float sc[kDqU];
#pragma unroll
    for (int u = 0; u < kDqU; ++u) {
      const int64_t c = min(c0 + u * kThreads, nchunks - 1);   // past the end: a repeated load, never used
      const int64_t e = c * 8, b = e >> 6;
      cc[u] = code8[b];
      sc[u] = c2[b >> 8];
      if (e + 7 < n) {
        p[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(packed + (e >> 1)));
      } else {
        p[u] = 0;
        for (int i = 0; i < 4; ++i)
          if (e + 2 * i < n) p[u] |= static_cast<uint32_t>(packed[(e >> 1) + i]) << (8 * i);
      }
    }
#pragma unroll
    for (int u = 0; u < kDqU; ++u) {
      const int64_t c = c0 + u * kThreads;
      if (c >= nchunks) break;
      const int64_t e = c * 8;
      const float chat = decode_absmax(t8[cc[u]], sc[u], mean);
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 lv = pairs[(p[u] >> (8 * i)) & 255u];
        o[i] = pack_bf16x2(lv.x * chat, lv.y * chat);
      }
      if (e + 7 < n) {
        const u32x4_t v = {o[0], o[1], o[2], o[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(out + e));
      } else {
        for (int i = 0; i < 8; ++i)
          if (e + i < n) out[e + i] = static_cast<uint16_t>(o[i >> 1] >> (16 * (i & 1)));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static int64_t tree_partials(int64_t len) { return (len + kTreeChunk - 1) / kTreeChunk; }

static unsigned grid_for(int64_t work_items, int64_t per_wg, int64_t cap) {
  int64_t g = (work_items + per_wg - 1) / per_wg;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return static_cast<unsigned>(g);
}

size_t quantize_ws_bytes(int64_t n) {
  if (n < 1) return 0;
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t p1 = tree_partials(nb);
  // absmax fp32 [nb] (padded to 256 B) | two ping-pong fp64 partial buffers [p1]
  const size_t a = ((static_cast<size_t>(nb) * 4 + 255) / 256) * 256;
  return a + 2 * static_cast<size_t>(p1) * 8;
}

hipError_t launch_quantize(const void *W, int in_type, int64_t n, int qtype, uint8_t *packed, uint8_t *code8,
                           float *c2, float *mean, void *ws, hipStream_t s) {
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const size_t a = ((static_cast<size_t>(nb) * 4 + 255) / 256) * 256;
  float *absmax = static_cast<float *>(ws);
  double *buf0 = reinterpret_cast<double *>(static_cast<char *>(ws) + a);
  double *buf1 = buf0 + tree_partials(nb);

  const dim3 g1(grid_for(nb * 16, kThreads * kQU, 16384));
  if (in_type == 1)
    hipLaunchKernelGGL(k_quant_blocks<1>, g1, dim3(kThreads), 0, s, W, n, qtype, packed, absmax);
  else if (in_type == 2)
    hipLaunchKernelGGL(k_quant_blocks<2>, g1, dim3(kThreads), 0, s, W, n, qtype, packed, absmax);
  else
    hipLaunchKernelGGL(k_quant_blocks<0>, g1, dim3(kThreads), 0, s, W, n, qtype, packed, absmax);
  int64_t len = nb;
  hipLaunchKernelGGL(k_tree_sum<float>, dim3(static_cast<unsigned>(tree_partials(len))), dim3(kThreads), 0,
                     s, absmax, len, buf0);
  len = tree_partials(len);
  double *cur = buf0, *nxt = buf1;
  while (len > kTreeChunk) {
    hipLaunchKernelGGL(k_tree_sum<double>, dim3(static_cast<unsigned>(tree_partials(len))), dim3(kThreads),
                       0, s, cur, len, nxt);
    len = tree_partials(len);
    double *t = cur; cur = nxt; nxt = t;
  }
  const int64_t nb2 = (nb + kGroup - 1) / kGroup;
  hipLaunchKernelGGL(k_quant_consts, dim3(grid_for(nb2, kThreads / 64, 4096)), dim3(kThreads), 0, s,
                     absmax, nb, cur, len, code8, c2, mean);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *packed, const uint8_t *code8, const float *c2,
                             const float *mean, int64_t n, int qtype, uint16_t *out, hipStream_t s) {
  hipLaunchKernelGGL(k_dequant, dim3(grid_for((n + 7) / 8, kThreads * kDqU, 16384)), dim3(kThreads), 0, s, packed,
                     code8, c2, mean, n, qtype, out);
  return hipGetLastError();
}

}  // namespace qlora
