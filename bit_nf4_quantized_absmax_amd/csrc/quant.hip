// NF4 + double-quantization codec kernels for gfx950.
//
// Quantize (automatone.win, "QLoRA paper explained", How it works / 4-bit
// NormalFloat and Double Quantization; creativeworksofknowledge.com, "QLoRA:
// Fine-Tune 70B on One GPU", The three innovations / 1-2):
//   pass 1  k_quant_blocks   one read of W: per-64 absmax, 4-bit codes,
//                            nibbles, and the fp64 sum of each workgroup's
//                            256 absmax values (one aligned subtree of the
//                            pairwise sum tree)
//   pass 2  k_quant_consts   the rest of the tree, mean, per-256 scale c2,
//                            8-bit constant codes
//   (k_tree_sum runs between them only when more than 8192 subtree sums
//   remain, i.e. for weights over 2^27 elements.)
// Dequantize: k_dequant     packed codes -> bf16, one read, one write.
//
// Bit-exactness rules: the 4-bit code of w is the count of table thresholds
// strictly below x = fl32(w / absmax) (IEEE quotient, correctly rounded); no
// fused multiply-add (-ffp-contract=off), bf16 conversion is
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

// ---------------------------------------------------------------------------
// Pass 1.  Workgroup w owns blocks [256 w, 256 w + 256), i.e. elements
// [16384 w, 16384 w + 16384).  Thread t loads all of its 16 chunks of 4
// consecutive elements (chunk i = elements 16384 w + 1024 i + 4 t ..) before
// coding the first, so each thread keeps 16 loads in flight; the 16 lanes
// t = 16 g .. 16 g + 15 of chunk i form block 16 i + g.  Elements past n do not
// exist: they load as 0 (which cannot raise a maximum of |w|) and pack as 0.
// The input is fp32 (kIn = 0) or 16-bit bit patterns, bf16 (1) or fp16 (2),
// which widen to fp32 exactly, so every input type codes its fp32 value.
//
// Coding without a division per element.  Multiplying x by 16 is exact, so
// the code is the count of thresholds tau with 16 tau < 16 x.  Cell k
// (k = -16..16) covers 16 x in [k - 1/2, k + 1/2) and stores the count lo of
// thresholds below the cell, the count of thresholds inside it (1, 2 for a
// repeated value, or 0) and 16 tau of the one threshold value inside it
// (+inf if none).  Every threshold of every table lies at least 2^-4 (in
// 16 x units) from a cell edge; a compile-time check below enforces it.
// The kernel forms y = w * fl32(16 * rcp(a)); for a >= 2^-100 (rcp accurate
// to 1 ulp, two more roundings) |y - 16 x| < 2^-17.  The cell is taken from
// y and the code is lo, plus the inside count if y > 16 tau.  This equals the
// exact code whenever |y - 16 tau| >= 2^-15: then y and 16 x lie on the same
// side of 16 tau, and any cell edge between them has no threshold within
// 2^-4 of it.  If one lane of the wave is closer than 2^-15 to its cell's
// threshold, or one block of the wave has a < 2^-100, the wave recodes that
// chunk from the correctly rounded quotient x = w / a, with the same cells.
// Codes of non-finite weights are unspecified (table indices stay clamped).
// ---------------------------------------------------------------------------
constexpr int kWgBlocks = 256;                           // blocks per workgroup of pass 1
constexpr int kWgElems = kWgBlocks * kBlock;             // 16384 elements
constexpr int kChunks = kWgElems / (kThreads * 4);       // 16 chunks of 4 per thread
constexpr int kCellUnit = 16;                            // cells per unit of x
constexpr int kCells = 2 * kCellUnit + 1;                // x in [-1, 1]
constexpr float kNearBand = 0x1p-15f;                    // |y - 16 tau| below this: exact recode
constexpr float kTinyAbsmax = 0x1p-100f;                 // below this: exact recode
constexpr int kCodecMaxGroup = 8;                        // weights per grouped launch

// Compile-time check of the cell property for the three 4-bit tables: each
// threshold at least 2^-4 from a cell edge (in 16 x units), ascending order.
constexpr double q4_threshold_value(uint32_t bits) {
  return static_cast<double>(__builtin_bit_cast(float, bits));
}
constexpr bool q4_cells_separate() {
  constexpr uint32_t th[3 * 15] = {QLORA_Q4_THRESH_BITS};
  for (int q = 0; q < 3; ++q) {
    for (int i = 0; i < 15; ++i) {
      const double y = 16.0 * q4_threshold_value(th[15 * q + i]);
      if (i > 0 && q4_threshold_value(th[15 * q + i]) < q4_threshold_value(th[15 * q + i - 1])) return false;
      double edge = static_cast<double>(static_cast<long long>(y < 0 ? y - 1.0 : y)) + 0.5;   // floor(y) + 1/2
      const double d0 = y - (edge - 1.0), d1 = edge - y, d2 = (edge + 1.0) - y;
      const double d = (d0 < 0 ? -d0 : d0) < (d1 < 0 ? -d1 : d1) ? (d0 < 0 ? -d0 : d0) : (d1 < 0 ? -d1 : d1);
      if ((d < (d2 < 0 ? -d2 : d2) ? d : (d2 < 0 ? -d2 : d2)) < 0.0625) return false;
    }
  }
  return true;
}
static_assert(q4_cells_separate(), "4-bit thresholds too close to a coding cell edge");
static_assert(kWgBlocks == kGroup, "a pass-1 workgroup writes whole groups of constants");

// Cell table of table qtype into c[0 .. kCells): (bits of 16 tau or +inf, lo | hi << 16).
__device__ __forceinline__ void build_cells(int qtype, uint2 *c) {
  const int t = threadIdx.x;
  if (t < kCells) {
    const int k = t - kCellUnit;
    const float lo = (k - 0.5f) / kCellUnit, hi = (k + 0.5f) / kCellUnit;   // exact: odd / 32
    uint32_t below = 0, inside = 0;
    float tau16 = INFINITY;
    for (int i = 0; i < 15; ++i) {
      const float th = u2f(cQ4Thresh[15 * qtype + i]);
      below += th < lo;
      if (th >= lo && th < hi) { ++inside; tau16 = th * 16.0f; }
    }
    c[t] = make_uint2(__float_as_uint(tau16), below | ((below + inside) << 16));
  }
}

// Cell of 16 x from y = 16 x (approximately): nearest integer, clamped.
__device__ __forceinline__ int cell_index(float y) {
  int k;
  asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(k) : "v"(y));   // floor(y + 1/2); NaN -> 0
  return min(max(k, -kCellUnit), kCellUnit);
}

// Maximum over the 16 lanes of a row (one block): non-negative floats order
// as their bit patterns.
__device__ __forceinline__ float row16_max(float a) {
  uint32_t u = __float_as_uint(a);
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0xB1, 0xF, 0xF, false)));   // lane ^ 1
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x4E, 0xF, 0xF, false)));   // lane ^ 2
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x141, 0xF, 0xF, false)));  // half mirror
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x140, 0xF, 0xF, false)));  // mirror
  return __uint_as_float(u);
}

template <int kIn>
__device__ __forceinline__ float widen16(uint32_t h) {
  return kIn == 1 ? u2f(h << 16) : static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// Raw chunk storage: 4 fp32 values, or 4 16-bit patterns in two dwords.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <int kIn> struct RawChunk { typedef u32x2_t type; };
template <> struct RawChunk<0> { typedef f32x4_t type; };

template <int kIn>
__device__ __forceinline__ f32x4_t widen_chunk(const typename RawChunk<kIn>::type &r) {
  if constexpr (kIn == 0) {
    return r;
  } else {
    f32x4_t v;
    v[0] = widen16<kIn>(r.x & 0xFFFFu);
    v[1] = widen16<kIn>(r.x >> 16);
    v[2] = widen16<kIn>(r.y & 0xFFFFu);
    v[3] = widen16<kIn>(r.y >> 16);
    return v;
  }
}

// The 16 chunks of one thread, coded; kFull: the workgroup's range lies wholly below n.
template <int kIn, bool kFull>
__device__ __forceinline__ void quant_chunks(const void *__restrict__ W, int64_t n, int qtype,
                                             uint8_t *__restrict__ packed, int64_t wg, const uint2 *cells,
                                             float *sA) {
  typedef typename RawChunk<kIn>::type raw_t;
  const int t = threadIdx.x;
  const int64_t e0 = wg * kWgElems;
  raw_t r[kChunks];
  if (kFull) {
    const raw_t *src = reinterpret_cast<const raw_t *>(static_cast<const char *>(W) + e0 * (kIn == 0 ? 4 : 2)) + t;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) r[i] = __builtin_nontemporal_load(src + i * kThreads);
  } else {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int64_t e = e0 + static_cast<int64_t>(i * kThreads + t) * 4;
      if constexpr (kIn == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) r[i][k] = (e + k < n) ? static_cast<const float *>(W)[e + k] : 0.0f;
      } else {
        const uint16_t *h = static_cast<const uint16_t *>(W);
        uint32_t q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = (e + k < n) ? h[e + k] : 0u;
        r[i] = u32x2_t{q[0] | (q[1] << 16), q[2] | (q[3] << 16)};
      }
    }
  }
  __syncthreads();   // cells ready
  const uint32_t zero_word = static_cast<uint32_t>(q4_zero_code(qtype)) * 0x1111u;
  uint16_t *dst = reinterpret_cast<uint16_t *>(packed + (e0 >> 1));
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const f32x4_t w = widen_chunk<kIn>(r[i]);
    const float a = row16_max(fmaxf(fmaxf(fabsf(w[0]), fabsf(w[1])), fmaxf(fabsf(w[2]), fabsf(w[3]))));
    const float r16 = 16.0f * __builtin_amdgcn_rcpf(a);
    uint32_t word = 0;
    bool near = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float y = w[k] * r16;
      const uint2 ce = cells[cell_index(y)];
      const float d = y - __uint_as_float(ce.x);
      near |= fabsf(d) < kNearBand;
      word |= ((ce.y >> (d > 0.0f ? 16u : 0u)) & 15u) << (4 * k);
    }
    if (__any(near || a < kTinyAbsmax)) {   // wave-uniform: recode from the exact quotient
      word = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float y = (w[k] / a) * 16.0f;
        const uint2 ce = cells[cell_index(y)];
        word |= ((ce.y >> (y > __uint_as_float(ce.x) ? 16u : 0u)) & 15u) << (4 * k);
      }
    }
    if (!(a > 0.0f)) word = zero_word;
    if (kFull) {
      __builtin_nontemporal_store(static_cast<uint16_t>(word), dst + i * kThreads + t);
    } else {
      const int64_t e = e0 + static_cast<int64_t>(i * kThreads + t) * 4;
      if (e + 3 >= n) word &= (e >= n) ? 0u : (e + 1 >= n ? 0xFu : (e + 2 >= n ? 0xFFu : 0xFFFu));
      if (e < n) packed[e >> 1] = static_cast<uint8_t>(word);
      if (e + 2 < n) packed[(e >> 1) + 1] = static_cast<uint8_t>(word >> 8);
    }
    sA[i * 16 + (t >> 4)] = a;   // the 16 lanes of the block store the same value
  }
}

// Pairwise fp64 sum of s[0 .. 256) by wave 0 (call after a barrier): lane l
// forms ((s[4l] + s[4l+1]) + (s[4l+2] + s[4l+3])), then six levels pair
// neighbouring lanes.  Returns the sum in lane 0.
template <typename T>
__device__ __forceinline__ double tree256_wave0(const T *s) {
  const int l = threadIdx.x;
  double r = (static_cast<double>(s[4 * l]) + static_cast<double>(s[4 * l + 1])) +
             (static_cast<double>(s[4 * l + 2]) + static_cast<double>(s[4 * l + 3]));
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const double lo = __shfl(r, 2 * l), hi = __shfl(r, 2 * l + 1);
    r = lo + hi;
  }
  return r;
}

// ---------------------------------------------------------------------------
// Grouped launches.  One launch serves up to kCodecMaxGroup weights (members):
// member j owns the workgroups [wg_begin[j], wg_begin[j + 1]) of the grid and
// each workgroup finds its member from blockIdx.x (uniform, scalar).  A
// single weight is a group of one.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int codec_member(const int *wg_begin, int count) {
  int i = 0;
#pragma unroll
  for (int j = 1; j < kCodecMaxGroup; ++j)
    i = (j < count && static_cast<int>(blockIdx.x) >= wg_begin[j]) ? j : i;
  return i;
}

struct QuantBlocksArgs {
  const void *W[kCodecMaxGroup];
  int64_t n[kCodecMaxGroup];
  uint8_t *packed[kCodecMaxGroup];
  float *absmax[kCodecMaxGroup];
  double *subtree[kCodecMaxGroup];
  int qtype[kCodecMaxGroup];
  int wg_begin[kCodecMaxGroup];
  int count;
};

template <int kIn>
__global__ __launch_bounds__(kThreads) void k_quant_blocks(const QuantBlocksArgs args) {
  __shared__ uint2 sCells[kCells];
  __shared__ float sA[kWgBlocks];
  const int m = codec_member(args.wg_begin, args.count);
  const int64_t wg = static_cast<int64_t>(blockIdx.x) - args.wg_begin[m];
  const int64_t n = args.n[m];
  const int qtype = args.qtype[m];
  build_cells(qtype, sCells);
  if ((wg + 1) * kWgElems <= n)
    quant_chunks<kIn, true>(args.W[m], n, qtype, args.packed[m], wg, sCells + kCellUnit, sA);
  else
    quant_chunks<kIn, false>(args.W[m], n, qtype, args.packed[m], wg, sCells + kCellUnit, sA);
  __syncthreads();
  // absmax holds whole groups of 256: blocks past nb (last workgroup) get 0.
  args.absmax[m][wg * kWgBlocks + threadIdx.x] = sA[threadIdx.x];
  if (threadIdx.x < 64) {
    const double r = tree256_wave0(sA);
    if (threadIdx.x == 0) args.subtree[m][wg] = r;
  }
}

// ---------------------------------------------------------------------------
// Tree levels for very large weights.  Workgroup g reduces
// in[2048 g, 2048 g + 2048) (zero beyond len) to one fp64 value with the
// neighbour-pairing tree: 8 values per thread ((v0+v1)+(v2+v3))+((v4+v5)+(v6+v7)),
// then level by level in LDS, s'[t] = s[2t] + s[2t+1].  Because chunks are
// aligned powers of two, applying this to subtree sums continues the global
// tree exactly.
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
// Pass 2.  Every wave first issues the read of its first group of
// constants; every workgroup then finishes the tree over the plen <= 8192
// subtree sums (thread t: sums 32 t .. 32 t + 31 by neighbour pairs in
// registers, then the 256 thread sums as in tree256_wave0), then
// mean = fl32(sum / nb).  One wave per group of 256 constants, 4 per lane:
// d = fl32(c - mean), c2 = max |d| over the group, code = number of T8
// thresholds below fl32(d / c2) (binary search over the 255 thresholds, with
// +inf as a 256th sentinel).  c2 = 0 -> code 127.
// ---------------------------------------------------------------------------
constexpr int kConstsMaxPartials = 32 * kThreads;   // 8192
static_assert(kThreads == 256, "one thread per 8-bit threshold-table entry");

struct QuantConstsArgs {
  const float *absmax[kCodecMaxGroup];
  int64_t nb[kCodecMaxGroup];
  const double *partials[kCodecMaxGroup];
  int64_t plen[kCodecMaxGroup];
  uint8_t *code8[kCodecMaxGroup];
  float *c2[kCodecMaxGroup];
  float *mean[kCodecMaxGroup];
  int wg_begin[kCodecMaxGroup];
  int wgs[kCodecMaxGroup];
  int count;
};

__global__ __launch_bounds__(kThreads) void k_quant_consts(const QuantConstsArgs args) {
  __shared__ float thr[256];
  __shared__ double s[kThreads];
  __shared__ float sMean;
  const int mem = codec_member(args.wg_begin, args.count);
  const float *__restrict__ absmax = args.absmax[mem];
  const int64_t nb = args.nb[mem];
  const double *__restrict__ partials = args.partials[mem];
  const int64_t plen = args.plen[mem];
  uint8_t *__restrict__ code8 = args.code8[mem];
  float *__restrict__ c2 = args.c2[mem];
  const int64_t wg = static_cast<int64_t>(blockIdx.x) - args.wg_begin[mem];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int64_t nb2 = (nb + kGroup - 1) / kGroup;
  const int64_t waves = static_cast<int64_t>(args.wgs[mem]) * (kThreads / 64);
  int64_t g = wg * (kThreads / 64) + (t >> 6);
  // The wave's first group of constants, the subtree sums and the threshold
  // table are all requested before any of them is used, so the three reads
  // overlap.  absmax is padded to whole groups (zeros past nb).
  f32x4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
  if (g < nb2) c = *reinterpret_cast<const f32x4_t *>(absmax + g * kGroup + lane * 4);
  {
    double v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = (32 * t + i < plen) ? partials[32 * t + i] : 0.0;
    const float th = (t < 255) ? u2f(cT8Thresh[t]) : INFINITY;   // kThreads == 256 entries
    thr[t] = th;
#pragma unroll
    for (int w = 16; w >= 1; w >>= 1)
#pragma unroll
      for (int j = 0; j < w; ++j) v[j] = v[2 * j] + v[2 * j + 1];
    s[t] = v[0];
  }
  __syncthreads();
  if (t < 64) {
    const double r = tree256_wave0(s);
    if (t == 0) sMean = static_cast<float>(r / static_cast<double>(nb));
  }
  __syncthreads();
  const float mean = sMean;
  if (wg == 0 && t == 0) args.mean[mem][0] = mean;

  for (; g < nb2; g += waves) {
    const int64_t idx = g * kGroup + lane * 4;
    float d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = (idx + i < nb) ? (c[i] - mean) : 0.0f;
    if (g + waves < nb2) c = *reinterpret_cast<const f32x4_t *>(absmax + (g + waves) * kGroup + lane * 4);
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

struct DequantArgs {
  const uint8_t *packed[kCodecMaxGroup];
  const uint8_t *code8[kCodecMaxGroup];
  const float *c2[kCodecMaxGroup];
  const float *mean[kCodecMaxGroup];
  uint16_t *out[kCodecMaxGroup];
  int64_t n[kCodecMaxGroup];
  int qtype[kCodecMaxGroup];
  int wg_begin[kCodecMaxGroup];
  int wgs[kCodecMaxGroup];
  int count;
};

__global__ __launch_bounds__(kThreads) void k_dequant(const DequantArgs args) {
  __shared__ float2 pairs[256];   // byte -> (level of its low nibble, level of its high nibble)
  __shared__ float t8[256];
  const int mem = codec_member(args.wg_begin, args.count);
  const uint8_t *__restrict__ packed = args.packed[mem];
  const uint8_t *__restrict__ code8 = args.code8[mem];
  const float *__restrict__ c2 = args.c2[mem];
  uint16_t *__restrict__ out = args.out[mem];
  const int64_t n = args.n[mem];
  const int qtype = args.qtype[mem];
  const int64_t wg = static_cast<int64_t>(blockIdx.x) - args.wg_begin[mem];
  for (int i = threadIdx.x; i < 256; i += kThreads) {
    pairs[i] = make_float2(u2f(cQ4Level[16 * qtype + (i & 15)]), u2f(cQ4Level[16 * qtype + (i >> 4)]));
    t8[i] = u2f(cT8Level[i]);
  }
  __syncthreads();
  const float mean = args.mean[mem][0];
  const int64_t nchunks = (n + 7) / 8;
  const int64_t span = static_cast<int64_t>(kThreads) * kDqU;
  for (int64_t c0 = wg * span + threadIdx.x; c0 < nchunks; c0 += static_cast<int64_t>(args.wgs[mem]) * span) {
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

static int64_t subtree_count(int64_t nb) { return (nb + kWgBlocks - 1) / kWgBlocks; }

size_t quantize_ws_bytes(int64_t n) {
  if (n < 1) return 0;
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t p = subtree_count(nb);
  // absmax fp32 [256 p] (whole groups; zeros past nb) | subtree sums fp64 [p] | next tree level fp64 [p / 2048]
  return static_cast<size_t>(p) * kWgBlocks * 4 + static_cast<size_t>(p + tree_partials(p)) * 8;
}

hipError_t launch_quantize_group(int count, const QuantJob *jobs, int in_type, hipStream_t s) {
  if (count < 1 || count > kCodecMaxGroup) return hipErrorInvalidValue;
  QuantBlocksArgs a1{};
  QuantConstsArgs a2{};
  a1.count = a2.count = count;
  int64_t grid1 = 0, grid2 = 0;
  for (int j = 0; j < count; ++j) {
    const QuantJob &q = jobs[j];
    const int64_t nb = (q.n + kBlock - 1) / kBlock;
    const int64_t len = subtree_count(nb);
    float *absmax = static_cast<float *>(q.ws);
    double *sub = reinterpret_cast<double *>(static_cast<char *>(q.ws) + static_cast<size_t>(len) * kWgBlocks * 4);
    a1.W[j] = q.W;
    a1.n[j] = q.n;
    a1.packed[j] = q.packed;
    a1.absmax[j] = absmax;
    a1.subtree[j] = sub;
    a1.qtype[j] = q.qtype;
    a1.wg_begin[j] = static_cast<int>(grid1);
    grid1 += len;
    a2.absmax[j] = absmax;
    a2.nb[j] = nb;
    a2.partials[j] = sub;
    a2.plen[j] = len;
    a2.code8[j] = q.code8;
    a2.c2[j] = q.c2;
    a2.mean[j] = q.mean;
    a2.wg_begin[j] = static_cast<int>(grid2);
    // At most 256 workgroups per member: each one repeats the tree over the
    // member's subtree sums, so fewer, longer workgroups read less.
    a2.wgs[j] = static_cast<int>(grid_for((nb + kGroup - 1) / kGroup, kThreads / 64, 256));
    grid2 += a2.wgs[j];
  }
  const dim3 g1(static_cast<unsigned>(grid1));
  if (in_type == 1)
    hipLaunchKernelGGL(k_quant_blocks<1>, g1, dim3(kThreads), 0, s, a1);
  else if (in_type == 2)
    hipLaunchKernelGGL(k_quant_blocks<2>, g1, dim3(kThreads), 0, s, a1);
  else
    hipLaunchKernelGGL(k_quant_blocks<0>, g1, dim3(kThreads), 0, s, a1);
  for (int j = 0; j < count; ++j) {
    if (a2.plen[j] > kConstsMaxPartials) {   // n > 2^27: one more tree level (len <= 2^17 -> at most 64 sums)
      double *level = a1.subtree[j] + a2.plen[j];
      hipLaunchKernelGGL(k_tree_sum<double>, dim3(static_cast<unsigned>(tree_partials(a2.plen[j]))), dim3(kThreads),
                         0, s, a1.subtree[j], a2.plen[j], level);
      a2.partials[j] = level;
      a2.plen[j] = tree_partials(a2.plen[j]);
    }
  }
  hipLaunchKernelGGL(k_quant_consts, dim3(static_cast<unsigned>(grid2)), dim3(kThreads), 0, s, a2);
  return hipGetLastError();
}

hipError_t launch_quantize(const void *W, int in_type, int64_t n, int qtype, uint8_t *packed, uint8_t *code8,
                           float *c2, float *mean, void *ws, hipStream_t s) {
  const QuantJob job{W, n, qtype, packed, code8, c2, mean, ws};
  return launch_quantize_group(1, &job, in_type, s);
}

hipError_t launch_dequantize_group(int count, const DequantJob *jobs, hipStream_t s) {
  if (count < 1 || count > kCodecMaxGroup) return hipErrorInvalidValue;
  DequantArgs a{};
  a.count = count;
  int64_t grid = 0;
  for (int j = 0; j < count; ++j) {
    const DequantJob &d = jobs[j];
    a.packed[j] = d.packed;
    a.code8[j] = d.code8;
    a.c2[j] = d.c2;
    a.mean[j] = d.mean;
    a.out[j] = d.out;
    a.n[j] = d.n;
    a.qtype[j] = d.qtype;
    a.wg_begin[j] = static_cast<int>(grid);
    a.wgs[j] = static_cast<int>(grid_for((d.n + 7) / 8, kThreads * kDqU, 16384));
    grid += a.wgs[j];
  }
  hipLaunchKernelGGL(k_dequant, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *packed, const uint8_t *code8, const float *c2,
                             const float *mean, int64_t n, int qtype, uint16_t *out, hipStream_t s) {
  const DequantJob job{packed, code8, c2, mean, n, qtype, out};
  return launch_dequantize_group(1, &job, s);
}

}  // namespace qlora
