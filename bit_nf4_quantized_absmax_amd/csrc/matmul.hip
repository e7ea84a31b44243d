// Fused NF4-dequant matmuls on gfx950 bf16 MFMA.
//
// Forward (automatone.win, "QLoRA paper explained", How it works: the frozen
// 4-bit weights are dequantized to BFloat16 on the fly for the math):
//     Y [M, N] = [X | s T] [deq(W) | B]^T
// i.e. the K loop over packed NF4 tiles plus one (r <= 64) or two (r <= 128)
// extra contraction steps that fold in the LoRA up-projection s T B^T.
//
// dX (same page: gradients flow through the frozen 4-bit base; gptget.net,
// "QLoRA: Efficient Finetuning of Quantized LLMs", Deep Analysis /
// Methodology: the backward matmul dequantizes to 16-bit):
//     dX [M, K] = [dY | s G] [deq(W) ; A]
// contraction over N: the dequantized tile is written transposed into LDS.
//
// Tiling (both kernels): 256 x 256 output tile per workgroup of 512 threads
// (8 waves as 2 x 4, 128 x 64 per wave = 8 x 4 MFMA 16x16x32 bf16 blocks),
// contraction step 64 (= one NF4 block per weight row in the forward), two
// LDS stages, rows padded by 16 bytes so the MFMA operand reads are
// bank-conflict free.  Each weight element of a tile is dequantized once per
// workgroup and shared by all 8 waves through LDS.
#include "common.h"
#include "launch.h"

namespace qlora {

__constant__ uint32_t cMMNF4Level[16] = {QLORA_NF4_LEVEL_BITS};
__constant__ uint32_t cMMT8Level[256] = {QLORA_T8_LEVEL_BITS};

constexpr int kBM = 256;        // output rows per tile (tokens)
constexpr int kBN = 256;        // output columns per tile
constexpr int kBK = 64;         // contraction step
constexpr int kLd = kBK + 8;    // LDS row stride in bf16 (144 bytes)
constexpr int kThreadsMM = 512;

struct MMShared {
  uint16_t a[2][kBM * kLd];     // left operand rows   (X / dY / s T / s G)
  uint16_t b[2][kBN * kLd];     // right operand rows  (deq(W) / B / deq(W)^T / A^T)
  float2 lut2[256];             // byte -> (NF4[low nibble], NF4[high nibble])
  float t8[256];
};

__device__ __forceinline__ void mm_init_tables(MMShared &sh) {
  for (int i = threadIdx.x; i < 256; i += kThreadsMM) {
    sh.lut2[i] = make_float2(u2f(cMMNF4Level[i & 15]), u2f(cMMNF4Level[i >> 4]));
    sh.t8[i] = u2f(cMMT8Level[i]);
  }
}

// One 64-wide contraction step of the 256 x 256 tile from LDS stage `buf`.
// Wave (wm, wn) owns rows 128 wm .. +127 and columns 64 wn .. +63.
__device__ __forceinline__ void mm_compute(const MMShared &sh, int buf, f32x4_t (&acc)[8][4]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int lrow = lane & 15, lk = (lane >> 4) * 8;
#pragma unroll
  for (int kk = 0; kk < kBK; kk += 32) {
    bf16x8_t av[8], bv[4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      av[i] = *reinterpret_cast<const bf16x8_t *>(&sh.a[buf][(wm * 128 + i * 16 + lrow) * kLd + kk + lk]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bv[j] = *reinterpret_cast<const bf16x8_t *>(&sh.b[buf][(wn * 64 + j * 16 + lrow) * kLd + kk + lk]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
  }
}

// Store the accumulators as bf16 (round to nearest even), guarded by M, N.
// MFMA 16x16 output layout: lane holds column (lane & 15), rows 4 (lane >> 4) + v.
__device__ __forceinline__ void mm_store(const f32x4_t (&acc)[8][4], uint16_t *out, int ld, int m0, int n0,
                                         int M, int N) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm * 128 + i * 16 + (lane >> 4) * 4 + v;
        if (row < M && col < N) out[static_cast<int64_t>(row) * ld + col] = f32_to_bf16(acc[i][j][v]);
      }
    }
}

// Left-operand tile: rows m0 .. m0+255 of a row-major bf16 matrix with row
// stride ld, columns c0 .. c0+63.  Thread t loads 16-byte chunks t + 512 i
// (row = chunk / 8, 8 columns each).  Columns must be in range (ld % 8 == 0,
// c0 + 64 <= number of columns); rows past `rows` read as zero.
struct LeftTile {
  uint4 v[4];
  __device__ __forceinline__ void load(const uint16_t *src, int64_t ld, int m0, int rows, int c0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = threadIdx.x + kThreadsMM * i;
      const int row = chunk >> 3, c8 = chunk & 7;
      if (m0 + row < rows)
        v[i] = *reinterpret_cast<const uint4 *>(src + static_cast<int64_t>(m0 + row) * ld + c0 + c8 * 8);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint16_t *dst) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = threadIdx.x + kThreadsMM * i;
      const int row = chunk >> 3, c8 = chunk & 7;
      *reinterpret_cast<uint4 *>(&dst[row * kLd + c8 * 8]) = v[i];
    }
  }
};

// A narrow [rows, r] bf16 matrix (T, G or B) as a 64-wide contraction tile:
// columns j0 .. j0+63 of it, zero past r, each element optionally multiplied
// by `scale` in fp32 and rounded back to bf16.  Element-wise loads: any r.
__device__ __forceinline__ void load_narrow_tile(uint16_t *dst, const uint16_t *src, int r, int m0, int rows,
                                                 int j0, float scale, bool scaled) {
  for (int idx = threadIdx.x; idx < kBM * kBK; idx += kThreadsMM) {
    const int row = idx >> 6, j = idx & 63;
    uint16_t v = 0;
    if (m0 + row < rows && j0 + j < r) {
      v = src[static_cast<int64_t>(m0 + row) * r + j0 + j];
      if (scaled) v = f32_to_bf16(bf16_to_f32(v) * scale);
    }
    dst[row * kLd + j] = v;
  }
}

// ===========================================================================
// Forward: Y = X deq(W)^T + s T B^T
// ===========================================================================

// Right-operand tile of the forward pass: weight rows n0 .. n0+255, K columns
// k0 .. k0+63 (one NF4 block per row).  Thread t covers row t/2, half t%2
// (32 codes = 16 packed bytes) and that row's block constant.
struct FwdWeightTile {
  uint4 p;
  uint32_t code;
  float c2;
  bool valid;
  __device__ __forceinline__ void load(const NF4View &w, int n0, int k0) {
    const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
    const int n = n0 + row;
    valid = n < w.N;
    if (valid) {
      const int64_t blk = (static_cast<int64_t>(n) * w.K + k0) >> 6;
      p = *reinterpret_cast<const uint4 *>(w.packed + (blk << 5) + half * 16);
      code = w.code8[blk];
      c2 = w.c2[blk >> 8];
    }
  }
  __device__ __forceinline__ void store(const MMShared &sh, uint16_t *dst, float mean) const {
    const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
    uint32_t o[16];
    if (valid) {
      const float chat = decode_absmax(sh.t8[code], c2, mean);
      const uint32_t words[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int wd = 0; wd < 4; ++wd)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float2 l = sh.lut2[(words[wd] >> (8 * b)) & 0xffu];
          o[wd * 4 + b] = pack_bf16x2(l.x * chat, l.y * chat);
        }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] = 0;
    }
    uint4 *d = reinterpret_cast<uint4 *>(&dst[row * kLd + half * 32]);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
};

__global__ __launch_bounds__(kThreadsMM) void k_matmul_fwd(const uint16_t *__restrict__ X, int M, NF4View w,
                                                           const uint16_t *__restrict__ T,
                                                           const uint16_t *__restrict__ B, int r, float scale,
                                                           uint16_t *__restrict__ Y) {
  __shared__ __attribute__((aligned(16))) MMShared sh;
  const int tiles_n = (w.N + kBN - 1) / kBN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int K = w.K;
  const float mean = w.mean[0];

  mm_init_tables(sh);
  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  LeftTile xa;
  FwdWeightTile wt;
  xa.load(X, K, m0, M, 0);
  wt.load(w, n0, 0);
  __syncthreads();  // tables ready
  xa.store(sh.a[0]);
  wt.store(sh, sh.b[0], mean);
  __syncthreads();

  const int KT = K / kBK;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      xa.load(X, K, m0, M, (kt + 1) * kBK);
      wt.load(w, n0, (kt + 1) * kBK);
    }
    mm_compute(sh, cur, acc);
    if (more) {
      xa.store(sh.a[cur ^ 1]);
      wt.store(sh, sh.b[cur ^ 1], mean);
    }
    __syncthreads();
  }

  // LoRA up-projection as extra contraction steps: [s T] [B]^T.
  for (int j0 = 0; j0 < r; j0 += kBK) {
    load_narrow_tile(sh.a[0], T, r, m0, M, j0, scale, true);
    load_narrow_tile(sh.b[0], B, r, n0, w.N, j0, 1.0f, false);
    __syncthreads();
    mm_compute(sh, 0, acc);
    __syncthreads();
  }
  mm_store(acc, Y, w.N, m0, n0, M, w.N);
}

// ===========================================================================
// dX = dY deq(W) + s G A
// ===========================================================================

// Right-operand tile of dX: weight rows n0 .. n0+63 (the contraction), K
// columns k0 .. k0+255 (the output), stored transposed as [k][n] in LDS.
// Thread t covers weight row t % 64 and 32 columns 32 (t / 64) .. +31 (half a
// block; both halves share one block constant).
struct DxWeightTile {
  uint4 p;
  uint32_t code;
  float c2;
  bool valid;
  __device__ __forceinline__ void load(const NF4View &w, int n0, int k0) {
    const int nrow = threadIdx.x & 63, seg = threadIdx.x >> 6;
    const int n = n0 + nrow;
    const int k = k0 + seg * 32;
    valid = (n < w.N) && (k < w.K);
    if (valid) {
      const int64_t e = static_cast<int64_t>(n) * w.K + k;
      p = *reinterpret_cast<const uint4 *>(w.packed + (e >> 1));
      code = w.code8[e >> 6];
      c2 = w.c2[e >> 14];
    }
  }
  __device__ __forceinline__ void store(const MMShared &sh, uint16_t *dst, float mean) const {
    const int nrow = threadIdx.x & 63, seg = threadIdx.x >> 6;
    if (valid) {
      const float chat = decode_absmax(sh.t8[code], c2, mean);
      const uint32_t words[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int wd = 0; wd < 4; ++wd)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float2 l = sh.lut2[(words[wd] >> (8 * b)) & 0xffu];
          const uint32_t pr = pack_bf16x2(l.x * chat, l.y * chat);
          const int kk = seg * 32 + wd * 8 + b * 2;
          dst[kk * kLd + nrow] = static_cast<uint16_t>(pr);
          dst[(kk + 1) * kLd + nrow] = static_cast<uint16_t>(pr >> 16);
        }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) dst[(seg * 32 + i) * kLd + nrow] = 0;
    }
  }
};

// A [r, K] rows j0 .. j0+63 (zero past r), columns k0 .. k0+255, transposed
// into LDS as [k][j].
__device__ __forceinline__ void load_a_transposed(uint16_t *dst, const uint16_t *A, int r, int K, int j0,
                                                  int k0) {
  for (int idx = threadIdx.x; idx < kBK * kBN; idx += kThreadsMM) {
    const int j = idx >> 8, k = idx & 255;
    uint16_t v = 0;
    if (j0 + j < r && k0 + k < K) v = A[static_cast<int64_t>(j0 + j) * K + k0 + k];
    dst[k * kLd + j] = v;
  }
}

__global__ __launch_bounds__(kThreadsMM) void k_matmul_dx(const uint16_t *__restrict__ dY, int M, NF4View w,
                                                          const uint16_t *__restrict__ G,
                                                          const uint16_t *__restrict__ A, int r, float scale,
                                                          uint16_t *__restrict__ dX) {
  __shared__ __attribute__((aligned(16))) MMShared sh;
  const int K = w.K, N = w.N;
  const int tiles_k = (K + kBN - 1) / kBN;
  const int tm = blockIdx.x / tiles_k, tk = blockIdx.x % tiles_k;
  const int m0 = tm * kBM, k0 = tk * kBN;
  const float mean = w.mean[0];

  mm_init_tables(sh);
  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The contraction runs over N in steps of 64; N % 8 == 0, so a 16-byte
  // chunk of dY is either wholly inside N or wholly past it.
  const int NT = (N + kBK - 1) / kBK;
  LeftTile ya;
  DxWeightTile wt;
  auto load_dy = [&](int n0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = threadIdx.x + kThreadsMM * i;
      const int row = chunk >> 3, c8 = chunk & 7;
      if (m0 + row < M && n0 + c8 * 8 < N)
        ya.v[i] = *reinterpret_cast<const uint4 *>(dY + static_cast<int64_t>(m0 + row) * N + n0 + c8 * 8);
      else
        ya.v[i] = make_uint4(0, 0, 0, 0);
    }
  };
  load_dy(0);
  wt.load(w, 0, k0);
  __syncthreads();
  ya.store(sh.a[0]);
  wt.store(sh, sh.b[0], mean);
  __syncthreads();

  for (int nt = 0; nt < NT; ++nt) {
    const int cur = nt & 1;
    const bool more = nt + 1 < NT;
    if (more) {
      load_dy((nt + 1) * kBK);
      wt.load(w, (nt + 1) * kBK, k0);
    }
    mm_compute(sh, cur, acc);
    if (more) {
      ya.store(sh.a[cur ^ 1]);
      wt.store(sh, sh.b[cur ^ 1], mean);
    }
    __syncthreads();
  }

  for (int j0 = 0; j0 < r; j0 += kBK) {
    load_narrow_tile(sh.a[0], G, r, m0, M, j0, scale, true);
    load_a_transposed(sh.b[0], A, r, K, j0, k0);
    __syncthreads();
    mm_compute(sh, 0, acc);
    __syncthreads();
  }
  mm_store(acc, dX, K, m0, k0, M, K);
}

// ---------------------------------------------------------------------------
hipError_t launch_matmul_fwd(const uint16_t *X, int M, const NF4View &w, const uint16_t *T,
                             const uint16_t *B, int r, float scale, uint16_t *Y, hipStream_t s) {
  const int tiles = ((M + kBM - 1) / kBM) * ((w.N + kBN - 1) / kBN);
  hipLaunchKernelGGL(k_matmul_fwd, dim3(tiles), dim3(kThreadsMM), 0, s, X, M, w, T, B, r, scale, Y);
  return hipGetLastError();
}

hipError_t launch_matmul_dx(const uint16_t *dY, int M, const NF4View &w, const uint16_t *G,
                            const uint16_t *A, int r, float scale, uint16_t *dX, hipStream_t s) {
  const int tiles = ((M + kBM - 1) / kBM) * ((w.K + kBN - 1) / kBN);
  hipLaunchKernelGGL(k_matmul_dx, dim3(tiles), dim3(kThreadsMM), 0, s, dY, M, w, G, A, r, scale, dX);
  return hipGetLastError();
}

}  // namespace qlora
