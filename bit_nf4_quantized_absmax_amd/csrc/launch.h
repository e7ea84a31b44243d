// Host-side launchers of the gfx950 kernels (internal to libqlora_mi355x).
// Arguments are validated by the C ABI layer before any of these is called;
// each returns the hipError_t of its launch(es).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qlora {

// ---- codec ---------------------------------------------------------------
// Workspace of one quantized weight: absmax fp32 in whole groups of 256 |
// subtree sums fp64 | one further tree level fp64.
size_t quantize_ws_bytes(int64_t n);
// W: fp32 (in_type 0), bf16 (1) or fp16 (2) elements.
hipError_t launch_quantize(const void *W, int in_type, int64_t n, int qtype, uint8_t *packed, uint8_t *code8,
                           float *c2, float *mean, void *ws, hipStream_t s);
hipError_t launch_dequantize(const uint8_t *packed, const uint8_t *code8, const float *c2,
                             const float *mean, int64_t n, int qtype, uint16_t *out, hipStream_t s);
// Up to 8 weights per call: two launches for the whole group (quantize; one
// more per member above 2^27 elements), one launch (dequantize).
struct QuantJob {
  const void *W;
  int64_t n;
  int qtype;
  uint8_t *packed;
  uint8_t *code8;
  float *c2;
  float *mean;
  void *ws;   // quantize_ws_bytes(n) bytes, 16-byte aligned
};
hipError_t launch_quantize_group(int count, const QuantJob *jobs, int in_type, hipStream_t s);
struct DequantJob {
  const uint8_t *packed;
  const uint8_t *code8;
  const float *c2;
  const float *mean;
  int64_t n;
  int qtype;
  uint16_t *out;
};
hipError_t launch_dequantize_group(int count, const DequantJob *jobs, hipStream_t s);

// ---- NF4 weight view passed to the matmul kernels ---------------------------
struct NF4View {
  const uint8_t *packed;
  const uint8_t *code8;
  const float *c2;
  const float *mean;
  int N;  // rows (output features)
  int K;  // columns (input features), multiple of 64
  int qtype;  // 4-bit level table: 0 NF4, 1 FP4, 2 Int4 (rows of QLORA_Q4_LEVEL_BITS)
};

// ---- large-M matmuls (T and G already carry the LoRA scale) ---------------------
// One product of a grouped launch: left operand L [M, contraction], the LoRA
// pair (Ln = T or G, Rn = B or A), mask (dropout dX only) and output.
struct MatmulJob {
  const uint16_t *L;
  const uint16_t *Ln;
  const uint16_t *Rn;
  const uint32_t *keep;
  uint16_t *out;
  NF4View w;
  int M;
  int r;
  const uint16_t *wd = nullptr;   // dequantized bf16 weight [w.N, w.K] (the pre-dequantized kernels)
};
// Up to 4 forward products (M >= 65 each) in one launch over their
// concatenated tile grids; each output as launch_matmul_fwd computes it.
hipError_t launch_matmul_fwd_group(int count, const MatmulJob *jobs, hipStream_t s);
// The same products from dequantized bf16 weights (job.wd; only w.N and w.K
// of job.w are read): forward groups of up to 4, and dX (w.N % 64 == 0).
// Outputs are bit-identical to the fused kernels' on the same weight.
hipError_t launch_pre_matmul_fwd_group(int count, const MatmulJob *jobs, hipStream_t s);
hipError_t launch_pre_matmul_dx(const MatmulJob &job, hipStream_t s);
// Y [M, N] = X deq(W)^T + T B^T
hipError_t launch_matmul_fwd(const uint16_t *X, int M, const NF4View &w, const uint16_t *T,
                             const uint16_t *B, int r, uint16_t *Y, hipStream_t s);
// ---- LoRA dropout (keep mask of the LoRA input) ------------------------------
// n = M K elements, K % 32 == 0; keep: uint32 [M][K / 32], bit k % 32.
hipError_t launch_dropout_mask(const uint16_t *X, int64_t n, uint64_t seed, uint32_t thresh, uint16_t *Xd,
                               uint32_t *keep, hipStream_t s);
hipError_t launch_dropout_apply(const uint16_t *X, int64_t n, const uint32_t *keep, uint16_t *Xd, hipStream_t s);
// dX = dY deq(W) + (G A) * keep
hipError_t launch_matmul_dx_drop(const uint16_t *dY, int M, const NF4View &w, const uint16_t *G,
                                 const uint16_t *A, int r, const uint32_t *keep, uint16_t *dX, hipStream_t s);

// ---- LoRA products of linears sharing one input X (q/k/v, gate/up) -----------
// Member i: R[i] (A_i for T, G_i for dA; rcols[i] columns per row), r[i],
// scale[i], out[i]; part[i] / plane[i]: its fp32 split partials (dA only).
constexpr int kLoraMaxShared = 8;
struct LoraShared {
  const uint16_t *R[kLoraMaxShared];
  uint16_t *out[kLoraMaxShared];
  float *part[kLoraMaxShared];
  int64_t plane[kLoraMaxShared];
  float scale[kLoraMaxShared];
  int rcols[kLoraMaxShared];
  int r[kLoraMaxShared];
  int y0[kLoraMaxShared + 1];   // first 64-column chunk of each member (prefix sums)
  int n;
};
// T_i = bf16(scale_i X A_i^T) for every member, X read once (bit-identical
// to launch_lora_down per member).
hipError_t launch_lora_down_shared(const uint16_t *X, int M, int K, int n, const uint16_t *const *A, const int *r,
                                   const float *scale, uint16_t *const *T, hipStream_t s);
// dA_i = G_i^T X for every member (G_i carries the scale), bit-identical to
// launch_lora_grad_w(X, G_i, ...) per member; workspace lora_dA_shared_ws_bytes.
size_t lora_dA_shared_ws_bytes(int M, int K, int n, const int *r);
hipError_t launch_lora_dA_shared(const uint16_t *X, int M, int K, int n, const uint16_t *const *G, const int *r,
                                 uint16_t *const *dA, void *ws, hipStream_t s);

// ---- small-M forward (M <= small_m_max()) -------------------------------------
// One linear of a group: Y = X deq(W)^T + T B^T.  T comes from Tin (bf16,
// already scaled) or, when P is set, is formed as bf16(scale * sum of the
// down-projection partials written to P by the first of the two launches).
// Tout (nullable) receives that T.
struct SmLinear {
  const uint16_t *X;
  NF4View w;
  const uint16_t *A;
  const uint16_t *B;
  const uint16_t *Tin;
  float *P;
  float *Pd;    // stream path: the down-projection partials [K / 256][M][r] fp32
  uint16_t *Y;
  uint16_t *Tout;
  int r;
  float scale;
  int S;        // set by launch_small_m: column chunks of the down-projection
  int kw;       // set by launch_small_m: columns per wave of the down-projection
  int jtiles;   // set by launch_small_m
};
constexpr int kSmMaxGroup = 8;
struct SmGroup {
  SmLinear lin[kSmMaxGroup];
  int down_start[kSmMaxGroup + 1];
  int main_start[kSmMaxGroup + 1];
  // Work plan (set by launch_small_m_gemv and launch_small_m_stream): first
  // item (row tile) of each linear, first unit of each linear (stream
  // kernel) and the GEMV kernels' chunks per item.
  int item0[kSmMaxGroup + 1];
  int cost0[kSmMaxGroup + 1];
  int nch[kSmMaxGroup];
  int xoff[kSmMaxGroup];   // byte offset of each linear's X in the GEMV kernel's LDS copy
  int toff[kSmMaxGroup];   // byte offset of each linear's T there
  int xs0[kSmMaxGroup + 1];   // first X copy slot (64 x 16 bytes) of each linear
  int dg0[kSmMaxGroup + 1];   // first (adapter row, chunk) item of each linear in k_sm_down_gemv
  int n;
  int M;
};
int small_m_max();
// Whether the small-M kernels take this case (M <= small_m_max(), r % 8 == 0).
bool small_m_ok(int64_t M, int r);
// fp32 partial buffer P of one linear: [S <= 4][M][r].
size_t small_m_ws_bytes(int M, int K, int r);
hipError_t launch_small_m(SmGroup &grp, hipStream_t s);
// Dequant-GEMV for M <= small_m_gemv_max() (S and the partials already
// prepared by launch_small_m).
int small_m_gemv_max();
// Whether the group takes the one-token path with X in LDS; if so the
// down-projection partials come from launch_small_m_down_gemv, one slice per
// 2048 columns (S = ceil(K / 2048)).
bool small_m_gemv_xl(const SmGroup &grp);
int small_m_gemv_slices(int K);
hipError_t launch_small_m_down_gemv(SmGroup &grp, hipStream_t s);
hipError_t launch_small_m_gemv(SmGroup &grp, hipStream_t s);
// Streaming path for 4 < M <= 64, K % 256 == 0 (down-projection, T and the
// product in three kernels); every linear's P is the start of its workspace
// region of small_m_stream_ws_bytes.
bool small_m_stream_ok(int64_t M, int K, int r);
bool small_m_stream_group_ok(const SmGroup &grp);
size_t small_m_stream_ws_bytes(int M, int N, int K, int r);
hipError_t launch_small_m_stream(SmGroup &grp, hipStream_t s);
// Small-M form of launch_matmul_fwd with T given (requires small_m_ok).
hipError_t launch_small_m_fwd(const uint16_t *X, int M, const NF4View &w, const uint16_t *T, const uint16_t *B,
                              int r, uint16_t *Y, hipStream_t s);
// dX [M, K] = dY deq(W) + G A
hipError_t launch_matmul_dx(const uint16_t *dY, int M, const NF4View &w, const uint16_t *G,
                            const uint16_t *A, int r, uint16_t *dX, hipStream_t s);

// ---- LoRA products ------------------------------------------------------------
// T [M, r] = scale X [M, K] A^T  (A [r, K]); K % 8 == 0.
hipError_t launch_lora_down(const uint16_t *X, int M, int K, const uint16_t *A, int r, float scale,
                            uint16_t *T, hipStream_t s);
// G [M, r] = scale dY [M, N] B  (B [N, r]); N % 8 == 0; ws (lora_grad_in_ws_bytes)
// holds a zero-padded copy of B when r % 8 != 0.
size_t lora_grad_in_ws_bytes(int N, int r);
hipError_t launch_lora_grad_in(const uint16_t *dY, int M, int N, const uint16_t *B, int r, float scale,
                               uint16_t *G, void *ws, hipStream_t s);
// out = P^T Q over M, P [M, D], Q [M, r]; stored as [r, D] (dA) or [D, r] (dB);
// D % 8 == 0; ws (lora_grad_ws_bytes): padded Q (r % 8 != 0) | split partials
// for sp M-splits (sp <= 0: the product's own choice, as launch_lora_grad_w).
size_t lora_grad_ws_bytes(int M, int D, int r, int sp);
// Up to 16 such products (dA and dB of up to 8 linears) in one k_lora_tn
// launch plus at most one partial-sum launch; each product as by
// launch_lora_grad_w with its own workspace (lora_grad_ws_bytes).
struct GradWJob {
  const uint16_t *P;
  const uint16_t *Q;
  int M;
  int D;
  int r;
  bool out_r_major;
  uint16_t *out;
  void *ws;
  int splits;   // M-splits of this product; 0: chosen for the product alone
};
hipError_t launch_lora_grad_w_group(int count, const GradWJob *jobs, hipStream_t s);
// M-splits shared by one linear's dA [r, K] and dB [N, r] launched together:
// chosen so that their tiles together fill the GPU in whole rounds.
int lora_grad_pair_splits(int M, int K, int N, int r);
// Splits used for one linear: the shared count when both dA and dB are
// computed, else the single product's own (tn_splits, as the shared-input dA).
int lora_grad_splits(int M, int K, int N, int r, bool dA, bool dB);
// Workspace of one of the pair's products (D = K for dA, N for dB), large
// enough for either split choice.
size_t lora_grad_pair_ws_bytes(int M, int D, int K, int N, int r);
hipError_t launch_lora_grad_w(const uint16_t *P, const uint16_t *Q, int M, int D, int r, bool out_r_major,
                              uint16_t *out, void *ws, hipStream_t s);

}  // namespace qlora
