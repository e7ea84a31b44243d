/*
 * qlora.h -- C ABI of libqlora_mi355x.so, the frozen-base QLoRA linear layer
 * on AMD Instinct MI355X (gfx950).
 *
 * The layer (automatone.win, "QLoRA paper explained", TL;DR and How it works;
 * aiwiki.com.my, "QLoRA", Key Concepts and Technology): the frozen base
 * weight W [N, K] is stored as 4-bit NormalFloat codes with one absmax
 * constant per block of 64 weights; the constants are themselves quantized
 * to 8-bit codes in groups of 256 around a per-tensor mean ("double
 * quantization", creativeworksofknowledge.com, "QLoRA: Fine-Tune 70B on One
 * GPU", The three innovations / 2).  Each pass dequantizes W to bf16 on the
 * fly inside the matmul and adds a 16-bit LoRA branch:
 *
 *     T  = s X A^T                  Y  = X deq(W)^T + T B^T
 *     G  = s dY B                   dX = dY deq(W) + G A
 *     dA = G^T X                    dB = dY^T T
 *
 * with s = alpha / r.  This is the pages' layer Y = X W^T + s X A^T B^T
 * with the scale folded into the rank-r intermediates: T and G carry s,
 * applied once in fp32 before their single rounding to bf16, so the fused
 * matmuls add T B^T and G A as plain contraction steps.  No gradient is
 * formed for W, which is frozen.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates no device memory and keeps no per-call state.  Scratch space
 *    is passed in as a workspace (size from the *_workspace_bytes queries).
 *  - bf16 tensors are passed as uint16_t bit patterns.  All tensors are
 *    row-major and contiguous; every pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously on it; the call returns without synchronizing.
 *  - The status is returned synchronously.  Arguments are validated before
 *    anything is launched: on any error nothing is launched or written.  A
 *    failed launch returns QLORA_ERR_HIP.
 *  - Gradients overwrite their outputs (no accumulation).
 *  - M = 0 (no tokens) is valid everywhere a token count is taken: the call
 *    validates its arguments, launches nothing and writes nothing (dA and dB,
 *    which would be zero, are left as they were).  Pointers to tensors with M
 *    rows (X, dY, Y, T, G, dX, keep masks) may then be NULL, as the storage of
 *    an empty tensor is.
 *  - The linear-layer calls take W [N, K] with K % 64 == 0 (a 64-block never
 *    straddles a row), N % 8 == 0 (16-byte rows of Y and dB) and every size
 *    below 2^31 (M * max(N, K) included); the codec calls take any
 *    rows, cols >= 1 with rows * cols < 2^31.
 *  - Results are deterministic: no floating-point atomics are used, so two
 *    calls on the same inputs give the same bits.
 *  - Inputs with NaN or Inf are outside the contract (outputs unspecified).
 */
#ifndef QLORA_MI355X_H
#define QLORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_INVALID_ARG = -1,       /* null/misaligned pointer, negative size, bad scale */
  QLORA_ERR_UNSUPPORTED_SHAPE = -2, /* K % 64 != 0, N % 8 != 0, r outside [1, 128], size >= 2^31 */
  QLORA_ERR_WORKSPACE = -3,         /* workspace missing or smaller than required */
  QLORA_ERR_HIP = -4,               /* a HIP runtime call or kernel launch failed */
  QLORA_ERR_SCRATCH_LIMIT = -5      /* qlora_linear_fwd_noalloc: needs more than the static scratch */
} qlora_status;

/* Size of the per-GPU static scratch array of qlora_linear_fwd_noalloc. */
#define QLORA_STATIC_SCRATCH_BYTES ((size_t)16 << 20)

/* 4-bit data types of the first-level codes: the 16-entry level table the
 * codes index.  Everything else in the format (blocks of 64, nearest level
 * with ties to the lower code, packing, the double-quantized constants) is
 * shared.  The pages compare NF4 with evenly spaced 4-bit integers and
 * exponent-spaced 4-bit floats (automatone.win, "QLoRA paper explained",
 * 4-bit NormalFloat; Results, FP4 vs NF4).
 *   NF4   quantiles of N(0, 1) with an exact zero, normalised to [-1, 1]
 *   FP4   E2M1 floats (0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives) / 6, ascending,
 *         codes 7 and 8 both zero (8 is never produced)
 *   INT4  k / 7 for k = -8 .. 7 (code 0, -8/7, is never produced) */
typedef enum { QLORA_Q4_NF4 = 0, QLORA_Q4_FP4 = 1, QLORA_Q4_INT4 = 2 } qlora_q4_type;

/* One quantized weight W [rows = N, cols = K], n = rows * cols elements,
 * flattened row-major.  Block b covers elements [64 b, 64 b + 64); group g
 * covers blocks [256 g, 256 g + 256); the last block and group may be partial.
 *   packed  [ceil(n/2)]   4-bit codes: byte j holds element 2j in its low
 *                         nibble and element 2j+1 in its high nibble; for odd
 *                         n the last high nibble is 0.
 *   code8   [nb]          8-bit code of block b's absmax, an index into the
 *                         ascending 256-entry constant table.
 *   c2      [nb2]         fp32 scale of group g (max |absmax - mean|).
 *   mean    [1]           fp32 mean of all block absmax values.
 * with nb = ceil(n/64) and nb2 = ceil(nb/256).  The library reads and writes
 * through these pointers; it does not own them. */
typedef struct {
  uint8_t *packed;
  uint8_t *code8;
  float *c2;
  float *mean;
  int64_t rows;
  int64_t cols;
  int32_t qtype;   /* qlora_q4_type; 0 (NF4) for a zero-initialised struct.
                      Set before qlora_quantize_nf4, which codes with this
                      type's table; every other call decodes with it.  A
                      value outside the enum is QLORA_ERR_INVALID_ARG. */
} qlora_nf4_weight;

/* Human-readable name of a status code (static string, never NULL). */
const char *qlora_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int qlora_version(void);

/* Largest M the forward sends to the decode-regime kernels (dequant-GEMV and
 * weight stream: the small-M case of the pages' dequantize-then-multiply,
 * automatone.win, "QLoRA paper explained", How it works); larger M take the
 * tiled MFMA matmuls.  64 by default; the environment variable
 * QLORA_SMALL_M_MAX (a decimal integer, clamped to [0, 64], read once per
 * process) lowers it for benchmarking the tiled kernels at small M, 0 sending
 * every M there.  Results stay within the matmul tolerance either way (the two
 * routes round differently).  Host-only; never touches the GPU. */
int qlora_small_m_max(void);

/* Storage sizes for n >= 1 elements: packed bytes, blocks (nb), groups (nb2).
 * Any output pointer may be NULL.  Host-only; never touches the GPU. */
int qlora_nf4_sizes(int64_t n, int64_t *packed_bytes, int64_t *nb, int64_t *nb2);

/* Workspace bytes needed by qlora_quantize_nf4 for n elements (0 if n < 1). */
size_t qlora_quantize_workspace_bytes(int64_t n);

/* Quantize fp32 W [out->rows, out->cols] into *out (storage as above).
 * Codes: x = fl32(w / absmax) (IEEE division), NF4 code = nearest of the 16
 * levels with ties to the lower index (absmax 0 -> code 7); the block
 * constants are centred on their mean (fp64 pairwise-tree sum in a fixed
 * order, divided by nb, rounded to fp32) and coded to the nearest entry of
 * the 8-bit table, ties low (group scale 0 -> code 127).  Bit-exact and
 * deterministic.  Pages: automatone.win, "QLoRA paper explained", How it
 * works / 4-bit NormalFloat and Double Quantization.
 * Requires rows, cols >= 1, rows * cols < 2^31 (UNSUPPORTED_SHAPE otherwise;
 * the largest LLaMA-65B weight has 1.8e8 elements) and ws_bytes >=
 * qlora_quantize_workspace_bytes. */
int qlora_quantize_nf4(const float *W, const qlora_nf4_weight *out, void *ws,
                       size_t ws_bytes, void *stream);

/* Element types of a 16-bit weight for qlora_quantize_nf4_16. */
typedef enum { QLORA_IN_BF16 = 1, QLORA_IN_FP16 = 2 } qlora_in_type;

/* Quantize a 16-bit W [out->rows, out->cols] (bf16 or fp16 bit patterns,
 * in_type) into *out.  Both types widen to fp32 exactly, so the result is
 * bit-identical to qlora_quantize_nf4 on the widened fp32 values, without an
 * fp32 copy of a 16-bit checkpoint.  (The pages load a pretrained model
 * straight into 4 bits with bf16 compute: creativeworksofknowledge.com,
 * "QLoRA: Fine-Tune 70B on One GPU", Code.)  Same rules and workspace as
 * qlora_quantize_nf4; an in_type outside the enum is QLORA_ERR_INVALID_ARG. */
int qlora_quantize_nf4_16(const uint16_t *W, int32_t in_type, const qlora_nf4_weight *out, void *ws,
                          size_t ws_bytes, void *stream);

/* Dequantize *w to bf16 out [rows, cols]:
 *   c_hat = fl32(fl32(T8[code8] * c2) + mean)      (no fused multiply-add)
 *   out   = bf16_rne(fl32(NF4[q] * c_hat))
 * Pages: automatone.win, "QLoRA paper explained", How it works (dequantize
 * to BFloat16 on the fly). */
int qlora_dequantize_nf4(const qlora_nf4_weight *w, uint16_t *out_bf16, void *stream);

/* Workspace bytes for qlora_quantize_nf4_group: the members'
 * qlora_quantize_workspace_bytes, each rounded up to 256 bytes, summed.  0 if
 * count < 1, count > 8, out is NULL or a member has rows or cols < 1 or
 * rows * cols >= 2^31.  Host-only; reads only rows and cols. */
size_t qlora_quantize_group_workspace_bytes(int count, const qlora_nf4_weight *out);

/* Quantize up to 8 weights in one call, for example the seven projections of
 * a layer as a checkpoint is loaded into 4 bits (creativeworksofknowledge.com,
 * "QLoRA: Fine-Tune 70B on One GPU", Code).  Member i codes W[i] (fp32 when
 * in_type = 0, else the 16-bit patterns of QLORA_IN_BF16 / QLORA_IN_FP16; one
 * in_type for the whole group) into out[i] with out[i].qtype's table, under
 * the rules of qlora_quantize_nf4.  Results are bit-identical to one
 * qlora_quantize_nf4 / qlora_quantize_nf4_16 call per member; the group takes
 * two launches in all (plus one per member above 2^27 elements) instead of two
 * per member.  ws: device memory of qlora_quantize_group_workspace_bytes
 * bytes, 16-byte aligned (each member's part starts on a 256-byte boundary).
 * W[i]: 16-byte aligned.  Every member is validated before any launch
 * (INVALID_ARG, UNSUPPORTED_SHAPE or WORKSPACE as for single calls; count
 * outside 1..8 or a NULL array is INVALID_ARG). */
int qlora_quantize_nf4_group(int count, const void *const *W, int32_t in_type, const qlora_nf4_weight *out,
                             void *ws, size_t ws_bytes, void *stream);

/* Dequantize up to 8 weights in one launch: w[i] -> out_bf16[i] (rows x cols,
 * 16-byte aligned), bit-identical to qlora_dequantize_nf4 per member.  Every
 * member is validated before the launch; count outside 1..8 or a NULL array
 * is INVALID_ARG.  Pages: automatone.win, "QLoRA paper explained", How it
 * works (dequantize to BFloat16 on the fly). */
int qlora_dequantize_nf4_group(int count, const qlora_nf4_weight *w, uint16_t *const *out_bf16, void *stream);

/* Workspace bytes for qlora_linear_fwd (is_bwd = 0) or qlora_linear_bwd
 * (is_bwd = 1) at these sizes.  0 if the shape is unsupported, and 0 for a
 * forward pass at M = 0.  A forward pass at 1 <= M <= 64 with r % 8 == 0
 * (the decode regime) always needs its workspace: it holds fp32 partial sums
 * of X A^T and, on the streaming route, the weight stream's tile sums and T. */
size_t qlora_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r, int is_bwd);

/* Forward: Y [M, N] = X [M, K] deq(W)^T + scale (X A^T) B^T.
 *   X [M, K], A [r, K], B [N, r], Y [M, N]: bf16.  W: N x K NF4 weight.
 *   T_out [M, r] (nullable): receives T = scale X A^T in bf16 (the LoRA
 *   intermediate with the scale applied once in fp32 before rounding, not
 *   the unscaled X A^T) for reuse in the backward pass; when NULL, T lives
 *   in the workspace.
 *   ws: device memory of qlora_linear_workspace_bytes(M, N, K, r, 0) bytes,
 *   16-byte aligned; it may be NULL only when that size is 0.
 *   At 1 <= M <= 64 with r % 8 == 0 the pass takes a decode-regime route that
 *   streams the packed weight once (bandwidth-bound): two launches at M <= 4
 *   (down-projection, dequant-GEMV) and for a single linear at M <= 16, four
 *   at 4 < M <= 64 when K % 256 == 0 and K <= 16384 (down-projection chunks,
 *   T, persistent weight stream, tile epilogue).  These routes apply each
 *   block constant to the bf16 level product in fp32 (bf16(NF4[q]) * c_hat)
 *   instead of rounding NF4[q] * c_hat to bf16 (within the same tolerance).
 *   Otherwise two MFMA tile kernels that dequantize exactly as
 *   qlora_dequantize_nf4 does.
 * Requires K % 64 == 0 (blocks never straddle rows), N % 8 == 0, 1 <= r <=
 * 128, M >= 0 (M = 0 launches nothing), M * max(N, K) < 2^31 (else
 * UNSUPPORTED_SHAPE).  Pages: automatone.win, "QLoRA paper
 * explained", How it works; creativeworksofknowledge.com, "QLoRA: Fine-Tune
 * 70B on One GPU", Code (r, lora_alpha, bias="none"). */
int qlora_linear_fwd(const uint16_t *X, int64_t M, const qlora_nf4_weight *W,
                     const uint16_t *A, const uint16_t *B, int32_t r, float scale,
                     uint16_t *Y, uint16_t *T_out, void *ws, size_t ws_bytes, void *stream);

/* qlora_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, rules and results as
 * qlora_linear_fwd (bit for bit: the same kernels); its scratch is a static
 * device array of QLORA_STATIC_SCRATCH_BYTES (16 MiB) per GPU, created when
 * the library is first used on that GPU and held until the process ends.
 * The call allocates nothing and calls no allocating routine.
 *   - Scratch needed: the decode-regime partials at 1 <= M <= 64 (r % 8 ==
 *     0; at most 13.4 MiB for the LLaMA-7B..65B shapes) or T [M, r] bf16
 *     when T_out is NULL.  A call that needs more returns
 *     QLORA_ERR_SCRATCH_LIMIT before launching anything.
 *   - The scratch of the current device is used: `stream` must belong to it.
 *   - Calls on one GPU share its scratch, which keeps the last call's
 *     contents (nothing in it needs clearing between calls).  Calls ordered
 *     on one stream are safe; calls that can overlap in time on the same GPU
 *     (different streams, several host threads) race on it and must be
 *     ordered by the caller. */
int qlora_linear_fwd_noalloc(const uint16_t *X, int64_t M, const qlora_nf4_weight *W,
                             const uint16_t *A, const uint16_t *B, int32_t r, float scale,
                             uint16_t *Y, uint16_t *T_out, void *stream);

/* One linear of a grouped forward call (all pointers device memory, same
 * layouts and rules as qlora_linear_fwd). */
typedef struct {
  const uint16_t *X;            /* [M, K] */
  const qlora_nf4_weight *W;    /* N x K (host pointer to the descriptor) */
  const uint16_t *A;            /* [r, K] */
  const uint16_t *B;            /* [N, r] */
  int32_t r;
  float scale;
  uint16_t *Y;                  /* [M, N] */
  uint16_t *T_out;              /* [M, r], nullable */
} qlora_linear_desc;

/* Shared-input LoRA products.  In a decoder layer q, k and v read the same
 * input X, and so do gate and up; the LoRA branch reads X once per linear for
 * T = s X A^T and once more for dA = G^T X.  These calls take up to 8 linears
 * ("members") that share X [M, K] and make one launch each, placed so that
 * every block of X is read from HBM once and served from L2 to the other
 * members.  Results are bit-identical to qlora_lora_down / the dA of
 * qlora_lora_grads per member.  Member arrays (A, G, r, scale, T, dA) are
 * host arrays of `count` entries; the tensors they point to are device
 * memory with the layouts of the single calls.  Rules: 1 <= count <= 8,
 * K % 8 == 0, 1 <= r[i] <= 128, finite scales (else INVALID_ARG /
 * UNSUPPORTED_SHAPE, nothing launched).  Page: automatone.win, "QLoRA paper
 * explained", How it works (adapters on every linear); creativeworksof
 * knowledge.com, "QLoRA: Fine-Tune 70B on One GPU", Code (all-linear targets).
 *   T[i] [M, r[i]] = bf16(scale[i] * X A[i]^T),  A[i] [r[i], K] */
int qlora_lora_down_shared(const uint16_t *X, int64_t M, int64_t K, int count, const uint16_t *const *A,
                           const int32_t *r, const float *scale, uint16_t *const *T, void *stream);
/* dA[i] [r[i], K] = bf16(G[i]^T X),  G[i] [M, r[i]] (already carries the scale);
 * ws of qlora_lora_dA_shared_workspace_bytes(M, K, count, r) bytes. */
size_t qlora_lora_dA_shared_workspace_bytes(int64_t M, int64_t K, int count, const int32_t *r);
int qlora_lora_dA_shared(const uint16_t *X, int64_t M, int64_t K, int count, const uint16_t *const *G,
                         const int32_t *r, uint16_t *const *dA, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for qlora_linear_fwd_group (0 if any shape is unsupported,
 * count < 1 or count > 8): the sum of the linears' forward workspaces. */
size_t qlora_linear_group_workspace_bytes(int count, const qlora_linear_desc *descs, int64_t M);

/* Forward of up to 8 linears that share the token count M, each as
 * qlora_linear_fwd computes it.  In the decode regime (1 <= M <= 64, every
 * r % 8 == 0, one 4-bit type) the whole group takes the launches of one
 * call, so that launch latency is paid once per group (for example the seven
 * projections of a layer); on the streaming route (4 < M <= 64) the fp32
 * summation order depends on the whole group, so results agree with single
 * calls within the tolerance, elsewhere bit for bit.  A decode-regime group
 * that mixes 4-bit types runs its linears one call at a time.  At larger M,
 * linears whose descriptors carry the same X pointer and K (q, k, v; gate,
 * up) get their T from one qlora_lora_down_shared launch, then every linear
 * runs its fused matmul (in launches of up to 4 that share one tile space);
 * results are bit-identical to single calls.  ws: device memory
 * of qlora_linear_group_workspace_bytes bytes, 16-byte aligned.  Validation of
 * every descriptor happens before any launch.  Pages: automatone.win,
 * "QLoRA paper explained", How it works; creativeworksofknowledge.com,
 * "QLoRA: Fine-Tune 70B on One GPU", Code (adapters on every linear). */
int qlora_linear_fwd_group(int count, const qlora_linear_desc *descs, int64_t M, void *ws, size_t ws_bytes,
                           void *stream);

/* Backward: given dY [M, N], X [M, K] and optionally T = scale X A^T [M, r]
 * as written by qlora_linear_fwd (NULL: recomputed), writes
 *   dX [M, K] = dY deq(W) + scale (dY B) A        (nullable: skipped)
 *   dA [r, K] = scale (dY B)^T X                  (nullable: skipped)
 *   dB [N, r] = scale dY^T T                      (nullable: skipped)
 * all bf16.  No gradient for W (frozen).  Same shape rules as the forward
 * (K % 64 == 0, N % 8 == 0, 1 <= r <= 128); M = 0 writes nothing.  T, when
 * given, must be the scaled T of the forward pass.  dA and dB are reduced
 * over M in a fixed order (deterministic).
 * Pages: automatone.win, "QLoRA paper explained", How it works (gradients
 * flow through the 4-bit base into the adapters only); gptget.net, "QLoRA:
 * Efficient Finetuning of Quantized LLMs", Deep Analysis / Methodology. */
int qlora_linear_bwd(const uint16_t *dY, const uint16_t *X, const uint16_t *T, int64_t M,
                     const qlora_nf4_weight *W, const uint16_t *A, const uint16_t *B,
                     int32_t r, float scale, uint16_t *dX, uint16_t *dA, uint16_t *dB,
                     void *ws, size_t ws_bytes, void *stream);

/* ---- The individual steps of the two passes (same conventions) ---------- */

/* T [M, r] = scale X [M, K] A^T, A [r, K]; bf16 in, fp32 accumulation, the
 * scale applied in fp32 before the single rounding to bf16.  K % 8 == 0. */
int qlora_lora_down(const uint16_t *X, int64_t M, int64_t K, const uint16_t *A, int32_t r,
                    float scale, uint16_t *T, void *stream);

/* Y [M, N] = X deq(W)^T + T B^T with T = scale X A^T [M, r] given: the fused
 * dequant-matmul with the LoRA up-projection folded in as one extra
 * contraction step.  No workspace. */
int qlora_nf4_matmul_fwd(const uint16_t *X, int64_t M, const qlora_nf4_weight *W,
                         const uint16_t *T, const uint16_t *B, int32_t r, uint16_t *Y,
                         void *stream);

/* Workspace bytes for qlora_lora_grad_in: at least 256 for a supported
 * shape, 0 if the shape is unsupported. */
size_t qlora_lora_grad_in_workspace_bytes(int64_t N, int32_t r);

/* G [M, r] = scale dY [M, N] B, B [N, r] (scale applied before rounding).
 * B is read transposed straight from its [N, r] layout; the workspace only
 * holds a zero-padded copy of B when r % 8 != 0.  ws: device memory of
 * qlora_lora_grad_in_workspace_bytes(N, r) bytes, 16-byte aligned.  Requires
 * N % 8 == 0, 1 <= r <= 128. */
int qlora_lora_grad_in(const uint16_t *dY, int64_t M, int64_t N, const uint16_t *B, int32_t r,
                       float scale, uint16_t *G, void *ws, size_t ws_bytes, void *stream);

/* One product of qlora_nf4_matmul_fwd_group: the arguments of
 * qlora_nf4_matmul_fwd. */
typedef struct {
  const uint16_t *X;
  int64_t M;
  const qlora_nf4_weight *W;
  const uint16_t *T;
  const uint16_t *B;
  int32_t r;
  uint16_t *Y;
} qlora_matmul_fwd_desc;

/* Up to 4 forward products that share M (for example q, k and v, or gate
 * and up) in one launch over their concatenated tile grids: the last partial
 * round of 256 x 256 tiles is shared instead of paid per product (gate and
 * up at M = 8192: 2 x 1376 tiles, 11 rounds of 256 CUs instead of 12).  Each
 * Y is bit-identical to qlora_nf4_matmul_fwd; decode-regime members
 * (M <= 64, r % 8 == 0) run one call each.  Every member is validated before
 * any launch; count outside 1..4, a NULL d or unequal M is INVALID_ARG.
 * Pages: automatone.win, "QLoRA paper explained", How it works. */
int qlora_nf4_matmul_fwd_group(int count, const qlora_matmul_fwd_desc *d, void *stream);

/* dX [M, K] = dY deq(W) + G A with G = scale dY B [M, r] given.  No workspace. */
int qlora_nf4_matmul_dx(const uint16_t *dY, int64_t M, const qlora_nf4_weight *W,
                        const uint16_t *G, const uint16_t *A, int32_t r, uint16_t *dX,
                        void *stream);

/* ---- The matmuls from a dequantized weight --------------------------------
 * The same products as qlora_nf4_matmul_fwd / _fwd_group / _dx, with the
 * weight given as its dequantized bf16 copy Wd [N, K] (row-major, 16-byte
 * aligned), i.e. what qlora_dequantize_nf4 (or _group) writes for it.  The
 * pages' recipe dequantizes the 4-bit weight to BFloat16 and then runs the
 * matmul (automatone.win, "QLoRA paper explained", How it works; gptget.net,
 * "QLoRA: Efficient Finetuning of Quantized LLMs", Deep Analysis /
 * Methodology: 16-bit matmuls in both passes).  With Wd from the dequantizer
 * the outputs are bit-identical to the fused entry points': the weight
 * values and the contraction order are the same.  A training step can
 * dequantize a layer's weights once (one grouped call) and use the copies
 * for both the forward and the dX products; on gfx950 that is faster than
 * expanding the codes inside every matmul tile (the caller holds N K 2 bytes
 * per weight meanwhile).  No workspace; no decode-regime route (any M >= 0
 * runs the 256 x 256 tiles).  Shape rules: K % 64 == 0, 1 <= r <= 128,
 * N % 8 == 0 for the forward and N % 64 == 0 for dX.  M = 0 launches
 * nothing. */
int qlora_deq_matmul_fwd(const uint16_t *X, int64_t M, const uint16_t *Wd, int64_t N, int64_t K,
                         const uint16_t *T, const uint16_t *B, int32_t r, uint16_t *Y, void *stream);

/* One product of qlora_deq_matmul_fwd_group: the arguments of
 * qlora_deq_matmul_fwd. */
typedef struct {
  const uint16_t *X;
  int64_t M;
  const uint16_t *Wd;
  int64_t N;
  int64_t K;
  const uint16_t *T;
  const uint16_t *B;
  int32_t r;
  uint16_t *Y;
} qlora_deq_matmul_fwd_desc;

/* Up to 4 such forward products sharing M in one launch over their
 * concatenated tile grids (as qlora_nf4_matmul_fwd_group); each Y equals
 * qlora_deq_matmul_fwd's.  Every member is validated before any launch;
 * count outside 1..4, a NULL d or unequal M is INVALID_ARG. */
int qlora_deq_matmul_fwd_group(int count, const qlora_deq_matmul_fwd_desc *d, void *stream);

int qlora_deq_matmul_dx(const uint16_t *dY, int64_t M, const uint16_t *Wd, int64_t N, int64_t K,
                        const uint16_t *G, const uint16_t *A, int32_t r, uint16_t *dX, void *stream);

/* Workspace bytes for qlora_lora_grads (at least 256; 0 if unsupported). */
size_t qlora_lora_grads_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r);

/* dA [r, K] = G^T X and/or dB [N, r] = dY^T T, with G = scale dY B and
 * T = scale X A^T as produced above (either output may be NULL).  The
 * contraction runs over M.  dA and dB share one contraction launch; when
 * their tiles do not fill the GPU, M is split and the fp32 split partials (in
 * the workspace) are summed in split order by one more launch
 * (deterministic).  The split count comes from the shape: one count for both
 * when both are computed (their tiles together fill the GPU in whole
 * rounds), else the single product's own, the one qlora_lora_dA_shared uses;
 * so dA's rounding can differ by whether dB is computed in the same call.  G and X are needed for dA (K % 8
 * == 0), dY and T for dB (N % 8 == 0).  M = 0 launches nothing and leaves dA
 * and dB as they were. */
int qlora_lora_grads(const uint16_t *X, const uint16_t *dY, const uint16_t *G,
                     const uint16_t *T, int64_t M, int64_t N, int64_t K, int32_t r,
                     uint16_t *dA, uint16_t *dB, void *ws, size_t ws_bytes, void *stream);

/* One linear's operands for qlora_lora_grads_group: the arguments of
 * qlora_lora_grads, same meanings and rules (dA or dB may be NULL). */
typedef struct {
  const uint16_t *X;
  const uint16_t *dY;
  const uint16_t *G;
  const uint16_t *T;
  int64_t M;
  int64_t N;
  int64_t K;
  int32_t r;
  uint16_t *dA;
  uint16_t *dB;
} qlora_lora_grads_desc;

/* Workspace bytes for qlora_lora_grads_group: the members'
 * qlora_lora_grads_workspace_bytes summed (0 if count < 1, count > 8, d is
 * NULL or a member's shape is unsupported). */
size_t qlora_lora_grads_group_workspace_bytes(int count, const qlora_lora_grads_desc *d);

/* dA and dB of up to 8 linears in one contraction launch plus at most one
 * partial-sum launch, for example at the end of a layer's backward pass when
 * every linear's G is known (adapters on every linear: creativeworksof
 * knowledge.com, "QLoRA: Fine-Tune 70B on One GPU", Code).  Every member is
 * computed exactly as by qlora_lora_grads (same tiles, splits and summation
 * order): results are bit-identical.  ws: device memory of
 * qlora_lora_grads_group_workspace_bytes bytes, 16-byte aligned; member i's
 * part starts after the parts of members 0 .. i-1.  Every member is validated
 * before any launch. */
int qlora_lora_grads_group(int count, const qlora_lora_grads_desc *d, void *ws, size_t ws_bytes, void *stream);

/* ---- LoRA dropout on the adapter input -----------------------------------
 * The pages' adapters drop their input with probability p (creativeworksof
 * knowledge.com, "QLoRA: Fine-Tune 70B on One GPU", Code: lora_dropout=0.05).
 * Keep mask: element e = m*K + k of X [M, K] is kept iff word e % 4 of
 * Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy as 1, 2,
 * 3", SC 2011) at counter (e / 4 as a 64-bit value in words 0 and 1, words 2
 * and 3 zero) under key (seed low 32 bits, seed high 32 bits) is >=
 * floor(p * 2^32).  The mask is stored as uint32 keep[M][K / 32], bit k % 32
 * of word k / 32 (16-byte aligned).  Inverted dropout: the LoRA scale
 * becomes s_eff = fl32(s / (1 - p)) (quotient in fp64); the dropped input
 * X_d = X where kept, +0 elsewhere.  The layer with dropout:
 *   T  = s_eff X_d A^T           Y  = X deq(W)^T + T B^T
 *   G  = s_eff dY B              dX = dY deq(W) + (G A) * keep
 *   dA = G^T X_d                 dB = dY^T T
 * Rules: 0 <= p < 1 finite (else INVALID_ARG), K % 32 == 0 for the mask
 * calls (the layer calls need K % 64 == 0 as usual). */

/* X_d [M, K] and keep from X [M, K], p and seed. */
int qlora_dropout_mask(const uint16_t *X, int64_t M, int64_t K, float p, uint64_t seed, uint16_t *X_drop,
                       uint32_t *keep, void *stream);
/* X_d from X and an existing keep mask (the backward pass). */
int qlora_dropout_apply(const uint16_t *X, int64_t M, int64_t K, const uint32_t *keep, uint16_t *X_drop,
                        void *stream);
/* dX [M, K] = dY deq(W) + (G A) * keep  (G = s_eff dY B, given). */
int qlora_nf4_matmul_dx_dropout(const uint16_t *dY, int64_t M, const qlora_nf4_weight *W, const uint16_t *G,
                                const uint16_t *A, int32_t r, const uint32_t *keep, uint16_t *dX, void *stream);
/* Workspace of the dropout layer calls: X_d plus the forward's T or the
 * backward's workspace (is_bwd). */
size_t qlora_linear_dropout_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r, int is_bwd);
/* Forward with dropout; writes keep_out [M][K / 32] for the backward pass and
 * T to T_out (nullable: workspace). */
int qlora_linear_fwd_dropout(const uint16_t *X, int64_t M, const qlora_nf4_weight *W, const uint16_t *A,
                             const uint16_t *B, int32_t r, float scale, float p, uint64_t seed, uint16_t *Y,
                             uint16_t *T_out, uint32_t *keep_out, void *ws, size_t ws_bytes, void *stream);
/* Backward with dropout, given the forward's keep mask; T as written by the
 * forward (NULL: recomputed from X_d); dX, dA, dB nullable as in
 * qlora_linear_bwd. */
int qlora_linear_bwd_dropout(const uint16_t *dY, const uint16_t *X, const uint16_t *T, int64_t M,
                             const qlora_nf4_weight *W, const uint16_t *A, const uint16_t *B, int32_t r, float scale,
                             float p, const uint32_t *keep, uint16_t *dX, uint16_t *dA, uint16_t *dB, void *ws,
                             size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_MI355X_H */
