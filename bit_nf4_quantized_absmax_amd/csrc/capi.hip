// C ABI of libqlora_mi355x: argument validation, workspace carving and the
// composite forward / backward passes.  Every check runs before anything is
// launched, so an error leaves all outputs untouched.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/qlora.h"
#include "launch.h"

using namespace qlora;

namespace {

constexpr int64_t kMaxElems = (int64_t{1} << 31) - 1;  // kernels index rows * cols in int32 where safe

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_weight(const qlora_nf4_weight *w) {
  if (!w) return QLORA_ERR_INVALID_ARG;
  if (w->rows < 1 || w->cols < 1) return QLORA_ERR_INVALID_ARG;
  if (w->rows > kMaxElems / w->cols) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (!w->packed || !w->code8 || !w->c2 || !w->mean) return QLORA_ERR_INVALID_ARG;
  if (!aligned(w->packed, 16) || !aligned(w->code8, 4) || !aligned(w->c2, 4) || !aligned(w->mean, 4))
    return QLORA_ERR_INVALID_ARG;
  if (w->qtype < QLORA_Q4_NF4 || w->qtype > QLORA_Q4_INT4) return QLORA_ERR_INVALID_ARG;
  return QLORA_OK;
}

// Shape rules of the matmul entry points.
int check_linear_shape(int64_t M, const qlora_nf4_weight *w, int32_t r, float scale) {
  int st = check_weight(w);
  if (st) return st;
  if (M < 0 || !isfinite(scale)) return QLORA_ERR_INVALID_ARG;
  const int64_t N = w->rows, K = w->cols;
  if (K % 64 != 0 || N % 8 != 0) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (r < 1 || r > 128) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (M > 0 && (M > kMaxElems / std::max(N, K))) return QLORA_ERR_UNSUPPORTED_SHAPE;
  return QLORA_OK;
}

bool bf16_ok(const void *p) { return p && aligned(p, 16); }
bool bf16_opt(const void *p) { return !p || aligned(p, 16); }

// Shape rules of the products from a dequantized weight Wd [N, K]: those of
// the fused kernels, and N % 64 == 0 for dX (its contraction over N has no
// zero-padded tail on this route).
int check_deq_shape(int64_t M, const uint16_t *Wd, int64_t N, int64_t K, int32_t r, bool dx) {
  if (M < 0 || N < 1 || K < 1 || !bf16_ok(Wd)) return QLORA_ERR_INVALID_ARG;
  if (K % 64 != 0 || N % (dx ? 64 : 8) != 0) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (N > kMaxElems / K) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (r < 1 || r > 128) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (M > 0 && (M > kMaxElems / std::max(N, K))) return QLORA_ERR_UNSUPPORTED_SHAPE;
  return QLORA_OK;
}
// A tensor with M rows: at M = 0 it has no storage and its pointer may be NULL.
bool rows_ok(const void *p, int64_t M) { return M == 0 ? bf16_opt(p) : bf16_ok(p); }

NF4View view_of(const qlora_nf4_weight *w) {
  return NF4View{w->packed, w->code8, w->c2, w->mean, static_cast<int>(w->rows), static_cast<int>(w->cols),
                 static_cast<int>(w->qtype)};
}

int from_hip(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP; }

size_t bf16_bytes(int64_t n) { return round_up(static_cast<size_t>(n) * 2, 256); }

// Workspace of the forward pass.  M <= small_m_max(): the fp32 partials of
// the down-projection (always needed), and where the streaming path applies
// its T copy, split-tile counters and pieces.  Larger M: T [M, r] when the
// caller passes no T_out.
size_t fwd_ws(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (small_m_ok(M, r)) {
    size_t b = small_m_ws_bytes(static_cast<int>(M), static_cast<int>(K), r);
    if (small_m_stream_ok(M, static_cast<int>(K), r))
      b = std::max(b, small_m_stream_ws_bytes(static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), r));
    return b;
  }
  return bf16_bytes(M * r);
}

// Workspace of the backward pass: T (recompute) | G | dA partials | dB partials.
struct BwdWs {
  size_t t, g, bt, pa, pb, total;
};
// Workspace of the backward pass: T (recompute) | G | B^T | dA partials | dB partials.
BwdWs bwd_ws(int64_t M, int64_t N, int64_t K, int32_t r) {
  BwdWs w;
  w.t = bf16_bytes(M * r);
  w.g = bf16_bytes(M * r);
  w.bt = lora_grad_in_ws_bytes(static_cast<int>(N), r);
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  w.pa = round_up(lora_grad_pair_ws_bytes(m, k, k, n, r), 256);
  w.pb = round_up(lora_grad_pair_ws_bytes(m, n, k, n, r), 256);
  w.total = w.t + w.g + w.bt + w.pa + w.pb;
  return w;
}

}  // namespace

// ---- static device scratch (qlora_linear_fwd_noalloc) -------------------------
// One file-scope device array per GPU, allocated when the library's code object
// is loaded on that GPU and held until the process ends.  Its host-side name
// is only a handle: the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is ever
// passed to kernels.
static __device__ __align__(256) uint8_t scratch[QLORA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array.
int current_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLORA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return QLORA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

}  // namespace

extern "C" {

const char *qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "QLORA_OK";
    case QLORA_ERR_INVALID_ARG: return "QLORA_ERR_INVALID_ARG: null, misaligned or out-of-range argument";
    case QLORA_ERR_UNSUPPORTED_SHAPE:
      return "QLORA_ERR_UNSUPPORTED_SHAPE: need K % 64 == 0, N % 8 == 0, 1 <= r <= 128, sizes < 2^31";
    case QLORA_ERR_WORKSPACE: return "QLORA_ERR_WORKSPACE: workspace missing or too small";
    case QLORA_ERR_HIP: return "QLORA_ERR_HIP: HIP runtime or launch failure";
    case QLORA_ERR_SCRATCH_LIMIT:
      return "QLORA_ERR_SCRATCH_LIMIT: the call needs more than the library's static scratch "
             "(QLORA_STATIC_SCRATCH_BYTES); pass T_out or use the workspace entry point";
    default: return "QLORA: unknown status";
  }
}

int qlora_version(void) { return 10000; }

int qlora_small_m_max(void) { return small_m_max(); }

int qlora_nf4_sizes(int64_t n, int64_t *packed_bytes, int64_t *nb, int64_t *nb2) {
  if (n < 1) return QLORA_ERR_INVALID_ARG;
  const int64_t b = (n + 63) / 64;
  if (packed_bytes) *packed_bytes = (n + 1) / 2;
  if (nb) *nb = b;
  if (nb2) *nb2 = (b + 255) / 256;
  return QLORA_OK;
}

size_t qlora_quantize_workspace_bytes(int64_t n) { return n < 1 ? 0 : quantize_ws_bytes(n); }

int qlora_quantize_nf4(const float *W, const qlora_nf4_weight *out, void *ws, size_t ws_bytes, void *stream) {
  int st = check_weight(out);
  if (st) return st;
  if (!W || !aligned(W, 16)) return QLORA_ERR_INVALID_ARG;
  const int64_t n = out->rows * out->cols;
  if (!ws || !aligned(ws, 16) || ws_bytes < quantize_ws_bytes(n)) return QLORA_ERR_WORKSPACE;
  return from_hip(launch_quantize(W, 0, n, out->qtype, out->packed, out->code8, out->c2, out->mean, ws,
                                  static_cast<hipStream_t>(stream)));
}

int qlora_quantize_nf4_16(const uint16_t *W, int32_t in_type, const qlora_nf4_weight *out, void *ws,
                          size_t ws_bytes, void *stream) {
  int st = check_weight(out);
  if (st) return st;
  if (in_type != QLORA_IN_BF16 && in_type != QLORA_IN_FP16) return QLORA_ERR_INVALID_ARG;
  if (!W || !aligned(W, 16)) return QLORA_ERR_INVALID_ARG;
  const int64_t n = out->rows * out->cols;
  if (!ws || !aligned(ws, 16) || ws_bytes < quantize_ws_bytes(n)) return QLORA_ERR_WORKSPACE;
  return from_hip(launch_quantize(W, in_type, n, out->qtype, out->packed, out->code8, out->c2, out->mean, ws,
                                  static_cast<hipStream_t>(stream)));
}

int qlora_dequantize_nf4(const qlora_nf4_weight *w, uint16_t *out_bf16, void *stream) {
  int st = check_weight(w);
  if (st) return st;
  if (!bf16_ok(out_bf16)) return QLORA_ERR_INVALID_ARG;
  return from_hip(launch_dequantize(w->packed, w->code8, w->c2, w->mean, w->rows * w->cols, w->qtype, out_bf16,
                                    static_cast<hipStream_t>(stream)));
}

constexpr int kCodecGroupMax = 8;

size_t qlora_quantize_group_workspace_bytes(int count, const qlora_nf4_weight *out) {
  if (count < 1 || count > kCodecGroupMax || !out) return 0;
  size_t total = 0;
  for (int i = 0; i < count; ++i) {
    if (out[i].rows < 1 || out[i].cols < 1 || out[i].rows > kMaxElems / out[i].cols) return 0;
    total += round_up(quantize_ws_bytes(out[i].rows * out[i].cols), 256);
  }
  return total;
}

int qlora_quantize_nf4_group(int count, const void *const *W, int32_t in_type, const qlora_nf4_weight *out,
                             void *ws, size_t ws_bytes, void *stream) {
  if (count < 1 || count > kCodecGroupMax || !W || !out) return QLORA_ERR_INVALID_ARG;
  if (in_type != 0 && in_type != QLORA_IN_BF16 && in_type != QLORA_IN_FP16) return QLORA_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    int st = check_weight(&out[i]);
    if (st) return st;
    if (!W[i] || !aligned(W[i], 16)) return QLORA_ERR_INVALID_ARG;
  }
  const size_t need = qlora_quantize_group_workspace_bytes(count, out);
  if (!ws || !aligned(ws, 16) || ws_bytes < need) return QLORA_ERR_WORKSPACE;
  QuantJob jobs[kCodecGroupMax];
  char *p = static_cast<char *>(ws);
  for (int i = 0; i < count; ++i) {
    const int64_t n = out[i].rows * out[i].cols;
    jobs[i] = QuantJob{W[i], n, out[i].qtype, out[i].packed, out[i].code8, out[i].c2, out[i].mean, p};
    p += round_up(quantize_ws_bytes(n), 256);
  }
  return from_hip(launch_quantize_group(count, jobs, in_type, static_cast<hipStream_t>(stream)));
}

int qlora_dequantize_nf4_group(int count, const qlora_nf4_weight *w, uint16_t *const *out_bf16, void *stream) {
  if (count < 1 || count > kCodecGroupMax || !w || !out_bf16) return QLORA_ERR_INVALID_ARG;
  DequantJob jobs[kCodecGroupMax];
  for (int i = 0; i < count; ++i) {
    int st = check_weight(&w[i]);
    if (st) return st;
    if (!bf16_ok(out_bf16[i])) return QLORA_ERR_INVALID_ARG;
    jobs[i] = DequantJob{w[i].packed, w[i].code8, w[i].c2, w[i].mean, w[i].rows * w[i].cols, w[i].qtype, out_bf16[i]};
  }
  return from_hip(launch_dequantize_group(count, jobs, static_cast<hipStream_t>(stream)));
}

size_t qlora_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r, int is_bwd) {
  if (M < 0 || N < 1 || K < 64 || K % 64 || N % 8 || r < 1 || r > 128) return 0;
  if (M > 0 && M > kMaxElems / std::max(N, K)) return 0;
  return is_bwd ? bwd_ws(M, N, K, r).total : fwd_ws(M, N, K, r);
}

int qlora_lora_down(const uint16_t *X, int64_t M, int64_t K, const uint16_t *A, int32_t r, float scale,
                    uint16_t *T, void *stream) {
  if (M < 0 || !isfinite(scale)) return QLORA_ERR_INVALID_ARG;
  if (K < 8 || K % 8 || r < 1 || r > 128) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (M > kMaxElems / K) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (!rows_ok(X, M) || !bf16_ok(A) || !rows_ok(T, M)) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  return from_hip(launch_lora_down(X, static_cast<int>(M), static_cast<int>(K), A, r, scale, T,
                                   static_cast<hipStream_t>(stream)));
}

// Shared-input members: 1..8, r in [1, 128] each, pointer arrays present.
static int check_shared(int64_t M, int64_t K, int count, const int32_t *r) {
  if (M < 0 || count < 1 || count > kLoraMaxShared || !r) return QLORA_ERR_INVALID_ARG;
  if (K < 8 || K % 8 || (M > 0 && M > kMaxElems / K)) return QLORA_ERR_UNSUPPORTED_SHAPE;
  for (int i = 0; i < count; ++i)
    if (r[i] < 1 || r[i] > 128) return QLORA_ERR_UNSUPPORTED_SHAPE;
  return QLORA_OK;
}

int qlora_lora_down_shared(const uint16_t *X, int64_t M, int64_t K, int count, const uint16_t *const *A,
                           const int32_t *r, const float *scale, uint16_t *const *T, void *stream) {
  int st = check_shared(M, K, count, r);
  if (st) return st;
  if (!A || !scale || !T || !rows_ok(X, M)) return QLORA_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i)
    if (!bf16_ok(A[i]) || !rows_ok(T[i], M) || !isfinite(scale[i])) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  return from_hip(launch_lora_down_shared(X, static_cast<int>(M), static_cast<int>(K), count, A, r, scale, T,
                                          static_cast<hipStream_t>(stream)));
}

size_t qlora_lora_dA_shared_workspace_bytes(int64_t M, int64_t K, int count, const int32_t *r) {
  if (check_shared(M, K, count, r)) return 0;
  return lora_dA_shared_ws_bytes(static_cast<int>(M), static_cast<int>(K), count, r);
}

int qlora_lora_dA_shared(const uint16_t *X, int64_t M, int64_t K, int count, const uint16_t *const *G,
                         const int32_t *r, uint16_t *const *dA, void *ws, size_t ws_bytes, void *stream) {
  int st = check_shared(M, K, count, r);
  if (st) return st;
  if (!G || !dA || !rows_ok(X, M)) return QLORA_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i)
    if (!rows_ok(G[i], M) || !bf16_ok(dA[i])) return QLORA_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 16) || ws_bytes < qlora_lora_dA_shared_workspace_bytes(M, K, count, r))
    return QLORA_ERR_WORKSPACE;
  if (M == 0) return QLORA_OK;
  return from_hip(launch_lora_dA_shared(X, static_cast<int>(M), static_cast<int>(K), count, G, r, dA, ws,
                                        static_cast<hipStream_t>(stream)));
}

size_t qlora_lora_grad_in_workspace_bytes(int64_t N, int32_t r) {
  if (N < 8 || N % 8 || N > kMaxElems / 128 || r < 1 || r > 128) return 0;
  return lora_grad_in_ws_bytes(static_cast<int>(N), r);
}

int qlora_lora_grad_in(const uint16_t *dY, int64_t M, int64_t N, const uint16_t *B, int32_t r, float scale,
                       uint16_t *G, void *ws, size_t ws_bytes, void *stream) {
  if (M < 0 || !isfinite(scale)) return QLORA_ERR_INVALID_ARG;
  if (N < 8 || N % 8 || r < 1 || r > 128) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (M > kMaxElems / N || N > kMaxElems / 128) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (!rows_ok(dY, M) || !bf16_ok(B) || !rows_ok(G, M)) return QLORA_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 16) || ws_bytes < qlora_lora_grad_in_workspace_bytes(N, r)) return QLORA_ERR_WORKSPACE;
  if (M == 0) return QLORA_OK;
  return from_hip(launch_lora_grad_in(dY, static_cast<int>(M), static_cast<int>(N), B, r, scale, G, ws,
                                      static_cast<hipStream_t>(stream)));
}

int qlora_nf4_matmul_fwd(const uint16_t *X, int64_t M, const qlora_nf4_weight *W, const uint16_t *T,
                         const uint16_t *B, int32_t r, uint16_t *Y, void *stream) {
  int st = check_linear_shape(M, W, r, 1.0f);
  if (st) return st;
  if (!rows_ok(X, M) || !rows_ok(T, M) || !bf16_ok(B) || !rows_ok(Y, M)) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  return from_hip(launch_matmul_fwd(X, static_cast<int>(M), view_of(W), T, B, r, Y,
                                    static_cast<hipStream_t>(stream)));
}

int qlora_nf4_matmul_dx(const uint16_t *dY, int64_t M, const qlora_nf4_weight *W, const uint16_t *G,
                        const uint16_t *A, int32_t r, uint16_t *dX, void *stream) {
  int st = check_linear_shape(M, W, r, 1.0f);
  if (st) return st;
  if (!rows_ok(dY, M) || !rows_ok(G, M) || !bf16_ok(A) || !rows_ok(dX, M)) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  return from_hip(launch_matmul_dx(dY, static_cast<int>(M), view_of(W), G, A, r, dX,
                                   static_cast<hipStream_t>(stream)));
}

int qlora_deq_matmul_fwd(const uint16_t *X, int64_t M, const uint16_t *Wd, int64_t N, int64_t K, const uint16_t *T,
                         const uint16_t *B, int32_t r, uint16_t *Y, void *stream) {
  const qlora_deq_matmul_fwd_desc d{X, M, Wd, N, K, T, B, r, Y};
  return qlora_deq_matmul_fwd_group(1, &d, stream);
}

int qlora_deq_matmul_fwd_group(int count, const qlora_deq_matmul_fwd_desc *d, void *stream) {
  if (count < 1 || count > 4 || !d) return QLORA_ERR_INVALID_ARG;
  const int64_t M = d[0].M;
  for (int i = 0; i < count; ++i) {
    if (d[i].M != M) return QLORA_ERR_INVALID_ARG;
    int st = check_deq_shape(M, d[i].Wd, d[i].N, d[i].K, d[i].r, false);
    if (st) return st;
    if (!rows_ok(d[i].X, M) || !rows_ok(d[i].T, M) || !bf16_ok(d[i].B) || !rows_ok(d[i].Y, M))
      return QLORA_ERR_INVALID_ARG;
  }
  if (M == 0) return QLORA_OK;
  MatmulJob jobs[4];
  for (int i = 0; i < count; ++i) {
    const NF4View shape{nullptr, nullptr, nullptr, nullptr, static_cast<int>(d[i].N), static_cast<int>(d[i].K), 0};
    jobs[i] = MatmulJob{d[i].X, d[i].T, d[i].B, nullptr, d[i].Y, shape, static_cast<int>(M), d[i].r, d[i].Wd};
  }
  return from_hip(launch_pre_matmul_fwd_group(count, jobs, static_cast<hipStream_t>(stream)));
}

int qlora_deq_matmul_dx(const uint16_t *dY, int64_t M, const uint16_t *Wd, int64_t N, int64_t K, const uint16_t *G,
                        const uint16_t *A, int32_t r, uint16_t *dX, void *stream) {
  int st = check_deq_shape(M, Wd, N, K, r, true);
  if (st) return st;
  if (!rows_ok(dY, M) || !rows_ok(G, M) || !bf16_ok(A) || !rows_ok(dX, M)) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  const NF4View shape{nullptr, nullptr, nullptr, nullptr, static_cast<int>(N), static_cast<int>(K), 0};
  const MatmulJob job{dY, G, A, nullptr, dX, shape, static_cast<int>(M), r, Wd};
  return from_hip(launch_pre_matmul_dx(job, static_cast<hipStream_t>(stream)));
}

size_t qlora_lora_grads_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (M < 0 || N < 1 || K < 1 || r < 1 || r > 128) return 0;
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  return round_up(lora_grad_pair_ws_bytes(m, k, k, n, r), 256) + round_up(lora_grad_pair_ws_bytes(m, n, k, n, r), 256);
}

int qlora_lora_grads(const uint16_t *X, const uint16_t *dY, const uint16_t *G, const uint16_t *T, int64_t M,
                     int64_t N, int64_t K, int32_t r, uint16_t *dA, uint16_t *dB, void *ws, size_t ws_bytes,
                     void *stream) {
  if (M < 0 || N < 1 || K < 1) return QLORA_ERR_INVALID_ARG;
  if (r < 1 || r > 128) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if ((dA && (K < 8 || K % 8)) || (dB && (N < 8 || N % 8))) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (M > 0 && M > kMaxElems / std::max(N, K)) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (!bf16_opt(dA) || !bf16_opt(dB)) return QLORA_ERR_INVALID_ARG;
  if (dA && (!rows_ok(X, M) || !rows_ok(G, M))) return QLORA_ERR_INVALID_ARG;
  if (dB && (!rows_ok(dY, M) || !rows_ok(T, M))) return QLORA_ERR_INVALID_ARG;
  const size_t pa = round_up(
      lora_grad_pair_ws_bytes(static_cast<int>(M), static_cast<int>(K), static_cast<int>(K), static_cast<int>(N), r), 256);
  if (!ws || !aligned(ws, 16) || ws_bytes < qlora_lora_grads_workspace_bytes(M, N, K, r))
    return QLORA_ERR_WORKSPACE;
  if (M == 0) return QLORA_OK;   // nothing to reduce: dA and dB are left as they were
  const int m = static_cast<int>(M);
  const int sp = lora_grad_splits(m, static_cast<int>(K), static_cast<int>(N), r, dA != nullptr, dB != nullptr);
  GradWJob jobs[2];
  int nj = 0;
  if (dA) jobs[nj++] = GradWJob{X, G, m, static_cast<int>(K), r, true, dA, ws, sp};
  if (dB) jobs[nj++] = GradWJob{dY, T, m, static_cast<int>(N), r, false, dB, static_cast<char *>(ws) + pa, sp};
  if (nj == 0) return QLORA_OK;
  return from_hip(launch_lora_grad_w_group(nj, jobs, static_cast<hipStream_t>(stream)));
}

size_t qlora_lora_grads_group_workspace_bytes(int count, const qlora_lora_grads_desc *d) {
  if (count < 1 || count > 8 || !d) return 0;
  size_t total = 0;
  for (int i = 0; i < count; ++i) {
    const size_t b = qlora_lora_grads_workspace_bytes(d[i].M, d[i].N, d[i].K, d[i].r);
    if (b == 0) return 0;
    total += b;
  }
  return total;
}

int qlora_lora_grads_group(int count, const qlora_lora_grads_desc *d, void *ws, size_t ws_bytes, void *stream) {
  if (count < 1 || count > 8 || !d) return QLORA_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    const qlora_lora_grads_desc &x = d[i];
    if (x.M < 0 || x.N < 1 || x.K < 1) return QLORA_ERR_INVALID_ARG;
    if (x.r < 1 || x.r > 128) return QLORA_ERR_UNSUPPORTED_SHAPE;
    if ((x.dA && (x.K < 8 || x.K % 8)) || (x.dB && (x.N < 8 || x.N % 8))) return QLORA_ERR_UNSUPPORTED_SHAPE;
    if (x.M > 0 && x.M > kMaxElems / std::max(x.N, x.K)) return QLORA_ERR_UNSUPPORTED_SHAPE;
    if (!bf16_opt(x.dA) || !bf16_opt(x.dB)) return QLORA_ERR_INVALID_ARG;
    if (x.dA && (!rows_ok(x.X, x.M) || !rows_ok(x.G, x.M))) return QLORA_ERR_INVALID_ARG;
    if (x.dB && (!rows_ok(x.dY, x.M) || !rows_ok(x.T, x.M))) return QLORA_ERR_INVALID_ARG;
  }
  const size_t need = qlora_lora_grads_group_workspace_bytes(count, d);
  if (!ws || !aligned(ws, 16) || ws_bytes < need) return QLORA_ERR_WORKSPACE;
  GradWJob jobs[16];
  int nj = 0;
  char *p = static_cast<char *>(ws);
  for (int i = 0; i < count; ++i) {
    const qlora_lora_grads_desc &x = d[i];
    const int xm = static_cast<int>(x.M), xk = static_cast<int>(x.K), xn = static_cast<int>(x.N);
    const int sp = lora_grad_splits(xm, xk, xn, x.r, x.dA != nullptr, x.dB != nullptr);
    const size_t pa = round_up(lora_grad_pair_ws_bytes(xm, xk, xk, xn, x.r), 256);
    if (x.M > 0) {
      const int m = static_cast<int>(x.M);
      if (x.dA) jobs[nj++] = GradWJob{x.X, x.G, m, static_cast<int>(x.K), x.r, true, x.dA, p, sp};
      if (x.dB) jobs[nj++] = GradWJob{x.dY, x.T, m, static_cast<int>(x.N), x.r, false, x.dB, p + pa, sp};
    }
    p += qlora_lora_grads_workspace_bytes(x.M, x.N, x.K, x.r);
  }
  if (nj == 0) return QLORA_OK;
  return from_hip(launch_lora_grad_w_group(nj, jobs, static_cast<hipStream_t>(stream)));
}

int qlora_linear_fwd(const uint16_t *X, int64_t M, const qlora_nf4_weight *W, const uint16_t *A,
                     const uint16_t *B, int32_t r, float scale, uint16_t *Y, uint16_t *T_out, void *ws,
                     size_t ws_bytes, void *stream) {
  int st = check_linear_shape(M, W, r, scale);
  if (st) return st;
  if (!rows_ok(X, M) || !bf16_ok(A) || !bf16_ok(B) || !rows_ok(Y, M) || !bf16_opt(T_out)) return QLORA_ERR_INVALID_ARG;
  if (small_m_ok(M, r)) {
    if (!ws || !aligned(ws, 16) || ws_bytes < fwd_ws(M, W->rows, W->cols, r)) return QLORA_ERR_WORKSPACE;
    SmGroup grp{};
    grp.n = 1;
    grp.M = static_cast<int>(M);
    SmLinear &L = grp.lin[0];
    L.X = X;
    L.w = view_of(W);
    L.A = A;
    L.B = B;
    L.P = static_cast<float *>(ws);
    L.Y = Y;
    L.Tout = T_out;
    L.r = r;
    L.scale = scale;
    return from_hip(launch_small_m(grp, static_cast<hipStream_t>(stream)));
  }
  uint16_t *T = T_out;
  if (!T && M > 0) {
    if (!ws || !aligned(ws, 16) || ws_bytes < fwd_ws(M, W->rows, W->cols, r)) return QLORA_ERR_WORKSPACE;
    T = static_cast<uint16_t *>(ws);
  }
  if (M == 0) return QLORA_OK;   // no workspace is needed (its size query gives 0)
  hipStream_t s = static_cast<hipStream_t>(stream);
  const NF4View v = view_of(W);
  const int m = static_cast<int>(M);
  hipError_t e = launch_lora_down(X, m, v.K, A, r, scale, T, s);
  if (e != hipSuccess) return QLORA_ERR_HIP;
  return from_hip(launch_matmul_fwd(X, m, v, T, B, r, Y, s));
}

int qlora_linear_fwd_noalloc(const uint16_t *X, int64_t M, const qlora_nf4_weight *W, const uint16_t *A,
                             const uint16_t *B, int32_t r, float scale, uint16_t *Y, uint16_t *T_out,
                             void *stream) {
  int st = check_linear_shape(M, W, r, scale);
  if (st) return st;
  if (!rows_ok(X, M) || !bf16_ok(A) || !bf16_ok(B) || !rows_ok(Y, M) || !bf16_opt(T_out)) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  // The workspace qlora_linear_fwd would use: the decode-regime partials, or T
  // when the caller keeps no T_out.  Nothing in it has to start at zero: every
  // byte the kernels read was written earlier in the same call.
  const size_t need = (small_m_ok(M, r) || !T_out) ? fwd_ws(M, W->rows, W->cols, r) : 0;
  if (need > QLORA_STATIC_SCRATCH_BYTES) return QLORA_ERR_SCRATCH_LIMIT;
  void *ptr = nullptr;
  if (need) {
    st = current_scratch(&ptr);
    if (st) return st;
  }
  return qlora_linear_fwd(X, M, W, A, B, r, scale, Y, T_out, ptr, need ? QLORA_STATIC_SCRATCH_BYTES : 0, stream);
}

static bool group_small_m(int count, const qlora_linear_desc *d, int64_t M) {
  for (int i = 0; i < count; ++i)
    if (!small_m_ok(M, d[i].r)) return false;
  return true;
}

// The decode-regime kernels build one level table per launch: a group whose
// linears mix 4-bit types runs them one call at a time.
static bool group_one_type(int count, const qlora_linear_desc *d) {
  for (int i = 1; i < count; ++i)
    if (d[i].W->qtype != d[0].W->qtype) return false;
  return true;
}

size_t qlora_linear_group_workspace_bytes(int count, const qlora_linear_desc *d, int64_t M) {
  if (count < 1 || count > kSmMaxGroup || !d) return 0;
  size_t total = 0;
  for (int i = 0; i < count; ++i) {
    if (!d[i].W || check_linear_shape(M, d[i].W, d[i].r, d[i].scale)) return 0;
    total += fwd_ws(M, d[i].W->rows, d[i].W->cols, d[i].r);
  }
  return total;   // decode regime: every linear's partials; larger M: every T at once
}

int qlora_linear_fwd_group(int count, const qlora_linear_desc *d, int64_t M, void *ws, size_t ws_bytes,
                           void *stream) {
  if (count < 1 || count > kSmMaxGroup || !d) return QLORA_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    if (!d[i].W) return QLORA_ERR_INVALID_ARG;
    int st = check_linear_shape(M, d[i].W, d[i].r, d[i].scale);
    if (st) return st;
    if (!rows_ok(d[i].X, M) || !bf16_ok(d[i].A) || !bf16_ok(d[i].B) || !rows_ok(d[i].Y, M) || !bf16_opt(d[i].T_out))
      return QLORA_ERR_INVALID_ARG;
  }
  const size_t need = qlora_linear_group_workspace_bytes(count, d, M);
  if (need && (!ws || !aligned(ws, 16) || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (M == 0) return QLORA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (group_small_m(count, d, M) && !group_one_type(count, d)) {
    char *p = static_cast<char *>(ws);
    for (int i = 0; i < count; ++i) {
      const size_t b = fwd_ws(M, d[i].W->rows, d[i].W->cols, d[i].r);
      int st = qlora_linear_fwd(d[i].X, M, d[i].W, d[i].A, d[i].B, d[i].r, d[i].scale, d[i].Y, d[i].T_out, p, b,
                                stream);
      if (st) return st;
      p += b;
    }
    return QLORA_OK;
  }
  if (group_small_m(count, d, M)) {
    SmGroup grp{};
    grp.n = count;
    grp.M = static_cast<int>(M);
    char *p = static_cast<char *>(ws);
    for (int i = 0; i < count; ++i) {
      SmLinear &L = grp.lin[i];
      L.X = d[i].X;
      L.w = view_of(d[i].W);
      L.A = d[i].A;
      L.B = d[i].B;
      L.P = reinterpret_cast<float *>(p);
      L.Y = d[i].Y;
      L.Tout = d[i].T_out;
      L.r = d[i].r;
      L.scale = d[i].scale;
      p += fwd_ws(M, d[i].W->rows, d[i].W->cols, d[i].r);
    }
    return from_hip(launch_small_m(grp, s));
  }
  // Larger M: every T first (one launch for the linears that read the same
  // X), then the fused matmuls.  T lives in T_out or in the linear's slice of
  // the workspace.
  uint16_t *T[kSmMaxGroup];
  char *p = static_cast<char *>(ws);
  for (int i = 0; i < count; ++i) {
    T[i] = d[i].T_out ? d[i].T_out : reinterpret_cast<uint16_t *>(p);
    p += fwd_ws(M, d[i].W->rows, d[i].W->cols, d[i].r);
  }
  const int m = static_cast<int>(M);
  bool done[kSmMaxGroup] = {};
  for (int i = 0; i < count; ++i) {
    if (done[i]) continue;
    const uint16_t *A[kSmMaxGroup];
    int32_t r[kSmMaxGroup];
    float sc[kSmMaxGroup];
    uint16_t *Ts[kSmMaxGroup];
    int n = 0;
    for (int j = i; j < count; ++j) {
      if (done[j] || d[j].X != d[i].X || d[j].W->cols != d[i].W->cols) continue;
      done[j] = true;
      A[n] = d[j].A;
      r[n] = d[j].r;
      sc[n] = d[j].scale;
      Ts[n] = T[j];
      ++n;
    }
    const int K = static_cast<int>(d[i].W->cols);
    hipError_t e = n > 1 ? launch_lora_down_shared(d[i].X, m, K, n, A, r, sc, Ts, s)
                         : launch_lora_down(d[i].X, m, K, A[0], r[0], sc[0], Ts[0], s);
    if (e != hipSuccess) return QLORA_ERR_HIP;
  }
  // The fused matmuls: members in the decode regime one call each, the others
  // in launches of up to 4 (one tile space per launch, so a launch's last
  // partial round of tiles is shared by its members).
  MatmulJob jobs[4];
  int nj = 0;
  for (int i = 0; i < count; ++i) {
    const qlora_linear_desc &x = d[i];
    if (small_m_ok(M, x.r)) {
      if (launch_matmul_fwd(x.X, m, view_of(x.W), T[i], x.B, x.r, x.Y, s) != hipSuccess) return QLORA_ERR_HIP;
      continue;
    }
    jobs[nj++] = MatmulJob{x.X, T[i], x.B, nullptr, x.Y, view_of(x.W), m, x.r};
    if (nj == 4) {
      if (launch_matmul_fwd_group(nj, jobs, s) != hipSuccess) return QLORA_ERR_HIP;
      nj = 0;
    }
  }
  if (nj > 0 && launch_matmul_fwd_group(nj, jobs, s) != hipSuccess) return QLORA_ERR_HIP;
  return QLORA_OK;
}

int qlora_nf4_matmul_fwd_group(int count, const qlora_matmul_fwd_desc *d, void *stream) {
  if (count < 1 || count > 4 || !d) return QLORA_ERR_INVALID_ARG;
  const int64_t M = d[0].M;
  for (int i = 0; i < count; ++i) {
    if (d[i].M != M) return QLORA_ERR_INVALID_ARG;
    int st = check_linear_shape(M, d[i].W, d[i].r, 1.0f);
    if (st) return st;
    if (!rows_ok(d[i].X, M) || !rows_ok(d[i].T, M) || !bf16_ok(d[i].B) || !rows_ok(d[i].Y, M))
      return QLORA_ERR_INVALID_ARG;
  }
  if (M == 0) return QLORA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int m = static_cast<int>(M);
  MatmulJob jobs[4];
  int nj = 0;
  for (int i = 0; i < count; ++i) {
    if (small_m_ok(M, d[i].r)) {   // the decode regime takes its own route, one call each
      if (launch_matmul_fwd(d[i].X, m, view_of(d[i].W), d[i].T, d[i].B, d[i].r, d[i].Y, s) != hipSuccess)
        return QLORA_ERR_HIP;
      continue;
    }
    jobs[nj++] = MatmulJob{d[i].X, d[i].T, d[i].B, nullptr, d[i].Y, view_of(d[i].W), m, d[i].r};
  }
  return nj > 0 ? from_hip(launch_matmul_fwd_group(nj, jobs, s)) : QLORA_OK;
}

int qlora_linear_bwd(const uint16_t *dY, const uint16_t *X, const uint16_t *T, int64_t M,
                     const qlora_nf4_weight *W, const uint16_t *A, const uint16_t *B, int32_t r, float scale,
                     uint16_t *dX, uint16_t *dA, uint16_t *dB, void *ws, size_t ws_bytes, void *stream) {
  int st = check_linear_shape(M, W, r, scale);
  if (st) return st;
  if (!rows_ok(dY, M) || !rows_ok(X, M) || !bf16_ok(A) || !bf16_ok(B)) return QLORA_ERR_INVALID_ARG;
  if (!bf16_opt(T) || !bf16_opt(dX) || !bf16_opt(dA) || !bf16_opt(dB)) return QLORA_ERR_INVALID_ARG;
  const BwdWs L = bwd_ws(M, W->rows, W->cols, r);
  if (!ws || !aligned(ws, 16) || ws_bytes < L.total) return QLORA_ERR_WORKSPACE;
  if (M == 0) return QLORA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const NF4View v = view_of(W);
  const int m = static_cast<int>(M);
  char *base = static_cast<char *>(ws);
  uint16_t *Tw = reinterpret_cast<uint16_t *>(base);
  uint16_t *G = reinterpret_cast<uint16_t *>(base + L.t);
  void *bt = base + L.t + L.g;
  void *pa = base + L.t + L.g + L.bt;
  void *pb = base + L.t + L.g + L.bt + L.pa;
  hipError_t e = hipSuccess;
  if (dX || dA) {
    e = launch_lora_grad_in(dY, m, v.N, B, r, scale, G, bt, s);
    if (e != hipSuccess) return QLORA_ERR_HIP;
  }
  if (dX) {
    e = launch_matmul_dx(dY, m, v, G, A, r, dX, s);
    if (e != hipSuccess) return QLORA_ERR_HIP;
  }
  const uint16_t *Tu = T;
  if (dB && !Tu) {
    e = launch_lora_down(X, m, v.K, A, r, scale, Tw, s);
    if (e != hipSuccess) return QLORA_ERR_HIP;
    Tu = Tw;
  }
  const int sp = lora_grad_splits(m, v.K, v.N, r, dA != nullptr, dB != nullptr);
  GradWJob jobs[2];
  int nj = 0;
  if (dA) jobs[nj++] = GradWJob{X, G, m, v.K, r, true, dA, pa, sp};
  if (dB) jobs[nj++] = GradWJob{dY, Tu, m, v.N, r, false, dB, pb, sp};
  if (nj > 0 && launch_lora_grad_w_group(nj, jobs, s) != hipSuccess) return QLORA_ERR_HIP;
  return QLORA_OK;
}

// ---- LoRA dropout -------------------------------------------------------------

static bool drop_p_ok(float p) { return isfinite(p) && p >= 0.0f && p < 1.0f; }
static uint32_t drop_thresh(float p) { return static_cast<uint32_t>(floor(static_cast<double>(p) * 4294967296.0)); }
static float drop_scale(float scale, float p) {
  return static_cast<float>(static_cast<double>(scale) / (1.0 - static_cast<double>(p)));
}

int qlora_dropout_mask(const uint16_t *X, int64_t M, int64_t K, float p, uint64_t seed, uint16_t *X_drop,
                       uint32_t *keep, void *stream) {
  if (M < 0 || !drop_p_ok(p)) return QLORA_ERR_INVALID_ARG;
  if (K < 32 || K % 32 || (M > 0 && M > kMaxElems / K)) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (!rows_ok(X, M) || !rows_ok(X_drop, M) || !rows_ok(keep, M)) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  return from_hip(launch_dropout_mask(X, M * K, seed, drop_thresh(p), X_drop, keep, static_cast<hipStream_t>(stream)));
}

int qlora_dropout_apply(const uint16_t *X, int64_t M, int64_t K, const uint32_t *keep, uint16_t *X_drop,
                        void *stream) {
  if (M < 0) return QLORA_ERR_INVALID_ARG;
  if (K < 32 || K % 32 || (M > 0 && M > kMaxElems / K)) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (!rows_ok(X, M) || !rows_ok(X_drop, M) || !rows_ok(keep, M)) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  return from_hip(launch_dropout_apply(X, M * K, keep, X_drop, static_cast<hipStream_t>(stream)));
}

int qlora_nf4_matmul_dx_dropout(const uint16_t *dY, int64_t M, const qlora_nf4_weight *W, const uint16_t *G,
                                const uint16_t *A, int32_t r, const uint32_t *keep, uint16_t *dX, void *stream) {
  int st = check_linear_shape(M, W, r, 1.0f);
  if (st) return st;
  if (!rows_ok(dY, M) || !rows_ok(G, M) || !bf16_ok(A) || !rows_ok(dX, M) || !rows_ok(keep, M))
    return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  return from_hip(launch_matmul_dx_drop(dY, static_cast<int>(M), view_of(W), G, A, r, keep, dX,
                                        static_cast<hipStream_t>(stream)));
}

size_t qlora_linear_dropout_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r, int is_bwd) {
  if (M < 0 || N < 1 || K < 64 || K % 64 || N % 8 || r < 1 || r > 128) return 0;
  if (M > 0 && M > kMaxElems / std::max(N, K)) return 0;
  const size_t xd = bf16_bytes(M * K);
  return xd + (is_bwd ? bwd_ws(M, N, K, r).total : bf16_bytes(M * r));
}

int qlora_linear_fwd_dropout(const uint16_t *X, int64_t M, const qlora_nf4_weight *W, const uint16_t *A,
                             const uint16_t *B, int32_t r, float scale, float p, uint64_t seed, uint16_t *Y,
                             uint16_t *T_out, uint32_t *keep_out, void *ws, size_t ws_bytes, void *stream) {
  int st = check_linear_shape(M, W, r, scale);
  if (st) return st;
  if (!drop_p_ok(p)) return QLORA_ERR_INVALID_ARG;
  if (!rows_ok(X, M) || !bf16_ok(A) || !bf16_ok(B) || !rows_ok(Y, M) || !bf16_opt(T_out)) return QLORA_ERR_INVALID_ARG;
  if (!rows_ok(keep_out, M)) return QLORA_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 16) || ws_bytes < qlora_linear_dropout_workspace_bytes(M, W->rows, W->cols, r, 0))
    return QLORA_ERR_WORKSPACE;
  if (M == 0) return QLORA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const NF4View v = view_of(W);
  const int m = static_cast<int>(M);
  uint16_t *Xd = static_cast<uint16_t *>(ws);
  uint16_t *T = T_out ? T_out : reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + bf16_bytes(M * v.K));
  hipError_t e = launch_dropout_mask(X, M * v.K, seed, drop_thresh(p), Xd, keep_out, s);
  if (e == hipSuccess) e = launch_lora_down(Xd, m, v.K, A, r, drop_scale(scale, p), T, s);
  if (e == hipSuccess) e = launch_matmul_fwd(X, m, v, T, B, r, Y, s);
  return from_hip(e);
}

int qlora_linear_bwd_dropout(const uint16_t *dY, const uint16_t *X, const uint16_t *T, int64_t M,
                             const qlora_nf4_weight *W, const uint16_t *A, const uint16_t *B, int32_t r, float scale,
                             float p, const uint32_t *keep, uint16_t *dX, uint16_t *dA, uint16_t *dB, void *ws,
                             size_t ws_bytes, void *stream) {
  int st = check_linear_shape(M, W, r, scale);
  if (st) return st;
  if (!drop_p_ok(p)) return QLORA_ERR_INVALID_ARG;
  if (!rows_ok(dY, M) || !rows_ok(X, M) || !bf16_ok(A) || !bf16_ok(B)) return QLORA_ERR_INVALID_ARG;
  if (!bf16_opt(T) || !bf16_opt(dX) || !bf16_opt(dA) || !bf16_opt(dB)) return QLORA_ERR_INVALID_ARG;
  if (!rows_ok(keep, M)) return QLORA_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 16) || ws_bytes < qlora_linear_dropout_workspace_bytes(M, W->rows, W->cols, r, 1))
    return QLORA_ERR_WORKSPACE;
  if (M == 0) return QLORA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const NF4View v = view_of(W);
  const int m = static_cast<int>(M);
  const float se = drop_scale(scale, p);
  const BwdWs L = bwd_ws(M, v.N, v.K, r);
  char *base = static_cast<char *>(ws);
  uint16_t *Xd = reinterpret_cast<uint16_t *>(base);
  base += bf16_bytes(M * v.K);
  uint16_t *Tw = reinterpret_cast<uint16_t *>(base);
  uint16_t *G = reinterpret_cast<uint16_t *>(base + L.t);
  void *bt = base + L.t + L.g;
  void *pa = base + L.t + L.g + L.bt;
  void *pb = base + L.t + L.g + L.bt + L.pa;
  hipError_t e = hipSuccess;
  if (dA || (dB && !T)) e = launch_dropout_apply(X, M * v.K, keep, Xd, s);
  if (e == hipSuccess && (dX || dA)) e = launch_lora_grad_in(dY, m, v.N, B, r, se, G, bt, s);
  if (e == hipSuccess && dX) e = launch_matmul_dx_drop(dY, m, v, G, A, r, keep, dX, s);
  const uint16_t *Tu = T;
  if (e == hipSuccess && dB && !Tu) {
    e = launch_lora_down(Xd, m, v.K, A, r, se, Tw, s);
    Tu = Tw;
  }
  const int sp = lora_grad_splits(m, v.K, v.N, r, dA != nullptr, dB != nullptr);
  GradWJob jobs[2];
  int nj = 0;
  if (dA) jobs[nj++] = GradWJob{Xd, G, m, v.K, r, true, dA, pa, sp};
  if (dB) jobs[nj++] = GradWJob{dY, Tu, m, v.N, r, false, dB, pb, sp};
  if (e == hipSuccess && nj > 0) e = launch_lora_grad_w_group(nj, jobs, s);
  return from_hip(e);
}

}  // extern "C"
