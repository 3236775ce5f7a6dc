// C ABI of libdsa (declared in include/dsa.h): argument checks, the gfx950
// check, workspace layout and kernel launches. Every check runs on the host
// before anything is enqueued; no entry point waits for the device.
#include <atomic>
#include <cstring>

#include "dsa_internal.h"

namespace {

using namespace dsa;

constexpr int kMaxTopk = 4096;
constexpr int kMaxDevices = 64;

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch[kMaxDevices];

dsa_status_t check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return DSA_ERROR_DEVICE;
  }
  if (dev >= kMaxDevices) return DSA_ERROR_NOT_SUPPORTED;
  int state = g_arch[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return DSA_ERROR_DEVICE;
    }
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? DSA_SUCCESS : DSA_ERROR_NOT_SUPPORTED;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

dsa_status_t to_status(hipError_t e) { return e == hipSuccess ? DSA_SUCCESS : DSA_ERROR_LAUNCH; }

// Shape checks of the indexer stage (T query tokens per batch row).
dsa_status_t check_indexer_shape(int B, int N, int H, int DI, int T = 1) {
  if (B < 1 || N < 1 || H < 1 || DI < 1 || T < 1) return DSA_ERROR_INVALID_VALUE;
  if (DI != 128 || H > 64 || T > kMaxTokens) return DSA_ERROR_NOT_SUPPORTED;
  if ((long long)B * T * N > 0x7FFFFFFFLL || B > 65535) return DSA_ERROR_NOT_SUPPORTED;
  return DSA_SUCCESS;
}

dsa_status_t check_topk_shape(int B, int N, int k, dsa_dtype_t dt) {
  if (B < 1 || N < 1 || k < 1 || k > N) return DSA_ERROR_INVALID_VALUE;
  if (dt != DSA_BF16 && dt != DSA_F32) return DSA_ERROR_INVALID_VALUE;
  if (k > kMaxTopk) return DSA_ERROR_NOT_SUPPORTED;
  if (B > 65535) return DSA_ERROR_NOT_SUPPORTED;
  return DSA_SUCCESS;
}

// Attention shape checks (reads batch, n, topk, window, q_heads, head_dim, scale).
dsa_status_t check_attend_dims(const dsa_dims_t* d) {
  if (!d) return DSA_ERROR_INVALID_VALUE;
  if (d->batch < 1 || d->n < 1 || d->topk < 1 || d->topk > d->n || d->window < 0 ||
      d->q_heads < 1 || d->head_dim < 1)
    return DSA_ERROR_INVALID_VALUE;
  if (!(d->scale == d->scale) || d->scale == __builtin_inff() || d->scale == -__builtin_inff())
    return DSA_ERROR_INVALID_VALUE;
  if (d->head_dim != 128 && d->head_dim != 512) return DSA_ERROR_NOT_SUPPORTED;
  if (d->q_heads % 16 != 0 || d->q_heads > 128) return DSA_ERROR_NOT_SUPPORTED;
  if (d->topk > kMaxTopk || d->batch > 65535) return DSA_ERROR_NOT_SUPPORTED;
  return DSA_SUCCESS;
}

// The attention dims of T query tokens per batch row: one query row each.
dsa_dims_t query_rows(const dsa_dims_t& d, int T) {
  dsa_dims_t r = d;
  r.batch = (int32_t)((long long)d.batch * T > 0x7FFFFFFFLL ? 0x7FFFFFFF : d.batch * T);
  return r;
}

// Workspace layout of the fused step (T query tokens per batch row).
struct StepLayout {
  size_t scores_off, idx_off, topk_off, attend_off, bytes;
  TopkPlan tk;
  AttendPlan at;
};

StepLayout step_layout(const dsa_dims_t& d, int T) {
  StepLayout L{};
  const dsa_dims_t dq = query_rows(d, T);
  L.tk = plan_topk(dq.batch, d.n, d.topk, DSA_F32);
  L.at = plan_attend(dq);
  size_t off = 0;
  L.scores_off = off;
  off = align_up(off + (size_t)dq.batch * d.n * sizeof(float), 256);
  L.idx_off = off;
  off = align_up(off + (size_t)dq.batch * d.topk * sizeof(int32_t), 256);
  L.topk_off = off;
  off = align_up(off + L.tk.bytes, 256);
  L.attend_off = off;
  off = align_up(off + L.at.bytes, 256);
  L.bytes = off;
  return L;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status_t s) {
  switch (s) {
    case DSA_SUCCESS: return "DSA_SUCCESS";
    case DSA_ERROR_INVALID_VALUE: return "DSA_ERROR_INVALID_VALUE: invalid argument";
    case DSA_ERROR_NOT_SUPPORTED: return "DSA_ERROR_NOT_SUPPORTED: shape or device not supported";
    case DSA_ERROR_WORKSPACE_TOO_SMALL: return "DSA_ERROR_WORKSPACE_TOO_SMALL: workspace too small";
    case DSA_ERROR_LAUNCH: return "DSA_ERROR_LAUNCH: kernel launch failed";
    case DSA_ERROR_DEVICE: return "DSA_ERROR_DEVICE: no usable HIP device";
  }
  return "DSA_ERROR_UNKNOWN";
}

dsa_status_t dsa_indexer_score(const void* q_idx, const void* k_idx, const float* w,
                               float* scores, int B, int N, int H_I, int D_I, void* stream) {
  if (!q_idx || !k_idx || !w || !scores) return DSA_ERROR_INVALID_VALUE;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(scores) ||
      (reinterpret_cast<uintptr_t>(w) & 3u))
    return DSA_ERROR_INVALID_VALUE;
  dsa_status_t s = check_indexer_shape(B, N, H_I, D_I);
  if (s != DSA_SUCCESS) return s;
  s = check_device();
  if (s != DSA_SUCCESS) return s;
  return to_status(launch_indexer_score(static_cast<const uint16_t*>(q_idx),
                                        static_cast<const uint16_t*>(k_idx), w, scores, B, N,
                                        H_I, 1, nullptr, static_cast<hipStream_t>(stream)));
}

dsa_status_t dsa_indexer_score_mt(const void* q_idx, const void* k_idx, const float* w,
                                  float* scores, int B, int T, int N, int H_I, int D_I,
                                  void* stream) {
  if (!q_idx || !k_idx || !w || !scores) return DSA_ERROR_INVALID_VALUE;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(scores) ||
      (reinterpret_cast<uintptr_t>(w) & 3u))
    return DSA_ERROR_INVALID_VALUE;
  dsa_status_t s = check_indexer_shape(B, N, H_I, D_I, T);
  if (s != DSA_SUCCESS) return s;
  s = check_device();
  if (s != DSA_SUCCESS) return s;
  return to_status(launch_indexer_score(static_cast<const uint16_t*>(q_idx),
                                        static_cast<const uint16_t*>(k_idx), w, scores, B, N,
                                        H_I, T, nullptr, static_cast<hipStream_t>(stream)));
}

dsa_status_t dsa_indexer_qproj(const void* x, const void* w_q, void* q_idx, int B, int d_in,
                               int H_I, int D_I, void* stream) {
  if (!x || !w_q || !q_idx) return DSA_ERROR_INVALID_VALUE;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(q_idx)) return DSA_ERROR_INVALID_VALUE;
  if (B < 1 || d_in < 1 || H_I < 1 || D_I < 1) return DSA_ERROR_INVALID_VALUE;
  if (D_I != 128 || H_I > 64 || d_in % 256 != 0 || B > 65535 * 16) return DSA_ERROR_NOT_SUPPORTED;
  if ((long long)H_I * D_I * d_in > 0x7FFFFFFFLL || (long long)B * d_in > 0x7FFFFFFFLL)
    return DSA_ERROR_NOT_SUPPORTED;
  dsa_status_t s = check_device();
  if (s != DSA_SUCCESS) return s;
  return to_status(launch_qproj(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_q),
                                static_cast<uint16_t*>(q_idx), B, d_in, H_I * D_I,
                                static_cast<hipStream_t>(stream)));
}

size_t dsa_topk_workspace_bytes(int B, int N, int k, dsa_dtype_t dtype) {
  if (check_topk_shape(B, N, k, dtype) != DSA_SUCCESS) return 0;
  return plan_topk(B, N, k, dtype).bytes;
}

}  // extern "C"

namespace {

dsa_status_t topk_impl(const void* scores, dsa_dtype_t dtype, int B, int N, const int32_t* lengths,
                       int k, int32_t* out_idx, void* out_val, int sorted_index, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!scores || !out_idx) return DSA_ERROR_INVALID_VALUE;
  if (!aligned16(scores) || !aligned16(ws) || (reinterpret_cast<uintptr_t>(out_idx) & 3u))
    return DSA_ERROR_INVALID_VALUE;
  if (out_val && (reinterpret_cast<uintptr_t>(out_val) & (dtype == DSA_BF16 ? 1u : 3u)))
    return DSA_ERROR_INVALID_VALUE;
  if (sorted_index != 0 && sorted_index != 1) return DSA_ERROR_INVALID_VALUE;
  dsa_status_t s = check_topk_shape(B, N, k, dtype);
  if (s != DSA_SUCCESS) return s;
  const TopkPlan plan = plan_topk(B, N, k, dtype);
  if (plan.bytes > 0 && !ws) return DSA_ERROR_INVALID_VALUE;
  if (ws_bytes < plan.bytes) return DSA_ERROR_WORKSPACE_TOO_SMALL;
  s = check_device();
  if (s != DSA_SUCCESS) return s;
  return to_status(launch_topk(scores, dtype, B, N, k, out_idx, out_val, sorted_index, lengths,
                               plan, ws, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

dsa_status_t dsa_topk(const void* scores, dsa_dtype_t dtype, int B, int N, int k,
                      int32_t* out_idx, void* out_val, int sorted_index, void* ws,
                      size_t ws_bytes, void* stream) {
  return topk_impl(scores, dtype, B, N, nullptr, k, out_idx, out_val, sorted_index, ws, ws_bytes,
                   stream);
}

dsa_status_t dsa_topk_ragged(const void* scores, dsa_dtype_t dtype, int B, int N,
                             const int32_t* lengths, int k, int32_t* out_idx, void* out_val,
                             int sorted_index, void* ws, size_t ws_bytes, void* stream) {
  if (!lengths || (reinterpret_cast<uintptr_t>(lengths) & 3u)) return DSA_ERROR_INVALID_VALUE;
  return topk_impl(scores, dtype, B, N, lengths, k, out_idx, out_val, sorted_index, ws, ws_bytes,
                   stream);
}

size_t dsa_sparse_attend_workspace_bytes(const dsa_dims_t* dims) {
  return dsa_sparse_attend_mt_workspace_bytes(dims, 1);
}

size_t dsa_sparse_attend_mt_workspace_bytes(const dsa_dims_t* dims, int T) {
  if (!dims || T < 1 || T > kMaxTokens) return 0;
  const dsa_dims_t dq = query_rows(*dims, T);
  if (check_attend_dims(&dq) != DSA_SUCCESS) return 0;
  // Never report 0 for a valid shape, so a zero result always means "invalid".
  const size_t b = plan_attend(dq).bytes;
  return b ? b : 256;
}

dsa_status_t dsa_sparse_attend(const void* q, const void* kv_cmp, const int32_t* idx,
                               const void* kv_win, void* out, const dsa_dims_t* dims, void* ws,
                               size_t ws_bytes, void* stream) {
  return dsa_sparse_attend_mt(q, kv_cmp, idx, kv_win, out, dims, 1, ws, ws_bytes, stream);
}

dsa_status_t dsa_sparse_attend_mt(const void* q, const void* kv_cmp, const int32_t* idx,
                                  const void* kv_win, void* out, const dsa_dims_t* dims, int T,
                                  void* ws, size_t ws_bytes, void* stream) {
  if (!dims || T < 1) return DSA_ERROR_INVALID_VALUE;
  if (T > kMaxTokens) return DSA_ERROR_NOT_SUPPORTED;
  const dsa_dims_t dq = query_rows(*dims, T);
  dsa_status_t s = check_attend_dims(&dq);
  if (s != DSA_SUCCESS) return s;
  if (!q || !kv_cmp || !idx || !out || !ws || (dims->window > 0 && !kv_win))
    return DSA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(kv_cmp) || !aligned16(out) || !aligned16(ws) ||
      (kv_win && !aligned16(kv_win)) || (reinterpret_cast<uintptr_t>(idx) & 3u))
    return DSA_ERROR_INVALID_VALUE;
  const AttendPlan plan = plan_attend(dq);
  if (ws_bytes < (plan.bytes ? plan.bytes : 256)) return DSA_ERROR_WORKSPACE_TOO_SMALL;
  s = check_device();
  if (s != DSA_SUCCESS) return s;
  return to_status(launch_attend(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv_cmp),
                                 idx, static_cast<const uint16_t*>(kv_win), static_cast<uint16_t*>(out),
                                 dq, plan, T, ws, static_cast<hipStream_t>(stream)));
}

size_t dsa_decode_step_workspace_bytes(const dsa_dims_t* dims) {
  return dsa_decode_step_mt_workspace_bytes(dims, 1);
}

size_t dsa_decode_step_mt_workspace_bytes(const dsa_dims_t* dims, int T) {
  if (!dims || T < 1 || T > kMaxTokens) return 0;
  const dsa_dims_t dq = query_rows(*dims, T);
  if (check_attend_dims(&dq) != DSA_SUCCESS) return 0;
  if (check_indexer_shape(dims->batch, dims->n, dims->idx_heads, dims->idx_dim, T) != DSA_SUCCESS)
    return 0;
  return step_layout(*dims, T).bytes;
}

}  // extern "C"

namespace {

dsa_status_t step_impl(const void* q_idx, const void* k_idx, const float* w, const void* q,
                       const void* kv_cmp, const void* kv_win, const int32_t* lengths, void* out,
                       int32_t* out_idx, const dsa_dims_t* dims, int T, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!dims || T < 1) return DSA_ERROR_INVALID_VALUE;
  if (T > kMaxTokens) return DSA_ERROR_NOT_SUPPORTED;
  const dsa_dims_t dq = query_rows(*dims, T);
  dsa_status_t s = check_attend_dims(&dq);
  if (s != DSA_SUCCESS) return s;
  s = check_indexer_shape(dims->batch, dims->n, dims->idx_heads, dims->idx_dim, T);
  if (s != DSA_SUCCESS) return s;
  if (!q_idx || !k_idx || !w || !q || !kv_cmp || !out || !ws || (dims->window > 0 && !kv_win))
    return DSA_ERROR_INVALID_VALUE;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(q) || !aligned16(kv_cmp) ||
      !aligned16(out) || !aligned16(ws) || (kv_win && !aligned16(kv_win)) ||
      (reinterpret_cast<uintptr_t>(w) & 3u) || (reinterpret_cast<uintptr_t>(out_idx) & 3u) ||
      (reinterpret_cast<uintptr_t>(lengths) & 3u))
    return DSA_ERROR_INVALID_VALUE;
  const StepLayout L = step_layout(*dims, T);
  if (ws_bytes < L.bytes) return DSA_ERROR_WORKSPACE_TOO_SMALL;
  s = check_device();
  if (s != DSA_SUCCESS) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base + L.scores_off);
  int32_t* sel = out_idx ? out_idx : reinterpret_cast<int32_t*>(base + L.idx_off);
  const dsa_dims_t& d = *dims;
  hipError_t e = launch_indexer_score(static_cast<const uint16_t*>(q_idx),
                                      static_cast<const uint16_t*>(k_idx), w, scores, d.batch, d.n,
                                      d.idx_heads, T, lengths, st);
  if (e != hipSuccess) return DSA_ERROR_LAUNCH;
  e = launch_topk(scores, DSA_F32, dq.batch, d.n, d.topk, sel, nullptr, 0, lengths, L.tk,
                  base + L.topk_off, st);
  if (e != hipSuccess) return DSA_ERROR_LAUNCH;
  e = launch_attend(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv_cmp), sel,
                    static_cast<const uint16_t*>(kv_win), static_cast<uint16_t*>(out), dq, L.at, T,
                    base + L.attend_off, st);
  return to_status(e);
}

}  // namespace

extern "C" {

dsa_status_t dsa_decode_step(const void* q_idx, const void* k_idx, const float* w, const void* q,
                             const void* kv_cmp, const void* kv_win, void* out, int32_t* out_idx,
                             const dsa_dims_t* dims, void* ws, size_t ws_bytes, void* stream) {
  return step_impl(q_idx, k_idx, w, q, kv_cmp, kv_win, nullptr, out, out_idx, dims, 1, ws,
                   ws_bytes, stream);
}

dsa_status_t dsa_decode_step_ragged(const void* q_idx, const void* k_idx, const float* w,
                                    const void* q, const void* kv_cmp, const void* kv_win,
                                    const int32_t* lengths, void* out, int32_t* out_idx,
                                    const dsa_dims_t* dims, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (!lengths) return DSA_ERROR_INVALID_VALUE;
  return step_impl(q_idx, k_idx, w, q, kv_cmp, kv_win, lengths, out, out_idx, dims, 1, ws,
                   ws_bytes, stream);
}

dsa_status_t dsa_decode_step_mt(const void* q_idx, const void* k_idx, const float* w,
                                const void* q, const void* kv_cmp, const void* kv_win,
                                const int32_t* lengths, void* out, int32_t* out_idx,
                                const dsa_dims_t* dims, int T, void* ws, size_t ws_bytes,
                                void* stream) {
  return step_impl(q_idx, k_idx, w, q, kv_cmp, kv_win, lengths, out, out_idx, dims, T, ws,
                   ws_bytes, stream);
}

}  // extern "C"
