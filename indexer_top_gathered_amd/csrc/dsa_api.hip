// C ABI of libdsa (declared in include/dsa.h): argument checks, the gfx950
// check, workspace layout and kernel launches. Every check runs on the host
// before anything is enqueued; no entry point waits for the device.
#include <atomic>
#include <cstring>
#include <mutex>

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

// Workspace of dsa_indexer_topk: the score rows (unless the caller takes
// them), then either the chunk cut's candidates or the two-stage top-k's.
struct IndexerTopkLayout {
  size_t scores_off, cand_off, cnt_off, tcut_off, topk_off, bytes;
  CutPlan cut;
  TopkPlan tk;
};

// The chunk cut serves rows longer than one workgroup's whole-row top-k:
// a row that fits one workgroup takes the indexer and that single top-k
// kernel, also two launches and each shorter (B=1, N=4096, k=256: 4.7 and
// 6.3 us against 6.8 and 5.9 us for the cut and its merge).
CutPlan indexer_cut_plan(int B, int N, int k) {
  CutPlan c = plan_cut(B, N, k);
  if (plan_topk(B, N, k, DSA_F32).fused) c.ok = false;
  return c;
}

IndexerTopkLayout indexer_topk_layout(int B, int N, int k, bool own_scores) {
  IndexerTopkLayout L{};
  L.cut = indexer_cut_plan(B, N, k);
  L.tk = plan_topk(B, N, k, DSA_F32);
  size_t off = 0;
  L.scores_off = off;
  if (own_scores) off = align_up(off + (size_t)B * N * sizeof(float), 256);
  if (L.cut.ok) {
    const size_t rows = (size_t)B * L.cut.chunks;
    L.cand_off = off;
    off = align_up(off + rows * L.cut.keep * sizeof(uint64_t), 256);
    L.cnt_off = off;
    off = align_up(off + rows * sizeof(uint32_t), 256);
    L.tcut_off = off;
    off = align_up(off + rows * sizeof(uint64_t), 256);
  } else {
    L.topk_off = off;
    off = align_up(off + L.tk.bytes, 256);
  }
  L.bytes = off ? off : 256;
  return L;
}

// The launches of dsa_indexer_topk (arguments already checked): the
// indexer with the chunk cut and the cut merge when the shape fits, else the
// indexer and the two-stage top-k.
hipError_t launch_indexer_topk(const void* q_idx, const void* k_idx, const float* w, float* scores,
                               int B, int N, int H, int k, int32_t* out_idx,
                               const IndexerTopkLayout& L, char* base, hipStream_t st) {
  hipError_t e;
  if (L.cut.ok) {
    uint64_t* cand = reinterpret_cast<uint64_t*>(base + L.cand_off);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(base + L.cnt_off);
    uint64_t* tcut = reinterpret_cast<uint64_t*>(base + L.tcut_off);
    e = launch_indexer_cut(static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx),
                           w, scores, B, N, H, L.cut, cand, cnt, tcut, st);
    if (e != hipSuccess) return e;
    return launch_topk_cut_merge(scores, B, N, k, L.cut, cand, cnt, tcut, out_idx, st);
  }
  e = launch_indexer_score(static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx),
                           w, scores, B, N, H, 1, nullptr, st);
  if (e != hipSuccess) return e;
  return launch_topk(scores, DSA_F32, B, N, k, out_idx, nullptr, 0, nullptr, L.tk,
                     base + L.topk_off, st);
}

// Workspace layout of the fused step (T query tokens per batch row). A
// plain one-token step takes dsa_indexer_topk's launches; ragged rows and
// several tokens take the indexer and the two-stage top-k.
struct StepLayout {
  size_t scores_off, idx_off, topk_off, attend_off, bytes;
  bool plain;             // no lengths, one token: dsa_indexer_topk's path
  IndexerTopkLayout itk;  // its buffers, at topk_off (the score rows at scores_off)
  TopkPlan tk;
  AttendPlan at;
};

StepLayout step_layout(const dsa_dims_t& d, int T, bool ragged) {
  StepLayout L{};
  const dsa_dims_t dq = query_rows(d, T);
  L.tk = plan_topk(dq.batch, d.n, d.topk, DSA_F32);
  L.at = plan_attend(dq);
  L.plain = T == 1 && !ragged;
  if (L.plain) L.itk = indexer_topk_layout(d.batch, d.n, d.topk, false);
  size_t off = 0;
  L.scores_off = off;
  off = align_up(off + (size_t)dq.batch * d.n * sizeof(float), 256);
  L.idx_off = off;
  off = align_up(off + (size_t)dq.batch * d.topk * sizeof(int32_t), 256);
  L.topk_off = off;
  off = align_up(off + (L.plain ? L.itk.bytes : L.tk.bytes), 256);
  L.attend_off = off;
  off = align_up(off + L.at.bytes, 256);
  L.bytes = off;
  return L;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status_t status) {
  // Callers may pass any int (an unknown code must give a name too), and an
  // out-of-range value may not be read as the enum in C++: take its bytes.
  int s;
  static_assert(sizeof(s) == sizeof(status), "dsa_status_t is an int-sized enum");
  std::memcpy(&s, &status, sizeof s);
  switch (s) {
    case DSA_SUCCESS: return "DSA_SUCCESS";
    case DSA_ERROR_INVALID_VALUE: return "DSA_ERROR_INVALID_VALUE: invalid argument";
    case DSA_ERROR_NOT_SUPPORTED: return "DSA_ERROR_NOT_SUPPORTED: shape or device not supported";
    case DSA_ERROR_WORKSPACE_TOO_SMALL: return "DSA_ERROR_WORKSPACE_TOO_SMALL: workspace too small";
    case DSA_ERROR_LAUNCH: return "DSA_ERROR_LAUNCH: kernel launch failed";
    case DSA_ERROR_DEVICE: return "DSA_ERROR_DEVICE: no usable HIP device";
    case DSA_ERROR_SCRATCH_LIMIT:
      return "DSA_ERROR_SCRATCH_LIMIT: the shape needs more workspace than the static scratch "
             "buffer of dsa_decode_step_noalloc holds (DSA_NOALLOC_SCRATCH_BYTES)";
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

int dsa_indexer_topk_chunks(int B, int N, int k) {
  if (check_topk_shape(B, N, k, DSA_F32) != DSA_SUCCESS) return 0;
  const CutPlan p = indexer_cut_plan(B, N, k);
  return p.ok ? p.chunks : 0;
}

size_t dsa_indexer_topk_workspace_bytes(int B, int N, int H_I, int k, int own_scores) {
  if (check_indexer_shape(B, N, H_I, 128) != DSA_SUCCESS) return 0;
  if (check_topk_shape(B, N, k, DSA_F32) != DSA_SUCCESS) return 0;
  return indexer_topk_layout(B, N, k, own_scores != 0).bytes;
}

dsa_status_t dsa_indexer_topk(const void* q_idx, const void* k_idx, const float* w, int B, int N,
                              int H_I, int D_I, int k, int32_t* out_idx, float* scores, void* ws,
                              size_t ws_bytes, void* stream) {
  if (!q_idx || !k_idx || !w || !out_idx || !ws) return DSA_ERROR_INVALID_VALUE;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(ws) ||
      (reinterpret_cast<uintptr_t>(w) & 3u) || (reinterpret_cast<uintptr_t>(out_idx) & 3u) ||
      (scores && !aligned16(scores)))
    return DSA_ERROR_INVALID_VALUE;
  dsa_status_t s = check_indexer_shape(B, N, H_I, D_I);
  if (s != DSA_SUCCESS) return s;
  s = check_topk_shape(B, N, k, DSA_F32);
  if (s != DSA_SUCCESS) return s;
  const IndexerTopkLayout L = indexer_topk_layout(B, N, k, scores == nullptr);
  if (ws_bytes < L.bytes) return DSA_ERROR_WORKSPACE_TOO_SMALL;
  s = check_device();
  if (s != DSA_SUCCESS) return s;
  char* base = static_cast<char*>(ws);
  float* sc = scores ? scores : reinterpret_cast<float*>(base + L.scores_off);
  return to_status(launch_indexer_topk(q_idx, k_idx, w, sc, B, N, H_I, k, out_idx, L, base,
                                       static_cast<hipStream_t>(stream)));
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

}  // extern "C"

namespace {

dsa_status_t attend_impl(const void* q, const void* kv_cmp, const int32_t* idx,
                         const void* kv_win, const float* sink, void* out,
                         const dsa_dims_t* dims, int T, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!dims || T < 1) return DSA_ERROR_INVALID_VALUE;
  if (T > kMaxTokens) return DSA_ERROR_NOT_SUPPORTED;
  const dsa_dims_t dq = query_rows(*dims, T);
  dsa_status_t s = check_attend_dims(&dq);
  if (s != DSA_SUCCESS) return s;
  if (!q || !kv_cmp || !idx || !out || !ws || (dims->window > 0 && !kv_win))
    return DSA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(kv_cmp) || !aligned16(out) || !aligned16(ws) ||
      (kv_win && !aligned16(kv_win)) || (reinterpret_cast<uintptr_t>(idx) & 3u) ||
      (reinterpret_cast<uintptr_t>(sink) & 3u))
    return DSA_ERROR_INVALID_VALUE;
  const AttendPlan plan = plan_attend(dq);
  if (ws_bytes < (plan.bytes ? plan.bytes : 256)) return DSA_ERROR_WORKSPACE_TOO_SMALL;
  s = check_device();
  if (s != DSA_SUCCESS) return s;
  return to_status(launch_attend(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv_cmp),
                                 idx, static_cast<const uint16_t*>(kv_win), static_cast<uint16_t*>(out),
                                 sink, dq, plan, T, ws, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

dsa_status_t dsa_sparse_attend(const void* q, const void* kv_cmp, const int32_t* idx,
                               const void* kv_win, void* out, const dsa_dims_t* dims, void* ws,
                               size_t ws_bytes, void* stream) {
  return attend_impl(q, kv_cmp, idx, kv_win, nullptr, out, dims, 1, ws, ws_bytes, stream);
}

dsa_status_t dsa_sparse_attend_sink(const void* q, const void* kv_cmp, const int32_t* idx,
                                    const void* kv_win, const float* sink, void* out,
                                    const dsa_dims_t* dims, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (!sink) return DSA_ERROR_INVALID_VALUE;
  return attend_impl(q, kv_cmp, idx, kv_win, sink, out, dims, 1, ws, ws_bytes, stream);
}

dsa_status_t dsa_sparse_attend_mt(const void* q, const void* kv_cmp, const int32_t* idx,
                                  const void* kv_win, void* out, const dsa_dims_t* dims, int T,
                                  void* ws, size_t ws_bytes, void* stream) {
  return attend_impl(q, kv_cmp, idx, kv_win, nullptr, out, dims, T, ws, ws_bytes, stream);
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
  // The larger of the two layouts, so one size serves the plain, ragged and
  // several-token calls alike.
  const size_t a = step_layout(*dims, T, false).bytes, b = step_layout(*dims, T, true).bytes;
  return a > b ? a : b;
}

}  // extern "C"

namespace {

// Pointer checks of the fused step (the workspace is checked by the caller).
dsa_status_t check_step_pointers(const void* q_idx, const void* k_idx, const float* w,
                                 const void* q, const void* kv_cmp, const void* kv_win,
                                 const int32_t* lengths, const void* out, const int32_t* out_idx,
                                 int window) {
  if (!q_idx || !k_idx || !w || !q || !kv_cmp || !out || (window > 0 && !kv_win))
    return DSA_ERROR_INVALID_VALUE;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(q) || !aligned16(kv_cmp) ||
      !aligned16(out) || (kv_win && !aligned16(kv_win)) ||
      (reinterpret_cast<uintptr_t>(w) & 3u) || (reinterpret_cast<uintptr_t>(out_idx) & 3u) ||
      (reinterpret_cast<uintptr_t>(lengths) & 3u))
    return DSA_ERROR_INVALID_VALUE;
  return DSA_SUCCESS;
}

dsa_status_t step_impl(const void* q_idx, const void* k_idx, const float* w, const void* q,
                       const void* kv_cmp, const void* kv_win, const int32_t* lengths, void* out,
                       int32_t* out_idx, const dsa_dims_t* dims, int T, void* ws,
                       size_t ws_bytes, void* stream, const float* sink = nullptr) {
  if (!dims || T < 1) return DSA_ERROR_INVALID_VALUE;
  if (T > kMaxTokens) return DSA_ERROR_NOT_SUPPORTED;
  const dsa_dims_t dq = query_rows(*dims, T);
  dsa_status_t s = check_attend_dims(&dq);
  if (s != DSA_SUCCESS) return s;
  s = check_indexer_shape(dims->batch, dims->n, dims->idx_heads, dims->idx_dim, T);
  if (s != DSA_SUCCESS) return s;
  s = check_step_pointers(q_idx, k_idx, w, q, kv_cmp, kv_win, lengths, out, out_idx, dims->window);
  if (s != DSA_SUCCESS) return s;
  if (!ws || !aligned16(ws) || (reinterpret_cast<uintptr_t>(sink) & 3u))
    return DSA_ERROR_INVALID_VALUE;
  const StepLayout L = step_layout(*dims, T, lengths != nullptr);
  if (ws_bytes < L.bytes) return DSA_ERROR_WORKSPACE_TOO_SMALL;
  s = check_device();
  if (s != DSA_SUCCESS) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base + L.scores_off);
  int32_t* sel = out_idx ? out_idx : reinterpret_cast<int32_t*>(base + L.idx_off);
  const dsa_dims_t& d = *dims;
  hipError_t e;
  if (L.plain) {
    // Where the attention kernel can select its own rows, the cut merge is
    // folded into it: the indexer with the chunk cut, then attention.
    const int per = L.itk.cut.ok ? attend_select_per(dq, L.at, L.itk.cut.chunks, L.itk.cut.keep) : 0;
    if (per > 0) {
      char* tb = base + L.topk_off;
      SelectArgs sa{};
      sa.cand = reinterpret_cast<const uint64_t*>(tb + L.itk.cand_off);
      sa.cnt = reinterpret_cast<const uint32_t*>(tb + L.itk.cnt_off);
      sa.tcut = reinterpret_cast<const uint64_t*>(tb + L.itk.tcut_off);
      sa.scores = scores;
      sa.idx_out = sel;
      sa.chunks = L.itk.cut.chunks;
      sa.keep = L.itk.cut.keep;
      e = launch_indexer_cut(static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx),
                             w, scores, d.batch, d.n, d.idx_heads, L.itk.cut,
                             reinterpret_cast<uint64_t*>(tb + L.itk.cand_off),
                             reinterpret_cast<uint32_t*>(tb + L.itk.cnt_off),
                             reinterpret_cast<uint64_t*>(tb + L.itk.tcut_off), st);
      if (e != hipSuccess) return DSA_ERROR_LAUNCH;
      e = launch_attend_select(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv_cmp),
                               static_cast<const uint16_t*>(kv_win), static_cast<uint16_t*>(out), sink,
                               dq, L.at, sa, per, base + L.attend_off, st);
      return to_status(e);
    }
    e = launch_indexer_topk(q_idx, k_idx, w, scores, d.batch, d.n, d.idx_heads, d.topk, sel,
                            L.itk, base + L.topk_off, st);
    if (e != hipSuccess) return DSA_ERROR_LAUNCH;
  } else {
    e = launch_indexer_score(static_cast<const uint16_t*>(q_idx),
                             static_cast<const uint16_t*>(k_idx), w, scores, d.batch, d.n,
                             d.idx_heads, T, lengths, st);
    if (e != hipSuccess) return DSA_ERROR_LAUNCH;
    e = launch_topk(scores, DSA_F32, dq.batch, d.n, d.topk, sel, nullptr, 0, lengths, L.tk,
                    base + L.topk_off, st);
    if (e != hipSuccess) return DSA_ERROR_LAUNCH;
  }
  e = launch_attend(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv_cmp), sel,
                    static_cast<const uint16_t*>(kv_win), static_cast<uint16_t*>(out), sink, dq,
                    L.at, T, base + L.attend_off, st);
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

dsa_status_t dsa_decode_step_sink(const void* q_idx, const void* k_idx, const float* w,
                                  const void* q, const void* kv_cmp, const void* kv_win,
                                  const float* sink, void* out, int32_t* out_idx,
                                  const dsa_dims_t* dims, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (!sink) return DSA_ERROR_INVALID_VALUE;
  return step_impl(q_idx, k_idx, w, q, kv_cmp, kv_win, nullptr, out, out_idx, dims, 1, ws,
                   ws_bytes, stream, sink);
}

dsa_status_t dsa_compress(const void* x, const float* w_gate, void* out, int B, int G, int D,
                          void* stream) {
  if (!x || !w_gate || !out) return DSA_ERROR_INVALID_VALUE;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(out)) return DSA_ERROR_INVALID_VALUE;
  if (B < 1 || G < 1 || D < 1) return DSA_ERROR_INVALID_VALUE;
  if (D % 8 != 0 || D > 1024) return DSA_ERROR_NOT_SUPPORTED;
  if ((long long)B * G * 4 * D > 0x7FFFFFFFLL) return DSA_ERROR_NOT_SUPPORTED;
  dsa_status_t s = check_device();
  if (s != DSA_SUCCESS) return s;
  return to_status(launch_compress(static_cast<const uint16_t*>(x), w_gate,
                                   static_cast<uint16_t*>(out), B * G, D,
                                   static_cast<hipStream_t>(stream)));
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

// ---------------------------------------------------------------- no allocation
// The workspace of dsa_decode_step_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends. Host code never uses the
// array's name as an address (on the host it names a stand-in, not device
// memory): the device address is looked up once per device with
// hipGetSymbolAddress and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device (looked up on the
// first call there), or an error status.
dsa_status_t scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return DSA_ERROR_DEVICE;
  }
  if (dev >= kMaxDevices) return DSA_ERROR_NOT_SUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return DSA_ERROR_DEVICE;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_SUCCESS;
}

}  // namespace

extern "C" {

dsa_status_t dsa_decode_step_noalloc(const void* q_idx, const void* k_idx, const float* w,
                                     const void* q, const void* kv_cmp, const void* kv_win,
                                     void* out, int32_t* out_idx, const dsa_dims_t* dims,
                                     void* stream) {
  if (!dims) return DSA_ERROR_INVALID_VALUE;
  dsa_status_t s = check_attend_dims(dims);
  if (s != DSA_SUCCESS) return s;
  s = check_indexer_shape(dims->batch, dims->n, dims->idx_heads, dims->idx_dim);
  if (s != DSA_SUCCESS) return s;
  s = check_step_pointers(q_idx, k_idx, w, q, kv_cmp, kv_win, nullptr, out, out_idx,
                          dims->window);
  if (s != DSA_SUCCESS) return s;
  const size_t need = step_layout(*dims, 1, false).bytes;
  if (need > (size_t)DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERROR_SCRATCH_LIMIT;
  s = check_device();
  if (s != DSA_SUCCESS) return s;
  void* ws = nullptr;
  s = scratch_ptr(&ws);
  if (s != DSA_SUCCESS) return s;
  return step_impl(q_idx, k_idx, w, q, kv_cmp, kv_win, nullptr, out, out_idx, dims, 1, ws,
                   (size_t)DSA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
