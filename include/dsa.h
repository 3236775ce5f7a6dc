/*
 * dsa.h - C ABI of the MI355X (gfx950) sparse-attention decode-step library.
 *
 * One decode step of DeepSeek-style sparse attention runs in three stages:
 *   1. lightning-indexer scoring of every compressed position,
 *   2. top-k selection of the best-scoring positions,
 *   3. multi-query attention over the selected compressed rows plus a window
 *      of recent raw rows.
 * The stages are described in "feat: Add DeepSeek-V4 CSA attention kernels"
 * (aws-neuron nki-library pull request 13), section "How the algorithm
 * works", steps 2-4; the top-k options follow the "DeepSelect" project page
 * (sorted_index and return_value), and the attention scale follows the
 * norm_factor of "Implementation: Deepspeedai DeepSpeed Inference PT
 * Binding" (Usage Examples).
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a HIP device pointer on the current device.
 *    Tensors are dense, row-major, and 16-byte aligned.
 *  - bf16 tensors hold IEEE bfloat16 bit patterns (2 bytes per element).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *    work is enqueued on it and the call returns without waiting for the
 *    device; outputs are ready once the stream reaches that point.
 *  - Ownership: the caller owns every buffer, including the workspace `ws`
 *    (size from the matching *_workspace_bytes call). The library allocates
 *    and frees no device memory and keeps no state between calls. Buffers
 *    must stay alive until the enqueued work completes. Calls that share a
 *    workspace must be ordered on one stream.
 *  - Errors: every argument is checked on the host before anything is
 *    enqueued. On a non-zero status nothing was launched. The device must be
 *    gfx950, else DSA_ERROR_NOT_SUPPORTED. A failed kernel launch returns
 *    DSA_ERROR_LAUNCH. No C++ exception crosses this interface.
 *  - Results are deterministic: the same inputs give the same bits.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define DSA_EXPORT __attribute__((visibility("default")))
#else
#define DSA_EXPORT
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DSA_BF16 = 0, DSA_F32 = 1 } dsa_dtype_t;

typedef enum {
  DSA_SUCCESS = 0,
  DSA_ERROR_INVALID_VALUE = 1,       /* null pointer, bad size, misalignment */
  DSA_ERROR_NOT_SUPPORTED = 2,       /* shape outside the compiled range, not gfx950 */
  DSA_ERROR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes below the *_workspace_bytes value */
  DSA_ERROR_LAUNCH = 4,              /* a kernel launch failed */
  DSA_ERROR_DEVICE = 5,              /* no usable HIP device */
  DSA_ERROR_SCRATCH_LIMIT = 6        /* beyond the static scratch of dsa_decode_step_noalloc */
} dsa_status_t;

/* Problem sizes of one decode step (the block shapes of "Launching a full
 * block" in the CSA pull request). */
typedef struct {
  int32_t batch;     /* B: independent decode tokens (>= 1) */
  int32_t n;         /* N: compressed positions per token (>= 1) */
  int32_t idx_heads; /* H_I: indexer heads, 1..64 */
  int32_t idx_dim;   /* D_I: indexer channels; must be 128 */
  int32_t topk;      /* k: selected positions, 1 <= k <= min(N, 4096) */
  int32_t window;    /* W: raw window rows, >= 0 */
  int32_t q_heads;   /* H_q: query heads, a multiple of 16, 16..128 */
  int32_t head_dim;  /* D: KV dim (K = V), 128 or 512 */
  float scale;       /* softmax scale applied to q.k, e.g. 1/sqrt(D) */
} dsa_dims_t;

/*
 * Lightning-indexer scores (CSA pull request, "How the algorithm works",
 * step 2): each head's query dotted with every key, clipped at zero, scaled
 * by the head's weight and added over heads:
 *   scores[b,j] = sum_{h<H_I} w[b,h] * max(0, sum_{d<D_I} q_idx[b,h,d] * k_idx[b,j,d])
 * q_idx  bf16 [B, H_I, D_I]; k_idx bf16 [B, N, D_I]; w float [B, H_I];
 * scores float [B, N] (output). Products are exact, sums run in float32
 * with a fixed order. Requires D_I == 128 and 1 <= H_I <= 64.
 */
DSA_EXPORT dsa_status_t dsa_indexer_score(const void* q_idx, const void* k_idx, const float* w,
                               float* scores, int B, int N, int H_I, int D_I,
                               void* stream);

/*
 * Indexer query projection (CSA pull request, "How the algorithm works",
 * step table, step 2: the indexer query is projected into 128 channels per
 * head; the pull request runs it as a hand-tiled GEMV):
 *   q_idx[b, h, c] = sum_i x[b, i] * w_q[h*D_I + c, i]
 * x bf16 [B, d_in] (the query input of each decode row); w_q bf16
 * [H_I*D_I, d_in] (row h*D_I + c holds the weights of head h, channel c);
 * q_idx bf16 [B, H_I, D_I] (output, the layout dsa_indexer_score reads).
 * Products are exact, sums run in float32 in a fixed order, and the result
 * is rounded to nearest even. Requires D_I == 128, 1 <= H_I <= 64 and d_in a
 * multiple of 256 (else DSA_ERROR_NOT_SUPPORTED). No workspace. With H_I = 1
 * and the key weights it gives the new token's indexer key ([B, 1, 128]),
 * which the caller appends to k_idx.
 */
DSA_EXPORT dsa_status_t dsa_indexer_qproj(const void* x, const void* w_q, void* q_idx, int B,
                               int d_in, int H_I, int D_I, void* stream);

/*
 * Top-k selection (CSA pull request, step 3; "DeepSelect" project page):
 * for each of the B rows of `scores` (dtype bf16 or float32, [B, N]) the k
 * positions with the largest value, ties broken by the lower index. -0.0 and
 * +0.0 compare equal; NaN inputs are not allowed (result unspecified).
 *   out_idx  int32 [B, k]: the selected positions. Their order is
 *            unspecified (but deterministic) when sorted_index == 0, and
 *            ascending when sorted_index == 1.
 *   out_val  [B, k] of the input dtype, or NULL: the scores at out_idx,
 *            bit-identical copies of the input.
 * Requires 1 <= k <= N and k <= 4096. ws/ws_bytes: workspace of at least
 * dsa_topk_workspace_bytes(B, N, k, dtype) bytes; its contents on entry do
 * not matter. That size is 0 for rows one workgroup takes whole (then ws may
 * be NULL), else it holds the per-segment candidates.
 */
DSA_EXPORT size_t dsa_topk_workspace_bytes(int B, int N, int k, dsa_dtype_t dtype);
DSA_EXPORT dsa_status_t dsa_topk(const void* scores, dsa_dtype_t dtype, int B, int N, int k,
                      int32_t* out_idx, void* out_val, int sorted_index, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * Indexer scores and top-k in one pass (CSA pull request, "Highlights":
 * indexer and top-k fused in one launch; "The top-k on the GPSIMD engine":
 * the scores are selected chunk by chunk as they are computed, and a final
 * top-k merges the chunks' results). The result is exactly
 * dsa_topk(dsa_indexer_score(...), k) as a set: the k positions with the
 * largest float32 score (the indexer's arithmetic, bit for bit), ties to the
 * lower index. Each row is scored in C interleaved chunks (every run of C
 * consecutive groups of 32 positions holds one group of each chunk, in an
 * order that rotates by one from run to run); each chunk keeps its exact
 * top few and the smallest
 * score it kept, and a merge selects the row's k-th kept candidate T*. When
 * no chunk dropped a candidate at or above T*, the merge's answer is exact;
 * a row where some chunk did (only rows that pile their top scores into few
 * chunks) is selected again, exactly, from its score row.
 *   q_idx bf16 [B, H_I, D_I]; k_idx bf16 [B, N, D_I]; w float [B, H_I] (as
 *   dsa_indexer_score); out_idx int32 [B, k] (output, in an unspecified but
 *   deterministic order); scores float [B, N] (output, as
 *   dsa_indexer_score writes them) or NULL to keep them in the workspace.
 * Requires the shapes of dsa_indexer_score and 1 <= k <= min(N, 4096).
 * ws: dsa_indexer_topk_workspace_bytes(B, N, H_I, k, scores == NULL) bytes;
 * its contents on entry do not matter. Shapes whose chunks would not fit,
 * and rows short enough for dsa_topk's one-workgroup path (N <= 8192), run
 * the indexer and dsa_topk's kernels instead (dsa_indexer_topk_chunks
 * returns 0), with the same result.
 */
DSA_EXPORT size_t dsa_indexer_topk_workspace_bytes(int B, int N, int H_I, int k,
                                                   int own_scores);
DSA_EXPORT dsa_status_t dsa_indexer_topk(const void* q_idx, const void* k_idx, const float* w,
                                         int B, int N, int H_I, int D_I, int k,
                                         int32_t* out_idx, float* scores, void* ws,
                                         size_t ws_bytes, void* stream);
/* The number C of interleaved chunks dsa_indexer_topk splits each row into,
 * or 0 when the shape takes the unfused kernels or is invalid. Row position
 * j lies in group g = j / 32, and group g belongs to chunk (g - g / C) mod C
 * (integer division). */
DSA_EXPORT int dsa_indexer_topk_chunks(int B, int N, int k);

/*
 * Sparse multi-query attention (CSA pull request, step 4, and "The top-k on
 * the GPSIMD engine"): every query head of a batch row attends over the
 * compressed rows the top-k picked followed by the window of recent raw
 * rows; one tensor holds both keys and values:
 *   R_b      = [kv_cmp[b, idx[b,i]] for i < k] followed by [kv_win[b,t] for t < W]
 *   out[b,h] = softmax_r(scale * q[b,h] . R_b[r]) @ R_b
 * q bf16 [B, H_q, D]; kv_cmp bf16 [B, N, D]; idx int32 [B, k] with values in
 * [0, N), or negative for an empty slot that takes no part (a batch row
 * left with no rows at all gets a zero output); values >= N are clamped and
 * the result is then unspecified;
 * kv_win bf16 [B, W, D] (may be NULL iff W == 0); out bf16 [B, H_q, D].
 * Softmax statistics and accumulation run in float32; out is rounded to
 * nearest even. Only dims->batch, n, topk, window, q_heads, head_dim, scale
 * are read. Workspace: dsa_sparse_attend_workspace_bytes(dims) bytes.
 */
DSA_EXPORT size_t dsa_sparse_attend_workspace_bytes(const dsa_dims_t* dims);
DSA_EXPORT dsa_status_t dsa_sparse_attend(const void* q, const void* kv_cmp, const int32_t* idx,
                               const void* kv_win, void* out, const dsa_dims_t* dims,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * The whole decode step: indexer scores -> top-k -> sparse attention, all on
 * `stream` with no host synchronisation; the score rows and the selected
 * indices stay in the workspace (as in the CSA pull request's Summary, where
 * neither returns to the host). Indexer and top-k run as dsa_indexer_topk.
 * Arguments as in the calls above. out_idx int32 [B, k] or NULL: when
 * given, receives the selected positions in the order dsa_indexer_topk
 * gives them. Workspace: dsa_decode_step_workspace_bytes(dims) (enough for
 * the ragged and several-token calls on the same dims too).
 */
DSA_EXPORT size_t dsa_decode_step_workspace_bytes(const dsa_dims_t* dims);
DSA_EXPORT dsa_status_t dsa_decode_step(const void* q_idx, const void* k_idx, const float* w,
                             const void* q, const void* kv_cmp, const void* kv_win,
                             void* out, int32_t* out_idx, const dsa_dims_t* dims,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * Ragged rows. The CSA pull request launches its block with one compressed
 * length T_c for the whole batch ("Launching a full block", with the
 * sequence length a driver option); a serving batch holds sequences of
 * different lengths. These calls take, in addition, lengths: int32 [B] in
 * device memory, row b holding lengths[b] valid positions (a value below 0
 * counts as 0, one above N as N). Positions at or beyond it take no part:
 * they are never selected, whatever their scores.
 *
 * dsa_topk_ragged: as dsa_topk over each row's valid prefix. When
 * lengths[b] < k, out_idx[b] holds the lengths[b] selected positions first
 * (ascending when sorted_index == 1) and -1 in the remaining slots, and
 * out_val (when given) holds negative infinity there. Workspace: as
 * dsa_topk_workspace_bytes(B, N, k, dtype).
 *
 * dsa_decode_step_ragged: the step with the ragged top-k; empty slots (-1)
 * take no part in attention. Workspace: dsa_decode_step_workspace_bytes.
 */
DSA_EXPORT dsa_status_t dsa_topk_ragged(const void* scores, dsa_dtype_t dtype, int B, int N,
                             const int32_t* lengths, int k, int32_t* out_idx,
                             void* out_val, int sorted_index, void* ws, size_t ws_bytes,
                             void* stream);
DSA_EXPORT dsa_status_t dsa_decode_step_ragged(const void* q_idx, const void* k_idx,
                                    const float* w, const void* q, const void* kv_cmp,
                                    const void* kv_win, const int32_t* lengths, void* out,
                                    int32_t* out_idx, const dsa_dims_t* dims, void* ws,
                                    size_t ws_bytes, void* stream);

/*
 * Several query tokens per batch row. Speculative (multi-token) decoding and
 * prompt chunks bring T > 1 query tokens per sequence in one step; the CSA
 * pull request's driver has a phase option (decode or prefill) and its
 * review asks for prefill profiles. Reading: the T tokens of batch row b
 * share its keys (k_idx[b] and kv_cmp[b]); each has its own indexer query
 * and weights, its own score row and selection, its own attention query and
 * window, and its own valid length. Token t of row b is query row b*T + t of
 * every per-token tensor, and is computed exactly as one decode row. The
 * indexer reads each key row once for all T tokens. 1 <= T <= 4.
 *
 * dsa_indexer_score_mt: q_idx bf16 [B, T, H_I, D_I]; k_idx bf16 [B, N, D_I];
 *   w float [B, T, H_I]; scores float [B, T, N]. Shape limits as
 *   dsa_indexer_score, with B*T*N < 2^31.
 * dsa_sparse_attend_mt: q bf16 [B, T, H_q, D]; kv_cmp bf16 [B, N, D]; idx
 *   int32 [B, T, k] (negative: empty slot); kv_win bf16 [B, T, W, D] (may be
 *   NULL iff W == 0); out bf16 [B, T, H_q, D]; dims->batch = B (rows of
 *   kv_cmp), B*T <= 65535. Workspace: dsa_sparse_attend_mt_workspace_bytes.
 * dsa_decode_step_mt: the step over those tensors, with lengths int32 [B, T]
 *   in device memory (token t of row b looks at its first lengths[b*T+t]
 *   positions, as dsa_decode_step_ragged) or NULL for full rows; out_idx
 *   int32 [B, T, k] or NULL. Workspace: dsa_decode_step_mt_workspace_bytes.
 * With T == 1 each call computes exactly what its one-token counterpart does.
 */
DSA_EXPORT dsa_status_t dsa_indexer_score_mt(const void* q_idx, const void* k_idx,
                                  const float* w, float* scores, int B, int T, int N,
                                  int H_I, int D_I, void* stream);
DSA_EXPORT size_t dsa_sparse_attend_mt_workspace_bytes(const dsa_dims_t* dims, int T);
DSA_EXPORT dsa_status_t dsa_sparse_attend_mt(const void* q, const void* kv_cmp,
                                  const int32_t* idx, const void* kv_win, void* out,
                                  const dsa_dims_t* dims, int T, void* ws, size_t ws_bytes,
                                  void* stream);
DSA_EXPORT size_t dsa_decode_step_mt_workspace_bytes(const dsa_dims_t* dims, int T);
DSA_EXPORT dsa_status_t dsa_decode_step_mt(const void* q_idx, const void* k_idx,
                                const float* w, const void* q, const void* kv_cmp,
                                const void* kv_win, const int32_t* lengths, void* out,
                                int32_t* out_idx, const dsa_dims_t* dims, int T, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * Attention sink (CSA pull request, "DMA Traffic Shaping", priority table:
 * the attention sink is one of the attention kernel's inputs; the pages give
 * no formula). Reading: sink float [H_q] holds one logit per query head, in
 * the units of scale * q.k, that takes part in the softmax normalisation
 * and brings no value vector:
 *   M = max(sink[h], max_r z[h,r]),  z[h,r] = scale * q[b,h] . R_b[r]
 *   out[b,h] = sum_r e^(z[h,r] - M) R_b[r] / (e^(sink[h] - M) + sum_r e^(z[h,r] - M))
 * A sink of -inf gives dsa_sparse_attend's result; a batch row with no rows
 * at all still gets zeros. sink must be non-NULL, 4-byte aligned, finite or
 * -inf. Everything else, workspaces included, as dsa_sparse_attend and
 * dsa_decode_step.
 */
DSA_EXPORT dsa_status_t dsa_sparse_attend_sink(const void* q, const void* kv_cmp,
                                    const int32_t* idx, const void* kv_win, const float* sink,
                                    void* out, const dsa_dims_t* dims, void* ws,
                                    size_t ws_bytes, void* stream);
DSA_EXPORT dsa_status_t dsa_decode_step_sink(const void* q_idx, const void* k_idx,
                                  const float* w, const void* q, const void* kv_cmp,
                                  const void* kv_win, const float* sink, void* out,
                                  int32_t* out_idx, const dsa_dims_t* dims, void* ws,
                                  size_t ws_bytes, void* stream);

/*
 * Compressor (CSA pull request, "How the algorithm works", step table, step
 * 1: every 4 raw tokens are folded into one compressed entry by a gated
 * weighted sum; the pages give no formula). Reading: the 4 raw KV rows x_i
 * of a group each get a gate score z_i = sum_d w_gate[d] * x_i[d], and
 *   out[b, g, :] = sum_i softmax(z)_i * x[b, 4g + i, :]
 * x bf16 [B, 4G, D] (group g of batch row b = its raw rows 4g .. 4g+3);
 * w_gate float [D] (the learned gate vector); out bf16 [B, G, D], rounded to
 * nearest even (row g of out is the compressed row the caller appends to
 * kv_cmp). Sums and the softmax run in float32 in a fixed order. D must be a
 * multiple of 8 and at most 1024. No workspace. A decode step calls it with
 * G = 1 every 4 tokens; a prompt with G = its length / 4.
 */
DSA_EXPORT dsa_status_t dsa_compress(const void* x, const float* w_gate, void* out, int B, int G,
                          int D, void* stream);

/*
 * For callers that cannot allocate device memory: code being captured into a
 * HIP graph, tight serving loops, or harnesses that forbid hipMalloc. The
 * same step as dsa_decode_step (same kernels, same results bit for bit), but
 * its workspace is a static device array of DSA_NOALLOC_SCRATCH_BYTES inside
 * the library instead of a caller buffer; the call itself allocates and
 * frees nothing. Each GPU the library runs on holds its own copy of that
 * array from the first call there until the process ends. Every call on one
 * GPU shares that GPU's copy, so calls that may overlap on one GPU (on
 * different streams, or from several host threads) race and must not be
 * issued; calls ordered on one stream are fine. Nothing in the scratch needs
 * to start at zero. A shape whose dsa_decode_step_workspace_bytes exceeds
 * DSA_NOALLOC_SCRATCH_BYTES returns DSA_ERROR_SCRATCH_LIMIT and launches
 * nothing (the production shape, B = 16, N = 32768, k = 1024, H_q = 128,
 * D = 512, needs about 19 MiB). Arguments and other errors as dsa_decode_step.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (64u << 20)
DSA_EXPORT dsa_status_t dsa_decode_step_noalloc(const void* q_idx, const void* k_idx,
                                     const float* w, const void* q, const void* kv_cmp,
                                     const void* kv_win, void* out, int32_t* out_idx,
                                     const dsa_dims_t* dims, void* stream);

/* A static, human-readable name for a status code (never NULL). */
DSA_EXPORT const char* dsa_status_string(dsa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
