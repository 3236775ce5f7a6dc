// Internal declarations shared by the HIP sources of libdsa (gfx950 only).
// Nothing here is part of the C ABI; see include/dsa.h for that.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kWave = 64;

// ---------------------------------------------------------------- keys
// Order-preserving map from an IEEE float32 bit pattern to an unsigned key:
// a larger float gives a larger key. -0.0 is first turned into +0.0 so that
// the two compare equal, as IEEE comparison says.
__device__ __forceinline__ uint32_t f32_key(uint32_t bits) {
  bits = (bits == 0x80000000u) ? 0u : bits;
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

// A 64-bit key that orders candidates the way top-k wants them: the value
// key in the high word, the complemented position in the low word, so a
// larger composite means a larger value or, for equal values, a lower index.
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t pos) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - pos);
}
__device__ __forceinline__ uint32_t composite_pos(uint64_t c) {
  return 0xFFFFFFFFu - (uint32_t)c;
}

// ---------------------------------------------------------------- wave ops
// Cross-lane primitives built on DPP row operations (VALU, a few cycles each)
// and readlane, instead of LDS-routed shuffles. Rows are 16 lanes.
namespace dpp {
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
constexpr int kXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141, kRowMirror = 0x140;
}  // namespace dpp

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_zero(uint32_t v) {  // lanes without a source read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_all(uint32_t v) {  // permutations: every lane has a source
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t lane_read(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
  x += dpp_zero<dpp::kRowShr1>(x);
  x += dpp_zero<dpp::kRowShr2>(x);
  x += dpp_zero<dpp::kRowShr4>(x);
  x += dpp_zero<dpp::kRowShr8>(x);
  x += dpp_zero<dpp::kRowBcast15, 0xA>(x);  // rows 1, 3 add the end of rows 0, 2
  x += dpp_zero<dpp::kRowBcast31, 0xC>(x);  // rows 2, 3 add the end of row 1
  return x;
}

// Reductions over the 64 lanes; the result is wave-uniform.
struct OpAdd { __device__ static uint32_t f(uint32_t a, uint32_t b) { return a + b; } };
struct OpMin { __device__ static uint32_t f(uint32_t a, uint32_t b) { return a < b ? a : b; } };
struct OpMax { __device__ static uint32_t f(uint32_t a, uint32_t b) { return a > b ? a : b; } };
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x) {
  x = Op::f(x, dpp_all<dpp::kXor1>(x));
  x = Op::f(x, dpp_all<dpp::kXor2>(x));
  x = Op::f(x, dpp_all<dpp::kRowHalfMirror>(x));
  x = Op::f(x, dpp_all<dpp::kRowMirror>(x));  // every lane holds its row's result
  return Op::f(Op::f(lane_read(x, 0), lane_read(x, 16)), Op::f(lane_read(x, 32), lane_read(x, 48)));
}
// One count into LDS histogram h at bucket `bin` per lane (kNoBin: none).
// When a whole wave hits one bucket (rows of tied scores), one lane adds 64:
// the wave's 64 atomics to one address would otherwise run one after
// another. Called by every lane of the wave.
constexpr uint32_t kNoBin = 0xFFFFFFFFu;
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t bin) {
  const uint32_t first = __builtin_amdgcn_readfirstlane(bin);
  if (__ballot(bin == first) == ~0ull) {  // uniform
    if ((threadIdx.x & (kWave - 1)) == 0 && first != kNoBin) atomicAdd(&h[first], (uint32_t)kWave);
  } else if (bin != kNoBin) {
    atomicAdd(&h[bin], 1u);
  }
}

__device__ __forceinline__ uint64_t u64_of(uint32_t lo, uint32_t hi) { return ((uint64_t)hi << 32) | lo; }
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_all64(uint64_t v) {
  return u64_of(dpp_all<CTRL>((uint32_t)v), dpp_all<CTRL>((uint32_t)(v >> 32)));
}
template <bool MIN>
__device__ __forceinline__ uint64_t wave_reduce64(uint64_t x) {
  auto f = [](uint64_t a, uint64_t b) { return MIN ? (a < b ? a : b) : (a > b ? a : b); };
  x = f(x, dpp_all64<dpp::kXor1>(x));
  x = f(x, dpp_all64<dpp::kXor2>(x));
  x = f(x, dpp_all64<dpp::kRowHalfMirror>(x));
  x = f(x, dpp_all64<dpp::kRowMirror>(x));
  uint64_t r = u64_of(lane_read((uint32_t)x, 0), lane_read((uint32_t)(x >> 32), 0));
#pragma unroll
  for (int row = 1; row < 4; ++row)
    r = f(r, u64_of(lane_read((uint32_t)x, 16 * row), lane_read((uint32_t)(x >> 32), 16 * row)));
  return r;
}

// The value of lane l ^ 16 (or l ^ 32) through v_permlane16_swap /
// v_permlane32_swap: plain VALU instructions, where __shfl_xor would be a
// ds_bpermute that waits in the LDS queue behind every outstanding LDS read.
// With both operands x, the swap returns (x of the lower lane, x of the
// upper lane) of each pair in every lane of the pair. Blocks are
// one-dimensional, so the lane is threadIdx.x mod 64.
__device__ __forceinline__ float lane_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_bf16. Lane l = 16*g + m supplies A[m][8g..8g+7] and
// B[8g..8g+7][m]; it receives D[4g+i][m] for i < 4.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// float -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two floats -> two bf16 in one word (lo = a), round to nearest even; one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Two floats -> two fp16 in one word (lo = a), round to nearest even; one
// v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
}
__device__ __forceinline__ float2 unpack_f16x2(uint32_t w) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
  return make_float2(v.x, v.y);
}

// ---------------------------------------------------------------- LDS DMA
// Byte address of an LDS location (the M0 value of an LDS DMA).
__device__ __forceinline__ uint32_t lds_byte_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at lds_byte + 16*l (M0 holds the wave-uniform LDS byte address). It
// is issued from inline assembly so that the compiler, which cannot tell
// these LDS writes apart from later LDS reads, does not wait for every
// outstanding copy before each read; the kernel waits with explicit vmcnt
// values instead. No register is written asynchronously. M0 is an input
// operand ("{m0}"), so the compiler writes it and knows it is in use; the
// s_nop gives the one wait state the ISA asks for between an M0 write and an
// LDS-DMA load.
__device__ __forceinline__ void dma_row16(const void* g, uint32_t lds_byte) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(g), "{m0}"(lds_byte) : "memory");
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error. Arguments are already checked.

// tokens (1..kMaxTokens) query tokens per batch row share its keys: q
// [B, tokens, H, 128], w [B, tokens, H], s [B, tokens, N]. lengths: int32
// [B, tokens] in device memory, or NULL for full rows; with it, a token's
// scores at or past its length are not written.
constexpr int kMaxTokens = 4;
hipError_t launch_indexer_score(const uint16_t* q, const uint16_t* k, const float* w,
                                float* s, int B, int N, int H, int tokens,
                                const int32_t* lengths, hipStream_t st);

// The indexer fused with a per-chunk cut of the top-k: chunk c of C
// interleaved chunks of row b (one group of 32 keys out of every C) keeps
// its top scores, between `target` and `keep` of them, as composites in cand
// [B, C, keep], their number in cnt [B, C], and in tcut [B, C] a composite
// that every kept one reaches and every dropped one lies below (0: the
// chunk kept all its scores). The scores are written to s as launch_indexer_score
// writes them.
struct CutPlan {
  bool ok;     // the shape fits the fused path
  int chunks;  // C
  int target;  // a chunk keeps at least this many of its top scores
  int keep;    // and at most this many (its candidate slots)
  int mcap;    // keys of the largest chunk
};
CutPlan plan_cut(int B, int N, int k);
hipError_t launch_indexer_cut(const uint16_t* q, const uint16_t* k, const float* w, float* s,
                              int B, int N, int H, const CutPlan& p, uint64_t* cand,
                              uint32_t* cnt, uint64_t* tcut, hipStream_t st);
// The row merge of the chunk cut: the k largest composites of each row's
// kept candidates, written to out_idx [B, k] when every chunk's cut lies at
// or below the row's k-th kept composite (then the answer is exact); other
// rows are selected again, exactly, from the float32 score rows.
hipError_t launch_topk_cut_merge(const float* scores, int B, int N, int k, const CutPlan& p,
                                 const uint64_t* cand, const uint32_t* cnt, const uint64_t* tcut,
                                 int32_t* out_idx, hipStream_t st);

// Indexer query projection: out bf16 [B, O] = x bf16 [B, d_in] @ w^T, w
// bf16 [O, d_in]; d_in a multiple of 256, O of 32.
hipError_t launch_qproj(const uint16_t* x, const uint16_t* w, uint16_t* out, int B, int d_in,
                        int O, hipStream_t st);

struct TopkPlan {
  bool fused;       // one workgroup per row does everything (no second kernel)
  int segs;         // segments per row
  int seg_len;      // elements per segment (all but the last segment)
  int vec;          // 16-byte vectors per thread per register block (1..16)
  // Full rows (no lengths) split into a power-of-two number of segments may
  // take the quota form: segment s holds the interleaved 128-byte pieces
  // that the rotation assigns it, keeps its `quota` largest scores (about
  // its share of the row's top k) in `slots` slots instead of its own top
  // k, and reports the cut below which it dropped everything; the merge
  // then checks that no cut reaches the row's k-th kept score. 0: off.
  int quota;
  int slots;        // candidate slots per segment in quota form
  size_t cand_off;  // byte offsets inside the workspace
  size_t cnt_off;
  size_t tcut_off;  // per-(row, segment) cuts, quota form only
  size_t bytes;     // total workspace bytes
};
TopkPlan plan_topk(int B, int N, int k, dsa_dtype_t dt);
// lengths: int32 [B] in device memory (row b's valid positions), or NULL
// for full rows.
hipError_t launch_topk(const void* scores, dsa_dtype_t dt, int B, int N, int k,
                       int32_t* out_idx, void* out_val, int sorted_index, const int32_t* lengths,
                       const TopkPlan& plan, void* ws, hipStream_t st);

struct AttendPlan {
  int splits;        // row splits per (batch, head group)
  int rows_per_split; // the most rows any split holds (its row list in LDS)
  int sel_rows;       // selected rows per split (a multiple of 32; the last split may hold fewer)
  int heads_per_wg;  // 16 * waves per workgroup
  size_t part_o_off; // fp16 [B, splits, Hq, D]: O / scale of its dim half
  size_t part_ml_off; // float4 [B, splits, Hq]: (running max, running sum, scale of dims
                      // [0, D/2), scale of dims [D/2, D))
  size_t bytes;
};
AttendPlan plan_attend(const dsa_dims_t& d);
// d.batch counts query rows; tokens consecutive query rows share one row of
// kv (kv holds d.batch / tokens rows).
// sink: float [q_heads] (one logit per query head, joining the softmax
// normalisation with no value vector), or NULL for none.
hipError_t launch_attend(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                         const uint16_t* win, uint16_t* out, const float* sink,
                         const dsa_dims_t& d, const AttendPlan& plan, int tokens, void* ws,
                         hipStream_t st);

// The chunk cut's candidates of the fused step, for an attention kernel that
// selects its own rows (SEL > 0): per batch row, C lists of keep composites
// with their counts and cuts (as the cut merge reads them), the score rows
// for a row the cut cannot vouch for, and where the selection goes.
struct SelectArgs {
  const uint64_t* cand;  // [B, C, keep]
  const uint32_t* cnt;   // [B, C]
  const uint64_t* tcut;  // [B, C]
  const float* scores;   // [B, N]
  int32_t* idx_out;      // [B, k], written by the split-0, head-group-0 workgroup of each row
  int chunks, keep;
};
// The attention kernel selecting its own rows (the cut merge folded in):
// the candidate slots per thread it takes for this shape (4 or 8), or 0
// when the shape has no such kernel (D = 512 with 64 heads per workgroup
// and at most 4096 candidates per row only).
int attend_select_per(const dsa_dims_t& d, const AttendPlan& p, int chunks, int keep);
// Attention whose workgroups select their rows from the chunk cut's
// candidates (sel), then the combine; the selection goes to sel.idx_out.
hipError_t launch_attend_select(const uint16_t* q, const uint16_t* kv, const uint16_t* win,
                                uint16_t* out, const float* sink, const dsa_dims_t& d,
                                const AttendPlan& p, const SelectArgs& sel, int per, void* ws,
                                hipStream_t st);


// Compressor: out bf16 [groups, D] from x bf16 [groups, 4, D] and the gate
// vector wg float [D]; D a multiple of 8, at most 1024.
hipError_t launch_compress(const uint16_t* x, const float* wg, uint16_t* out, int groups, int D,
                           hipStream_t st);

}  // namespace dsa
