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

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error. Arguments are already checked.

hipError_t launch_indexer_score(const uint16_t* q, const uint16_t* k, const float* w,
                                float* s, int B, int N, int H, hipStream_t st);

struct TopkPlan {
  int segs;         // segments per row
  int seg_len;      // elements per segment (all but the last segment)
  size_t cand_off;  // byte offsets inside the workspace
  size_t cnt_off;
  size_t bytes;     // total workspace bytes
};
TopkPlan plan_topk(int B, int N, int k, dsa_dtype_t dt);
hipError_t launch_topk(const void* scores, dsa_dtype_t dt, int B, int N, int k,
                       int32_t* out_idx, void* out_val, int sorted_index,
                       const TopkPlan& plan, void* ws, hipStream_t st);

struct AttendPlan {
  int splits;        // row splits per (batch, head group)
  int rows_per_split;
  int heads_per_wg;  // 16 * waves per workgroup
  size_t part_o_off; // float [B, splits, Hq, D]
  size_t part_ml_off; // float2 [B, splits, Hq] (running max, running sum)
  size_t bytes;
};
AttendPlan plan_attend(const dsa_dims_t& d);
hipError_t launch_attend(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                         const uint16_t* win, uint16_t* out, const dsa_dims_t& d,
                         const AttendPlan& plan, void* ws, hipStream_t st);

}  // namespace dsa
