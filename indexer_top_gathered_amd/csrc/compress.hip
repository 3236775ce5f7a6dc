// Compressor on gfx950 ("feat: Add DeepSeek-V4 CSA attention kernels", "How
// the algorithm works", step table, step 1: every 4 raw tokens become one
// compressed entry through a gated weighted sum). Reading: each raw KV row
// x_i of a group of 4 gets a gate score z_i = wg . x_i, the softmax of the
// four scores weights the rows, and the compressed row is the weighted sum
//   out[d] = sum_i softmax(z)_i * x_i[d]      (bf16, rounded to nearest even)
//
// The work is a few KB per group and bandwidth-bound, so one wave takes one
// group: each lane loads 16-byte chunks (8 dims) of the four rows and of
// the gate, the four dot products are summed over the wave by a fixed
// butterfly (lane 0's sums are taken, so the result does not depend on the
// lane), the softmax runs in float32 and the weighted sum is formed with the
// rows still in registers.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kCmpWaves = 4;  // groups per workgroup

// Sum over the 64 lanes in a fixed order; every lane gets lane 0's total.
__device__ __forceinline__ float wave_sum_f32(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// CH: 16-byte chunks of a row per lane (D <= 512 * CH).
template <int CH>
__global__ __launch_bounds__(kCmpWaves * kWave) void compress_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wg, uint16_t* __restrict__ out,
    int groups, int D) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gid = blockIdx.x * kCmpWaves + (int)threadIdx.x / kWave;
  if (gid >= groups) return;  // uniform per wave
  const uint16_t* rows = x + (size_t)gid * 4 * D;
  const int nchunks = D / 8;
  u32x4 v[CH][4];
  float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = lane + c * kWave;
    if (ch < nchunks) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[c][i] = *reinterpret_cast<const u32x4*>(rows + (size_t)i * D + ch * 8);
      const float4 w0 = *reinterpret_cast<const float4*>(wg + ch * 8);
      const float4 w1 = *reinterpret_cast<const float4*>(wg + ch * 8 + 4);
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t word = v[c][i][j >> 1];
          const float xv = bf16_bits_to_f32((uint16_t)((j & 1) ? (word >> 16) : (word & 0xFFFFu)));
          z[i] = fmaf(wv[j], xv, z[i]);
        }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[c][i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = wave_sum_f32(z[i]);
  const float zm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
  float a[4], l = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __expf(z[i] - zm);
    l += a[i];
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] *= inv;
  uint16_t* orow = out + (size_t)gid * D;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = lane + c * kWave;
    if (ch < nchunks) {
      u32x4 r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float acc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float s = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t word = v[c][i][q];
            s = fmaf(a[i], bf16_bits_to_f32((uint16_t)(h ? (word >> 16) : (word & 0xFFFFu))), s);
          }
          acc[h] = s;
        }
        r[q] = pack_bf16x2(acc[0], acc[1]);
      }
      *reinterpret_cast<u32x4*>(orow + ch * 8) = r;
    }
  }
}

}  // namespace

hipError_t launch_compress(const uint16_t* x, const float* wg, uint16_t* out, int groups, int D,
                           hipStream_t st) {
  const dim3 grid((unsigned)((groups + kCmpWaves - 1) / kCmpWaves));
  const dim3 block(kCmpWaves * kWave);
  if (D <= 512)
    hipLaunchKernelGGL(compress_kernel<1>, grid, block, 0, st, x, wg, out, groups, D);
  else
    hipLaunchKernelGGL(compress_kernel<2>, grid, block, 0, st, x, wg, out, groups, D);
  return hipGetLastError();
}

}  // namespace dsa
