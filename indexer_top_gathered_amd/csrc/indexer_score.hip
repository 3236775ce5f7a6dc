// Lightning-indexer scoring on gfx950 ("feat: Add DeepSeek-V4 CSA attention
// kernels", section "How the algorithm works", step 2: a multi-query product
// of the indexer query with every compressed key, a ReLU and a per-head
// weight, summed over heads).
//
//   s[b,j] = sum_h w[b,h] * max(0, q[b,h,:] . k[b,j,:]),   D_I = 128
//
// Per batch row this is a [H x 128] x [128 x N] product followed by a
// weighted ReLU reduction over H, so it is streamed as MFMA tiles with the
// heads as the M dimension and 16 keys as the N dimension. The key rows are
// read straight from HBM into the B operand: lane 16g+m loads 16 contiguous
// bytes of key m at channel 32*kk + 8g, so four lanes cover 64 contiguous
// bytes of a row per instruction and every byte of k is read exactly once.
// The query fragments and weights stay in registers for the whole sweep.
// Each lane ends with four heads of one key; the head sum finishes with two
// cross-lane steps. Summation order is fixed, so results are deterministic.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kIsWaves = 4;
constexpr int kIsThreads = kIsWaves * kWave;
constexpr int kIsTiles = 2;                       // 16-key tiles per wave step
constexpr int kIsKeysPerStep = 16 * kIsTiles;     // keys per wave per step
constexpr int kIsKeysPerRound = kIsWaves * kIsKeysPerStep;  // 128 per workgroup round
constexpr int kDI = 128;

template <int MT>  // MT = number of 16-head tiles (1..4)
__global__ __launch_bounds__(kIsThreads) void indexer_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ w, float* __restrict__ s, int N, int H, int keys_per_wg) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int m = lane & 15;
  const int g = lane >> 4;

  // A operand: query fragments, head (16*mt + m), channels 32*kk + 8g .. +8.
  bf16x8 qa[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int head = mt * 16 + m;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (head < H) {
        qa[mt][kk] = *reinterpret_cast<const bf16x8*>(q + ((size_t)b * H + head) * kDI + kk * 32 + g * 8);
      } else {
        qa[mt][kk] = bf16x8{};
      }
    }
  }
  // Weights of the heads this lane's accumulators hold: 16*mt + 4g + i.
  float wv[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = mt * 16 + g * 4 + i;
      wv[mt][i] = head < H ? w[(size_t)b * H + head] : 0.0f;
    }

  const uint16_t* krow = k + (size_t)b * N * kDI;
  float* srow = s + (size_t)b * N;
  const int start = blockIdx.x * keys_per_wg;
  const int end = min(N, start + keys_per_wg);

  // Key fragments of one wave step: lane 16g+m holds key (key0 + 16t + m),
  // channels 32*kk + 8g .. +8. Keys past N are clamped to N-1 (their columns
  // are computed and never stored), so every load is unconditional.
  auto load_keys = [&](bf16x8 (&kb)[kIsTiles][4], int key0) {
#pragma unroll
    for (int t = 0; t < kIsTiles; ++t) {
      const int key = min(key0 + t * 16 + m, N - 1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kb[t][kk] = __builtin_nontemporal_load(
            reinterpret_cast<const bf16x8*>(krow + (size_t)key * kDI + kk * 32 + g * 8));
    }
  };
  auto score_step = [&](const bf16x8 (&kb)[kIsTiles][4], int key0) {
    f32x4 acc[kIsTiles][MT];
#pragma unroll
    for (int t = 0; t < kIsTiles; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int t = 0; t < kIsTiles; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = mfma16x16x32(qa[mt][kk], kb[t][kk], acc[t][mt]);

    // Weighted ReLU over this lane's heads, per key tile.
    float p[kIsTiles];
#pragma unroll
    for (int t = 0; t < kIsTiles; ++t) {
      float sum = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum += wv[mt][i] * fmaxf(acc[t][mt][i], 0.0f);
      p[t] = sum;
    }
    // Sum over the four lane groups. Lanes with even g keep tile 0, odd g
    // keep tile 1: one exchange with g^1 hands over the other tile, one with
    // g^2 completes the sum.
    float mine = (g & 1) ? p[1] : p[0];
    const float other = (g & 1) ? p[0] : p[1];
    mine += __shfl_xor(other, 16);
    mine += __shfl_xor(mine, 32);
    if (g < 2) {
      const int key = key0 + g * 16 + m;
      if (key < N) srow[key] = mine;
    }
  };

  // Two key buffers in turn: the loads of the next step are in flight while
  // this step is computed. Each load sits on a path where the compiler can
  // see exactly which loads are outstanding, so a step waits only for its
  // own buffer.
  bf16x8 ka[kIsTiles][4], kb[kIsTiles][4];
  int key0 = start + wave * kIsKeysPerStep;
  if (key0 < end) {
    load_keys(ka, key0);
    while (true) {
      if (key0 + kIsKeysPerRound >= end) {
        score_step(ka, key0);
        break;
      }
      load_keys(kb, key0 + kIsKeysPerRound);
      score_step(ka, key0);
      key0 += kIsKeysPerRound;
      if (key0 + kIsKeysPerRound >= end) {
        score_step(kb, key0);
        break;
      }
      load_keys(ka, key0 + kIsKeysPerRound);
      score_step(kb, key0);
      key0 += kIsKeysPerRound;
    }
  }
}

}  // namespace

hipError_t launch_indexer_score(const uint16_t* q, const uint16_t* k, const float* w,
                                float* s, int B, int N, int H, hipStream_t st) {
  // Each wave keeps its query fragments (up to 16 KB per batch row) in
  // registers for its whole sweep. Aim for one round of about 256 workgroups
  // (one per CU measured fastest), each sweeping at least 8 and at most 32
  // rounds of 128 keys so the query loads stay small next to the key stream.
  const long long per_row_rounds = (N + kIsKeysPerRound - 1) / kIsKeysPerRound;
  long long rounds = ((long long)B * per_row_rounds + 255) / 256;
  if (rounds < 8) rounds = 8;
  if (rounds > 32) rounds = 32;
  if (rounds > per_row_rounds) rounds = per_row_rounds;
  if (rounds < 1) rounds = 1;
  const int keys_per_wg = (int)rounds * kIsKeysPerRound;
  dim3 grid((N + keys_per_wg - 1) / keys_per_wg, B);
  dim3 block(kIsThreads);
  const int mt = (H + 15) / 16;
  switch (mt) {
    case 1: hipLaunchKernelGGL(indexer_score_kernel<1>, grid, block, 0, st, q, k, w, s, N, H, keys_per_wg); break;
    case 2: hipLaunchKernelGGL(indexer_score_kernel<2>, grid, block, 0, st, q, k, w, s, N, H, keys_per_wg); break;
    case 3: hipLaunchKernelGGL(indexer_score_kernel<3>, grid, block, 0, st, q, k, w, s, N, H, keys_per_wg); break;
    default: hipLaunchKernelGGL(indexer_score_kernel<4>, grid, block, 0, st, q, k, w, s, N, H, keys_per_wg); break;
  }
  return hipGetLastError();
}

}  // namespace dsa
