// Lightning-indexer scoring on gfx950 ("feat: Add DeepSeek-V4 CSA attention
// kernels", section "How the algorithm works", step 2: a multi-query product
// of the indexer query with every compressed key, a ReLU and a per-head
// weight, summed over heads).
//
//   s[b,j] = sum_h w[b,h] * max(0, q[b,h,:] . k[b,j,:]),   D_I = 128
//
// Per batch row this is a [H x 128] x [128 x N] product followed by a
// weighted ReLU reduction over H, so it is streamed as MFMA tiles with the
// heads as the M dimension and 16 keys as the N dimension. An MFMA B operand
// wants 16 different keys per 16 lanes (64 bytes of each per instruction);
// loaded that way a key row costs twice the cache-line requests of a
// contiguous read, which bounds the load rate. So keys are loaded in whole
// 1 KB runs (4 keys per instruction; three register buffers per wave, two
// steps in flight while one is computed), written
// to a per-wave LDS area with each key's 16-byte chunks XOR-swizzled by the
// key index, and read back in MFMA layout without bank conflicts. Every byte
// of k is read from HBM exactly once. The query fragments and weights stay
// in registers for the whole sweep. Each lane ends with four heads of one
// key; the head sum finishes with two cross-lane steps. Summation order is
// fixed, so results are deterministic.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kIsWaves = 8;
constexpr int kIsThreads = kIsWaves * kWave;
constexpr int kIsTiles = 2;                       // 16-key tiles per wave step
constexpr int kIsKeysPerStep = 16 * kIsTiles;     // keys per wave per step
constexpr int kIsKeysPerRound = kIsWaves * kIsKeysPerStep;  // 256 per workgroup round
constexpr int kDI = 128;

// One workgroup's sweep over keys [start, end) of batch row b: start is a
// multiple of 256 keys, end at most the row's valid length. st: this wave's
// 8 KB LDS staging area.
template <int MT>  // MT = number of 16-head tiles (1..4)
__device__ __forceinline__ void sweep_row(const uint16_t* __restrict__ q,
                                          const uint16_t* __restrict__ k,
                                          const float* __restrict__ w, float* __restrict__ s,
                                          int b, int N, int H, int start, int end, u32x4* st) {
  // The thread index passes through an empty asm statement, so that the
  // values derived from it are formed per call: a caller that sweeps
  // several rows in a loop does not keep them live across its iterations.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
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

  // Keys are loaded with whole 1 KB runs per instruction (4 keys x 256 B,
  // lane l: key 4j + l/16, 16-byte chunk l%16), then written to this wave's
  // LDS area with the chunk of key q at slot (chunk ^ q%16), so that the MFMA
  // fragment reads (16 different keys, one chunk) hit 16 different slots.
  auto load_step = [&](u32x4 (&r)[8], int key0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = min(key0 + 4 * j + (lane >> 4), end - 1);
      r[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(krow + (size_t)key * kDI) + (lane & 15));
    }
  };
  auto score_step = [&](const u32x4 (&r)[8], int key0) {
    // stage: key q = 4j + lane/16, chunk c = lane%16 -> slot q*16 + (c ^ (q & 15))
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = 4 * j + (lane >> 4);
      st[q * 16 + ((lane & 15) ^ (q & 15))] = r[j];
    }
    bf16x8 kb[kIsTiles][4];
#pragma unroll
    for (int t = 0; t < kIsTiles; ++t)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int q = 16 * t + m;
        kb[t][kk] = __builtin_bit_cast(bf16x8, st[q * 16 + ((4 * kk + g) ^ m)]);
      }
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
    float mine = (g & 1) ? p[1] : p[0];
    const float other = (g & 1) ? p[0] : p[1];
    mine += lane_xor16(other);
    mine += lane_xor32(mine);
    if (g < 2) {
      const int key = key0 + g * 16 + m;
      if (key < end) srow[key] = mine;
    }
  };
  // Three register buffers in turn: two steps of loads in flight while one
  // step is staged and computed.
  u32x4 ra[8], rb[8], rc[8];
  int key0 = start + wave * kIsKeysPerStep;
  const int nsteps = key0 < end ? (end - key0 + kIsKeysPerRound - 1) / kIsKeysPerRound : 0;
  if (nsteps > 0) load_step(ra, key0);
  if (nsteps > 1) load_step(rb, key0 + kIsKeysPerRound);
  for (int i = 0; i < nsteps; i += 3) {
    if (i + 2 < nsteps) load_step(rc, key0 + (i + 2) * kIsKeysPerRound);
    score_step(ra, key0 + i * kIsKeysPerRound);
    if (i + 1 >= nsteps) break;
    if (i + 3 < nsteps) load_step(ra, key0 + (i + 3) * kIsKeysPerRound);
    score_step(rb, key0 + (i + 1) * kIsKeysPerRound);
    if (i + 2 >= nsteps) break;
    if (i + 4 < nsteps) load_step(rb, key0 + (i + 4) * kIsKeysPerRound);
    score_step(rc, key0 + (i + 2) * kIsKeysPerRound);
  }
}

template <int MT>
__global__ __launch_bounds__(kIsThreads) void indexer_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ w, float* __restrict__ s, int N, int H, int keys_per_wg) {
  __shared__ u32x4 stage_lds[kIsWaves][32 * 16];  // 8 KB per wave: 32 keys x 16 chunks
  const int b = blockIdx.y;
  const int start = blockIdx.x * keys_per_wg;
  const int end = min(N, start + keys_per_wg);
  sweep_row<MT>(q, k, w, s, b, N, H, start, end, stage_lds[threadIdx.x / kWave]);
}

// Ragged rows (lengths given): keys at or past a row's length are neither
// read nor scored. The rounds of 256 keys that hold valid keys, taken over
// all rows in order, are split evenly over the workgroups, so every
// workgroup streams about the same number of valid keys whatever the mix of
// lengths; a workgroup's share may span rows, and it loads the query
// fragments of each row it enters.
__device__ __forceinline__ uint32_t valid_rounds(const int32_t* lengths, int b, int N) {
  const int len = min(max(lengths[b], 0), N);
  return (uint32_t)((len + kIsKeysPerRound - 1) / kIsKeysPerRound);
}

template <int MT>
__global__ __launch_bounds__(kIsThreads) void indexer_score_ragged_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ w, float* __restrict__ s, int B, int N, int H,
    const int32_t* __restrict__ lengths) {
  __shared__ u32x4 stage_lds[kIsWaves][32 * 16];
  const int lane = threadIdx.x & (kWave - 1);
  // Every wave derives the same split: all rows' valid rounds, then this
  // workgroup's range [lo, hi) of them.
  uint32_t total = 0;
  for (int b0 = 0; b0 < B; b0 += kWave) {
    const uint32_t r = b0 + lane < B ? valid_rounds(lengths, b0 + lane, N) : 0u;
    total += wave_reduce<OpAdd>(r);
  }
  const uint32_t lo = (uint32_t)((uint64_t)blockIdx.x * total / gridDim.x);
  const uint32_t hi = (uint32_t)((uint64_t)(blockIdx.x + 1) * total / gridDim.x);
  if (lo >= hi) return;  // uniform
  // Walk this range a row at a time. Only wave-uniform values (the next
  // round, and the first row and cumulative rounds of the current chunk of
  // 64 rows) live across a row's sweep.
  uint32_t cur = lo;
  int b0 = 0;
  uint32_t base = 0;
  while (cur < hi && b0 < B) {
    const uint32_t r = b0 + lane < B ? valid_rounds(lengths, b0 + lane, N) : 0u;
    const uint32_t incl = base + wave_scan_incl(r);
    const uint64_t past = __ballot(incl <= cur);  // rows wholly before cur
    if (past == ~0ull) {  // cur lies beyond this chunk
      base = lane_read(incl, kWave - 1);
      b0 += kWave;
      continue;
    }
    const int j = __builtin_ctzll(~past);  // the row holding round cur
    const uint32_t e0 = lane_read(incl - r, j), e1 = lane_read(incl, j);
    const int b = b0 + j;
    const int len = min(max(lengths[b], 0), N);
    const int start = (int)((cur - e0) * kIsKeysPerRound);
    const int end = min(len, (int)((min(hi, e1) - e0) * kIsKeysPerRound));
    sweep_row<MT>(q, k, w, s, b, N, H, start, end, stage_lds[threadIdx.x / kWave]);
    cur = min(hi, e1);
  }
}

// Several query tokens per batch row (draft tokens, or a chunk of a prompt)
// share the row's keys. The workgroup streams and stages each key step once,
// exactly as above, and scores it for every token in turn, so the keys are
// read from HBM once for all the tokens. Registers hold one token's query
// fragments, so all the tokens' query rows and weights are staged in LDS at
// the start (rows padded to 272 B: the 16 lanes of a fragment read land on
// different banks) and each token's are read back once per pair of steps.
// Per token the arithmetic and its order are those of the one-token kernel.
constexpr int kQPitch = kDI * 2 + 16;  // bytes per staged query row

template <int MT>
__global__ __launch_bounds__(kIsThreads) void indexer_score_mt_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ w, float* __restrict__ s, int N, int H, int T, int keys_per_wg,
    const int32_t* __restrict__ lengths) {
  extern __shared__ u32x4 lds_mt[];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int m = lane & 15;
  const int g = lane >> 4;

  // Each token's valid length; the keys swept are those of the longest.
  int tlen[kMaxTokens];
  int rmax = 0;
#pragma unroll
  for (int t = 0; t < kMaxTokens; ++t) {
    tlen[t] = t < T ? (lengths ? min(max(lengths[b * T + t], 0), N) : N) : 0;
    rmax = max(rmax, tlen[t]);
  }
  const int start = blockIdx.x * keys_per_wg;
  if (start >= rmax) return;  // uniform
  const int end = min(rmax, start + keys_per_wg);

  // LDS: the 8 waves' key stages (8 KB each), then the query rows of all
  // tokens (T x MT*16 rows of kQPitch bytes, zero past H), then the weights.
  constexpr int kRowsPerToken = MT * 16;
  u32x4* st = lds_mt + wave * (32 * 16);
  char* qs = reinterpret_cast<char*>(lds_mt + kIsWaves * 32 * 16);
  float* wl = reinterpret_cast<float*>(qs + (size_t)T * kRowsPerToken * kQPitch);
  for (int c = threadIdx.x; c < T * kRowsPerToken * 16; c += kIsThreads) {
    const int row = c >> 4, chunk = c & 15;
    const int t = row / kRowsPerToken, head = row % kRowsPerToken;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (head < H)
      v = *reinterpret_cast<const u32x4*>(q + (((size_t)b * T + t) * H + head) * kDI + chunk * 8);
    *reinterpret_cast<u32x4*>(qs + (size_t)row * kQPitch + chunk * 16) = v;
  }
  for (int i = threadIdx.x; i < T * kRowsPerToken; i += kIsThreads) {
    const int t = i / kRowsPerToken, head = i % kRowsPerToken;
    wl[i] = head < H ? w[((size_t)b * T + t) * H + head] : 0.0f;
  }
  __syncthreads();

  const uint16_t* krow = k + (size_t)b * N * kDI;
  auto load_step = [&](u32x4 (&r)[8], int key0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = min(key0 + 4 * j + (lane >> 4), end - 1);
      r[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(krow + (size_t)key * kDI) + (lane & 15));
    }
  };
  // Steps are scored in pairs: the two steps' key fragments stay in
  // registers, so each token's query fragments are read from LDS once per
  // 64 keys and feed 16 MFMAs each.
  auto stage_read = [&](const u32x4 (&r)[8], bf16x8 (&kb)[kIsTiles][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int qk = 4 * j + (lane >> 4);
      st[qk * 16 + ((lane & 15) ^ (qk & 15))] = r[j];
    }
#pragma unroll
    for (int tt = 0; tt < kIsTiles; ++tt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int qk = 16 * tt + m;
        kb[tt][kk] = __builtin_bit_cast(bf16x8, st[qk * 16 + ((4 * kk + g) ^ m)]);
      }
  };
  auto score_pair = [&](const bf16x8 (&ka)[kIsTiles][4], const bf16x8 (&kc)[kIsTiles][4], int key0,
                        bool two) __attribute__((always_inline)) {
    for (int t = 0; t < T; ++t) {
      const char* qt = qs + (size_t)t * kRowsPerToken * kQPitch;
      float p[2 * kIsTiles] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        bf16x8 qa[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          qa[kk] = *reinterpret_cast<const bf16x8*>(qt + (size_t)(mt * 16 + m) * kQPitch + kk * 64 + g * 16);
        f32x4 acc[2 * kIsTiles];
#pragma unroll
        for (int u = 0; u < 2 * kIsTiles; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int tt = 0; tt < kIsTiles; ++tt) {
            acc[tt] = mfma16x16x32(qa[kk], ka[tt][kk], acc[tt]);
            acc[kIsTiles + tt] = mfma16x16x32(qa[kk], kc[tt][kk], acc[kIsTiles + tt]);
          }
        const float4 wq = *reinterpret_cast<const float4*>(wl + t * kRowsPerToken + mt * 16 + g * 4);
        const float wv[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
        for (int u = 0; u < 2 * kIsTiles; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[u] += wv[i] * fmaxf(acc[u][i], 0.0f);
      }
      int tl = tlen[0];
#pragma unroll
      for (int u = 1; u < kMaxTokens; ++u) tl = t == u ? tlen[u] : tl;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float mine = (g & 1) ? p[2 * h + 1] : p[2 * h];
        const float other = (g & 1) ? p[2 * h] : p[2 * h + 1];
        mine += lane_xor16(other);
        mine += lane_xor32(mine);
        if (g < 2 && (h == 0 || two)) {
          const int key = key0 + h * kIsKeysPerRound + g * 16 + m;
          if (key < tl) s[((size_t)b * T + t) * N + key] = mine;
        }
      }
    }
  };
  // Two register buffers: a pair's loads are issued as soon as the previous
  // pair is staged, and land while that pair is scored.
  u32x4 ra[8], rb[8];
  bf16x8 ka[kIsTiles][4], kc[kIsTiles][4];
  int key0 = start + wave * kIsKeysPerStep;
  const int nsteps = key0 < end ? (end - key0 + kIsKeysPerRound - 1) / kIsKeysPerRound : 0;
  if (nsteps > 0) load_step(ra, key0);
  if (nsteps > 1) load_step(rb, key0 + kIsKeysPerRound);
  for (int i = 0; i < nsteps; i += 2) {
    const bool two = i + 1 < nsteps;
    stage_read(ra, ka);
    if (two) stage_read(rb, kc);
    if (i + 2 < nsteps) load_step(ra, key0 + (i + 2) * kIsKeysPerRound);
    if (i + 3 < nsteps) load_step(rb, key0 + (i + 3) * kIsKeysPerRound);
    score_pair(ka, kc, key0 + i * kIsKeysPerRound, two);
  }
}

template <int MT>
hipError_t launch_mt(const uint16_t* q, const uint16_t* k, const float* w, float* s, int N, int H,
                     int T, int keys_per_wg, const int32_t* lengths, dim3 grid, hipStream_t st) {
  const size_t lds = (size_t)kIsWaves * 32 * 16 * sizeof(u32x4) +
                     (size_t)T * MT * 16 * (kQPitch + sizeof(float));
  auto kern = indexer_score_mt_kernel<MT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(kIsThreads), lds, st, q, k, w, s, N, H, T, keys_per_wg,
                     lengths);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_score(const uint16_t* q, const uint16_t* k, const float* w,
                                float* s, int B, int N, int H, int tokens,
                                const int32_t* lengths, hipStream_t st) {
  // Each wave keeps its query fragments (up to 16 KB per batch row) in
  // registers for its whole sweep. Aim for one round of about 256 workgroups
  // (one per CU measured fastest), each sweeping at most 32 rounds of 256
  // keys; large calls take at least 8 rounds per workgroup so the query
  // loads stay small next to the key stream, while small calls (fewer than
  // 256 * 8 rounds in all) spread over as many workgroups as they can fill.
  const long long per_row_rounds = (N + kIsKeysPerRound - 1) / kIsKeysPerRound;
  const long long total_rounds = (long long)B * per_row_rounds;
  long long rounds = (total_rounds + 255) / 256;
  if (rounds < 8 && total_rounds >= 256 * 8) rounds = 8;
  if (rounds > 32) rounds = 32;
  if (rounds > per_row_rounds) rounds = per_row_rounds;
  if (rounds < 1) rounds = 1;
  const int keys_per_wg = (int)rounds * kIsKeysPerRound;
  dim3 grid((N + keys_per_wg - 1) / keys_per_wg, B);
  dim3 block(kIsThreads);
  const int mt = (H + 15) / 16;
  if (tokens > 1) {
    switch (mt) {
      case 1: return launch_mt<1>(q, k, w, s, N, H, tokens, keys_per_wg, lengths, grid, st);
      case 2: return launch_mt<2>(q, k, w, s, N, H, tokens, keys_per_wg, lengths, grid, st);
      case 3: return launch_mt<3>(q, k, w, s, N, H, tokens, keys_per_wg, lengths, grid, st);
      default: return launch_mt<4>(q, k, w, s, N, H, tokens, keys_per_wg, lengths, grid, st);
    }
  }
  if (lengths) {
    // One workgroup per CU (fewer when the rows hold fewer rounds in all),
    // each taking an equal share of the valid rounds.
    const dim3 rgrid((unsigned)(total_rounds < 256 ? total_rounds : 256));
    switch (mt) {
      case 1: hipLaunchKernelGGL(indexer_score_ragged_kernel<1>, rgrid, block, 0, st, q, k, w, s, B, N, H, lengths); break;
      case 2: hipLaunchKernelGGL(indexer_score_ragged_kernel<2>, rgrid, block, 0, st, q, k, w, s, B, N, H, lengths); break;
      case 3: hipLaunchKernelGGL(indexer_score_ragged_kernel<3>, rgrid, block, 0, st, q, k, w, s, B, N, H, lengths); break;
      default: hipLaunchKernelGGL(indexer_score_ragged_kernel<4>, rgrid, block, 0, st, q, k, w, s, B, N, H, lengths); break;
    }
    return hipGetLastError();
  }
  switch (mt) {
    case 1: hipLaunchKernelGGL(indexer_score_kernel<1>, grid, block, 0, st, q, k, w, s, N, H, keys_per_wg); break;
    case 2: hipLaunchKernelGGL(indexer_score_kernel<2>, grid, block, 0, st, q, k, w, s, N, H, keys_per_wg); break;
    case 3: hipLaunchKernelGGL(indexer_score_kernel<3>, grid, block, 0, st, q, k, w, s, N, H, keys_per_wg); break;
    default: hipLaunchKernelGGL(indexer_score_kernel<4>, grid, block, 0, st, q, k, w, s, N, H, keys_per_wg); break;
  }
  return hipGetLastError();
}

}  // namespace dsa
