// Lightning-indexer scoring on gfx950 ("feat: Add DeepSeek-V4 CSA attention
// kernels", section "How the algorithm works", step 2). Every indexer head's
// query is dotted with each compressed key; negative dot products are
// clipped to zero, each head's result is scaled by that head's weight, and
// the heads are added up.
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
#include <cmath>

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kIsWaves = 8;
constexpr int kIsThreads = kIsWaves * kWave;
constexpr int kIsTiles = 2;                       // 16-key tiles per wave step
constexpr int kIsKeysPerStep = 16 * kIsTiles;     // keys per wave per step
constexpr int kIsKeysPerRound = kIsWaves * kIsKeysPerStep;  // 256 per workgroup round
constexpr int kDI = 128;

// Interleaved chunks of a row: its groups of 32 keys are taken C at a time
// (super-group L holds groups L*C .. L*C + C-1) and chunk c gets group
// L*C + (c + L) mod C of each, so every chunk samples the whole row evenly
// (a rising row gives every chunk the same share of its top k), and one
// chunk's consecutive groups are never a power-of-two stride apart (which
// measured 1.5 us slower on the production shape: the loads of a workgroup
// then pile onto few memory channels).
__device__ __forceinline__ int chunk_group(int c, int C, int L) { return L * C + (c + L) % C; }
__device__ __forceinline__ int chunk_group_count(int c, int C, int groups) {
  const int full = groups / C, rem = groups % C;
  return full + ((c + full) % C < rem ? 1 : 0);
}

// One workgroup's sweep over keys [start, end) of batch row b: start is a
// multiple of 256 keys, end at most the row's valid length. st: this wave's
// 8 KB LDS staging area.
//
// CUT sweeps take chunk c of C interleaved chunks of the row instead (one
// group of 32 keys per wave step; start is unused, end is N). Each score's
// order key also goes to keep[local index] in LDS (local index = 32 * (the
// group's rank in the chunk) + offset; 0 for a position past N), for the
// cut that follows the sweep.
template <int MT, bool CUT = false>  // MT = number of 16-head tiles (1..4)
__device__ __forceinline__ void sweep_row(const uint16_t* __restrict__ q,
                                          const uint16_t* __restrict__ k,
                                          const float* __restrict__ w, float* __restrict__ s,
                                          int b, int N, int H, int start, int end, u32x4* st,
                                          int c = 0, int C = 1, uint32_t* keep = nullptr,
                                          uint32_t* key_lo = nullptr, uint32_t* key_hi = nullptr) {
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
  // CUT: the smallest and largest order key this lane wrote to keep[].
  uint32_t klo = 0xFFFFFFFFu, khi = 0u;

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
  auto score_step = [&](const u32x4 (&r)[8], int key0, int local0) {
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
      if constexpr (CUT) {
        const uint32_t kx = f32_key(__float_as_uint(mine));
        keep[local0 + g * 16 + m] = key < end ? kx : 0u;
        if (key < end) {
          klo = min(klo, kx);
          khi = max(khi, kx);
        }
      }
    }
  };
  // Three register buffers in turn: two steps of loads in flight while one
  // step is staged and computed.
  u32x4 ra[8], rb[8], rc[8];
  int key0 = start + wave * kIsKeysPerStep;
  int nsteps = key0 < end ? (end - key0 + kIsKeysPerRound - 1) / kIsKeysPerRound : 0;
  if constexpr (CUT) {
    // Step i of this wave takes the chunk's group 8i + wave.
    const int groups = (N + kIsKeysPerStep - 1) / kIsKeysPerStep;
    const int mine_groups = chunk_group_count(c, C, groups);
    nsteps = wave < mine_groups ? (mine_groups - wave + kIsWaves - 1) / kIsWaves : 0;
  }
  auto key_at = [&](int i) {
    if constexpr (CUT) return chunk_group(c, C, i * kIsWaves + wave) * kIsKeysPerStep;
    return key0 + i * kIsKeysPerRound;
  };
  auto local_at = [&](int i) { return (i * kIsWaves + wave) * kIsKeysPerStep; };
  if (nsteps > 0) load_step(ra, key_at(0));
  if (nsteps > 1) load_step(rb, key_at(1));
  for (int i = 0; i < nsteps; i += 3) {
    if (i + 2 < nsteps) load_step(rc, key_at(i + 2));
    score_step(ra, key_at(i), local_at(i));
    if (i + 1 >= nsteps) break;
    if (i + 3 < nsteps) load_step(ra, key_at(i + 3));
    score_step(rb, key_at(i + 1), local_at(i + 1));
    if (i + 2 >= nsteps) break;
    if (i + 4 < nsteps) load_step(rb, key_at(i + 4));
    score_step(rc, key_at(i + 2), local_at(i + 2));
  }
  if constexpr (CUT) {  // the wave's key range, for the cut's histogram
    *key_lo = wave_reduce<OpMin>(klo);
    *key_hi = wave_reduce<OpMax>(khi);
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

// ---------------------------------------------------------------- chunk cut
// The indexer fused with the first half of the top-k ("feat: Add DeepSeek-V4
// CSA attention kernels", "The top-k on the GPSIMD engine": the score and
// the top-k run together chunk by chunk, and a last top-k merges the chunks'
// results). Each workgroup scores chunk c of C interleaved chunks of its row
// (see sweep_row), keeps every score's order key in LDS, and then keeps the
// chunk's exact top KL under (value desc, position asc), written as 64-bit
// composites, together with t_c, the smallest kept composite (0 when the
// chunk kept every score it has). A merge kernel then selects the row's k-th
// composite T* among the kept ones; when every t_c <= T*, no dropped score
// can be in the row's top k and the merge's answer is exact.

constexpr int kCutBins = 2048;  // buckets of a cut round (11 bits)

struct CutScratch {
  uint32_t wsum[kIsWaves];
  uint32_t wmin[kIsWaves], wmax[kIsWaves];
  uint64_t wcomp[kIsWaves];
  uint32_t digit, above, in_bucket;
};

// Exclusive block-wide scan in thread order; *total gets the sum.
__device__ __forceinline__ uint32_t cut_scan(uint32_t v, uint32_t* total, CutScratch& cs) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint32_t inc = wave_scan_incl(v);
  if (lane == kWave - 1) cs.wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kIsWaves; ++w) {
    const uint32_t x = cs.wsum[w];
    before += (w < wave) ? x : 0u;
    all += x;
  }
  __syncthreads();  // wsum is written again by the next scan
  *total = all;
  return before + inc - v;
}

// Wave 0 finds the bucket of hist[0..kCutBins) that holds the need-th
// largest entry (buckets in ascending key order) and publishes it.
__device__ __forceinline__ void cut_pick(const uint32_t* hist, uint32_t need, CutScratch& cs) {
  constexpr int PER = kCutBins / kWave;  // 32 buckets per lane
  const int tid = threadIdx.x;
  if (tid < kWave) {
    // Lane l sums the buckets ending at kCutBins-1-PER*l, so lane order is
    // descending bucket order.
    const int base = kCutBins - PER * (tid + 1);
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(hist + base + 4 * j);
      local += x[0] + x[1] + x[2] + x[3];
    }
    const uint32_t inc = wave_scan_incl(local);
    const int first = __ffsll((long long)__ballot(inc >= need)) - 1;
    const uint32_t run = lane_read(inc - local, first);
    const int top = kCutBins - 1 - PER * first;
    const uint32_t cj = tid < PER ? hist[top - tid] : 0u;
    const uint32_t incj = wave_scan_incl(cj);
    const int j = __ffsll((long long)__ballot(tid < PER && run + incj >= need)) - 1;
    if (tid == j) {
      cs.digit = (uint32_t)(top - j);
      cs.above = run + incj - cj;
      cs.in_bucket = cj;
    }
  }
  __syncthreads();
}

// The chunk's exact top KL (or all of its valid keys when it has no more).
// keep[0..M): order keys by local index, 0 = no score. The selection is
// "key > t_gt, or key == t_eq among the first need_eq such keys by index",
// found by range-adaptive 11-bit histogram rounds over the keys, starting
// from keys [lo, hi], which hold the KL-th largest, with need of the KL
// inside it (every key above hi is in). Each round first takes the actual
// range of the keys inside [lo, hi], so a range that holds one tied value
// ends the search at once (quantised scores: one round of contended
// histogram atomics less per cut). Expects the histogram clear and leaves
// it so.
__device__ __noinline__ void chunk_cut_exact(const uint32_t* keep, int M, int valid, int KL, int b,
                                             int c, int C, uint32_t* hist, CutScratch& cs,
                                             uint64_t* __restrict__ cand,
                                             uint32_t* __restrict__ cnt,
                                             uint64_t* __restrict__ tcut, uint32_t lo = 1u,
                                             uint32_t hi = 0xFFFFFFFFu, uint32_t need = 0u) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  int64_t t_gt = 0;        // keys above it are in
  uint32_t t_eq = 0, need_eq = 0;
  const bool all = valid <= KL;
  if (!all) {
    if (need == 0u) need = (uint32_t)KL;
    for (int round = 0; round < 5; ++round) {  // 11-bit rounds: 3 narrow any 32-bit range
      uint32_t a = 0xFFFFFFFFu, z = 0;
      for (int i = tid; i < M; i += kIsThreads) {
        const uint32_t x = keep[i];
        if (x >= lo && x <= hi) {
          a = min(a, x);
          z = max(z, x);
        }
      }
      a = wave_reduce<OpMin>(a);
      z = wave_reduce<OpMax>(z);
      if (lane == 0) {
        cs.wmin[wave] = a;
        cs.wmax[wave] = z;
      }
      __syncthreads();
#pragma unroll
      for (int w = 0; w < kIsWaves; ++w) {
        a = min(a, cs.wmin[w]);
        z = max(z, cs.wmax[w]);
      }
      __syncthreads();  // wmin/wmax are written again by the next round
      lo = a;
      hi = z;
      if (lo == hi) {  // what is left ties on one key: take the first `need` of them
        t_gt = lo;
        t_eq = lo;
        need_eq = need;
        break;
      }
      const uint32_t range = hi - lo;
      const int shift = max(0, 31 - __clz(range) - 10);
      for (int i = tid; i < M; i += kIsThreads) {
        const uint32_t x = keep[i];
        hist_add(hist, (x >= lo && x <= hi) ? ((x - lo) >> shift) : kNoBin);
      }
      __syncthreads();
      cut_pick(hist, need, cs);
      const uint32_t digit = cs.digit, above = cs.above, in_bucket = cs.in_bucket;
      for (int i = tid; i < kCutBins; i += kIsThreads) hist[i] = 0;
      __syncthreads();  // every thread has read the pick; the histogram is clear
      need -= above;
      const uint32_t blo = lo + (digit << shift);
      if (in_bucket == need) {  // the whole bucket is in: every key >= blo
        t_gt = (int64_t)blo - 1;
        need_eq = 0;
        break;
      }
      const uint32_t bhi = blo + ((1u << shift) - 1u);
      lo = blo;
      hi = bhi < hi ? bhi : hi;
    }
  }
  // Compaction in index order: thread t takes [t*per, t*per + per).
  const int per = (M + kIsThreads - 1) / kIsThreads;
  const int i0 = min(M, tid * per), i1 = min(M, i0 + per);
  uint32_t ngt = 0, neq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t x = keep[i];
    ngt += (x != 0u && (int64_t)x > t_gt) ? 1u : 0u;
    neq += (x != 0u && x == t_eq && need_eq) ? 1u : 0u;
  }
  uint32_t totals;
  const uint32_t before = cut_scan(ngt | (neq << 16), &totals, cs);
  const uint32_t gt_before = before & 0xFFFFu, eq_before = before >> 16;
  uint32_t eq_seen = eq_before;
  uint32_t at = gt_before + min(need_eq, eq_before);
  uint64_t* out = cand + ((size_t)b * C + c) * KL;
  uint64_t least = ~(uint64_t)0;
  int grp = i0 >> 5;  // the row offset of the group of 32 holding key i
  int grp_row = chunk_group(c, C, grp) * kIsKeysPerStep;
  for (int i = i0; i < i1; ++i) {
    const uint32_t x = keep[i];
    if (x == 0u) continue;
    bool sel = (int64_t)x > t_gt;
    if (need_eq && x == t_eq) {
      sel = sel || eq_seen < need_eq;
      ++eq_seen;
    }
    if (sel && at < (uint32_t)KL) {
      // local index i = 32 * (the group's rank in the chunk) + offset
      if ((i >> 5) != grp) {
        grp = i >> 5;
        grp_row = chunk_group(c, C, grp) * kIsKeysPerStep;
      }
      const uint64_t cp = composite(x, (uint32_t)(grp_row + (i & 31)));
      out[at++] = cp;
      least = cp < least ? cp : least;
    }
  }
  least = wave_reduce64<true>(least);
  if (lane == 0) cs.wcomp[wave] = least;
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int w = 0; w < kIsWaves; ++w) least = cs.wcomp[w] < least ? cs.wcomp[w] : least;
    cnt[(size_t)b * C + c] = min((uint32_t)KL, (totals & 0xFFFFu) + min(need_eq, totals >> 16));
    tcut[(size_t)b * C + c] = all ? 0ull : least;
  }
}

// The chunk's cut: all of its scores at or above a bucket edge that leaves
// at least `target` of them (one histogram round of 2048 buckets over the
// chunk's key range), written in index order, with t_c = the edge as a
// composite (every dropped composite lies below it). A chunk with at most
// `cap` scores keeps them all (t_c = 0); when the edge would leave more than
// `cap` (a heavy bucket of ties), the exact cut to `cap` takes over.
// Expects the histogram clear and cs.wmin/wmax holding each wave's smallest
// and largest key, behind a barrier.
__device__ void chunk_cut(const uint32_t* keep, int M, int valid, int target, int cap, int b,
                          int c, int C, uint32_t* hist, CutScratch& cs,
                          uint64_t* __restrict__ cand, uint32_t* __restrict__ cnt,
                          uint64_t* __restrict__ tcut) {
  const int tid = threadIdx.x;
  uint32_t edge = 1;  // keys >= edge are kept (real keys are >= 1)
  if (valid > cap) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
    for (int w = 0; w < kIsWaves; ++w) {
      lo = min(lo, cs.wmin[w]);
      hi = max(hi, cs.wmax[w]);
    }
    const uint32_t range = hi - lo;
    const int shift = range == 0 ? 0 : max(0, 31 - __clz(range) - 10);
    for (int i = tid; i < M; i += kIsThreads) {
      const uint32_t x = keep[i];
      if (x) atomicAdd(&hist[(x - lo) >> shift], 1u);
    }
    __syncthreads();
    cut_pick(hist, (uint32_t)target, cs);
    const uint32_t digit = cs.digit, kept = cs.above + cs.in_bucket;
    if (kept > (uint32_t)cap) {  // uniform
      // The cap-th largest key lies in this bucket too (above < target <=
      // cap < kept): the exact cut starts there.
      for (int i = tid; i < kCutBins; i += kIsThreads) hist[i] = 0;
      __syncthreads();  // every thread has read the pick; the histogram is clear
      const uint32_t blo = lo + (digit << shift);
      const uint32_t bhi = min(hi, blo + ((1u << shift) - 1u));
      chunk_cut_exact(keep, M, valid, cap, b, c, C, hist, cs, cand, cnt, tcut, blo, bhi,
                      (uint32_t)cap - cs.above);
      return;
    }
    // (The compaction below writes neither the pick nor the histogram.)
    edge = lo + (digit << shift);
  }
  // Compaction in index order: thread t takes [t*per, t*per + per).
  const int per = (M + kIsThreads - 1) / kIsThreads;
  const int i0 = min(M, tid * per), i1 = min(M, i0 + per);
  uint32_t n = 0;
  for (int i = i0; i < i1; ++i) n += keep[i] >= edge ? 1u : 0u;
  uint32_t total;
  uint32_t at = cut_scan(n, &total, cs);
  uint64_t* out = cand + ((size_t)b * C + c) * cap;
  int grp = i0 >> 5;  // a thread's keys lie in one or two groups of 32: their row offset is kept
  int grp_row = chunk_group(c, C, grp) * kIsKeysPerStep;
  for (int i = i0; i < i1; ++i) {
    const uint32_t x = keep[i];
    if (x >= edge && at < (uint32_t)cap) {
      if ((i >> 5) != grp) {
        grp = i >> 5;
        grp_row = chunk_group(c, C, grp) * kIsKeysPerStep;
      }
      out[at++] = composite(x, (uint32_t)(grp_row + (i & 31)));
    }
  }
  if (tid == 0) {
    cnt[(size_t)b * C + c] = min(total, (uint32_t)cap);
    tcut[(size_t)b * C + c] = valid > cap ? ((uint64_t)edge << 32) : 0ull;
  }
}

template <int MT>
__global__ __launch_bounds__(kIsThreads) void indexer_score_cut_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ w, float* __restrict__ s, int N, int H, int C, int target,
    int cap, uint64_t* __restrict__ cand, uint32_t* __restrict__ cnt,
    uint64_t* __restrict__ tcut) {
  __shared__ u32x4 stage_lds[kIsWaves][32 * 16];  // 8 KB per wave; the cut's histogram after
  __shared__ CutScratch cs;
  extern __shared__ uint32_t keep[];              // the chunk's order keys
  const int b = blockIdx.y;
  const int c = blockIdx.x;
  uint32_t klo, khi;
  sweep_row<MT, true>(q, k, w, s, b, N, H, 0, N, stage_lds[threadIdx.x / kWave], c, C, keep, &klo,
                      &khi);
  // Each wave's key range goes to LDS, and wave 0 clears its staging area
  // (its own LDS operations run in order), which the cut's histogram takes,
  // before the barrier that ends the sweep.
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    cs.wmin[wave] = klo;
    cs.wmax[wave] = khi;
  }
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 32 * 16 / kWave; ++i) stage_lds[0][i * kWave + threadIdx.x] = u32x4{0u, 0u, 0u, 0u};
  }
  const int groups = (N + kIsKeysPerStep - 1) / kIsKeysPerStep;
  const int M = chunk_group_count(c, C, groups) * kIsKeysPerStep;
  // The row's last group may be partial: it is group (groups-1) mod C of
  // super-group (groups-1) / C, which belongs to chunk (its slot - L) mod C.
  const int lastL = (groups - 1) / C;
  const int owner = (((groups - 1) % C - lastL) % C + C) % C;
  const int valid = M - (c == owner ? groups * kIsKeysPerStep - N : 0);
  __syncthreads();  // every key is in keep[], the key ranges and the clear histogram are in place
  chunk_cut(keep, M, valid, target, cap, b, c, C, reinterpret_cast<uint32_t*>(&stage_lds[0][0]),
            cs, cand, cnt, tcut);
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

// Keys per workgroup. Each wave keeps its query fragments (up to 16 KB per
// batch row) in registers for its whole sweep. Aim for one round of about
// 256 workgroups (one per CU measured fastest), each sweeping at most 32
// rounds of 256 keys; large calls take at least 8 rounds per workgroup so
// the query loads stay small next to the key stream, while small calls
// (fewer than 256 * 8 rounds in all) spread over as many workgroups as they
// can fill.
int indexer_keys_per_wg(int B, int N) {
  const long long per_row_rounds = (N + kIsKeysPerRound - 1) / kIsKeysPerRound;
  const long long total_rounds = (long long)B * per_row_rounds;
  long long rounds = (total_rounds + 255) / 256;
  if (rounds < 8 && total_rounds >= 256 * 8) rounds = 8;
  if (rounds > 32) rounds = 32;
  if (rounds > per_row_rounds) rounds = per_row_rounds;
  if (rounds < 1) rounds = 1;
  return (int)rounds * kIsKeysPerRound;
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
  const long long per_row_rounds = (N + kIsKeysPerRound - 1) / kIsKeysPerRound;
  const long long total_rounds = (long long)B * per_row_rounds;
  const int keys_per_wg = indexer_keys_per_wg(B, N);
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

CutPlan plan_cut(int B, int N, int k) {
  CutPlan p{};
  const int kpw = indexer_keys_per_wg(B, N);
  const int C = (N + kpw - 1) / kpw;
  const int groups = (N + kIsKeysPerStep - 1) / kIsKeysPerStep;
  const int mcap = (groups + C - 1) / C * kIsKeysPerStep;  // keys of the largest chunk
  // A chunk keeps at least its expected share of k plus 4 standard
  // deviations of a random row's spread plus 16: a chunk then holds more of
  // the row's top k than it keeps with a probability below 1e-4 even at
  // k/C = 1 (rising rows spread evenly over interleaved chunks). Room for
  // twice that, rounded up to 8 and capped by the chunk: a heavier bucket at
  // the cut's edge (tied scores) takes the exact cut. Where an eighth more
  // (at least 8) brings a row's slots down to 2048, 4 per merging thread,
  // the keep is that tight instead: at B = 16, N = 32768, k = 1024 (C = 16,
  // target 113) keep 128 instead of 232 took the step from 59.5 to 57.5 us.
  // (At B = 64, N = 262144, k = 2048 the tight keep sent 16 % of the stress
  // rows' chunks to the exact cut, and it would not reach 4 per thread.)
  const double share = (double)k / C;
  long long target = (long long)(share + 4.0 * sqrt(share) + 16.0) + 1;
  if (target > mcap) target = mcap;
  long long cap = (target + (target / 8 > 8 ? target / 8 : 8) + 7) / 8 * 8;
  if ((long long)C * cap > 2048) cap = (2 * target + 7) / 8 * 8;
  if (cap > mcap) cap = mcap;
  p.chunks = C;
  p.target = (int)target;
  p.keep = (int)cap;
  p.mcap = mcap;
  // The merge holds at most 16384 candidates per row; the LDS copy of a
  // chunk's keys at most 32 KB.
  p.ok = (long long)C * target >= k && (long long)C * cap <= 16384 && mcap <= 8192 && C <= 1024;
  return p;
}

hipError_t launch_indexer_cut(const uint16_t* q, const uint16_t* k, const float* w, float* s,
                              int B, int N, int H, const CutPlan& p, uint64_t* cand,
                              uint32_t* cnt, uint64_t* tcut, hipStream_t st) {
  const dim3 grid((unsigned)p.chunks, (unsigned)B);
  const dim3 block(kIsThreads);
  const size_t lds = (size_t)p.mcap * sizeof(uint32_t);
  const int mt = (H + 15) / 16;
  // With the static staging area the workgroup holds more than 64 KB of LDS.
  const void* kern = mt == 1 ? reinterpret_cast<const void*>(indexer_score_cut_kernel<1>)
                   : mt == 2 ? reinterpret_cast<const void*>(indexer_score_cut_kernel<2>)
                   : mt == 3 ? reinterpret_cast<const void*>(indexer_score_cut_kernel<3>)
                             : reinterpret_cast<const void*>(indexer_score_cut_kernel<4>);
  const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  switch (mt) {
    case 1: hipLaunchKernelGGL(indexer_score_cut_kernel<1>, grid, block, lds, st, q, k, w, s, N, H, p.chunks, p.target, p.keep, cand, cnt, tcut); break;
    case 2: hipLaunchKernelGGL(indexer_score_cut_kernel<2>, grid, block, lds, st, q, k, w, s, N, H, p.chunks, p.target, p.keep, cand, cnt, tcut); break;
    case 3: hipLaunchKernelGGL(indexer_score_cut_kernel<3>, grid, block, lds, st, q, k, w, s, N, H, p.chunks, p.target, p.keep, cand, cnt, tcut); break;
    default: hipLaunchKernelGGL(indexer_score_cut_kernel<4>, grid, block, lds, st, q, k, w, s, N, H, p.chunks, p.target, p.keep, cand, cnt, tcut); break;
  }
  return hipGetLastError();
}

}  // namespace dsa
