// Exact selection of the k largest 64-bit composites (order key of the
// value in the high word, complemented position in the low word) by one
// workgroup, shared by the top-k merge and by the attention kernel that
// selects its own rows (the chunk cut's merge folded into attention).
//
// One histogram round over the candidates' value keys (2048 buckets over
// their actual range) finds the bucket of the K-th largest. A bucket that is
// not taken whole is gathered and ranked entry against entry (up to 512
// entries); a heavier one goes to a radix select whose 10-bit digits split
// the remaining range into 1024 equal buckets per round.
#pragma once

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kMergeThreads = 512;
constexpr int kMaxWaves = 16;
constexpr int kBins = 1024;        // buckets of an exact-select round
constexpr int kBinBits = 10;
constexpr int kHBins = 2048;       // buckets of a one-round histogram (11 bits)
constexpr int kHBinBits = 11;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct Scratch {
  alignas(16) uint32_t hist[2][kHBins];
  uint64_t wlo[kMaxWaves], whi[kMaxWaves];
  uint32_t wsum[kMaxWaves];                                 // block scans
  uint32_t wcnt[kMaxWaves], wmin[kMaxWaves], wmax[kMaxWaves];  // count/min/max reductions
  uint32_t digit, above, in_bucket;
  uint32_t n_app;  // entries appended to an LDS list
  uint64_t pick;   // a composite published to the block
};

// How many entries of list[0..n8) are above x; n8 is a multiple of 8 and
// the list is zero-padded to it (real composites are non-zero). Every lane
// reads the same 16-byte slots (broadcast reads), four at a time.
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t count_above(const uint64_t* list, uint32_t n8, uint64_t x) {
  const u64x2* L = reinterpret_cast<const u64x2*>(list);
  uint32_t r = 0;
  for (uint32_t i = 0; i < n8 / 2; i += 4) {
    const u64x2 a = L[i], b = L[i + 1], c = L[i + 2], d = L[i + 3];
    r += (a.x > x ? 1u : 0u) + (a.y > x ? 1u : 0u) + (b.x > x ? 1u : 0u) + (b.y > x ? 1u : 0u) +
         (c.x > x ? 1u : 0u) + (c.y > x ? 1u : 0u) + (d.x > x ? 1u : 0u) + (d.y > x ? 1u : 0u);
  }
  return r;
}

// Exclusive block-wide scan in thread order; *total gets the sum. One
// barrier: every caller passes another barrier before wsum is written again.
template <int THREADS>
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total, Scratch& sc) {
  constexpr int W = THREADS / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint32_t inc = wave_scan_incl(v);
  if (lane == kWave - 1) sc.wsum[wave] = inc;
  lds_barrier();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const uint32_t s = sc.wsum[w];
    before += (w < wave) ? s : 0u;
    all += s;
  }
  *total = all;
  return before + inc - v;
}

// Wave 0 finds the digit whose bucket holds the need-th largest entry of
// hist[0..NB) and publishes it; ends with a barrier. Two wave scans: one
// over per-lane sums of PER bins, then one over the PER bins of the lane
// that holds the answer (one bin per lane).
template <int NB>
__device__ void pick_digit(const uint32_t* hist, uint32_t need, Scratch& sc, uint32_t& digit,
                           uint32_t& above, uint32_t& in_bucket) {
  constexpr int PER = NB / kWave;
  static_assert(PER % 4 == 0 && PER <= kWave, "lanes read their bins as 16-byte vectors");
  const int tid = threadIdx.x;
  if (tid < kWave) {
    // Lane l owns the PER contiguous bins ending at NB-1-PER*l (read as
    // 16-byte vectors; a scalar stride-PER pattern would hit one LDS bank
    // many times over), so lane order is descending bin order.
    const int base = NB - PER * (tid + 1);
    uint32_t local = 0;
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(hist + base + 4 * q);
      local += x[0] + x[1] + x[2] + x[3];
    }
    const uint32_t inc = wave_scan_incl(local);
    const int first = __ffsll((long long)__ballot(inc >= need)) - 1;  // uniform
    const uint32_t run = (uint32_t)__builtin_amdgcn_readlane((int)(inc - local), first);
    // Lane j takes bin NB-1-PER*first-j, again in descending order.
    const int top = NB - 1 - PER * first;
    const uint32_t cj = tid < PER ? hist[top - tid] : 0u;
    const uint32_t incj = wave_scan_incl(cj);
    const int j = __ffsll((long long)__ballot(tid < PER && run + incj >= need)) - 1;
    if (tid == j) {
      sc.digit = (uint32_t)(top - j);
      sc.above = run + incj - cj;
      sc.in_bucket = cj;
    }
  }
  lds_barrier();
  digit = sc.digit;
  above = sc.above;
  in_bucket = sc.in_bucket;
}

// The same exact select over entries held in registers: PER slots per
// thread, 0 = empty (real composites are non-zero). No LDS reads per pass.
template <int THREADS, int PER>
__device__ void regs_range(const uint64_t (&v)[PER], uint64_t& lo, uint64_t& hi, Scratch& sc) {
  constexpr int W = THREADS / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint64_t a = ~(uint64_t)0, z = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool in = v[j] && v[j] >= lo && v[j] <= hi;
    a = (in && v[j] < a) ? v[j] : a;
    z = (in && v[j] > z) ? v[j] : z;
  }
  a = wave_reduce64<true>(a);
  z = wave_reduce64<false>(z);
  if (lane == 0) {
    sc.wlo[wave] = a;
    sc.whi[wave] = z;
  }
  lds_barrier();
#pragma unroll
  for (int w = 0; w < W; ++w) {
    a = sc.wlo[w] < a ? sc.wlo[w] : a;
    z = sc.whi[w] > z ? sc.whi[w] : z;
  }
  lo = a;
  hi = z;
}

template <int THREADS, int PER>
__device__ uint64_t select_exact_regs(const uint64_t (&v)[PER], int K, Scratch& sc,
                                      uint64_t lo = 1, uint64_t hi = ~(uint64_t)0) {
  const int tid = threadIdx.x;
  regs_range<THREADS, PER>(v, lo, hi, sc);
  uint32_t need = (uint32_t)K;
  uint64_t result = lo;
  for (int round = 0; round < 8; ++round) {
    const uint64_t range = hi - lo;
    if (range == 0) {
      result = lo;
      break;
    }
    const int hb = 63 - __clzll((long long)range);
    const int shift = hb >= kBinBits ? hb - (kBinBits - 1) : 0;
    uint32_t* cur = sc.hist[round & 1];
    uint32_t* nxt = sc.hist[(round + 1) & 1];
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (v[j] && v[j] >= lo && v[j] <= hi) atomicAdd(&cur[(uint32_t)((v[j] - lo) >> shift)], 1u);
    for (int i = tid; i < kBins; i += THREADS) nxt[i] = 0;
    lds_barrier();
    uint32_t digit, above, in_bucket;
    pick_digit<kBins>(cur, need, sc, digit, above, in_bucket);
    for (int i = tid; i < kBins; i += THREADS) cur[i] = 0;  // ordered by the next barrier
    need -= above;
    const uint64_t blo = lo + ((uint64_t)digit << shift);
    result = blo;
    if (in_bucket == need) break;
    const uint64_t bhi = blo + (((uint64_t)1 << shift) - 1);
    lo = blo;
    hi = bhi < hi ? bhi : hi;
    regs_range<THREADS, PER>(v, lo, hi, sc);
  }
  lds_barrier();
  return result;
}

// Exact top k of one float32 (or bf16) row read from global memory by one
// workgroup: emit(at, i) is called for the at-th winner i, at = 0, 1, ...
// in ascending position order. The rows that a chunk cut (the fused
// indexer's) or a segment quota (the top-k's) could not settle come here:
// radix rounds over the value keys (2048 buckets over the remaining key
// range, one pass over the row each), then the ties at the k-th value taken
// by lowest position. Slow (several passes over the row by one workgroup)
// and rare: a random row never comes here at the benchmarked shapes, a
// sorted one neither (chunks and segments are interleaved), only rows built
// to pile their top k into few chunks do.
template <bool BF16 = false, typename Emit>
__device__ __noinline__ void row_topk_from_scores(const void* __restrict__ row, int N, int k,
                                                  Emit emit, Scratch& sc) {
  constexpr int T = kMergeThreads;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  // A bf16 value is the float32 with its bits in the high half.
  auto key_at = [&](int i) {
    return BF16 ? f32_key((uint32_t)reinterpret_cast<const uint16_t*>(row)[i] << 16)
                : f32_key(reinterpret_cast<const uint32_t*>(row)[i]);
  };
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
  for (int i = tid; i < N; i += T) {
    const uint32_t x = key_at(i);
    lo = min(lo, x);
    hi = max(hi, x);
  }
  lo = wave_reduce<OpMin>(lo);
  hi = wave_reduce<OpMax>(hi);
  if (lane == 0) {
    sc.wmin[wave] = lo;
    sc.wmax[wave] = hi;
  }
  for (int i = tid; i < kHBins; i += T) sc.hist[0][i] = 0;
  lds_barrier();
#pragma unroll
  for (int w = 0; w < T / kWave; ++w) {
    lo = min(lo, sc.wmin[w]);
    hi = max(hi, sc.wmax[w]);
  }
  // Selected: key > t_gt, or key == t_eq among the first need_eq such keys.
  int64_t t_gt = -1;
  uint32_t t_eq = 0, need_eq = 0;
  uint32_t need = (uint32_t)k;
  if (k < N) {
    for (int round = 0; round < 4; ++round) {
      if (lo == hi) {
        t_gt = lo;
        t_eq = lo;
        need_eq = need;
        break;
      }
      const uint32_t range = hi - lo;
      const int shift = max(0, 31 - __clz(range) - (kHBinBits - 1));
      for (int i = tid; i < N; i += T) {
        const uint32_t x = key_at(i);
        if (x >= lo && x <= hi) atomicAdd(&sc.hist[0][(x - lo) >> shift], 1u);
      }
      lds_barrier();
      uint32_t digit, above, in_bucket;
      pick_digit<kHBins>(sc.hist[0], need, sc, digit, above, in_bucket);
      for (int i = tid; i < kHBins; i += T) sc.hist[0][i] = 0;
      lds_barrier();
      need -= above;
      const uint32_t blo = lo + (digit << shift);
      if (in_bucket == need) {
        t_gt = (int64_t)blo - 1;
        break;
      }
      const uint32_t bhi = blo + ((1u << shift) - 1u);
      lo = blo;
      hi = bhi < hi ? bhi : hi;
    }
  }
  // Winners in position order, a block of 4 positions per thread at a time.
  uint32_t gt_done = 0, eq_done = 0;
  for (int base = 0; base < N; base += 4 * T) {
    uint32_t x[4];
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = base + 4 * tid + e;
      x[e] = i < N ? key_at(i) : 0u;
      ngt += (i < N && (int64_t)x[e] > t_gt) ? 1u : 0u;
      neq += (i < N && need_eq && x[e] == t_eq) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t before = block_exclusive_scan<T>(ngt | (neq << 16), &tot, sc);
    uint32_t eq_seen = eq_done + (before >> 16);
    uint32_t at = gt_done + (before & 0xFFFFu) + min(need_eq, eq_seen);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = base + 4 * tid + e;
      if (i >= N) continue;
      bool sel = (int64_t)x[e] > t_gt;
      if (need_eq && x[e] == t_eq) {
        sel = sel || eq_seen < need_eq;
        ++eq_seen;
      }
      if (sel && at < (uint32_t)k) emit(at++, i);
    }
    gt_done += tot & 0xFFFFu;
    eq_done += tot >> 16;
    lds_barrier();  // wsum is written again by the next block's scan
  }
}

// The selection of a row's k winners from its candidate lists, by one
// workgroup of kMergeThreads threads: segs lists of slots entries each at
// src (list j holds cnt_row[j] valid composites), at most kMergeThreads *
// kPer slots in all. On return v[] holds this thread's slots (0 = empty)
// and the winners are the slots with v[j] >= thr, min(k, valid) of them;
// this thread's first winner is number pos of nkeep in (thread, slot)
// order. With CUT, the lists are the chunk cut's, tcut_row[j] is the cut of
// list j, and false is returned when the kept candidates cannot vouch for
// the row's top k (some chunk dropped a composite at or above the k-th
// kept one, or fewer than k were kept): the caller then selects the row
// from its scores. Expects nothing of sc; leaves it dirty.
template <int kPer, bool CUT>
__device__ __forceinline__ bool merge_candidates(const uint64_t* __restrict__ src,
                                                 const uint32_t* __restrict__ cnt_row,
                                                 const uint64_t* __restrict__ tcut_row, int segs,
                                                 int slots, int k, Scratch& sc, uint64_t (&v)[kPer],
                                                 uint64_t& thr, uint32_t& pos, uint32_t& nkeep) {
  const int tid = threadIdx.x;
  // Every slot of the row at once: slot q = tid + j*512 is entry q % slots
  // of segment q / slots, valid below that segment's count. All loads, the
  // counts included, are issued unconditionally (clamped into the row's
  // slots, which lie inside the workspace) so they overlap; validity is
  // applied after.
  const int nslots = segs * slots;
  uint32_t c[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int q = min(tid + j * kMergeThreads, nslots - 1);
    v[j] = src[q];
    c[j] = cnt_row[q / slots];
  }
  // With CUT, the largest of the lists' cuts, loaded with them.
  uint64_t cut = 0;
  if constexpr (CUT) {
    for (int j = tid; j < segs; j += kMergeThreads) {
      const uint64_t t = tcut_row[j];
      cut = t > cut ? t : cut;
    }
  }
  for (int i = tid; i < kHBins; i += kMergeThreads) {
    sc.hist[0][i] = 0;
    sc.hist[1][i] = 0;
  }
  if (tid == 0) sc.n_app = 0;
  uint32_t nvalid = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int q = tid + j * kMergeThreads;
    const bool ok = q < nslots && (uint32_t)(q % slots) < min((uint32_t)slots, c[j]);
    v[j] = ok ? v[j] : 0;
    nvalid += ok ? 1u : 0u;
  }
  // Count, smallest and largest value key of the valid entries.
  uint32_t total, kmin, kmax;
  {
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t key = (uint32_t)(v[j] >> 32);
      lo = v[j] ? min(lo, key) : lo;
      hi = v[j] ? max(hi, key) : hi;
    }
    const uint32_t n = wave_reduce<OpAdd>(nvalid);
    lo = wave_reduce<OpMin>(lo);
    hi = wave_reduce<OpMax>(hi);
    if constexpr (CUT) cut = wave_reduce64<false>(cut);
    if (lane == 0) {  // wcnt/wmin/wmax: not written again here; whi only behind later barriers
      sc.wcnt[wave] = n;
      sc.wmin[wave] = lo;
      sc.wmax[wave] = hi;
      if constexpr (CUT) sc.whi[wave] = cut;
    }
    lds_barrier();
    total = 0;
    kmin = 0xFFFFFFFFu;
    kmax = 0;
#pragma unroll
    for (int w = 0; w < kMergeThreads / kWave; ++w) {
      total += sc.wcnt[w];
      kmin = min(kmin, sc.wmin[w]);
      kmax = max(kmax, sc.wmax[w]);
      if constexpr (CUT) cut = sc.whi[w] > cut ? sc.whi[w] : cut;
    }
  }
  // The k-th largest composite. One histogram round over the value keys
  // (2048 buckets over [kmin, kmax]) finds its bucket; if that bucket is not
  // taken whole, its few entries are gathered in LDS and ranked against one
  // another (composites are distinct, so exactly one has rank need-1). A
  // bucket of more than 512 entries (heavy ties) takes the general select.
  thr = 0;
  if ((int)total > k) {
    const uint32_t range = kmax - kmin;
    const int shift = range == 0 ? 0 : max(0, 31 - __clz(range) - (kHBinBits - 1));
    uint32_t* h = sc.hist[0];
    // The largest candidate sets (16 or more slots per thread, k of 2048 and
    // up) take the wave-aggregated count, which pays off on rows of many tied
    // scores (bf16 stress rows, 64 x 262144, k = 2048: 76.8 -> 71.0 us); on
    // the smaller sets its ballot costs more than it saves (+1-2 %).
    if constexpr (kPer >= 16) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) hist_add(h, v[j] ? (((uint32_t)(v[j] >> 32) - kmin) >> shift) : kNoBin);
    } else {
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (v[j]) atomicAdd(&h[((uint32_t)(v[j] >> 32) - kmin) >> shift], 1u);
    }
    lds_barrier();
    uint32_t digit, above, in_bucket;
    pick_digit<kHBins>(h, (uint32_t)k, sc, digit, above, in_bucket);
    const uint32_t need = (uint32_t)k - above;
    const uint32_t blo = kmin + (digit << shift);
    if (in_bucket == need) {
      thr = (uint64_t)blo << 32;  // the whole bucket is in
    } else if (in_bucket <= (uint32_t)kMergeThreads) {
      uint64_t* list = reinterpret_cast<uint64_t*>(sc.hist[1]);  // 1024 entries
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (v[j] && (((uint32_t)(v[j] >> 32) - kmin) >> shift) == digit)
          list[atomicAdd(&sc.n_app, 1u)] = v[j];
      }
      const uint32_t n8 = (in_bucket + 7u) & ~7u;
      if ((uint32_t)tid >= in_bucket && (uint32_t)tid < n8) list[tid] = 0;
      lds_barrier();
      if (tid < (int)in_bucket) {
        const uint64_t x = list[tid];
        const uint32_t r = count_above(list, n8, x);
        if (r == need - 1) sc.pick = x;
      }
      lds_barrier();
      thr = sc.pick;
    } else {
      // Heavy bucket: start the exact select from its own entries.
      for (int i = tid; i < kHBins; i += kMergeThreads) h[i] = 0;  // ordered by the next barrier
      const uint64_t bhi = min((uint64_t)kmax, (uint64_t)blo + (((uint64_t)1 << shift) - 1));
      thr = select_exact_regs<kMergeThreads, kPer>(v, (int)need, sc, (uint64_t)blo << 32,
                                                   (bhi << 32) | 0xFFFFFFFFull);
    }
  }
  if constexpr (CUT) {
    // T*, the row's k-th largest kept composite, is the smallest winner,
    // and every winner is >= thr (or, when all kept entries win, >= the
    // smallest kept value key). Every chunk that dropped scores dropped only
    // composites below its cut t_c, so when all t_c are at most that bound,
    // nothing dropped can reach T*: T* is at most the row's true k-th
    // composite and the winners are exact. (A bound below T* can only send a
    // row to the fallback needlessly, never pass a wrong one.)
    const uint64_t bound = (int)total > k ? thr : ((uint64_t)kmin << 32);
    if ((int)total < k || cut > bound) return false;  // uniform
  }
  // Winners in (thread, slot) order.
  uint32_t keep = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) keep += (v[j] && v[j] >= thr) ? 1u : 0u;
  pos = block_exclusive_scan<kMergeThreads>(keep, &nkeep, sc);
  return true;
}

}  // namespace
}  // namespace dsa
