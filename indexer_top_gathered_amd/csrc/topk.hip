// Top-k selection on gfx950 ("feat: Add DeepSeek-V4 CSA attention kernels",
// step 3, and its chunked score/top-k pipeline in "The top-k on the GPSIMD
// engine"; "DeepSelect" project page: a threshold that only rises, early
// rejection of everything below it, and a worst-case guarantee that does not
// depend on the order of the data).
//
// The answer is exact under the order (value desc, index asc): every score
// is mapped to a 64-bit composite (order-preserving value key in the high
// word, complemented position in the low word), so the k largest composites
// are the unique answer. The kernels never sort.
//
// Stage 1, one workgroup per (row, segment). The segment is read from HBM
// straight into registers in blocks of V 16-byte vectors per thread, all
// loads of a block in flight together, and a block's scores become order
// keys when it is taken up (bf16 keys two per 32-bit word). A threshold
// comes cheaply from "group maxima": group (thread t, element e) holds
// element e of every vector of thread t, so its members are spread evenly
// over the block. If at least k groups have a maximum >= T then at least k
// scores are >= T, so T may reject everything below it; one histogram round
// over about 2k group maxima gives such a T. Random rows let a few percent
// through and sorted rows about k, because the spread-out groups see the
// whole range. The first block's groups also take in the blocks already
// loaded behind it (up to two more), so its T covers all of them whatever
// their order, and those blocks are admitted against it. Each vector is
// first tested by its maximum, so most are dismissed with a handful of
// instructions; survivors go to an LDS list in thread order (block prefix
// sum). A later block of a long segment is filtered by the exact k-th
// candidate so far (after the blocks the first T covers, the list is cut
// to its exact top k); if its survivors would
// overflow the list (a row rising along the segment), the block's own group
// maxima give a higher bound, the list is cut to it, and later blocks are
// held to it. Only if that overflows too is the block taken one vector at a
// time with exact selects in between. At most 2k candidates leave the
// segment; more are first cut to exactly k.
//
// Quota form (full rows in a power-of-two number of segments): a segment
// only has to pass on its part of the row's top k, about k/S. It takes
// interleaved 128-byte pieces of the row (so a sorted row spreads its top k
// over all segments), runs everything above with a quota q (about k/S plus
// four standard deviations of a random row's spread) in place of k, keeps at
// most 2q candidates, and reports its cut: every composite it dropped lies
// below it. Stage 2 checks that no cut reaches the row's k-th kept
// composite, which makes the kept set exact, and otherwise selects the row
// again from its scores.
//
// Stage 2, one workgroup per row: load every segment's candidates into
// registers at once, select the row's k-th composite exactly, and write the
// k winners (indices, optional value copies), in buffer order or sorted by
// index.
//
// Exact selection: one histogram round over the candidates' value keys
// (2048 buckets over their actual range) finds the bucket of the K-th
// largest. A bucket of up to 512 entries is gathered and ranked entry
// against entry; a heavier one whose entries tie on one value is resolved by
// position through a bitmap; any other goes to a radix select whose 10-bit
// digits split the remaining range into 1024 equal buckets per round, so
// each round narrows it 1024-fold whatever the value distribution.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "select_k.h"

namespace dsa {
namespace {

constexpr int kTkThreads = 512;    // stage-1 workgroups of a segmented row
constexpr int kRowThreads = 512;   // one workgroup for a whole row
// Rows of at most this many vectors per thread are taken whole by one
// workgroup; for longer rows the per-thread work of one workgroup outweighs
// the second kernel of the segmented path (on the 16 x 32768 float32
// decode-step rows: 16.9 us whole vs 15.7 us segmented; a 1024-thread
// workgroup taking such a row as one block was 1.5 us slower than the
// segmented path inside the decode step).
constexpr int kRowFusedVec = 4;
constexpr int kTkMaxVec = 8;       // vectors per thread per register block
// LDS candidates of a stage-1 workgroup: k (<= 4096) plus one vector of
// every thread (THREADS * 8 bf16).
template <int THREADS>
constexpr int seg_cap() { return 4096 + THREADS * 8; }
constexpr int kMergeCap = 16384;   // candidate slots per row in stage 2

// Quota form of the segmented path: the row is cut into pieces of 128 bytes
// (64 bf16 or 32 float32 scores), and run r of S consecutive pieces gives
// its piece at slot (s + r) mod S to segment s. Every run holds one piece
// of each segment and the order rotates from run to run, so a row sorted
// along its positions spreads its top k evenly over the segments. S is a
// power of two. Positions inside a segment ("local") keep the row's order.
__host__ __device__ __forceinline__ int64_t piece_pos(int64_t l, int s, int log_s, int log_p) {
  const int64_t r = l >> log_p;
  const int64_t j = (s + r) & (((int64_t)1 << log_s) - 1);
  return (((r << log_s) | j) << log_p) | (l & (((int64_t)1 << log_p) - 1));
}
// The number of positions of a row of N that segment s holds.
__host__ __device__ __forceinline__ int64_t piece_seg_len(int64_t N, int s, int log_s, int log_p) {
  const int64_t run = (int64_t)1 << (log_s + log_p);
  const int64_t full = N / run, rem = N % run;
  const int64_t j = (s + full) & (((int64_t)1 << log_s) - 1);
  int64_t extra = rem - (j << log_p);
  extra = extra < 0 ? 0 : extra;
  extra = extra > ((int64_t)1 << log_p) ? ((int64_t)1 << log_p) : extra;
  return (full << log_p) + extra;
}

// Per-half unsigned maximum of two words holding two 16-bit keys each: one
// v_pk_max_u16. (Written as assembly: 16-bit vector element access was
// miscompiled, element 0 being returned for every index, so 16-bit vector
// types are avoided throughout.)
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_u16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}


// Block-wide min and max of the entries of buf[0..cnt) inside [lo, hi];
// every thread gets both. One barrier; the wlo/whi slots are reused only
// after further barriers.
template <int THREADS>
__device__ void bucket_range(const uint64_t* buf, int cnt, uint64_t& lo, uint64_t& hi, Scratch& sc) {
  constexpr int W = THREADS / kWave;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  uint64_t a = ~(uint64_t)0, z = 0;
  for (int i = tid; i < cnt; i += THREADS) {
    const uint64_t e = buf[i];
    if (e >= lo && e <= hi) {
      a = e < a ? e : a;
      z = e > z ? e : z;
    }
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

// Exact: the T for which exactly K of the distinct entries of buf[0..cnt)
// inside [lo, hi] (all of them by default) are >= T (1 <= K <= their
// number). Each round splits the entries' actual range into 1024 equal
// buckets, keeps the bucket holding the K-th largest, and then shrinks the
// range to the entries inside that bucket. Expects both hist halves clear
// behind a barrier and leaves them clear.
template <int THREADS>
__device__ __forceinline__ uint64_t select_exact(const uint64_t* buf, int cnt, int K, Scratch& sc,
                                                 uint64_t lo = 0, uint64_t hi = ~(uint64_t)0) {
  const int tid = threadIdx.x;
  bucket_range<THREADS>(buf, cnt, lo, hi, sc);
  uint32_t need = (uint32_t)K;
  uint64_t result = lo;
  for (int round = 0; round < 8; ++round) {  // 10-bit rounds: 7 narrow any 64-bit range
    const uint64_t range = hi - lo;
    if (range == 0) {
      result = lo;
      break;
    }
    const int hb = 63 - __clzll((long long)range);
    const int shift = hb >= kBinBits ? hb - (kBinBits - 1) : 0;
    uint32_t* cur = sc.hist[round & 1];
    uint32_t* nxt = sc.hist[(round + 1) & 1];
    for (int i = tid; i < cnt; i += THREADS) {
      const uint64_t e = buf[i];
      if (e >= lo && e <= hi) atomicAdd(&cur[(uint32_t)((e - lo) >> shift)], 1u);
    }
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
    bucket_range<THREADS>(buf, cnt, lo, hi, sc);
  }
  lds_barrier();
  return result;
}


// Keep the entries >= thr of buf[0..cnt), in order; returns the new count.
template <int THREADS, int MAXPER>
__device__ __noinline__ int block_compact(uint64_t* buf, int cnt, uint64_t thr, Scratch& sc) {
  const int per = (cnt + THREADS - 1) / THREADS;
  const int lo = min(cnt, (int)threadIdx.x * per);
  const int hi = min(cnt, lo + per);
  uint64_t v[MAXPER];
  uint32_t keep = 0;
#pragma unroll
  for (int j = 0; j < MAXPER; ++j) {
    const int i = lo + j;
    v[j] = (i < hi) ? buf[i] : 0;
    keep += (i < hi && v[j] >= thr) ? 1u : 0u;
  }
  uint32_t total;
  uint32_t pos = block_exclusive_scan<THREADS>(keep, &total, sc);  // orders reads before writes
#pragma unroll
  for (int j = 0; j < MAXPER; ++j) {
    const int i = lo + j;
    if (i < hi && v[j] >= thr) buf[pos++] = v[j];
  }
  lds_barrier();
  return (int)total;
}

// ---------------------------------------------------------------- keys
// bf16: two 16-bit order keys per word, computed on the raw pair. A negative
// half becomes its complement, a non-negative one gets its top bit set. The
// pattern 0xFFFF (used for padding) maps to 0, below every real score. -0.0
// maps to 0x7FFF, one below +0.0; canon16 merges the two.
__device__ __forceinline__ uint32_t bf16_pair_keys(uint32_t w) {
  const uint32_t neg = (w >> 15) & 0x00010001u;
  return w ^ (neg * 0x7FFFu) ^ 0x80008000u;
}
__device__ __forceinline__ uint32_t canon16(uint32_t k16) { return k16 == 0x7FFFu ? 0x8000u : k16; }
// The float32 order key of the bf16 value with (canonical) 16-bit key k16.
__device__ __forceinline__ uint32_t key32_of_key16(uint32_t k16) {
  return (k16 << 16) | (k16 < 0x8000u ? 0xFFFFu : 0u);
}
// float32 keys without the -0 merge (padding 0xFFFFFFFF maps to 0).
__device__ __forceinline__ uint32_t f32_raw_key(uint32_t bits) {
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}
__device__ __forceinline__ uint32_t canon32(uint32_t k) { return k == 0x7FFFFFFFu ? 0x80000000u : k; }

// The raw score bits of a winner, from its composite's value key (the
// inverse of the order key) without reading the row again. Only a zero
// score is read back: the key merged -0 into +0.
template <bool BF16>
__device__ __forceinline__ uint32_t winner_bits(uint64_t c, const char* row, uint32_t p) {
  const uint32_t key = (uint32_t)(c >> 32);
  if (key == 0x80000000u)
    return BF16 ? (uint32_t)reinterpret_cast<const uint16_t*>(row)[p] : reinterpret_cast<const uint32_t*>(row)[p];
  if (BF16) {
    const uint32_t k16 = key >> 16;
    return k16 >= 0x8000u ? (k16 & 0x7FFFu) : (~k16 & 0xFFFFu);
  }
  return key >= 0x80000000u ? (key & 0x7FFFFFFFu) : ~key;
}

template <bool BF16>
__device__ __forceinline__ uint32_t elem_key32(const u32x4& kv, int e) {
  if (BF16) {
    const uint32_t w = kv[e >> 1];
    return key32_of_key16(canon16((e & 1) ? (w >> 16) : (w & 0xFFFFu)));
  }
  return canon32(kv[e]);
}
template <bool BF16>
__device__ __forceinline__ uint32_t elem_rawkey(const u32x4& kv, int e) {
  if (BF16) {
    const uint32_t w = kv[e >> 1];
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
  }
  return kv[e];
}

// One thread's vector of raw scores at row position p0, wholly inside the
// row and 16-byte aligned.
template <bool BF16>
__device__ __forceinline__ u32x4 load_raw_full(const void* row, int64_t p0) {
  const u32x4* src = BF16 ? reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(row) + p0)
                          : reinterpret_cast<const u32x4*>(reinterpret_cast<const uint32_t*>(row) + p0);
  return __builtin_nontemporal_load(src);
}
// The same for any vector: positions past `end` get the padding pattern
// (all ones), whose key is 0. p0 is the vector's position in the segment's
// order (checked against end), g0 the row position it is read from.
template <bool BF16, bool ALIGNED>
__device__ __forceinline__ u32x4 load_raw(const void* row, int64_t p0, int64_t end, int64_t g0) {
  constexpr int E = BF16 ? 8 : 4;
  u32x4 r;
  if (ALIGNED && p0 + E <= end) {
    r = load_raw_full<BF16>(row, g0);
  } else {
    r = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (p0 + e < end) {
        if (BF16) {
          const uint32_t h = reinterpret_cast<const uint16_t*>(row)[g0 + e];
          r[e >> 1] = (e & 1) ? ((r[e >> 1] & 0xFFFFu) | (h << 16)) : ((r[e >> 1] & 0xFFFF0000u) | h);
        } else {
          r[e] = reinterpret_cast<const uint32_t*>(row)[g0 + e];
        }
      }
    }
  }
  return r;
}
// Raw scores -> order keys, in place.
template <bool BF16>
__device__ __forceinline__ void to_keys(u32x4& r) {
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = BF16 ? bf16_pair_keys(r[j]) : f32_raw_key(r[j]);
}

// From below: a T with at least K of the G group maxima per thread (raw
// keys, 0 = none) >= T: the lower edge of the bucket that holds the K-th
// largest maximum, in one histogram round whose 2048 buckets split the
// maxima's actual [lo, hi]; 1 when fewer than K maxima exist. Leaves
// hist[0] clear.
template <int THREADS, int G>
__device__ uint32_t group_threshold(const uint32_t (&g)[G], int K, Scratch& sc) {
  constexpr int W = THREADS / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint32_t lo = 0xFFFFFFFFu, hi = 0, n = 0;
#pragma unroll
  for (int e = 0; e < G; ++e) {
    if (g[e]) {
      lo = min(lo, g[e]);
      hi = max(hi, g[e]);
      ++n;
    }
  }
  n = wave_reduce<OpAdd>(n);
  lo = wave_reduce<OpMin>(lo);
  hi = wave_reduce<OpMax>(hi);
  // wcnt/wmin/wmax are written again only behind later barriers (block
  // scans use wsum), so no second barrier is needed.
  if (lane == 0) {
    sc.wcnt[wave] = n;
    sc.wmin[wave] = lo;
    sc.wmax[wave] = hi;
  }
  lds_barrier();
  n = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    n += sc.wcnt[w];
    lo = min(lo, sc.wmin[w]);
    hi = max(hi, sc.wmax[w]);
  }
  if ((int)n < K) return 1u;  // uniform
  const uint32_t range = hi - lo;
  if (range == 0) return lo;
  const int hb = 31 - __clz(range);
  const int shift = hb >= kHBinBits ? hb - (kHBinBits - 1) : 0;
  uint32_t* h = sc.hist[0];
  // A wave whose first maxima all tie (rows of quantised or sorted scores)
  // takes wave-aggregated counts; checking once per wave keeps the other
  // rows at plain atomics (bf16 stress rows 66.5 -> 62.0 us, float32 88.0 ->
  // 78.6 us; per-count checks cost the bf16 64 x 131072 top-k 0.4-0.7 us).
  if (__ballot(g[0] == (uint32_t)__builtin_amdgcn_readfirstlane(g[0])) == ~0ull) {  // uniform
#pragma unroll
    for (int e = 0; e < G; ++e) hist_add(h, g[e] >= lo ? ((g[e] - lo) >> shift) : kNoBin);
  } else {
#pragma unroll
    for (int e = 0; e < G; ++e)
      if (g[e] >= lo) atomicAdd(&h[(g[e] - lo) >> shift], 1u);
  }
  lds_barrier();
  uint32_t digit, above, in_bucket;
  pick_digit<kHBins>(h, (uint32_t)K, sc, digit, above, in_bucket);
  for (int i = threadIdx.x; i < kHBins; i += THREADS) h[i] = 0;  // ordered by later barriers
  return lo + (digit << shift);
}

// The admitted scores of this thread's vectors as composites at cand[at...],
// in (vector, element) order; pos_of maps a vector's position in the
// segment's order to the one the composite carries.
struct SamePos {
  __device__ int64_t operator()(int64_t p) const { return p; }
};
template <bool BF16, int V, int THREADS, typename PosOf = SamePos>
__device__ __forceinline__ void write_admitted(uint64_t* cand, uint32_t at, const u32x4 (&kv)[V],
                                               uint64_t adm, int64_t base, PosOf pos_of = PosOf{}) {
  constexpr int E = BF16 ? 8 : 4;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    uint32_t m = (uint32_t)(adm >> (v * E)) & ((1u << E) - 1u);
    const int64_t p0 = pos_of(base + ((int64_t)v * THREADS + threadIdx.x) * E);
    while (m) {
      const int e = __ffs(m) - 1;
      m &= m - 1;
      uint32_t key;
      if (BF16) {
        const uint32_t w = kv[v][e >> 1];
        key = key32_of_key16(canon16((e & 1) ? (w >> 16) : (w & 0xFFFFu)));
      } else {
        key = canon32(kv[v][e]);
      }
      cand[at++] = composite(key, (uint32_t)(p0 + e));
    }
  }
}

// Admission bits of vector v: raw key >= t0 and, when have_thr, composite > thr.
template <bool BF16>
__device__ __forceinline__ uint32_t admit_vector(const u32x4& kv, uint32_t t0, bool have_thr,
                                                 uint64_t thr, int64_t p0) {
  constexpr int E = BF16 ? 8 : 4;
  uint32_t vmax;
  if (BF16) {
    const uint32_t m = max_u16x2(max_u16x2(kv[0], kv[1]), max_u16x2(kv[2], kv[3]));
    vmax = max(m & 0xFFFFu, m >> 16);
  } else {
    vmax = max(max(kv[0], kv[1]), max(kv[2], kv[3]));
  }
  uint32_t bits = 0;
  if (vmax >= t0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      bool ok = elem_rawkey<BF16>(kv, e) >= t0;
      if (have_thr && ok) ok = composite(elem_key32<BF16>(kv, e), (uint32_t)(p0 + e)) > thr;
      bits |= ok ? (1u << e) : 0u;
    }
  }
  return bits;
}

// The K-th largest of the distinct composites buf[0..cnt) (K < cnt), as a
// threshold: exactly K entries are >= it. One histogram round over the
// value keys (2048 buckets over their actual range) finds its bucket; a
// bucket that is not taken whole is gathered into a list and ranked entry
// against entry; a bucket of more than THREADS entries (heavy ties) takes
// the general select, except when all of its entries tie on one value: then
// the K-th is the entry of that value with the need-th smallest position,
// found through a bitmap of positions (entries lie in [pos0, pos0 + npos);
// npos <= 65536). Expects both histograms clear and leaves them dirty.
template <int THREADS>
__device__ __noinline__ uint64_t select_k_lds(const uint64_t* buf, int cnt, int K, Scratch& sc,
                                              uint32_t pos0, uint32_t npos) {
  constexpr int W = THREADS / kWave;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
  for (int i = tid; i < cnt; i += THREADS) {
    const uint32_t key = (uint32_t)(buf[i] >> 32);
    lo = min(lo, key);
    hi = max(hi, key);
  }
  lo = wave_reduce<OpMin>(lo);
  hi = wave_reduce<OpMax>(hi);
  if (lane == 0) {
    sc.wmin[wave] = lo;
    sc.wmax[wave] = hi;
  }
  if (tid == 0) sc.n_app = 0;
  lds_barrier();
#pragma unroll
  for (int w = 0; w < W; ++w) {
    lo = min(lo, sc.wmin[w]);
    hi = max(hi, sc.wmax[w]);
  }
  const uint32_t range = hi - lo;
  const int shift = range == 0 ? 0 : max(0, 31 - __clz(range) - (kHBinBits - 1));
  uint32_t* h = sc.hist[0];
  // Wave-aggregated counts: an exact cut runs over rows of many tied scores
  // (stress rows) as often as over others, and costs the same otherwise.
  for (int i = tid; i < cnt; i += THREADS) hist_add(h, ((uint32_t)(buf[i] >> 32) - lo) >> shift);
  lds_barrier();
  uint32_t digit, above, in_bucket;
  pick_digit<kHBins>(h, (uint32_t)K, sc, digit, above, in_bucket);
  const uint32_t need = (uint32_t)K - above;
  const uint32_t blo = lo + (digit << shift);
  if (in_bucket == need) return (uint64_t)blo << 32;  // the whole bucket is in (uniform)
  if (in_bucket <= (uint32_t)THREADS && in_bucket <= (uint32_t)(kHBins / 2)) {
    uint64_t* list = reinterpret_cast<uint64_t*>(sc.hist[1]);  // kHBins / 2 entries
    for (int i = tid; i < cnt; i += THREADS) {
      const uint64_t x = buf[i];
      if ((((uint32_t)(x >> 32) - lo) >> shift) == digit) list[atomicAdd(&sc.n_app, 1u)] = x;
    }
    const uint32_t n8 = (in_bucket + 7u) & ~7u;
    if ((uint32_t)tid >= in_bucket && (uint32_t)tid < n8) list[tid] = 0;
    lds_barrier();
    if (tid < (int)in_bucket) {
      const uint64_t x = list[tid];
      const uint32_t r = count_above(list, n8, x);
      if (r == need - 1) sc.pick = x;  // exactly one entry has this rank
    }
    lds_barrier();
    return sc.pick;
  }
  // A heavy bucket (many ties): the K-th largest is the need-th largest of
  // the bucket's own entries.
  for (int i = tid; i < kHBins; i += THREADS) h[i] = 0;  // ordered by the next barrier
  const uint64_t bhi = min((uint64_t)hi, (uint64_t)blo + (((uint64_t)1 << shift) - 1));
  uint64_t clo = (uint64_t)blo << 32, chi = (bhi << 32) | 0xFFFFFFFFull;
  bucket_range<THREADS>(buf, cnt, clo, chi, sc);
  if ((uint32_t)(clo >> 32) == (uint32_t)(chi >> 32) && npos <= 32u * kHBins) {  // uniform
    // One value: larger composites are smaller positions, so the answer is
    // the tied entry with the need-th smallest position.
    constexpr int WPT = kHBins / THREADS;  // bitmap words per thread
    const uint32_t val = (uint32_t)(clo >> 32);
    for (int i = tid; i < cnt; i += THREADS) {
      const uint64_t x = buf[i];
      if ((uint32_t)(x >> 32) == val) {
        const uint32_t p = composite_pos(x) - pos0;
        atomicOr(&h[p >> 5], 1u << (p & 31));
      }
    }
    lds_barrier();
    uint32_t w[WPT], c = 0;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      w[j] = h[tid * WPT + j];
      c += __popc(w[j]);
    }
    uint32_t before_total;
    const uint32_t before = block_exclusive_scan<THREADS>(c, &before_total, sc);
    if (before < need && need <= before + c) {
      uint32_t r = need - before;  // 1-based rank inside this thread's words
#pragma unroll
      for (int j = 0; j < WPT; ++j) {
        const uint32_t pc = __popc(w[j]);
        if (r > 0 && r <= pc) {
          uint32_t m = w[j];
          for (uint32_t q = 1; q < r; ++q) m &= m - 1;  // drop the r-1 lowest set bits
          const uint32_t p = (uint32_t)(tid * WPT + j) * 32u + (uint32_t)(__ffs(m) - 1);
          sc.pick = composite(val, pos0 + p);
          r = 0;
        } else if (r > 0) {
          r -= pc;
        }
      }
    }
    lds_barrier();
    return sc.pick;
  }
  return select_exact<THREADS>(buf, cnt, (int)need, sc, clo, chi);
}

// FUSED (one segment covering the whole row): after stage 1 the workgroup
// also selects the row's k winners from its LDS candidates and writes them,
// so no stage 2 runs.
// Output slots [from, k) of a row that has fewer than k valid positions
// (ragged rows): index -1 and, when values are returned, negative infinity.
template <bool BF16, int THREADS>
__device__ __forceinline__ void pad_row(int32_t* oi, void* out_val, size_t out_off, int from, int k) {
  for (int i = from + (int)threadIdx.x; i < k; i += THREADS) {
    oi[i] = -1;
    if (out_val) {
      if (BF16) reinterpret_cast<uint16_t*>(out_val)[out_off + i] = 0xFF80u;
      else reinterpret_cast<uint32_t*>(out_val)[out_off + i] = 0xFF800000u;
    }
  }
}

template <bool BF16, int kPer, int THREADS>
__device__ void write_winners_from_lds(const uint64_t* cand, int cnt, uint64_t thr, const char* row,
                                       int N, int k, int32_t* oi, void* out_val, size_t out_off,
                                       int sorted_index, uint32_t* pos_lds, Scratch& sc);

// QUOTA (full rows, segs a power of two): segment sidx takes the pieces the
// rotation assigns it (positions in the kernel are local to the segment),
// keeps at least its `quota` largest scores, at most `slots`, and writes its
// cut to tcut_out: every composite it dropped lies below it.
template <bool BF16, bool ALIGNED, int V, int THREADS, bool FUSED, bool QUOTA>
__global__ __launch_bounds__(THREADS) void topk_segment_kernel(
    const void* __restrict__ scores, int N, int k, int seg_len, int segs,
    uint64_t* __restrict__ cand_out, uint32_t* __restrict__ cnt_out,
    int32_t* __restrict__ out_idx, void* __restrict__ out_val, int sorted_index,
    const int32_t* __restrict__ lengths, int quota, int slots, uint64_t* __restrict__ tcut_out) {
  constexpr int E = BF16 ? 8 : 4;
  constexpr int CAP = seg_cap<THREADS>();
  constexpr int kLogPiece = BF16 ? 6 : 5;
  static_assert(V * E <= 64, "the admission mask holds 64 bits");
  static_assert(!(FUSED && QUOTA), "a whole row has no segments");
  extern __shared__ uint64_t cand[];  // CAP entries
  __shared__ Scratch sc;
  const int b = blockIdx.y;
  const int sidx = blockIdx.x;
  const size_t esz = BF16 ? 2 : 4;
  const void* row = reinterpret_cast<const char*>(scores) + (size_t)b * (size_t)N * esz;
  const int log_s = QUOTA ? __ffs(segs) - 1 : 0;
  const int64_t seg_start = QUOTA ? 0 : (int64_t)sidx * seg_len;
  // Ragged rows: positions at or past the row's length take no part.
  const int64_t row_end = lengths ? (int64_t)min(max(lengths[b], 0), N) : (int64_t)N;
  const int64_t seg_end = QUOTA ? piece_seg_len(N, sidx, log_s, kLogPiece) : min(row_end, seg_start + seg_len);
  // The row position of a segment position.
  auto row_pos = [sidx, log_s](int64_t p) -> int64_t {
    return QUOTA ? piece_pos(p, sidx, log_s, kLogPiece) : p;
  };
  // The count a segment keeps above its cut, and its output slots.
  const int kk = QUOTA ? quota : k;
  const int out_cap = QUOTA ? slots : 2 * k;
  // The raw-key threshold t as the smallest composite of its value.
  auto value_floor = [](uint32_t t) -> uint64_t {
    return (uint64_t)(BF16 ? key32_of_key16(canon16(t)) : canon32(t)) << 32;
  };
  // QUOTA: the largest bound below which composites were dropped so far.
  uint64_t tc = 0;
  constexpr int64_t kBlock = (int64_t)THREADS * V * E;
  if (seg_end <= seg_start) {  // nothing valid in this segment (uniform)
    if (FUSED) pad_row<BF16, THREADS>(out_idx + (size_t)b * k, out_val, (size_t)b * k, 0, k);
    else if (threadIdx.x == 0) {
      cnt_out[(size_t)b * segs + sidx] = 0;
      if (QUOTA) tcut_out[(size_t)b * segs + sidx] = 0;
    }
    return;
  }

  for (int i = threadIdx.x; i < kHBins; i += THREADS) {
    sc.hist[0][i] = 0;
    sc.hist[1][i] = 0;
  }
  int cnt = 0;
  bool have_thr = false;
  uint64_t thr = 0;  // once set: admit only composites > thr
  uint32_t t_floor = 0;  // raw key that the segment's k-th largest is known to reach
  // The first block's threshold is taken over the group maxima of every
  // block already loaded (up to three): a group then spans those blocks, so
  // the bound does not depend on their order (a row rising along the
  // segment no longer sets it from its lowest block), and the following
  // blocks it covers are admitted against it with no threshold of their own.
  int cover = 0;        // following blocks the first block's threshold covers
  // QUOTA: the first threshold was extended over every block of the segment
  // (no exact cut after the blocks it was taken on; see below).
  bool extended = false;
  uint32_t pair_t = 0;  // that threshold (raw key)

  // Register blocks of THREADS*V*E scores. The first block sets a threshold
  // from its group maxima and is cut to its exact top k; later blocks are
  // only filtered against that k-th composite (which every later winner must
  // beat).
  //
  // A block wholly inside the segment (all but possibly the last) is read
  // by straight-line 16-byte loads, so all of them are in flight before the
  // first is used; scores become keys only when the block is taken up.
  // Blocks are loaded into a ring of three register buffers, two blocks
  // ahead of the one being taken up, so a block's loads have two blocks'
  // processing time to land. (Rotating names through an unrolled loop keeps
  // the buffers in place: a register copy of a block still in flight would
  // wait for it.)
  auto load_block = [&](u32x4 (&r)[V], int64_t at) __attribute__((always_inline)) {
    if (ALIGNED && at + kBlock <= seg_end) {  // uniform
#pragma unroll
      for (int v = 0; v < V; ++v) r[v] = load_raw_full<BF16>(row, row_pos(at + ((int64_t)v * THREADS + threadIdx.x) * E));
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int64_t p = at + ((int64_t)v * THREADS + threadIdx.x) * E;
        r[v] = load_raw<BF16, ALIGNED>(row, p, seg_end, row_pos(p));
      }
    }
  };
  // Takes up the block held in kv, at row position base; true when the
  // segment is finished (its survivors written straight to the workspace).
  // fold: how many of the loaded blocks nx, nx2 (raw scores) the first
  // block's threshold also covers.
  auto take_block = [&](u32x4 (&kv)[V], int64_t base, const u32x4 (&nx)[V], const u32x4 (&nx2)[V],
                        int fold) __attribute__((always_inline)) -> bool {
#pragma unroll
    for (int v = 0; v < V; ++v) to_keys<BF16>(kv[v]);
    const int fold_now = (!have_thr && cover == 0) ? fold : 0;
    // The E group maxima over vectors [v0, v1) of this thread, as raw keys,
    // into g[0..E).
    auto group_maxima = [&](uint32_t* g, int v0, int v1) __attribute__((always_inline)) {
      if (BF16) {
        uint32_t m[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) m[j] = kv[v0][j];
#pragma unroll
        for (int v = v0 + 1; v < v1; ++v)
#pragma unroll
          for (int j = 0; j < 4; ++j) m[j] = max_u16x2(m[j], kv[v][j]);
        if (fold_now > 0) {  // uniform
#pragma unroll
          for (int v = v0; v < v1; ++v)
#pragma unroll
            for (int j = 0; j < 4; ++j) m[j] = max_u16x2(m[j], bf16_pair_keys(nx[v][j]));
        }
        if (fold_now > 1) {  // uniform
#pragma unroll
          for (int v = v0; v < v1; ++v)
#pragma unroll
            for (int j = 0; j < 4; ++j) m[j] = max_u16x2(m[j], bf16_pair_keys(nx2[v][j]));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          g[2 * j] = m[j] & 0xFFFFu;
          g[2 * j + 1] = m[j] >> 16;
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          g[e] = kv[v0][e];
#pragma unroll
          for (int v = v0 + 1; v < v1; ++v) g[e] = max(g[e], kv[v][e]);
          if (fold_now > 0) {  // uniform
#pragma unroll
            for (int v = v0; v < v1; ++v) g[e] = max(g[e], f32_raw_key(nx[v][e]));
          }
          if (fold_now > 1) {  // uniform
#pragma unroll
            for (int v = v0; v < v1; ++v) g[e] = max(g[e], f32_raw_key(nx2[v][e]));
          }
        }
      }
    };
    // A threshold from this block's group maxima (raw keys): at least k
    // scores of the block, hence of the segment, are >= it. A group is
    // element e of every vector of this thread or, when k asks for more
    // groups than that, of every vector in one of S equal parts of them.
    constexpr uint32_t kNegZero = BF16 ? 0x8000u : 0x80000000u;
    auto split_threshold = [&](auto parts) __attribute__((always_inline)) -> uint32_t {
      constexpr int S = decltype(parts)::value;
      uint32_t gs[S * E];
#pragma unroll
      for (int p = 0; p < S; ++p) group_maxima(gs + p * E, p * (V / S), (p + 1) * (V / S));
      uint32_t t = group_threshold<THREADS, S * E>(gs, kk, sc);
      if (t == kNegZero) t -= 1;
      return t;
    };
    auto block_threshold = [&]() __attribute__((always_inline)) -> uint32_t {
      // About 2k groups: fewer, larger groups cost fewer histogram atomics
      // and still leave a threshold near the k-th largest score; with fewer
      // than k groups the threshold would admit the whole block. (With
      // k <= 4096 and 512 threads, 2k groups take at most 4E per thread for
      // float32 and 2E for bf16.) bf16 segments in quota form take about 4k
      // groups: a finer threshold on rows of tied levels (bf16 stress rows
      // 34.7 -> 28.8 us; float32 rows, which would need the split, were 1 us
      // slower with it).
      const int gpt = ((BF16 && QUOTA ? 4 : 2) * kk + THREADS - 1) / THREADS;  // wanted groups per thread
      if constexpr (!BF16 && V >= 4) {
        if (gpt > 2 * E) return split_threshold(std::integral_constant<int, 4>{});  // uniform
      }
      if constexpr (V >= 2) {
        if (gpt > E) return split_threshold(std::integral_constant<int, 2>{});  // uniform
      }
      uint32_t g[E];
      group_maxima(g, 0, V);
      // Fold the E maxima per thread in halves (a zero slot means "no
      // group") while half of them still give 2k groups.
#pragma unroll
      for (int half = E / 2; half >= 1; half /= 2) {
        if (gpt <= half) {  // uniform
#pragma unroll
          for (int j = 0; j < half; ++j) {
            g[j] = max(g[j], g[j + half]);
            g[j + half] = 0;
          }
        }
      }
      uint32_t t = group_threshold<THREADS, E>(g, kk, sc);
      // Raw keys place -0 one below +0; admitting from one lower keeps the tie.
      if (t == kNegZero) t -= 1;
      return t;
    };
    auto admit_block = [&](uint32_t t) __attribute__((always_inline)) -> uint64_t {
      uint64_t a = 0;
#pragma unroll
      for (int v = 0; v < V; ++v)
        a |= (uint64_t)admit_vector<BF16>(kv[v], t, false, thr,
                                          base + ((int64_t)v * THREADS + threadIdx.x) * E)
             << (v * E);
      return a;
    };
    uint32_t t0;
    if (have_thr) {
      // Raw-key bound of the k-th composite for the vector test.
      const uint32_t key32 = (uint32_t)(thr >> 32);
      t0 = BF16 ? (key32 >> 16) : key32;
      if (t0 == (BF16 ? 0x8000u : 0x80000000u)) t0 -= 1;
      t0 = max(t0, t_floor);
    } else if (cover > 0) {
      // The first block's threshold holds for this block too (raised by a
      // later block's own threshold, if one was taken).
      t0 = max(pair_t, t_floor);
      --cover;
    } else {
      t0 = block_threshold();
      if (fold_now > 0) {
        pair_t = t0;
        cover = fold_now;
      }
    }
    // Admission: raw key >= t0. Once an exact threshold exists, t0 is its
    // value key, so ties at that value are admitted too (harmless extra
    // candidates; the position test is left to the overflow path below).
    uint64_t adm = admit_block(t0);
    uint32_t total;
    uint32_t excl = block_exclusive_scan<THREADS>((uint32_t)__popcll(adm), &total, sc);
    if (__builtin_expect((have_thr || extended) && cnt + (int)total > CAP, 0)) {
      // A later block that beats the running threshold almost everywhere
      // (a row rising along the segment): its own group maxima give a
      // higher bound, and the segment's k-th largest is at least that.
      // Listed candidates below it can go, and later blocks are held to it.
      const uint32_t t2 = block_threshold();
      if (t2 > t0) {  // uniform
        t0 = t2;
        t_floor = t2;
        adm = admit_block(t0);
        excl = block_exclusive_scan<THREADS>((uint32_t)__popcll(adm), &total, sc);
        lds_barrier();  // every thread has read the scan's totals
        cnt = block_compact<THREADS, CAP / THREADS>(cand, cnt, value_floor(t2), sc);
      }
    }
    // Everything this block drops lies below t0's value (or below an exact
    // cut already taken into tc).
    if (QUOTA) tc = max(tc, value_floor(t0));
    if (!FUSED && base == seg_start && base + kBlock >= seg_end && (int)total <= out_cap) {
      // The whole segment in one block and its survivors fit the output
      // slots: write them straight to the workspace.
      write_admitted<BF16, V, THREADS>(cand_out + ((size_t)b * segs + sidx) * (size_t)out_cap, excl, kv,
                                       adm, base, row_pos);
      if (threadIdx.x == 0) {
        cnt_out[(size_t)b * segs + sidx] = total;
        if (QUOTA) tcut_out[(size_t)b * segs + sidx] = tc;  // a value bound: no position to map
      }
      return true;
    }
    if (cnt + (int)total <= CAP) {
      write_admitted<BF16, V, THREADS>(cand, (uint32_t)cnt + excl, kv, adm, base);
      cnt += (int)total;
      lds_barrier();
    } else {
      // Too many survivors: one vector at a time (each adds at most
      // THREADS*E entries), with an exact select whenever the next might not
      // fit; each vector is filtered against the thresholds current at its
      // turn.
#pragma unroll
      for (int v = 0; v < V; ++v) {
        if (cnt + THREADS * E > CAP && cnt > kk) {
          const uint64_t t = select_k_lds<THREADS>(cand, cnt, kk, sc, (uint32_t)seg_start, (uint32_t)(seg_end - seg_start));
          if (QUOTA) tc = max(tc, t);
          cnt = block_compact<THREADS, CAP / THREADS>(cand, cnt, t, sc);
          for (int i = threadIdx.x; i < kHBins; i += THREADS) {
            sc.hist[0][i] = 0;
            sc.hist[1][i] = 0;
          }
          lds_barrier();
          thr = t - 1;  // t > 0: real composites have a non-zero high word
          have_thr = true;
        }
        const int64_t p0 = base + ((int64_t)v * THREADS + threadIdx.x) * E;
        const uint64_t vbits = (uint64_t)admit_vector<BF16>(kv[v], t0, have_thr, thr, p0) << (v * E);
        uint32_t vt;
        const uint32_t vx = block_exclusive_scan<THREADS>((uint32_t)__popcll(vbits), &vt, sc);
        write_admitted<BF16, V, THREADS>(cand, (uint32_t)cnt + vx, kv, vbits, base);
        cnt += (int)vt;
        lds_barrier();
      }
    }
    // After the first block: cut to the exact top k so that later blocks
    // are filtered by the k-th composite.
    // Quota form: when the candidates listed so far, scaled to the whole
    // segment, still fit the output slots, the first threshold is kept for
    // the remaining blocks instead (it is a bound for the segment: at least
    // kk of the blocks it was taken on reach it), which saves the exact cut;
    // the final cut to the slots runs only if the list outgrows them.
    if (QUOTA && !have_thr && cover == 0 && !extended && base + kBlock < seg_end) {
      const int64_t done = (base - seg_start) / kBlock + 1;
      const int64_t all = (seg_end - seg_start + kBlock - 1) / kBlock;
      if ((int64_t)cnt * all <= (int64_t)out_cap * done) {  // uniform
        cover = (int)(all - done);
        extended = true;
      }
    }
    if (base + kBlock < seg_end && cnt > kk && !have_thr && cover == 0) {
      const uint64_t t = select_k_lds<THREADS>(cand, cnt, kk, sc, (uint32_t)seg_start, (uint32_t)(seg_end - seg_start));
      if (QUOTA) tc = max(tc, t);
      cnt = block_compact<THREADS, CAP / THREADS>(cand, cnt, t, sc);
      for (int i = threadIdx.x; i < kHBins; i += THREADS) {
        sc.hist[0][i] = 0;
        sc.hist[1][i] = 0;
      }
      lds_barrier();
      thr = t - 1;
      have_thr = true;
    }
    return false;
  };
  if constexpr (FUSED) {
    // A whole row is one register block (the plan sizes V so).
    u32x4 ka[V];
    load_block(ka, seg_start);
    take_block(ka, seg_start, ka, ka, 0);
  } else {
    u32x4 ka[V], kb[V], kc[V];
    load_block(ka, seg_start);
    if (seg_start + kBlock < seg_end) load_block(kb, seg_start + kBlock);
    for (int64_t base = seg_start; base < seg_end; base += 3 * kBlock) {
      if (base + 2 * kBlock < seg_end) load_block(kc, base + 2 * kBlock);
      if (take_block(ka, base, kb, kc, base != seg_start ? 0 : (base + 2 * kBlock < seg_end ? 2 : (base + kBlock < seg_end ? 1 : 0)))) return;
      if (base + kBlock >= seg_end) break;
      if (base + 3 * kBlock < seg_end) load_block(ka, base + 3 * kBlock);
      if (take_block(kb, base + kBlock, kc, ka, 0)) return;
      if (base + 2 * kBlock >= seg_end) break;
      if (base + 4 * kBlock < seg_end) load_block(kb, base + 4 * kBlock);
      if (take_block(kc, base + 2 * kBlock, ka, kb, 0)) return;
    }
  }
  if (FUSED) {
    // The row's candidates are all here: select the k winners and write them.
    const uint64_t t = cnt > k ? select_k_lds<THREADS>(cand, cnt, k, sc, (uint32_t)seg_start, (uint32_t)(seg_end - seg_start)) : (uint64_t)0;
    write_winners_from_lds<BF16, CAP / THREADS, THREADS>(
        cand, cnt, t, reinterpret_cast<const char*>(row), N, k, out_idx + (size_t)b * k, out_val,
        (size_t)b * k, sorted_index, reinterpret_cast<uint32_t*>(cand + CAP), sc);
    return;
  }
  // At most 2k candidates leave the segment (more are cut to exactly k); in
  // quota form at most `slots` (more are cut to exactly that many).
  if (cnt > out_cap) {
    const uint64_t t = select_k_lds<THREADS>(cand, cnt, QUOTA ? out_cap : k, sc, (uint32_t)seg_start,
                                             (uint32_t)(seg_end - seg_start));
    cnt = block_compact<THREADS, CAP / THREADS>(cand, cnt, t, sc);
    if (QUOTA) tc = max(tc, t);
  }
  cnt = min(cnt, out_cap);
  // Quota form: composites leave with row positions (the map keeps the
  // order of a segment's positions, so every comparison inside the segment,
  // the cut's included, comes out the same).
  auto to_row = [&](uint64_t x) -> uint64_t {
    if (!QUOTA || (uint32_t)x == 0u) return x;  // a value bound carries no position
    return (x & 0xFFFFFFFF00000000ull) | (uint64_t)(0xFFFFFFFFu - (uint32_t)row_pos(composite_pos(x)));
  };
  uint64_t* out = cand_out + ((size_t)b * segs + sidx) * (size_t)out_cap;
  for (int i = threadIdx.x; i < cnt; i += THREADS) out[i] = to_row(cand[i]);
  if (threadIdx.x == 0) {
    cnt_out[(size_t)b * segs + sidx] = (uint32_t)cnt;
    if (QUOTA) tcut_out[(size_t)b * segs + sidx] = to_row(tc);
  }
}

// The winners (entries >= thr, exactly k of them, or all cnt <= k) of an
// LDS candidate list: indices (and value copies) in list order, or sorted
// by index through pos_lds (P = next power of two >= k entries).
template <bool BF16, int kPer, int THREADS>
__device__ void write_winners_from_lds(const uint64_t* cand, int cnt, uint64_t thr, const char* row,
                                       int N, int k, int32_t* oi, void* out_val, size_t out_off,
                                       int sorted_index, uint32_t* pos_lds, Scratch& sc) {
  const int tid = threadIdx.x;
  // Thread t takes entries [t*per, t*per + per).
  const int per = (cnt + THREADS - 1) / THREADS;
  const int lo = min(cnt, tid * per);
  const int hi = min(cnt, lo + per);
  uint64_t v[kPer];
  uint32_t keep = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = lo + j;
    v[j] = (i < hi) ? cand[i] : 0;
    keep += (i < hi && v[j] >= thr) ? 1u : 0u;
  }
  uint32_t nkeep;
  uint32_t pos = block_exclusive_scan<THREADS>(keep, &nkeep, sc);
  if (!sorted_index) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (lo + j < hi && v[j] >= thr && pos < (uint32_t)k) {
        const uint32_t p = min(composite_pos(v[j]), (uint32_t)(N - 1));
        oi[pos] = (int32_t)p;
        if (out_val) {
          const uint32_t bits = winner_bits<BF16>(v[j], row, p);
          if (BF16) reinterpret_cast<uint16_t*>(out_val)[out_off + pos] = (uint16_t)bits;
          else reinterpret_cast<uint32_t*>(out_val)[out_off + pos] = bits;
        }
        ++pos;
      }
    }
    pad_row<BF16, THREADS>(oi, out_val, out_off, (int)min(nkeep, (uint32_t)k), k);
    return;
  }
  int P = 1;
  while (P < k) P <<= 1;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (lo + j < hi && v[j] >= thr && pos < (uint32_t)k) pos_lds[pos++] = min(composite_pos(v[j]), (uint32_t)(N - 1));
  for (int i = (int)min(nkeep, (uint32_t)k) + tid; i < P; i += THREADS) pos_lds[i] = 0xFFFFFFFFu;
  lds_barrier();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < P / 2; t += THREADS) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool up = ((i & size) == 0);
        const uint32_t x = pos_lds[i], y = pos_lds[j];
        if ((x > y) == up) {
          pos_lds[i] = y;
          pos_lds[j] = x;
        }
      }
      lds_barrier();
    }
  }
  const int nout = (int)min(nkeep, (uint32_t)k);
  for (int i = tid; i < nout; i += THREADS) {
    const uint32_t p = pos_lds[i];
    oi[i] = (int32_t)p;
    if (out_val) {
      if (BF16) reinterpret_cast<uint16_t*>(out_val)[out_off + i] = reinterpret_cast<const uint16_t*>(row)[p];
      else reinterpret_cast<uint32_t*>(out_val)[out_off + i] = reinterpret_cast<const uint32_t*>(row)[p];
    }
  }
  pad_row<BF16, THREADS>(oi, out_val, out_off, nout, k);
}

template <bool BF16, int kPer, bool CUT = false>  // kPer: candidate slots per thread (segs * slots <= 512 * kPer)
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(
    const void* __restrict__ scores, int N, int k, int segs, int slots,
    const uint64_t* __restrict__ cand_in, const uint32_t* __restrict__ cnt_in,
    const uint64_t* __restrict__ tcut_in,
    int32_t* __restrict__ out_idx, void* __restrict__ out_val, int sorted_index) {
  extern __shared__ uint32_t pos_lds[];  // k positions (sorted path)
  __shared__ Scratch sc;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  uint64_t v[kPer];
  uint64_t thr;
  uint32_t pos, nkeep;
  int32_t* oi = out_idx + (size_t)b * k;
  const size_t esz = BF16 ? 2 : 4;
  const char* row = reinterpret_cast<const char*>(scores) + (size_t)b * (size_t)N * esz;
  if (!merge_candidates<kPer, CUT>(cand_in + (size_t)b * segs * slots, cnt_in + (size_t)b * segs,
                                   CUT ? tcut_in + (size_t)b * segs : nullptr, segs, slots, k, sc,
                                   v, thr, pos, nkeep)) {
    // The row again from its scores; winners come in ascending position
    // order, which is also the sorted-by-index order.
    row_topk_from_scores<BF16>(row, N, k,
                               [oi, out_val, row, b, k](uint32_t at, int i) {
                                 oi[at] = i;
                                 if (out_val) {
                                   if (BF16) reinterpret_cast<uint16_t*>(out_val)[(size_t)b * k + at] = reinterpret_cast<const uint16_t*>(row)[i];
                                   else reinterpret_cast<uint32_t*>(out_val)[(size_t)b * k + at] = reinterpret_cast<const uint32_t*>(row)[i];
                                 }
                               },
                               sc);
    return;
  }
  if (!sorted_index) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (v[j] && v[j] >= thr && pos < (uint32_t)k) {
        const uint32_t p = min(composite_pos(v[j]), (uint32_t)(N - 1));
        oi[pos] = (int32_t)p;
        if (out_val) {
          const uint32_t bits = winner_bits<BF16>(v[j], row, p);
          if (BF16) reinterpret_cast<uint16_t*>(out_val)[(size_t)b * k + pos] = (uint16_t)bits;
          else reinterpret_cast<uint32_t*>(out_val)[(size_t)b * k + pos] = bits;
        }
        ++pos;
      }
    }
    // A ragged row with fewer than k valid positions: -1 in the rest.
    pad_row<BF16, kMergeThreads>(oi, out_val, (size_t)b * k, (int)min(nkeep, (uint32_t)k), k);
    return;
  }
  // Sorted by index: the winners' positions go to LDS, padded to a power of
  // two, then a bitonic sort.
  int P = 1;
  while (P < k) P <<= 1;
  const int nout = (int)min(nkeep, (uint32_t)k);
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (v[j] && v[j] >= thr && pos < (uint32_t)k) pos_lds[pos++] = min(composite_pos(v[j]), (uint32_t)(N - 1));
  for (int i = nout + tid; i < P; i += kMergeThreads) pos_lds[i] = 0xFFFFFFFFu;
  lds_barrier();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < P / 2; t += kMergeThreads) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool up = ((i & size) == 0);
        const uint32_t x = pos_lds[i], y = pos_lds[j];
        if ((x > y) == up) {
          pos_lds[i] = y;
          pos_lds[j] = x;
        }
      }
      lds_barrier();
    }
  }
  for (int i = tid; i < nout; i += kMergeThreads) {
    const uint32_t p = pos_lds[i];
    oi[i] = (int32_t)p;
    if (out_val) {
      if (BF16) reinterpret_cast<uint16_t*>(out_val)[(size_t)b * k + i] = reinterpret_cast<const uint16_t*>(row)[p];
      else reinterpret_cast<uint32_t*>(out_val)[(size_t)b * k + i] = reinterpret_cast<const uint32_t*>(row)[p];
    }
  }
  pad_row<BF16, kMergeThreads>(oi, out_val, (size_t)b * k, nout, k);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  // These workgroups use more than 64 KB of LDS (gfx950 has 160 KB per CU).
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Stage-1 launch state: the workspace lists and the launch's options.
struct Stage1Args {
  uint64_t* cand;
  uint32_t* cnt;
  uint64_t* tcut;  // quota form only
  int32_t* out_idx;
  void* out_val;
  int sorted_index;
  const int32_t* lengths;
};

template <bool BF16, bool AL, int V, int THREADS, bool FUSED, bool QUOTA>
hipError_t launch_seg(const void* scores, int B, int N, int k, const TopkPlan& p, const Stage1Args& a,
                      hipStream_t st) {
  int P = 1;
  while (P < k) P <<= 1;
  const size_t lds = (size_t)seg_cap<THREADS>() * sizeof(uint64_t) + (FUSED ? (size_t)P * sizeof(uint32_t) : 0);
  auto kern = topk_segment_kernel<BF16, AL, V, THREADS, FUSED, QUOTA>;
  hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.segs, B), dim3(THREADS), lds, st, scores, N, k, p.seg_len, p.segs,
                     a.cand, a.cnt, a.out_idx, a.out_val, a.sorted_index, a.lengths, p.quota, p.slots,
                     a.tcut);
  return hipGetLastError();
}

template <bool BF16, bool AL, int THREADS, bool FUSED, bool QUOTA>
hipError_t launch_seg_v(const void* scores, int B, int N, int k, const TopkPlan& p, const Stage1Args& a,
                        hipStream_t st) {
  switch (p.vec) {
    case 1: return launch_seg<BF16, AL, 1, THREADS, FUSED, QUOTA>(scores, B, N, k, p, a, st);
    case 2: return launch_seg<BF16, AL, 2, THREADS, FUSED, QUOTA>(scores, B, N, k, p, a, st);
    case 4: return launch_seg<BF16, AL, 4, THREADS, FUSED, QUOTA>(scores, B, N, k, p, a, st);
    default: return launch_seg<BF16, AL, 8, THREADS, FUSED, QUOTA>(scores, B, N, k, p, a, st);
  }
}

template <bool BF16, bool AL>
hipError_t launch_stage1(const void* scores, int B, int N, int k, const TopkPlan& p, const Stage1Args& a,
                         bool quota, hipStream_t st) {
  if (p.fused) return launch_seg_v<BF16, AL, kRowThreads, true, false>(scores, B, N, k, p, a, st);
  if constexpr (AL) {
    if (quota) return launch_seg_v<BF16, AL, kTkThreads, false, true>(scores, B, N, k, p, a, st);
  }
  return launch_seg_v<BF16, AL, kTkThreads, false, false>(scores, B, N, k, p, a, st);
}

}  // namespace

TopkPlan plan_topk(int B, int N, int k, dsa_dtype_t dt) {
  TopkPlan p{};
  const int E = dt == DSA_BF16 ? 8 : 4;
  // A row that one workgroup covers in one register block is taken whole
  // by that workgroup (one kernel, no candidates in memory); longer rows are
  // split into segments that a second kernel merges.
  const int max_vec = kRowFusedVec;
  if ((long long)N <= (long long)kRowThreads * max_vec * E) {
    const long long chunk = (long long)kRowThreads * E;
    long long vec = ((long long)N + chunk - 1) / chunk;
    int v = 1;
    while (v < vec && v < max_vec) v <<= 1;
    p.fused = true;
    p.vec = v;
    p.segs = 1;
    p.seg_len = N;
    p.cand_off = p.cnt_off = 0;
    p.bytes = 0;
    return p;
  }
  const long long chunk = (long long)kTkThreads * E;  // one vector per thread
  // About one workgroup per CU over the call; each row's candidates
  // (segs * 2k) must fit the merge buffer.
  long long segs = (256 + B - 1) / B;
  const long long max_by_len = (N + 16383) / 16384;  // at least 16K scores per segment
  const long long max_by_merge = kMergeCap / (2LL * k);
  if (segs > max_by_len) segs = max_by_len;
  if (segs > max_by_merge) segs = max_by_merge;
  if (segs > 64) segs = 64;
  if (segs < 1) segs = 1;
  long long seg_len = (N + segs - 1) / segs;
  seg_len = (seg_len + chunk - 1) / chunk * chunk;
  segs = (N + seg_len - 1) / seg_len;
  const long long vec = seg_len / chunk;  // vectors per thread over the segment
  int v = 1;
  while (v < vec && v < kTkMaxVec) v <<= 1;
  p.fused = false;
  p.vec = v;
  p.segs = (int)segs;
  p.seg_len = (int)seg_len;
  // Quota form: segment s keeps about its share of the row's top k, the
  // share's mean plus four standard deviations of a random row's spread
  // plus 17 (the indexer's chunk cut uses the same margin), in twice that
  // many slots, so the group-maxima threshold (which admits a little more
  // than the count it is set for) rarely needs an exact cut. It needs a
  // power-of-two segment count and slots within the lists' 2k stride, and a
  // segment of at most 65536 positions keeps the tie select's position
  // bitmap. It pays with four or more segments (the merge's candidates
  // shrink: bf16 64 x 131072, k = 512: 15.9 -> 14.6 us) or segments of
  // several register blocks (fewer exact cuts: float32 128 x 129280,
  // k = 1024: 37.3 -> 36.4 us); two one-block segments per row gain nothing
  // in the merge and were 0.2-0.6 us slower (float32 16-64 x 32768,
  // k = 1024), so they keep every segment's top k.
  p.quota = 0;
  p.slots = 2 * k;
  const bool one_block = seg_len <= (long long)kTkThreads * kTkMaxVec * E;
  if (segs >= 2 && (segs & (segs - 1)) == 0 && (segs >= 4 || !one_block)) {
    const double share = (double)k / (double)segs;
    const int quota = (int)ceil(share + 4.0 * sqrt(share) + 17.0);
    int slots = (2 * quota + 7) / 8 * 8;
    // The merge holds 4, 8, 16 or 32 slots per thread: segments of three or
    // more blocks take all of the slots that count gives them, so they cut
    // their lists only when these outgrow that (stage 1 then skips the exact
    // cut it would otherwise take after its first blocks; the merge's
    // per-thread work is the same). Shorter segments take no such cut and
    // keep 2q (the larger lists cost the bf16 64 x 131072 rows 0.15 us and
    // the bf16 stress rows 0.1 us in the merge's loads).
    if (seg_len > 2LL * kTkThreads * v * E) {
      const long long need = segs * (long long)slots;
      const int per = need <= kMergeThreads * 4 ? 4 : need <= kMergeThreads * 8 ? 8 : need <= kMergeThreads * 16 ? 16 : 32;
      slots = std::max(slots, std::min(2 * k, (int)((long long)kMergeThreads * per / segs) / 8 * 8));
    }
    const int log_s = __builtin_ctzll((unsigned long long)segs), log_p = dt == DSA_BF16 ? 6 : 5;
    int64_t longest = 0;
    for (int sg = 0; sg < (int)segs; ++sg) longest = std::max(longest, piece_seg_len(N, sg, log_s, log_p));
    if (slots <= 2 * k && quota < k && longest <= 65536) {
      p.quota = quota;
      p.slots = slots;
    }
  }
  p.cand_off = 0;
  p.cnt_off = align_up((size_t)B * p.segs * (size_t)(2 * k) * sizeof(uint64_t), 256);
  p.tcut_off = align_up(p.cnt_off + (size_t)B * p.segs * sizeof(uint32_t), 256);
  p.bytes = align_up(p.tcut_off + (size_t)(p.quota ? B * p.segs : 0) * sizeof(uint64_t), 256);
  return p;
}

hipError_t launch_topk(const void* scores, dsa_dtype_t dt, int B, int N, int k,
                       int32_t* out_idx, void* out_val, int sorted_index, const int32_t* lengths,
                       const TopkPlan& plan, void* ws, hipStream_t st) {
  char* base = reinterpret_cast<char*>(ws);
  uint64_t* cand = reinterpret_cast<uint64_t*>(base + plan.cand_off);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(base + plan.cnt_off);
  uint64_t* tcut = plan.quota ? reinterpret_cast<uint64_t*>(base + plan.tcut_off) : nullptr;
  const bool bf16 = dt == DSA_BF16;
  const int E = bf16 ? 8 : 4;
  const bool aligned = (N % E) == 0 && (reinterpret_cast<uintptr_t>(scores) % 16) == 0;
  // The quota form takes full, aligned rows; ragged or unaligned ones keep
  // every segment's top k.
  const bool quota = !plan.fused && plan.quota > 0 && lengths == nullptr && aligned;
  const Stage1Args a{cand, cnt, tcut, out_idx, out_val, sorted_index, lengths};
  hipError_t e;
  if (bf16) e = aligned ? launch_stage1<true, true>(scores, B, N, k, plan, a, quota, st)
                        : launch_stage1<true, false>(scores, B, N, k, plan, a, quota, st);
  else e = aligned ? launch_stage1<false, true>(scores, B, N, k, plan, a, quota, st)
                   : launch_stage1<false, false>(scores, B, N, k, plan, a, quota, st);
  if (e != hipSuccess || plan.fused) return e;
  int P = 1;
  while (P < k) P <<= 1;
  const size_t merge_lds = (size_t)P * sizeof(uint32_t);
  const int stride = quota ? plan.slots : 2 * k;  // slots per segment list
  const int slots = plan.segs * stride;
  const int per = slots <= 512 * 4 ? 4 : slots <= 512 * 8 ? 8 : slots <= 512 * 16 ? 16 : 32;
#define DSA_MERGE(BF, PER, CUT)                                                                 \
  do {                                                                                          \
    e = allow_lds(topk_merge_kernel<BF, PER, CUT>, merge_lds);                                  \
    if (e != hipSuccess) return e;                                                              \
    hipLaunchKernelGGL((topk_merge_kernel<BF, PER, CUT>), dim3(B), dim3(kMergeThreads), merge_lds, \
                       st, scores, N, k, plan.segs, stride, cand, cnt, CUT ? tcut : nullptr,    \
                       out_idx, out_val, sorted_index);                                         \
  } while (0)
#define DSA_MERGE_PER(BF, CUT)                                                                  \
  do {                                                                                          \
    if (per == 4) DSA_MERGE(BF, 4, CUT); else if (per == 8) DSA_MERGE(BF, 8, CUT);              \
    else if (per == 16) DSA_MERGE(BF, 16, CUT); else DSA_MERGE(BF, 32, CUT);                    \
  } while (0)
  if (bf16) {
    if (quota) DSA_MERGE_PER(true, true); else DSA_MERGE_PER(true, false);
  } else {
    if (quota) DSA_MERGE_PER(false, true); else DSA_MERGE_PER(false, false);
  }
#undef DSA_MERGE_PER
#undef DSA_MERGE
  return hipGetLastError();
}

hipError_t launch_topk_cut_merge(const float* scores, int B, int N, int k, const CutPlan& p,
                                 const uint64_t* cand, const uint32_t* cnt, const uint64_t* tcut,
                                 int32_t* out_idx, hipStream_t st) {
  int P = 1;
  while (P < k) P <<= 1;
  const size_t merge_lds = (size_t)P * sizeof(uint32_t);
  const int slots = p.chunks * p.keep;
  const int per = slots <= 512 * 4 ? 4 : slots <= 512 * 8 ? 8 : slots <= 512 * 16 ? 16 : 32;
  hipError_t e;
#define DSA_CUT_MERGE(PER)                                                                       \
  do {                                                                                           \
    e = allow_lds(topk_merge_kernel<false, PER, true>, merge_lds);                               \
    if (e != hipSuccess) return e;                                                               \
    hipLaunchKernelGGL((topk_merge_kernel<false, PER, true>), dim3(B), dim3(kMergeThreads),      \
                       merge_lds, st, scores, N, k, p.chunks, p.keep, cand, cnt, tcut, out_idx,  \
                       nullptr, 0);                                                              \
  } while (0)
  if (per == 4) DSA_CUT_MERGE(4);
  else if (per == 8) DSA_CUT_MERGE(8);
  else if (per == 16) DSA_CUT_MERGE(16);
  else DSA_CUT_MERGE(32);
#undef DSA_CUT_MERGE
  return hipGetLastError();
}

}  // namespace dsa
