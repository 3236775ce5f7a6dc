// Top-k selection on gfx950 ("feat: Add DeepSeek-V4 CSA attention kernels",
// step 3, and its chunked score/top-k pipeline in "The top-k on the GPSIMD
// engine"; "DeepSelect" project page: a dynamic threshold that starts at
// minus infinity, blocks visited in a random order that does not depend on
// the data, and early rejection of everything below the threshold).
//
// The answer is exact under the order (value desc, index asc): every score
// is mapped to a 64-bit composite key (order-preserving value key in the
// high word, complemented position in the low word), so the k largest
// composites are the unique answer.
//
// Stage 1, one workgroup per (row, segment): stream the segment once in
// sub-chunks of 4096 scores, visiting the sub-chunks in a Weyl-sequence
// order (a golden-ratio stride coprime to the count). Each thread rejects
// its 8 scores with one compare against the running threshold; survivors
// are appended to an LDS candidate buffer in a fixed order (wave prefix
// sums, waves in index order). When the buffer could overflow on the next
// sub-chunk, an exact radix select finds the k-th largest composite, the
// buffer is compacted to k entries and that composite becomes the new
// threshold. Anything at or below it can never enter this segment's top-k.
// The segment ends with its exact top-min(k, length) in the workspace.
//
// Stage 2, one workgroup per row: load the segments' candidates into LDS,
// radix-select the row's k-th composite, and write the k winners (indices,
// optional value copies) either in buffer order or sorted by index.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkEpt = 8;                           // scores per thread per sub-chunk
constexpr int kTkSub = kTkThreads * kTkEpt;         // 4096 scores per sub-chunk
constexpr int kMergeThreads = 1024;
constexpr int kMergeWaves = kMergeThreads / kWave;
constexpr int kMaxK = 4096;
constexpr int kSegCap = 8192;                       // LDS candidates per segment (>= kMaxK + kTkSub)
constexpr int kMergeCap = 8192;                     // candidates per row in stage 2

// LDS-only barrier: wait for this wave's LDS traffic, then meet the others.
// Pending global loads (prefetches) are left in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t gcd_u32(uint32_t a, uint32_t b) {
  while (b) {
    uint32_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    uint32_t o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// Shared scratch of the block-wide helpers below.
struct SelectScratch {
  uint32_t hist[256];
  uint32_t wave_sum[kMergeWaves];
  uint32_t digit, above, in_bucket;
};

// Exclusive block-wide scan of one count per thread, in thread order.
// Returns the exclusive prefix; *total receives the sum. Two barriers.
template <int THREADS>
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total, SelectScratch& sc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  constexpr int WAVES = THREADS / kWave;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) sc.wave_sum[wave] = inc;
  lds_barrier();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w2 = 0; w2 < WAVES; ++w2) {
    const uint32_t ws = sc.wave_sum[w2];
    before += (w2 < wave) ? ws : 0u;
    all += ws;
  }
  lds_barrier();
  *total = all;
  return before + inc - v;
}

// Radix select over the LDS buffer buf[0..cnt): returns T such that exactly
// K entries are >= T (entries are distinct). Digits of 8 bits from the top,
// skipping bit ranges that cannot differ between candidates: only
// `key_levels` bytes of the value key carry information (2 for bf16 scores,
// whose low key half follows from the sign, 4 for float32), and of the
// complemented position only the low `pos_bits` bits vary. Stops as soon as
// the bucket holding the K-th entry is taken whole.
template <int THREADS>
__device__ uint64_t block_select_kth(const uint64_t* buf, int cnt, int K, int key_levels,
                                     int pos_bits, SelectScratch& sc) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  uint64_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)K;
  int shift = 56;
  int level = 0;
  for (;;) {
    for (int i = tid; i < 256; i += THREADS) sc.hist[i] = 0;
    lds_barrier();
    for (int i = tid; i < cnt; i += THREADS) {
      const uint64_t e = buf[i];
      if ((e & mask) == prefix) atomicAdd(&sc.hist[(uint32_t)(e >> shift) & 255u], 1u);
    }
    lds_barrier();
    if (tid < kWave) {
      // Lane l owns bins 255-4l .. 252-4l, so lane order is descending digits.
      uint32_t c[4];
      uint32_t local = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = sc.hist[255 - 4 * lane - j];
        local += c[j];
      }
      const uint32_t inc = wave_inclusive_scan(local);
      const uint64_t hit = __ballot(inc >= need);
      const int first = __ffsll((long long)hit) - 1;
      if (lane == first) {
        uint32_t run = inc - local;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (run + c[j] >= need) {
            sc.digit = 255u - 4u * lane - j;
            sc.above = run;
            sc.in_bucket = c[j];
            break;
          }
          run += c[j];
        }
      }
    }
    lds_barrier();
    const uint32_t digit = sc.digit, above = sc.above, in_bucket = sc.in_bucket;
    need -= above;
    prefix |= (uint64_t)digit << shift;
    mask |= (uint64_t)0xFF << shift;
    if (in_bucket == need) break;
    // Next digit. Overlapping the last position digit with bits already
    // fixed is harmless: those bits match the prefix for every counted entry.
    ++level;
    if (level < key_levels) {
      shift = 56 - 8 * level;
    } else if (level == key_levels) {
      // Entering the position digits. The skipped bits are the same for
      // every entry still in play, so the prefix must carry their actual
      // values: for bf16 scores the low half of the value key is 0x0000 for
      // a non-negative value and 0xFFFF for a negative one (the sign sits
      // in the prefix's top bit); above the low pos_bits bits the
      // complemented position is all ones.
      if (key_levels == 2) {
        const uint64_t low_key = (prefix >> 63) ? 0u : 0xFFFFu;
        prefix |= low_key << 32;
        mask |= (uint64_t)0xFFFF << 32;
      }
      const uint64_t high_ones = pos_bits >= 32 ? 0 : ((uint64_t)(0xFFFFFFFFu >> pos_bits) << pos_bits);
      prefix |= high_ones;
      mask |= high_ones;
      shift = max(pos_bits - 8, 0);
    } else {
      if (shift == 0) break;  // unreachable for distinct entries
      shift = max(shift - 8, 0);
    }
  }
  return prefix;
}

// Keep the entries >= thr, preserving their order; returns the new count.
// Each thread moves a contiguous run of entries through registers.
template <int THREADS, int MAXPER>
__device__ int block_compact(uint64_t* buf, int cnt, uint64_t thr, SelectScratch& sc) {
  const int tid = threadIdx.x;
  const int per = (cnt + THREADS - 1) / THREADS;  // <= MAXPER by construction
  const int lo = min(cnt, tid * per);
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
  uint32_t pos = block_exclusive_scan<THREADS>(keep, &total, sc);  // also orders reads before writes
#pragma unroll
  for (int j = 0; j < MAXPER; ++j) {
    const int i = lo + j;
    if (i < hi && v[j] >= thr) buf[pos++] = v[j];
  }
  lds_barrier();
  return (int)total;
}

template <bool BF16>
__device__ __forceinline__ uint32_t load_key(const void* row, int64_t j) {
  if (BF16) {
    const uint16_t h = reinterpret_cast<const uint16_t*>(row)[j];
    return f32_key((uint32_t)h << 16);
  } else {
    return f32_key(reinterpret_cast<const uint32_t*>(row)[j]);
  }
}

// Loads the 8 keys of one thread's slot. Positions at or past `end` get key 0,
// whose composite (0 in the high word) is below every real score's.
template <bool BF16, bool ALIGNED>
__device__ __forceinline__ void load_keys(const void* row, int64_t j0, int64_t end, uint32_t key[kTkEpt]) {
  if (ALIGNED && j0 + kTkEpt <= end) {
    if (BF16) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          reinterpret_cast<const uint16_t*>(row) + j0));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[2 * e] = f32_key(v[e] << 16);
        key[2 * e + 1] = f32_key(v[e] & 0xFFFF0000u);
      }
    } else {
      const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint32_t*>(row) + j0);
      const u32x4 v0 = __builtin_nontemporal_load(p);
      const u32x4 v1 = __builtin_nontemporal_load(p + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[e] = f32_key(v0[e]);
        key[4 + e] = f32_key(v1[e]);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kTkEpt; ++e) key[e] = (j0 + e < end) ? load_key<BF16>(row, j0 + e) : 0u;
  }
}

struct SegShared {
  SelectScratch sc;
  uint32_t wave_cnt[kTkWaves];
};

template <bool BF16, bool ALIGNED>
__global__ __launch_bounds__(kTkThreads) void topk_segment_kernel(
    const void* __restrict__ scores, int N, int k, int seg_len, int segs, int pos_bits,
    uint64_t* __restrict__ cand_out, uint32_t* __restrict__ cnt_out) {
  extern __shared__ uint64_t cand[];  // kSegCap entries
  __shared__ SegShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int b = blockIdx.y;
  const int sidx = blockIdx.x;
  const size_t esz = BF16 ? 2 : 4;
  const void* row = reinterpret_cast<const char*>(scores) + (size_t)b * (size_t)N * esz;
  const int64_t seg_start = (int64_t)sidx * seg_len;
  const int64_t seg_end = min((int64_t)N, seg_start + seg_len);
  const int L = (int)(seg_end - seg_start);
  const int nsub = (L + kTkSub - 1) / kTkSub;
  constexpr int key_levels = BF16 ? 2 : 4;

  // Visiting order: p(it) = (c0 + a*it) mod nsub with gcd(a, nsub) = 1 and a
  // near nsub/phi, so consecutive visits land far apart for any input.
  uint32_t a = (uint32_t)(nsub * 0.6180339887f);
  if (a < 1) a = 1;
  while (gcd_u32(a, (uint32_t)nsub) != 1u) ++a;
  const uint32_t c0 = (uint32_t)(((uint64_t)b * 2654435761u + (uint64_t)sidx * 40503u) % (uint64_t)nsub);

  uint64_t thr = 0;  // admit composites > thr
  int cnt = 0;
  bool have_thr = false;

  uint32_t nxt[kTkEpt];
  {
    const int64_t j0 = seg_start + (int64_t)(c0 % nsub) * kTkSub + tid * kTkEpt;
    load_keys<BF16, ALIGNED>(row, j0, seg_end, nxt);
  }
  for (int it = 0; it < nsub; ++it) {
    const uint32_t p = (uint32_t)((c0 + (uint64_t)a * it) % (uint64_t)nsub);
    const int64_t j0 = seg_start + (int64_t)p * kTkSub + tid * kTkEpt;
    uint32_t key[kTkEpt];
#pragma unroll
    for (int e = 0; e < kTkEpt; ++e) key[e] = nxt[e];
    if (it + 1 < nsub) {
      const uint32_t pn = (uint32_t)((c0 + (uint64_t)a * (it + 1)) % (uint64_t)nsub);
      load_keys<BF16, ALIGNED>(row, seg_start + (int64_t)pn * kTkSub + tid * kTkEpt, seg_end, nxt);
    }
    // Filter: one compare of the largest key against the threshold's key
    // rejects the whole slot in the common case.
    uint32_t kmax = key[0];
#pragma unroll
    for (int e = 1; e < kTkEpt; ++e) kmax = max(kmax, key[e]);
    const uint32_t thr_key = (uint32_t)(thr >> 32);
    uint32_t pass_mask = 0;
    if (kmax >= thr_key) {
#pragma unroll
      for (int e = 0; e < kTkEpt; ++e) {
        const uint64_t c = composite(key[e], (uint32_t)(j0 + e));
        pass_mask |= (key[e] != 0u && c > thr) ? (1u << e) : 0u;
      }
    }
    const uint32_t npass = __popc(pass_mask);
    uint32_t excl = 0;
    if (__ballot(npass != 0) != 0) {
      const uint32_t inc = wave_inclusive_scan(npass);
      excl = inc - npass;
      if (lane == kWave - 1) sh.wave_cnt[wave] = inc;
    } else if (lane == 0) {
      sh.wave_cnt[wave] = 0;
    }
    lds_barrier();
    uint32_t base = (uint32_t)cnt, total = 0;
#pragma unroll
    for (int w2 = 0; w2 < kTkWaves; ++w2) {
      const uint32_t wc = sh.wave_cnt[w2];
      base += (w2 < wave) ? wc : 0u;
      total += wc;
    }
    if (pass_mask) {
      uint32_t at = base + excl;
#pragma unroll
      for (int e = 0; e < kTkEpt; ++e)
        if (pass_mask & (1u << e)) cand[at++] = composite(key[e], (uint32_t)(j0 + e));
    }
    cnt += (int)total;
    lds_barrier();
    // Select when the next sub-chunk might not fit, and once early (at 2k
    // candidates) so that a useful threshold exists from then on.
    if (cnt > k && (cnt > kSegCap - kTkSub || (!have_thr && cnt >= 2 * k))) {
      const uint64_t t = block_select_kth<kTkThreads>(cand, cnt, k, key_levels, pos_bits, sh.sc);
      cnt = block_compact<kTkThreads, kSegCap / kTkThreads>(cand, cnt, t, sh.sc);
      thr = t ? t - 1 : 0;  // t > 0 whenever more than k candidates exist
      have_thr = true;
    }
  }
  if (cnt > k) {
    const uint64_t t = block_select_kth<kTkThreads>(cand, cnt, k, key_levels, pos_bits, sh.sc);
    cnt = block_compact<kTkThreads, kSegCap / kTkThreads>(cand, cnt, t, sh.sc);
  }
  cnt = min(cnt, k);  // never more than the k slots this segment owns
  uint64_t* out = cand_out + ((size_t)b * segs + sidx) * (size_t)k;
  for (int i = tid; i < cnt; i += kTkThreads) out[i] = cand[i];
  if (tid == 0) cnt_out[(size_t)b * segs + sidx] = (uint32_t)cnt;
}

struct MergeShared {
  SelectScratch sc;
  uint32_t seg_off[65];
};

template <bool BF16>
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(
    const void* __restrict__ scores, int N, int k, int segs, int pos_bits,
    const uint64_t* __restrict__ cand_in, const uint32_t* __restrict__ cnt_in,
    int32_t* __restrict__ out_idx, void* __restrict__ out_val, int sorted_index) {
  extern __shared__ uint64_t buf[];  // kMergeCap entries
  __shared__ MergeShared sh;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  if (tid == 0) {
    uint32_t off = 0;
    for (int s2 = 0; s2 < segs; ++s2) {
      sh.seg_off[s2] = off;
      off += min((uint32_t)k, cnt_in[(size_t)b * segs + s2]);
    }
    sh.seg_off[segs] = off;
  }
  lds_barrier();
  const int total = (int)sh.seg_off[segs];
  for (int s2 = 0; s2 < segs; ++s2) {
    const int o = (int)sh.seg_off[s2];
    const int c = (int)sh.seg_off[s2 + 1] - o;
    const uint64_t* src = cand_in + ((size_t)b * segs + s2) * (size_t)k;
    for (int i = tid; i < c; i += kMergeThreads) buf[o + i] = src[i];
  }
  lds_barrier();
  uint64_t thr = 0;
  if (total > k) thr = block_select_kth<kMergeThreads>(buf, total, k, BF16 ? 2 : 4, pos_bits, sh.sc);

  // Winners in buffer order: thread t owns a contiguous run of entries.
  constexpr int kPer = kMergeCap / kMergeThreads;
  const int per = (total + kMergeThreads - 1) / kMergeThreads;
  const int lo = min(total, tid * per);
  const int hi = min(total, lo + per);
  uint32_t keep = 0;
  uint64_t v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = lo + j;
    v[j] = (i < hi) ? buf[i] : 0;
    keep += (i < hi && v[j] >= thr) ? 1u : 0u;
  }
  uint32_t nkeep;
  uint32_t pos = block_exclusive_scan<kMergeThreads>(keep, &nkeep, sh.sc);
  int32_t* oi = out_idx + (size_t)b * k;
  const size_t esz = BF16 ? 2 : 4;
  const char* row = reinterpret_cast<const char*>(scores) + (size_t)b * (size_t)N * esz;
  if (!sorted_index) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = lo + j;
      if (i < hi && v[j] >= thr && pos < (uint32_t)k) {
        const uint32_t p = min(composite_pos(v[j]), (uint32_t)(N - 1));
        oi[pos] = (int32_t)p;
        if (out_val) {
          if (BF16) reinterpret_cast<uint16_t*>(out_val)[(size_t)b * k + pos] = reinterpret_cast<const uint16_t*>(row)[p];
          else reinterpret_cast<uint32_t*>(out_val)[(size_t)b * k + pos] = reinterpret_cast<const uint32_t*>(row)[p];
        }
        ++pos;
      }
    }
    return;
  }
  // Sorted by index: place the winners' positions in LDS (reusing the front
  // of the buffer as 32-bit slots after everyone has read it), pad to a power
  // of two and run a bitonic sort.
  lds_barrier();
  uint32_t* pos_lds = reinterpret_cast<uint32_t*>(buf);
  int P = 1;
  while (P < k) P <<= 1;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = lo + j;
    if (i < hi && v[j] >= thr && pos < (uint32_t)k) pos_lds[pos++] = min(composite_pos(v[j]), (uint32_t)(N - 1));
  }
  for (int i = k + tid; i < P; i += kMergeThreads) pos_lds[i] = 0xFFFFFFFFu;
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
  for (int i = tid; i < k; i += kMergeThreads) {
    const uint32_t p = pos_lds[i];
    oi[i] = (int32_t)p;
    if (out_val) {
      if (BF16) reinterpret_cast<uint16_t*>(out_val)[(size_t)b * k + i] = reinterpret_cast<const uint16_t*>(row)[p];
      else reinterpret_cast<uint32_t*>(out_val)[(size_t)b * k + i] = reinterpret_cast<const uint32_t*>(row)[p];
    }
  }
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

TopkPlan plan_topk(int B, int N, int k, dsa_dtype_t dt) {
  (void)dt;
  TopkPlan p{};
  // Aim for about two workgroups per CU over the whole call, but keep each
  // row's candidates (segs * k) within the merge buffer.
  long long want = (512 + B - 1) / B;
  const long long max_by_len = (N + kTkSub - 1) / kTkSub;
  const long long max_by_merge = kMergeCap / k;
  long long segs = want;
  if (segs > max_by_len) segs = max_by_len;
  if (segs > max_by_merge) segs = max_by_merge;
  if (segs > 64) segs = 64;
  if (segs < 1) segs = 1;
  long long seg_len = (N + segs - 1) / segs;
  seg_len = (seg_len + kTkSub - 1) / kTkSub * kTkSub;
  segs = (N + seg_len - 1) / seg_len;
  p.segs = (int)segs;
  p.seg_len = (int)seg_len;
  p.cand_off = 0;
  p.cnt_off = align_up((size_t)B * p.segs * (size_t)k * sizeof(uint64_t), 256);
  p.bytes = align_up(p.cnt_off + (size_t)B * p.segs * sizeof(uint32_t), 256);
  return p;
}

template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  // Workgroups here use more than 64 KB of LDS (gfx950 has 160 KB per CU).
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_topk(const void* scores, dsa_dtype_t dt, int B, int N, int k,
                       int32_t* out_idx, void* out_val, int sorted_index,
                       const TopkPlan& plan, void* ws, hipStream_t st) {
  uint64_t* cand = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + plan.cand_off);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) + plan.cnt_off);
  const bool bf16 = dt == DSA_BF16;
  const int vec = bf16 ? 8 : 4;
  const bool aligned = (N % vec) == 0 && (reinterpret_cast<uintptr_t>(scores) % 16) == 0;
  int pos_bits = 1;
  while (pos_bits < 32 && ((uint32_t)(N - 1) >> pos_bits) != 0) ++pos_bits;
  const size_t seg_lds = (size_t)kSegCap * sizeof(uint64_t);
  const size_t merge_lds = (size_t)kMergeCap * sizeof(uint64_t);
  dim3 g1(plan.segs, B);
  hipError_t e = hipSuccess;
#define DSA_SEG(BF, AL)                                                                        \
  do {                                                                                         \
    e = allow_lds(topk_segment_kernel<BF, AL>, seg_lds);                                       \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL((topk_segment_kernel<BF, AL>), g1, dim3(kTkThreads), seg_lds, st, scores, \
                       N, k, plan.seg_len, plan.segs, pos_bits, cand, cnt);                    \
  } while (0)
  if (bf16) {
    if (aligned) DSA_SEG(true, true); else DSA_SEG(true, false);
  } else {
    if (aligned) DSA_SEG(false, true); else DSA_SEG(false, false);
  }
#undef DSA_SEG
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (bf16) {
    e = allow_lds(topk_merge_kernel<true>, merge_lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((topk_merge_kernel<true>), dim3(B), dim3(kMergeThreads), merge_lds, st, scores, N, k, plan.segs, pos_bits, cand, cnt, out_idx, out_val, sorted_index);
  } else {
    e = allow_lds(topk_merge_kernel<false>, merge_lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((topk_merge_kernel<false>), dim3(B), dim3(kMergeThreads), merge_lds, st, scores, N, k, plan.segs, pos_bits, cand, cnt, out_idx, out_val, sorted_index);
  }
  return hipGetLastError();
}

}  // namespace dsa
