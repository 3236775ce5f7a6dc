// Sparse multi-query decode attention on gfx950 ("feat: Add DeepSeek-V4 CSA
// attention kernels", "How the algorithm works", step 4; "The top-k on the
// GPSIMD engine"). Each batch row attends over the compressed rows its top-k
// picked plus its recent raw rows; one tensor serves as both keys and
// values, so a row is fetched from HBM once and used for both products.
//
//   R_b = kv_cmp[b, idx[b, :]] ++ kv_win[b, :]          (k + W rows of D)
//   out[b,h,:] = softmax_r(scale * q[b,h,:] . R_b[r,:]) @ R_b
//
// Each workgroup takes one batch row, a group of 16*HG query heads and a
// split of the rows (a share of the selected rows, and on some splits first a
// tile of the window); each 16-head group is served by DSPLIT waves
// that own 1/DSPLIT of the head dims each (they add up their halves of the
// logits through LDS). Rows are copied 32 at a time from HBM straight into
// LDS (row-major, padded), and each staged row is used twice:
//   S^T = R Q^T  : MFMA A operand = 16 rows x 32 dims read straight from
//                  LDS (ds_read_b128), B operand = the wave's query
//                  fragments, kept in registers;
//   O^T = R^T P^T: A operand = 16 dims x 32 rows from the same LDS tile via
//                  ds_read_b64_tr_b16 (a 4x4 transposing read), B operand =
//                  the probabilities, which the S^T result already holds in
//                  the right lanes (lane 16g+m: rows 4g..4g+3 of head m).
// A lane therefore owns one head throughout, so the running max, the
// rescale factor and the running sum need no cross-lane traffic except two
// reductions per tile. The tiles are software-pipelined: the logits of tile
// t+1 are computed while tile t is finished. The online softmax runs in
// float32. A single split writes bf16 output directly; several splits write
// partials (max, sum, and the unnormalised O in fp16 with one float32 scale
// per head and dim half) that a combine kernel merges with the log-sum-exp
// rule.
#include <cfloat>

#include "select_k.h"

namespace dsa {
namespace {

constexpr int kTile = 32;          // rows per LDS tile
constexpr int kMaxSplitTiles = 64; // rows per split <= 2048
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Lazy-rescale margin in base-2 units: weights stay below 2^11.5 (about e^8).
constexpr float kRescale2 = 11.5f;
constexpr int kStages = 3;         // LDS tiles
// Row-list entry of an empty slot (a negative index: no row, ragged rows).
constexpr int kEmpty = -0x7FFFFFFF - 1;

// SEL > 0: the workgroup first selects its batch row's k rows itself from
// the chunk cut's candidates (merge_candidates with SEL slots per thread,
// the cut merge's selection, in the same order), instead of reading idx;
// every workgroup of the row repeats the selection (it is latency, not
// work), and one of them also writes it out.
template <int D, int HG, int DSPLIT, int SEL = 0>
__global__ __launch_bounds__(HG * DSPLIT * kWave) void sparse_attend_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ win,
    uint16_t* __restrict__ out, uint16_t* __restrict__ part_o, float* __restrict__ part_ml,
    const float* __restrict__ sink, int N, int k, int W, int Hq, float scale,
    int rows_per_split, int sel_rows, int splits, int nitems, int hgroups, int tokens,
    SelectArgs sel) {
  static_assert(SEL == 0 || HG * DSPLIT * kWave == kMergeThreads,
                "the selection runs on kMergeThreads threads");
  constexpr int WAVES = HG * DSPLIT;
  constexpr int THREADS = WAVES * kWave;
  constexpr int HW = HG * 16;           // query heads per workgroup
  constexpr int DW = D / DSPLIT;        // dims of q and O owned by one wave
  constexpr int KS = DW / 32;           // S^T k-steps per wave
  constexpr int DTW = DW / 16;          // 16-dim output tiles per wave
  constexpr int ROW_WORDS = D / 2 + 4;  // 16 bytes of padding per row
  constexpr int ROW_LANES = D / 8;      // lanes that copy one row (16 bytes each)
  constexpr int kRowsPerWave = kTile / WAVES;
  constexpr int XWORDS = DSPLIT > 1 ? 2 * WAVES * kWave * 8 : 0;  // S^T exchange, by tile parity
  extern __shared__ uint32_t lds[];
  uint32_t* Rbuf = lds;  // kStages tiles
  f32x4* xbuf = reinterpret_cast<f32x4*>(lds + kStages * kTile * ROW_WORDS);
  int32_t* srow = reinterpret_cast<int32_t*>(lds + kStages * kTile * ROW_WORDS + XWORDS);
  int32_t* wempty = srow + rows_per_split;  // per wave: saw an empty slot

  // Workgroup -> work item (batch, split, head group), batch-major.
  // Workgroups are dispatched to the 8 XCDs round robin, so XCD x runs ids
  // x, x+8, ...; those take the x-th contiguous eighth of the work items.
  // Every workgroup of one batch row then sits on one XCD: its query, its
  // gathered rows and its partials are fetched from HBM once and shared
  // through that XCD's L2.
  const int L = blockIdx.x;
  const int item = (L % 8) * (int)(gridDim.x / 8) + L / 8;
  if (item >= nitems) return;  // padding workgroup (uniform)
  const int hg = item % hgroups;
  const int pair = item / hgroups;
  const int b = pair / splits;
  const int split = pair % splits;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int m = lane & 15;
  const int g = lane >> 4;
  // Wave (hq, dh): 16 heads, and the dh-th 1/DSPLIT of the dims for the
  // query fragments and the output accumulators.
  const int hq = wave % HG;
  const int dh = wave / HG;
  const int h = hg * HW + hq * 16 + m;  // the head this lane owns
  const int dbase = dh * DW;
  // This split's rows, in local order: first its tiles of the window (the
  // window's tiles are dealt round robin to the splits, starting after the
  // last split that holds selected rows), then its share of the k selected
  // rows, sel_rows per split in selection order. Slots past the window or
  // past k are empty. A split that starts with a window tile can copy it
  // before its selected rows are known.
  const int tiles_sel = (k + kTile - 1) / kTile;
  const int tps = sel_rows / kTile;                   // selected tiles per split
  const int s_sel = (tiles_sel + tps - 1) / tps;      // splits that hold selected rows
  const int nwt = (W + kTile - 1) / kTile;            // window tiles
  const int j0 = ((split - s_sel) % splits + splits) % splits;  // this split's first window tile
  const int wt = j0 < nwt ? (nwt - 1 - j0) / splits + 1 : 0;
  const int wrows = wt * kTile;
  const int sbase = split * sel_rows;
  const int nsel = max(0, min(k, sbase + sel_rows) - sbase);
  const int ntiles = wt + (nsel + kTile - 1) / kTile;
  const int r0 = 0, r1 = ntiles * kTile;  // local rows; every tile is full, empty slots are masked
  const bool has_pad = nsel % kTile != 0 || (wt > 0 && (j0 + (wt - 1) * splits + 1) * kTile > W);
  // Encoded source of local window row i (< wrows): -(j+1) for window row j,
  // kEmpty past the window.
  auto win_enc = [&](int i) -> int {
    const int j = (j0 + (i / kTile) * splits) * kTile + (i % kTile);
    return j < W ? -j - 1 : kEmpty;
  };
  const int32_t* irow = SEL == 0 ? idx + (size_t)b * k : nullptr;  // with SEL, idx is unused
  // SEL == 0: the encoded source of local row i: >= 0 a compressed row
  // (indices >= N clamped), kEmpty an empty slot, other negatives window
  // row -(v+1).
  auto src_enc = [&](int i) -> int {
    if (i < wrows) return win_enc(i);
    const int r = sbase + (i - wrows);
    if (r >= sbase + nsel) return kEmpty;
    const int v = irow[r];
    return v < 0 ? kEmpty : (v >= N ? N - 1 : v);
  };
  // Query row b is token b % tokens of batch row b / tokens, whose
  // compressed rows it gathers from.
  const uint16_t* kvb = kv + (size_t)(b / tokens) * N * D;
  const uint16_t* winb = win ? win + (size_t)b * W * D : nullptr;

  // The first two tiles' copies go out first, their row indices read with
  // wave-uniform scalar loads (all issued before any is used), so they need
  // neither the row list in LDS nor a barrier. A row is copied by one
  // instruction, ROW_LANES lanes of 16 bytes each (at D = 128 the other
  // lanes are masked off, so rows keep their padding). (With SEL the rows
  // are known only after the selection below.)
  if constexpr (SEL == 0) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int vr[2][kRowsPerWave];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) vr[tile][i] = src_enc(min(tile * kTile + wv * kRowsPerWave + i, r1 - 1));
    const uint32_t rbase = lds_byte_addr(Rbuf);  // tile slot j starts at rbase + j*kTile*ROW_WORDS*4
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      if (tile < ntiles) {
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
          const int rr = wv * kRowsPerWave + i;
          const int v = vr[tile][i];
          // An empty slot copies row 0 (finite data; its weight is zero).
          const uint16_t* src = v >= 0 ? kvb + (size_t)v * D : (v == kEmpty ? kvb : winb + (size_t)(-v - 1) * D);
          const uint32_t at = __builtin_amdgcn_readfirstlane(
              rbase + (uint32_t)((tile * kTile + rr) * ROW_WORDS * 4));
          if (ROW_LANES == kWave || lane < ROW_LANES) dma_row16(src + (lane % ROW_LANES) * 8, at);
        }
      }
    }
  }

  // Query fragments (B operand of S^T): head h, dims dbase + 32*kk + 8g .. +8.
  bf16x8 qf[KS];
  const uint16_t* qrow = q + ((size_t)b * Hq + h) * D + dbase;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + kk * 32 + g * 8);

  // The split's source rows for the later tiles: >= 0 a compressed row,
  // kEmpty an empty slot (negative index), other negatives window row
  // -(v+1). Each wave notes whether it met an empty slot.
  if constexpr (SEL == 0) {
    bool saw_empty = false;
    for (int i = tid; i < r1; i += THREADS) {
      const int v = src_enc(i);
      saw_empty |= v == kEmpty;
      srow[i] = v;
    }
    const bool wave_saw_empty = __ballot(saw_empty) != 0;  // all lanes take part
    if (lane == 0) wempty[wave] = wave_saw_empty ? 1 : 0;
  } else {
    // A split that starts with window tiles copies the first two of them
    // now (their rows are known), so they land while the selection runs.
    // The selection then works in the third tile slot, which the tile loop
    // takes only after its first barrier; the q loads are in flight too.
    // Winner number pos (in the cut merge's order) is selected row pos of
    // the batch row; this split keeps [sbase, sbase + nsel) of them. The
    // selection never leaves an empty slot.
    {
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      const uint32_t rbase = lds_byte_addr(Rbuf);
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        if (tile < wt) {
#pragma unroll
          for (int i = 0; i < kRowsPerWave; ++i) {
            const int rr = wv * kRowsPerWave + i;
            const int v = win_enc(tile * kTile + rr);
            const uint16_t* src = v == kEmpty ? kvb : winb + (size_t)(-v - 1) * D;
            const uint32_t at = __builtin_amdgcn_readfirstlane(
                rbase + (uint32_t)((tile * kTile + rr) * ROW_WORDS * 4));
            if (ROW_LANES == kWave || lane < ROW_LANES) dma_row16(src + (lane % ROW_LANES) * 8, at);
          }
        }
      }
    }
    static_assert(sizeof(Scratch) <= kTile * ROW_WORDS * sizeof(uint32_t), "the selection fits a tile slot");
    Scratch& sc = *reinterpret_cast<Scratch*>(lds + 2 * kTile * ROW_WORDS);
    const size_t lists = (size_t)b * sel.chunks;
    int32_t* const io = (split == 0 && hg == 0) ? sel.idx_out + (size_t)b * k : nullptr;
    uint64_t cv[SEL];
    uint64_t thr;
    uint32_t pos, nkeep;
    if (merge_candidates<SEL, true>(sel.cand + lists * sel.keep, sel.cnt + lists, sel.tcut + lists,
                                    sel.chunks, sel.keep, k, sc, cv, thr, pos, nkeep)) {
#pragma unroll
      for (int j = 0; j < SEL; ++j) {
        if (cv[j] && cv[j] >= thr && pos < (uint32_t)k) {
          const int p = (int)min(composite_pos(cv[j]), (uint32_t)(N - 1));
          if ((int)pos >= sbase && (int)pos < sbase + nsel) srow[wrows + (int)pos - sbase] = p;
          if (io) io[pos] = p;
          ++pos;
        }
      }
    } else {
      int32_t* const sr = srow + wrows;
      const int lo = sbase, hi = sbase + nsel;
      row_topk_from_scores(sel.scores + (size_t)b * N, N, k,
                           [sr, lo, hi, io](uint32_t at, int i) {
                             if ((int)at >= lo && (int)at < hi) sr[at - lo] = i;
                             if (io) io[at] = i;
                           }, sc);
    }
    for (int i = tid; i < wrows; i += THREADS) srow[i] = win_enc(i);
    for (int i = wrows + nsel + tid; i < r1; i += THREADS) srow[i] = kEmpty;
    if (lane == 0) wempty[wave] = has_pad ? 1 : 0;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the selection's stores
    lds_barrier();  // the row list is complete and the tile slots are free
  }
  // Settle the query loads here: otherwise the compiler places their waits
  // inside the tile loop, where they would also wait for the row copies in
  // flight.
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) asm volatile("" : "+v"(qf[kk]));

  f32x4 o[DTW];
#pragma unroll
  for (int dt = 0; dt < DTW; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The softmax runs in base 2: logits are scaled by scale*log2(e), so every
  // weight is one exp2. mrun is in those units.
  const float scale2 = scale * kLog2e;
  // Running max of the scaled logits of head h. It starts at -FLT_MAX, not
  // -inf: a split whose slots are all empty keeps it, and its weights
  // exp2(-inf - mrun) are still 0 with a finite (m, l = 0) partial.
  float mrun = -FLT_MAX;
  float lrun = 0.0f;       // this lane's share of the running sum

  // Rows are copied from HBM straight into the LDS tiles (global_load_lds).
  // Each wave copies kRowsPerWave rows of a tile; the waits are explicit
  // vmcnt values over this wave's own copies, and a barrier publishes the
  // tile. Rows past r1 repeat the last valid row (finite data; their weights
  // are zero).
  auto dma = [&](int tile) {
    uint32_t* dst = Rbuf + (tile % kStages) * kTile * ROW_WORDS;
    const int t0 = r0 + tile * kTile;
    int vr[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) vr[i] = srow[min(t0 + wave * kRowsPerWave + i, r1 - 1) - r0];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int rr = wave * kRowsPerWave + i;
      const int v = __builtin_amdgcn_readfirstlane(vr[i]);
      // An empty slot copies row 0 (finite data; its weight is zero).
      const uint16_t* src = (v >= 0 ? kvb + (size_t)v * D : (v == kEmpty ? kvb : winb + (size_t)(-v - 1) * D)) +
                            (lane % ROW_LANES) * 8;
      const uint32_t at = __builtin_amdgcn_readfirstlane(lds_byte_addr(dst + rr * ROW_WORDS));
      if (ROW_LANES == kWave || lane < ROW_LANES) dma_row16(src, at);
    }
  };

  // Partial S^T (this wave's dims) of a tile: rows 0..15 and 16..31.
  // Lane (m, g): s0[i] is row 4g+i, s1[i] is row 16+4g+i, head m.
  auto partial_s = [&](int tile, f32x4& s0, f32x4& s1) {
    const uint32_t* R = Rbuf + (tile % kStages) * kTile * ROW_WORDS;
    s0 = f32x4{0.f, 0.f, 0.f, 0.f};
    s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int w0 = (dbase >> 1) + kk * 16 + g * 4;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&R[m * ROW_WORDS + w0]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&R[(16 + m) * ROW_WORDS + w0]);
      s0 = mfma16x16x32(a0, qf[kk], s0);
      s1 = mfma16x16x32(a1, qf[kk], s1);
    }
  };

  if constexpr (SEL > 0) {  // the first two tiles, less the window tiles already copied
    if (ntiles > 0 && wt < 1) dma(0);
    if (ntiles > 1 && wt < 2) dma(1);
  }

  // Software pipeline over tiles: iteration t computes the (partial) logits
  // of tile t+1 while it finishes tile t (exchange, softmax, PV), so the
  // matrix work of one overlaps the vector work of the other. kStages = 3
  // LDS tiles: t (PV), t+1 (S^T) and t+2 in flight.
  // Tile 0 has landed once at most tile 1's copies are outstanding.
  if (ntiles > 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kRowsPerWave) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();  // tile 0 and the row list visible
  int any_empty_v = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) any_empty_v |= wempty[w];
  // The same in every lane; made scalar so the tile loop branches on it.
  const bool any_empty = __builtin_amdgcn_readfirstlane(any_empty_v) != 0;
  f32x4 s0, s1;   // partial logits of the tile about to be finished
  partial_s(0, s0, s1);
  if (DSPLIT > 1) {
    xbuf[(0 * WAVES + wave) * 2 * kWave + lane] = s0;
    xbuf[(0 * WAVES + wave) * 2 * kWave + kWave + lane] = s1;
  }

  // Adds the partner wave's half of tile t's logits to s0, s1: the two
  // waves of a head group each hold half of the dot products, and both form
  // the same sums (addition is commutative), so they run identical softmax
  // states.
  auto exchange = [&](int t) __attribute__((always_inline)) {
    if (DSPLIT > 1) {
      const int partner = (DSPLIT - 1 - dh) * HG + hq;
      const f32x4* xb = xbuf + ((t & 1) * WAVES + partner) * 2 * kWave;
      s0 += xb[lane];
      s1 += xb[kWave + lane];
    }
  };
  // This wave's partial logits of tile t into s0, s1, and to its partner.
  auto next_logits = [&](int t) __attribute__((always_inline)) {
    partial_s(t, s0, s1);
    if (DSPLIT > 1) {
      f32x4* xw = xbuf + ((t & 1) * WAVES + wave) * 2 * kWave;
      xw[lane] = s0;
      xw[kWave + lane] = s1;
    }
  };
  // Softmax and O^T += R^T P^T of tile t, from its logits c0, c1.
  auto finish = [&](int t, const f32x4 c0, const f32x4 c1) __attribute__((always_inline)) {
    const int t0 = r0 + t * kTile;
    float z[8];
    float mx = -INFINITY;
    if (t0 + kTile <= r1) {  // a full tile (uniform)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = c0[i] * scale2;
        z[4 + i] = c1[i] * scale2;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = (t0 + 4 * g + i < r1) ? c0[i] * scale2 : -INFINITY;
        z[4 + i] = (t0 + 16 + 4 * g + i < r1) ? c1[i] * scale2 : -INFINITY;
      }
    }
    if (any_empty) {  // uniform: empty slots get no weight
      const int4 e0 = *reinterpret_cast<const int4*>(srow + t * kTile + 4 * g);
      const int4 e1 = *reinterpret_cast<const int4*>(srow + t * kTile + 16 + 4 * g);
      z[0] = e0.x == kEmpty ? -INFINITY : z[0];
      z[1] = e0.y == kEmpty ? -INFINITY : z[1];
      z[2] = e0.z == kEmpty ? -INFINITY : z[2];
      z[3] = e0.w == kEmpty ? -INFINITY : z[3];
      z[4] = e1.x == kEmpty ? -INFINITY : z[4];
      z[5] = e1.y == kEmpty ? -INFINITY : z[5];
      z[6] = e1.z == kEmpty ? -INFINITY : z[6];
      z[7] = e1.w == kEmpty ? -INFINITY : z[7];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, z[i]);
    mx = fmaxf(mx, lane_xor16(mx));
    mx = fmaxf(mx, lane_xor32(mx));
    // Lazy rescaling: the weights are taken relative to a reference mrun that
    // only moves when a tile's maximum exceeds it by more than kRescale2, so
    // the weights stay below 2^kRescale2 and the accumulators are rescaled
    // (for the whole wave at once) on few tiles only. The first tile always
    // sets the reference (mrun starts at -FLT_MAX); a tile of empty slots
    // only (mx = -inf) never does.
    if (__ballot(mx > mrun + kRescale2) != 0) {
      const float mnew = fmaxf(mrun, mx);  // finite: the tile holds at least one row
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
      mrun = mnew;
      lrun *= alpha;
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt) {
        o[dt][0] *= alpha;
        o[dt][1] *= alpha;
        o[dt][2] *= alpha;
        o[dt][3] *= alpha;
      }
    }
    u32x4 pw;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t pk = pack_bf16x2(__builtin_amdgcn_exp2f(z[2 * i] - mrun),
                                      __builtin_amdgcn_exp2f(z[2 * i + 1] - mrun));
      // The sum uses the rounded weights the MFMA sees: a dot product of the
      // packed pair with (1, 1).
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk),
                                             __builtin_bit_cast(bf16x2_t, 0x3F803F80u), psum, false);
      pw[i] = pk;
    }
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
    lrun += psum;

    // O^T += R^T P^T over this wave's dims. Within each 16-lane group, lane
    // j points at row (4g + j/4) [then 16 + 4g + j/4], dims 16*dt + 4*(j%4)
    // .. +4; the transposing read hands lane j the 4 rows at dim 16*dt + j.
    const uint32_t* R = Rbuf + (t % kStages) * kTile * ROW_WORDS;
    const int ra = 4 * g + (m >> 2);
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt) {
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      const int col = (dbase >> 1) + dt * 8 + 2 * (m & 3);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(&R[ra * ROW_WORDS + col]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(&R[(16 + ra) * ROW_WORDS + col]));
      // Concatenate as whole vectors (element-wise inserts of bit-cast
      // halves were folded into copies of element 0 by the compiler).
      const i16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[dt] = mfma16x16x32(__builtin_bit_cast(bf16x8, cat), pb, o[dt]);
    }
  };

  int t_first = 0;
  if (SEL > 0 && wt > 0 && ntiles > 1) {
    // A split that starts with a window tile copied it before its selection;
    // it finishes that tile before waiting for tile 1, whose copies went out
    // after the selection, so their latency overlaps tile 0's softmax and
    // P.V instead of delaying them.
    lds_barrier();  // publishes tile 0's partial logits
    exchange(0);
    const f32x4 c0 = s0, c1 = s1;
    finish(0, c0, c1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();  // tile 1 visible; every wave is done with tile 0's logits
    if (2 < ntiles) dma(2);
    next_logits(1);
    t_first = 1;
  }
  for (int t = t_first; t < ntiles; ++t) {
    // Tile t+1 has landed once no copy issued after it is outstanding (tile
    // t+2 is issued below). The barrier also publishes the partial logits of
    // tile t and tells that every wave finished tile t-1, whose slot then
    // takes tile t+2.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (t + 2 < ntiles) dma(t + 2);
    exchange(t);
    const f32x4 c0 = s0, c1 = s1;  // logits of tile t
    if (t + 1 < ntiles) next_logits(t + 1);
    finish(t, c0, c1);
  }

  // Full sum over the four lane groups that share head m.
  float l = lrun + lane_xor16(lrun);
  l += lane_xor32(l);
  // Lane (m, g) holds O[h][dbase + 16*dt + 4g + i]. Results leave through
  // LDS so that each store is 16 contiguous bytes per lane and whole head
  // rows per instruction (straight from the MFMA layout, a store would put
  // 8 bytes per lane into 16 rows 1 KiB apart). Every wave has passed the
  // last tile's barrier, so the two tile slots other than the last tile's
  // are free; each wave stages its own 16 rows there (no barrier needed).
  // words(dt) gives the lane's two packed words of its 4 values at dt; row0
  // is the wave's first head row of the destination (rows D apart).
  constexpr int kPitch = DW * 2 + 8;        // bytes per staged head row (8 of padding)
  constexpr int kSlotBytes = kTile * ROW_WORDS * 4;
  constexpr int kPerSlot = kSlotBytes / (16 * kPitch);  // waves' rows per tile slot
  static_assert(WAVES <= 2 * kPerSlot, "the staged rows fit two tile slots");
  constexpr int CH = DW * 2 / 16;           // 16-byte chunks per head row
  constexpr int HPI = kWave / CH;           // head rows per store instruction
  static_assert(CH * HPI == kWave && 16 % HPI == 0, "whole head rows per store");
  auto store_rows = [&](auto words, uint16_t* row0) __attribute__((always_inline)) {
    const int last = (ntiles - 1) % kStages;
    const int tslot = (last + 1 + wave / kPerSlot) % kStages;
    char* wrows = reinterpret_cast<char*>(Rbuf) + tslot * kSlotBytes + (wave % kPerSlot) * 16 * kPitch;
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt)
      *reinterpret_cast<uint2*>(wrows + m * kPitch + (dt * 16 + g * 4) * 2) = words(dt);
#pragma unroll
    for (int j = 0; j < 16 / HPI; ++j) {
      const int hh = j * HPI + lane / CH, c = lane % CH;
      const uint2 a0 = *reinterpret_cast<const uint2*>(wrows + hh * kPitch + c * 16);
      const uint2 a1 = *reinterpret_cast<const uint2*>(wrows + hh * kPitch + c * 16 + 8);
      *reinterpret_cast<u32x4*>(row0 + (size_t)hh * D + c * 8) = u32x4{a0.x, a0.y, a1.x, a1.y};
    }
  };
  if (splits == 1) {
    // A sink (one logit of head h, no value vector) joins the normalisation:
    // with M = max(running max, sink), the sum becomes l 2^(mrun - M) +
    // 2^(sink - M) and O is scaled by 2^(mrun - M). A sink of -inf changes
    // nothing; a batch row with no rows keeps O = 0.
    float oscale = 1.0f;
    if (sink) {
      const float s2 = sink[h] * kLog2e;
      const float M = fmaxf(mrun, s2);
      oscale = __builtin_amdgcn_exp2f(mrun - M);
      l = l * oscale + __builtin_amdgcn_exp2f(s2 - M);
    }
    const float inv = l > 0.0f ? oscale / l : 0.0f;  // no row at all: zeros
    store_rows([&](int dt) __attribute__((always_inline)) {
                 return make_uint2(pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv),
                                   pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv));
               },
               out + ((size_t)b * Hq + (h - m)) * D + dbase);
  } else {
    // Partials in fp16, scaled by the largest magnitude of this wave's
    // share of O[h] (so every value lies in [-1, 1] and keeps 11 significant
    // bits); the scale goes with the running max and sum.
    float amax = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(o[dt][i]));
    amax = fmaxf(amax, lane_xor16(amax));
    amax = fmaxf(amax, lane_xor32(amax));
    const float sc = amax > 0.0f ? amax : 1.0f;
    const float inv = 1.0f / sc;
    const size_t slot = ((size_t)b * splits + split) * Hq + h;
    store_rows([&](int dt) __attribute__((always_inline)) {
                 return make_uint2(pack_f16x2(o[dt][0] * inv, o[dt][1] * inv),
                                   pack_f16x2(o[dt][2] * inv, o[dt][3] * inv));
               },
               part_o + (slot - m) * D + dbase);
    if (g == 0) {
      float* ml = part_ml + slot * 4;
      if (dh == 0) {
        ml[0] = mrun * kLn2;  // natural-log units for the combine
        ml[1] = l;
      }
      ml[2 + dh] = sc;
      if (DSPLIT == 1) ml[3] = sc;
    }
  }
}

// Log-sum-exp merge of the split partials. A head's D dims are taken by D/8
// threads, 8 dims (16 bytes of fp16) each, and a workgroup of 256 threads
// takes 256/(D/8) heads of one batch row. Splits are taken 8 at a time with
// every load of a chunk issued before any is used (indices past the last
// split are clamped and weighted zero), so a chunk costs one memory latency.
template <int D>
__global__ __launch_bounds__(256) void attend_combine_kernel(
    const uint16_t* __restrict__ part_o, const float4* __restrict__ part_ml,
    const float* __restrict__ sink, uint16_t* __restrict__ out, int Hq, int splits, int nitems) {
  constexpr int TPH = D / 8;      // threads per head
  constexpr int HPW = 256 / TPH;  // heads per workgroup (divides Hq, a multiple of 16)
  constexpr int SC = 8;
  // The same XCD placement as the attention kernel: batch row b is merged on
  // the XCD whose L2 holds its partials.
  const int wg = blockIdx.x;
  const int item = (wg % 8) * (int)(gridDim.x / 8) + wg / 8;
  if (item >= nitems) return;  // padding workgroup (uniform)
  const int bh = item * HPW + (int)threadIdx.x / TPH;
  const int b = bh / Hq;
  const int h = bh % Hq;
  const int d = ((int)threadIdx.x % TPH) * 8;
  const bool upper = d >= D / 2;  // which scale covers these dims
  const size_t base = (size_t)b * splits * Hq + h;  // slot of split 0
  float M = -INFINITY, L = 0.0f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int s0 = 0; s0 < splits; s0 += SC) {
    float4 ml[SC];
    u32x4 v[SC];
#pragma unroll
    for (int j = 0; j < SC; ++j) {
      const size_t slot = base + (size_t)min(s0 + j, splits - 1) * Hq;
      ml[j] = part_ml[slot];
      v[j] = *reinterpret_cast<const u32x4*>(part_o + slot * D + d);
    }
    float Mc = M;
#pragma unroll
    for (int j = 0; j < SC; ++j) Mc = fmaxf(Mc, ml[j].x);
    // Every partial max is finite (a split with no rows wrote -FLT_MAX ln 2
    // and l = 0), so Mc is too and r is 0 on the first chunk (M = -inf).
    const float r = __expf(M - Mc);
    L *= r;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= r;
#pragma unroll
    for (int j = 0; j < SC; ++j) {
      const float f = (s0 + j < splits) ? __expf(ml[j].x - Mc) : 0.0f;
      L += ml[j].y * f;
      const float fs = f * (upper ? ml[j].w : ml[j].z);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float2 a = unpack_f16x2(v[j][q]);
        acc[2 * q] += a.x * fs;
        acc[2 * q + 1] += a.y * fs;
      }
    }
    M = Mc;
  }
  if (sink) {  // the sink's term of the normalisation (natural-log units, as M)
    const float Ms = fmaxf(M, sink[h]);
    const float r = __expf(M - Ms);
    L = L * r + __expf(sink[h] - Ms);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= r;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;  // no row at all: zeros
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q] * inv, acc[2 * q + 1] * inv);
  *reinterpret_cast<u32x4*>(out + ((size_t)b * Hq + h) * D + d) = o;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

template <int D, int HG, int DSPLIT, int SEL = 0>
hipError_t launch_attend_t(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                           const uint16_t* win, uint16_t* out, uint16_t* po, float* pml,
                           const float* sink, const dsa_dims_t& d, const AttendPlan& p,
                           int tokens, hipStream_t st, const SelectArgs& sel = SelectArgs{}) {
  constexpr int WAVES = HG * DSPLIT;
  constexpr int ROW_WORDS = D / 2 + 4;
  constexpr int XWORDS = DSPLIT > 1 ? 2 * WAVES * kWave * 8 : 0;
  const size_t lds = ((size_t)kStages * kTile * ROW_WORDS + XWORDS) * sizeof(uint32_t) +
                     ((size_t)p.rows_per_split + WAVES) * sizeof(int32_t);
  auto kern = sparse_attend_kernel<D, HG, DSPLIT, SEL>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int hgroups = d.q_heads / (16 * HG);
  const int nitems = d.batch * p.splits * hgroups;
  const int grid = (nitems + 7) / 8 * 8;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(WAVES * kWave), lds, st, q, kv, idx, win, out, po,
                     pml, sink, d.n, d.topk, d.window, d.q_heads, d.scale, p.rows_per_split,
                     p.sel_rows, p.splits, nitems, hgroups, tokens, sel);
  return hipGetLastError();
}

// The split combine (several splits only).
hipError_t launch_combine(uint16_t* po, float* pml, const float* sink, uint16_t* out,
                          const dsa_dims_t& d, const AttendPlan& p, hipStream_t st) {
  const int Hq = d.q_heads;
  const int hpw = 256 / (d.head_dim / 8);  // heads per combine workgroup
  const int nitems = d.batch * Hq / hpw;
  const int grid = (nitems + 7) / 8 * 8;
  if (d.head_dim == 512)
    hipLaunchKernelGGL((attend_combine_kernel<512>), dim3(grid), dim3(256), 0, st, po,
                       reinterpret_cast<const float4*>(pml), sink, out, Hq, p.splits, nitems);
  else
    hipLaunchKernelGGL((attend_combine_kernel<128>), dim3(grid), dim3(256), 0, st, po,
                       reinterpret_cast<const float4*>(pml), sink, out, Hq, p.splits, nitems);
  return hipGetLastError();
}

}  // namespace

AttendPlan plan_attend(const dsa_dims_t& d) {
  AttendPlan p{};
  p.heads_per_wg = (d.q_heads % 64 == 0) ? 64 : (d.q_heads % 32 == 0 ? 32 : 16);
  const int hgroups = d.q_heads / p.heads_per_wg;
  // About 256 workgroups in total. The selected rows are shared out in whole
  // tiles, the same number per split, and the window's tiles are dealt round
  // robin to the splits after the last one that holds selected rows; every
  // split holds at least one tile, and at most kMaxSplitTiles (the row list
  // in LDS). At the production shape (k = 1024, W = 128, 8 splits) each
  // split holds 4 tiles of selected rows and splits 0-3 one window tile
  // more, which they copy while they select their rows.
  const int tiles_sel = (d.topk + kTile - 1) / kTile;
  const int tiles_win = (d.window + kTile - 1) / kTile;
  long long want = (256 + (long long)d.batch * hgroups - 1) / ((long long)d.batch * hgroups);
  if (want > tiles_sel + tiles_win) want = tiles_sel + tiles_win;
  if (want < 1) want = 1;
  for (int S = (int)want;; ++S) {
    const int tps = (tiles_sel + S - 1) / S;
    const int s_sel = (tiles_sel + tps - 1) / tps;
    const int splits = S < s_sel + tiles_win ? S : s_sel + tiles_win;
    const int wmax = (tiles_win + splits - 1) / splits;
    if (tps + wmax <= kMaxSplitTiles || S >= tiles_sel + tiles_win) {
      p.sel_rows = tps * kTile;
      p.splits = splits;
      p.rows_per_split = (tps + wmax) * kTile;
      break;
    }
  }
  if (p.splits > 1) {
    p.part_o_off = 0;
    p.part_ml_off = align_up((size_t)d.batch * p.splits * d.q_heads * d.head_dim * sizeof(uint16_t), 256);
    p.bytes = align_up(p.part_ml_off + (size_t)d.batch * p.splits * d.q_heads * 4 * sizeof(float), 256);
  } else {
    p.part_o_off = p.part_ml_off = 0;
    p.bytes = 0;
  }
  return p;
}

hipError_t launch_attend(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                         const uint16_t* win, uint16_t* out, const float* sink,
                         const dsa_dims_t& d, const AttendPlan& p, int tokens, void* ws,
                         hipStream_t st) {
  uint16_t* po = p.splits > 1 ? reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(ws) + p.part_o_off) : nullptr;
  float* pml = p.splits > 1 ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + p.part_ml_off) : nullptr;
  const int hgw = p.heads_per_wg / 16;  // 16-head groups per workgroup
  hipError_t e;
  if (d.head_dim == 512) {
    if (hgw == 4) e = launch_attend_t<512, 4, 2>(q, kv, idx, win, out, po, pml, sink, d, p, tokens, st);
    else if (hgw == 2) e = launch_attend_t<512, 2, 2>(q, kv, idx, win, out, po, pml, sink, d, p, tokens, st);
    else e = launch_attend_t<512, 1, 2>(q, kv, idx, win, out, po, pml, sink, d, p, tokens, st);
  } else {
    if (hgw == 4) e = launch_attend_t<128, 4, 1>(q, kv, idx, win, out, po, pml, sink, d, p, tokens, st);
    else if (hgw == 2) e = launch_attend_t<128, 2, 1>(q, kv, idx, win, out, po, pml, sink, d, p, tokens, st);
    else e = launch_attend_t<128, 1, 1>(q, kv, idx, win, out, po, pml, sink, d, p, tokens, st);
  }
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_combine(po, pml, sink, out, d, p, st);
}

int attend_select_per(const dsa_dims_t& d, const AttendPlan& p, int chunks, int keep) {
  if (d.head_dim != 512 || p.heads_per_wg != 64) return 0;  // 512-thread workgroups only
  // Every workgroup repeats its row's selection; that is free only while all
  // of them run at once (one per CU of the 256). With more, the selection's
  // latency comes once per round of workgroups, and the merge kernel, which
  // selects each row once, is faster (B = 64, N = 262144, k = 2048: 1024
  // workgroups, the step 869 us with the merge kernel, 915 with the selection
  // inside attention).
  const long long wgs = (long long)d.batch * p.splits * (d.q_heads / p.heads_per_wg);
  if (wgs > 256) return 0;
  const long long slots = (long long)chunks * keep;
  return slots <= 512 * 4 ? 4 : slots <= 512 * 8 ? 8 : 0;
}

hipError_t launch_attend_select(const uint16_t* q, const uint16_t* kv, const uint16_t* win,
                                uint16_t* out, const float* sink, const dsa_dims_t& d,
                                const AttendPlan& p, const SelectArgs& sel, int per, void* ws,
                                hipStream_t st) {
  uint16_t* po = p.splits > 1 ? reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(ws) + p.part_o_off) : nullptr;
  float* pml = p.splits > 1 ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + p.part_ml_off) : nullptr;
  hipError_t e = per == 4
      ? launch_attend_t<512, 4, 2, 4>(q, kv, nullptr, win, out, po, pml, sink, d, p, 1, st, sel)
      : launch_attend_t<512, 4, 2, 8>(q, kv, nullptr, win, out, po, pml, sink, d, p, 1, st, sel);
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_combine(po, pml, sink, out, d, p, st);
}

}  // namespace dsa
