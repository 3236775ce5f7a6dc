// Indexer query projection on gfx950 ("feat: Add DeepSeek-V4 CSA attention
// kernels", section "How the algorithm works", step table, step 2: the
// indexer query is projected into 128 channels per head before scoring; the
// pull request runs it as a hand-tiled GEMV, nki_indexer_qproj_gemv).
//
//   q[b, o] = sum_i x[b, i] * w[o, i],   o < O = H_I * 128
//
// With a decode batch of up to 16 rows this is a skinny product whose cost
// is reading w once (O x d_in bf16). MFMA 16x16x32 takes 16 outputs as M and
// the batch rows as N (rows past B read as zero). A workgroup of 8 waves owns
// 32 outputs and its waves split d_in eight ways. Loaded in the MFMA operand
// layout, a wave's read of w touches 16 rows in 64-byte pieces per
// instruction and streamed at about 3.4 TB/s; so w is read as the indexer
// reads its keys: each instruction takes 1 KB of four rows (256 B of each,
// 16 lanes per row), the pieces are written to the wave's LDS area with each
// row's 16-byte chunks XOR-swizzled by the row index, and read back in MFMA
// layout without bank conflicts. Three register buffers keep two pieces of
// loads in flight while one is staged and multiplied. The eight waves'
// partial tiles are added in LDS in a fixed order, so results are
// deterministic. x is small and is read from L2, each piece's fragments
// with the piece's loads. Output: bf16, rounded to nearest even from the fp32
// sums.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kQpWaves = 8;
constexpr int kQpThreads = kQpWaves * kWave;
constexpr int kQpOut = 32;    // outputs per workgroup: 2 tiles of 16
constexpr int kQpCols = 128;  // columns of w per piece: 256 B of each of 32 rows

__global__ __launch_bounds__(kQpThreads) void qproj_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, uint16_t* __restrict__ out,
    int B, int d_in, int O) {
  __shared__ u32x4 stage_lds[kQpWaves][kQpOut * 16];  // 8 KB per wave: 32 rows x 16 chunks
  __shared__ f32x4 part[kQpWaves][2][kWave];          // every wave's two partial tiles
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int m = lane & 15;
  const int g = lane >> 4;
  const int o0 = blockIdx.x * kQpOut;
  const int b0 = blockIdx.y * 16;
  const bool has_row = b0 + m < B;  // this lane's batch row exists (B operand)
  u32x4* st = stage_lds[wave];

  // This wave's columns [c0, c1) of w (a multiple of 32 wide), in pieces of
  // kQpCols; the last piece may be partial, its missing chunks read as zero.
  const int span = d_in / kQpWaves;
  const int c0 = wave * span;
  const int c1 = c0 + span;
  const int npieces = (span + kQpCols - 1) / kQpCols;
  const uint16_t* xr = x + (size_t)(has_row ? b0 + m : 0) * d_in;

  // Piece p: instruction j covers rows 4j .. 4j+3; lane l takes row
  // 4j + l/16, 16-byte chunk l%16. The piece's x fragments (B operand,
  // one per 32 columns) are loaded with it.
  constexpr int KK = kQpCols / 32;
  auto load_piece = [&](u32x4 (&r)[8], bf16x8 (&bx)[KK], int p) __attribute__((always_inline)) {
    const int col = c0 + p * kQpCols + (lane & 15) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 4 * j + (lane >> 4);
      r[j] = col < c1 ? __builtin_nontemporal_load(
                            reinterpret_cast<const u32x4*>(w + (size_t)(o0 + row) * d_in + col))
                      : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int xc = c0 + p * kQpCols + kk * 32 + g * 8;
      bx[kk] = (has_row && xc < c1) ? *reinterpret_cast<const bf16x8*>(xr + xc) : bf16x8{};
    }
  };
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  auto mul_piece = [&](const u32x4 (&r)[8], const bf16x8 (&bx)[KK]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 4 * j + (lane >> 4);
      st[row * 16 + ((lane & 15) ^ (row & 15))] = r[j];
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, st[m * 16 + ((4 * kk + g) ^ m)]);
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, st[(16 + m) * 16 + ((4 * kk + g) ^ m)]);
      acc0 = mfma16x16x32(a0, bx[kk], acc0);
      acc1 = mfma16x16x32(a1, bx[kk], acc1);
    }
  };
  u32x4 ra[8], rb[8], rc[8];
  bf16x8 xa[KK], xb[KK], xc[KK];
  if (npieces > 0) load_piece(ra, xa, 0);
  if (npieces > 1) load_piece(rb, xb, 1);
  for (int p = 0; p < npieces; p += 3) {
    if (p + 2 < npieces) load_piece(rc, xc, p + 2);
    mul_piece(ra, xa);
    if (p + 1 >= npieces) break;
    if (p + 3 < npieces) load_piece(ra, xa, p + 3);
    mul_piece(rb, xb);
    if (p + 2 >= npieces) break;
    if (p + 4 < npieces) load_piece(rb, xb, p + 4);
    mul_piece(rc, xc);
  }

  // Lane (m, g) holds outputs o0 + 16t + 4g + i of batch row b0 + m.
  part[wave][0][lane] = acc0;
  part[wave][1][lane] = acc1;
  __syncthreads();
  if (wave < 2) {
    f32x4 sum = part[0][wave][lane];
#pragma unroll
    for (int v = 1; v < kQpWaves; ++v) {
      const f32x4 q = part[v][wave][lane];
      sum[0] += q[0];
      sum[1] += q[1];
      sum[2] += q[2];
      sum[3] += q[3];
    }
    if (has_row) {
      uint2 o;
      o.x = pack_bf16x2(sum[0], sum[1]);
      o.y = pack_bf16x2(sum[2], sum[3]);
      *reinterpret_cast<uint2*>(out + (size_t)(b0 + m) * O + o0 + 16 * wave + 4 * g) = o;
    }
  }
}

}  // namespace

hipError_t launch_qproj(const uint16_t* x, const uint16_t* w, uint16_t* out, int B, int d_in,
                        int O, hipStream_t st) {
  const dim3 grid(O / kQpOut, (B + 15) / 16);
  hipLaunchKernelGGL(qproj_kernel, grid, dim3(kQpThreads), 0, st, x, w, out, B, d_in, O);
  return hipGetLastError();
}

}  // namespace dsa
