// Latent D / U dense projections: Q8_0 weights x q8_1 activations.
//
// Page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1", the
// lat_dense_w11.cu commit message: the two dense projections of a latent
// layer (D into the latent rows, U back out) run as Q8_0 x q8_1 integer dots
// per 32-value block, and D rounds its products to the latent rows' q8_1
// blocks with the rule of the other q8_1 stores, writing fp32 rows too when
// they are asked for.
//
//   y[t][n] = sum over blocks b of d_w[n][b] * d_x[t][b] * I[t][n][b],
//   I[t][n][b] = sum over the block's 32 values of qw * qx   (int32, exact).
//
// Work item: 64 weight rows x 128 tokens, one workgroup of 4 waves; wave
// (wr, wc) owns rows 32 wr .. +31 and tokens 64 wc .. +63, i.e. two 32x32
// output tiles that share the weight fragment.  Per 32-value block and tile:
// one v_mfma_i32_32x32x32_i8 whose accumulator input is the bit pattern of
// 1.5 * 2^23, so the int32 result read as fp32 is exactly 1.5 * 2^23 + I
// (|I| <= 2^19); then
//     t   = fma(that, d_x, -(1.5 * 2^23) * d_x)   = fp32(d_x * I), one rounding
//     acc = fma(d_w, t, acc)
// (1.5 * 2^23 * d_x is exact in fp32: d_x is an fp16 value).  Two VALU
// operations per (row, token, block): that fold, not the MFMA, bounds the
// kernel.  Lane layout of a 32x32 tile: token = lane & 31, rows
// 8 q + 4 (lane >> 5) + i (q, i < 4), so d_x is one value per lane and d_w
// four 16-byte LDS reads shared by both tiles.
//
// K steps of kKB blocks, double-buffered in LDS and with two register sets
// of loads in flight: the workgroup's threads load 16-byte halves of weight
// and activation blocks (buffer loads; Q8_0 rows are 34-byte blocks, read
// unaligned) and the fp16 scales, the lanes of one load instruction walking
// a few contiguous row segments (a lane per row would touch a cache line per
// lane), and write them to LDS as (block, half) planes of 16-byte row slots,
// so a fragment read is 1 KiB contiguous.
//
// Batches of at most kSmallTok tokens take k_dense_small instead: GEMV
// shaped, one workgroup of up to 16 waves per 32 output rows (one q8_1 block
// of every token's output) when only q8_1 output is asked for, else per 4
// rows (a CU keeps a bounded number of loads in flight, so the weight stream
// needs many CUs), followed for q8_1 output by the rounding kernel on the
// fp32 rows.  The lanes of a wave take consecutive blocks of one row
// (coalesced weight reads, issued first into registers), the activation rows
// are copied into LDS once in contiguous 16-byte chunks, integer dots by
// v_dot4, the fold per block in fp32, a butterfly sum across the lanes of a
// row, and the q8_1 rounding from LDS.
//
// Work items are dealt XCD-major: workgroup w runs on XCD w % 8 and takes
// item (w % 8) * ceil(items / 8) + w / 8 of an order that sweeps groups of
// row tiles (about kGroupBytes of weights) over every token tile, so an XCD
// works through a contiguous stretch of that order and its L2 keeps the
// group's weight rows (when all of W exceeds an XCD's 4 MiB L2, the plain
// token-major order streams W from memory again for every token tile).
#include <type_traits>

#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsWG = 64;   // weight rows per work item
constexpr int kTokWG = 128;   // tokens per work item
constexpr int kLogKB = 2;
constexpr int kKB = 1 << kLogKB;  // 32-value blocks per K step
constexpr int kXcds = 8;
constexpr int kGroupBytes = 2 << 20;  // weight bytes of the row tiles of one sweep over the token tiles
// LDS slots of 16 bytes: (block, half) planes of rows/tokens, each plane
// padded by 16 bytes so that the lanes of a load instruction, which walk the
// (block, half) planes of one row, write to different banks.
constexpr int kAPlane = kRowsWG * 16 + 16;
constexpr int kBPlane = kTokWG * 16 + 16;
constexpr int kDwStride = kRowsWG + 4;  // floats; 16-byte multiple, 4 banks apart
constexpr int kDxStride = kTokWG + 4;

struct Smem {
  int8_t a[2][2 * kKB * kAPlane];   // weight codes, plane 2 b + half, row r at 16 r
  int8_t b[2][2 * kKB * kBPlane];   // activation codes, plane 2 b + half, token t at 16 t
  float dw[2][kKB * kDwStride + 4];  // weight block scales [block][row]; the last word takes stores of no task
  float dx[2][kKB * kDxStride + 4];  // activation block scales [block][token]; likewise
};
static_assert(kRowsWG == 64 && kTokWG == 128 && kThreads == 256 && kKB >= 2,
              "the loader deals 64 rows and 128 tokens per step over 256 threads");

template <bool PROBE>
__global__ __launch_bounds__(kThreads) void k_dense_q8_0(const uint8_t* __restrict__ x, const uint8_t* __restrict__ w,
                                                         int T, int N, int K, int n_rt, int n_tt, int group_rows,
                                                         int items, int per_xcd,
                                                         float* __restrict__ y_f32, uint8_t* __restrict__ y_q8,
                                                         ProbeRows probe) {
  __shared__ __align__(16) Smem sm;
  const int wg = blockIdx.x;
  const int item = (wg % kXcds) * per_xcd + wg / kXcds;
  if (item >= items) return;
  // grouped order: group_rows row tiles at a time, swept over every token tile
  const int group = item / (group_rows * n_tt);
  const int within = item - group * group_rows * n_tt;
  const int g_rows = min(group_rows, n_rt - group * group_rows);
  const int tt = within / g_rows, rt = group * group_rows + (within - (within / g_rows) * g_rows);
  const int row0 = rt * kRowsWG, tok0 = tt * kTokWG;
  const int nb = K / 32;
  const int n_steps = (nb + kKB - 1) / kKB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave & 1, wc = wave >> 1;

  // ---- loader: fixed per-thread roles ----
  // Per step the workgroup moves kKB blocks of its 64 weight rows and 128
  // tokens.  Task q = tid + 256 i walks (half, block) fastest, so the lanes of
  // one load instruction read a few contiguous row segments (kKB blocks of a
  // row are adjacent in memory): weight half-block (row q >> (kLogKB + 1),
  // block (q >> 1) & (kKB - 1), half q & 1), activation half-block likewise
  // with tokens, and the scales (row or token q >> kLogKB, block
  // q & (kKB - 1)).
  constexpr int kA = kKB / 2, kB = kKB;                           // 16-byte loads per thread
  constexpr int kSA = (kRowsWG * kKB + kThreads - 1) / kThreads;  // weight scales per thread
  constexpr int kSB = (kTokWG * kKB + kThreads - 1) / kThreads;   // activation scales per thread
  const rsrc_t rw = make_rsrc(w, (uint32_t)((int64_t)N * nb * kQ80Bytes));
  const rsrc_t rx = make_rsrc(x, (uint32_t)((int64_t)T * nb * kQ81Bytes));
  int a_off[kA], b_off[kB], sa_off[kSA], sb_off[kSB];
  int a_blk[kA], b_blk[kB], sa_blk[kSA], sb_blk[kSB];
  int a_lds[kA], b_lds[kB], sa_lds[kSA], sb_lds[kSB];
#pragma unroll
  for (int i = 0; i < kA; ++i) {
    const int q = tid + kThreads * i, rl = q >> (kLogKB + 1), r = row0 + rl, h = q & 1;
    a_blk[i] = (q >> 1) & (kKB - 1);
    a_off[i] = r < N ? (r * nb + a_blk[i]) * kQ80Bytes + 2 + 16 * h : kOutOfRange;
    a_lds[i] = (2 * a_blk[i] + h) * kAPlane + 16 * rl;
  }
#pragma unroll
  for (int j = 0; j < kB; ++j) {
    const int q = tid + kThreads * j, tl = q >> (kLogKB + 1), t = tok0 + tl, h = q & 1;
    b_blk[j] = (q >> 1) & (kKB - 1);
    b_off[j] = t < T ? (t * nb + b_blk[j]) * kQ81Bytes + 4 + 16 * h : kOutOfRange;
    b_lds[j] = (2 * b_blk[j] + h) * kBPlane + 16 * tl;
  }
#pragma unroll
  for (int i = 0; i < kSA; ++i) {
    const int q = tid + kThreads * i, rl = q >> kLogKB, r = row0 + rl;
    sa_blk[i] = q & (kKB - 1);
    sa_off[i] = (q < kRowsWG * kKB && r < N) ? (r * nb + sa_blk[i]) * kQ80Bytes : kOutOfRange;
    sa_lds[i] = q < kRowsWG * kKB ? sa_blk[i] * kDwStride + rl : kKB * kDwStride;
  }
#pragma unroll
  for (int i = 0; i < kSB; ++i) {
    const int q = tid + kThreads * i, tl = q >> kLogKB, t = tok0 + tl;
    sb_blk[i] = q & (kKB - 1);
    sb_off[i] = (q < kTokWG * kKB && t < T) ? (t * nb + sb_blk[i]) * kQ81Bytes : kOutOfRange;
    sb_lds[i] = q < kTokWG * kKB ? sb_blk[i] * kDxStride + tl : kKB * kDxStride;
  }

  // Two register sets of loaded data: set k & 1 holds step k until staged.
  uint4 ra[2][kA], rb[2][kB];
  uint32_t rsa[2][kSA], rsb[2][kSB];
  auto load = [&](auto set_tag, int step) {
    constexpr int S = decltype(set_tag)::value;
    // blocks past the end of K read as zeros (offset beyond the buffer)
    const int kb0 = step * kKB;
    const int sw = __builtin_amdgcn_readfirstlane(kb0 * kQ80Bytes);
    const int sx = __builtin_amdgcn_readfirstlane(kb0 * kQ81Bytes);
#pragma unroll
    for (int i = 0; i < kA; ++i) ra[S][i] = buf_u128(rw, kb0 + a_blk[i] < nb ? a_off[i] : kOutOfRange, sw);
#pragma unroll
    for (int j = 0; j < kB; ++j) rb[S][j] = buf_u128(rx, kb0 + b_blk[j] < nb ? b_off[j] : kOutOfRange, sx);
#pragma unroll
    for (int i = 0; i < kSA; ++i) rsa[S][i] = buf_u16(rw, kb0 + sa_blk[i] < nb ? sa_off[i] : kOutOfRange, sw);
#pragma unroll
    for (int i = 0; i < kSB; ++i) rsb[S][i] = buf_u16(rx, kb0 + sb_blk[i] < nb ? sb_off[i] : kOutOfRange, sx);
  };
  auto stage = [&](auto set_tag, int buf) {
    constexpr int S = decltype(set_tag)::value;
#pragma unroll
    for (int i = 0; i < kA; ++i) *reinterpret_cast<uint4*>(sm.a[buf] + a_lds[i]) = ra[S][i];
#pragma unroll
    for (int j = 0; j < kB; ++j) *reinterpret_cast<uint4*>(sm.b[buf] + b_lds[j]) = rb[S][j];
    // no branches here (see the pipeline below): spare tasks store to a spare word
#pragma unroll
    for (int i = 0; i < kSA; ++i) sm.dw[buf][sa_lds[i]] = half_bits_to_float(rsa[S][i]);
#pragma unroll
    for (int i = 0; i < kSB; ++i) sm.dx[buf][sb_lds[i]] = half_bits_to_float(rsb[S][i]);
  };

  // ---- consumer state ----
  const int col = lane & 31, kh = lane >> 5;
  const bool rows_live = row0 + 32 * wr < N;  // wave-uniform (N % 32 == 0)
  v16i magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits,
                kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits};
  // opaque to the optimizer: the 16 registers stay live instead of being
  // rebuilt (8 v_mov_b64) before every block's MFMAs
  asm volatile("" : "+v"(magic));
  float acc[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;

  auto compute = [&](int buf, int step) {
    if (!rows_live) return;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      const int blk = step * kKB + kb;
      if (blk >= nb) break;
      const v4i va = *reinterpret_cast<const v4i*>(sm.a[buf] + (2 * kb + kh) * kAPlane + 16 * (32 * wr + col));
      const v4i vb0 = *reinterpret_cast<const v4i*>(sm.b[buf] + (2 * kb + kh) * kBPlane + 16 * (64 * wc + col));
      const v4i vb1 =
          *reinterpret_cast<const v4i*>(sm.b[buf] + (2 * kb + kh) * kBPlane + 16 * (64 * wc + 32 + col));
      const v16i r0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb0, magic, 0, 0, 0);
      const v16i r1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb1, magic, 0, 0, 0);
      const float dx0 = sm.dx[buf][kb * kDxStride + 64 * wc + col];
      const float dx1 = sm.dx[buf][kb * kDxStride + 64 * wc + 32 + col];
      const float m0 = -kMagic * dx0, m1 = -kMagic * dx1;
      float dwv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 d4 = *reinterpret_cast<const float4*>(&sm.dw[buf][kb * kDwStride + 32 * wr + 8 * q + 4 * kh]);
        dwv[4 * q] = d4.x;
        dwv[4 * q + 1] = d4.y;
        dwv[4 * q + 2] = d4.z;
        dwv[4 * q + 3] = d4.w;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float t0 = __builtin_fmaf(as_float(r0[i]), dx0, m0);
        const float t1 = __builtin_fmaf(as_float(r1[i]), dx1, m1);
        acc[0][i] = __builtin_fmaf(dwv[i], t0, acc[0][i]);
        acc[1][i] = __builtin_fmaf(dwv[i], t1, acc[1][i]);
      }
      if (PROBE) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int t = tok0 + 64 * wc + 32 * j + col;
          if (t < T) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int r = row0 + 32 * wr + 8 * (i >> 2) + 4 * kh + (i & 3) - probe.row0;
              if (r >= 0 && r < probe.rows)
                probe.out[((int64_t)t * probe.rows + r) * nb + blk] = (j ? r1[i] : r0[i]) - kMagicBits;
            }
          }
        }
      }
    }
  };

  // ---- pipeline ----
  // Step g: the MFMAs of step g from LDS buffer g & 1; then step g+1 (register
  // set (g+1) & 1) is staged into the other buffer and the loads of step g+3
  // go into the freed set; barrier.  Loads are in flight for two steps, and
  // staging comes after the MFMAs so that its wait for the loads (the
  // compiler's count is conservative on the loop's first half) is mostly
  // covered.  Loads and stores are issued on every step, also past the last
  // one (those loads are out of range and return zeros without touching
  // memory), so no branch blurs the compiler's wait counts.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  load(S0{}, 0);
  load(S1{}, 1);
  stage(S0{}, 0);
  load(S0{}, 2);
  __syncthreads();
  for (int g = 0; g < n_steps; g += 2) {
    compute(0, g);
    stage(S1{}, 1);
    load(S1{}, g + 3);
    __syncthreads();
    if (g + 1 >= n_steps) break;
    compute(1, g + 1);
    stage(S0{}, 0);
    load(S0{}, g + 4);
    __syncthreads();
  }

  // ---- epilogue ----
  if (!rows_live) return;
  const int nrow = row0 + 32 * wr;  // first row of this wave's 32 (one q8_1 block of a token's output)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = tok0 + 64 * wc + 32 * j + col;
    if (y_f32 && t < T) {
      float* dst = y_f32 + (int64_t)t * N + nrow + 4 * kh;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(dst + 8 * q) =
            float4{acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
    }
    if (y_q8) {
      // q8_1 rule over the token's 32 rows (16 here, 16 in lane ^ 32):
      // amax, d = amax / 127, id = 1 / d, q = round-half-away(v * id), IEEE fp32
#pragma clang fp contract(off)
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(acc[j][i]));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const float d = amax / 127.0f;
      const float id = d != 0.0f ? 1.0f / d : 0.0f;
      uint32_t pk[4];
      int sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        pk[q] = pack_codes(round_half_away(acc[j][4 * q] * id), round_half_away(acc[j][4 * q + 1] * id),
                           round_half_away(acc[j][4 * q + 2] * id), round_half_away(acc[j][4 * q + 3] * id));
        sum = __builtin_amdgcn_sdot4((int)pk[q], 0x01010101, sum, false);
      }
      sum += __shfl_xor(sum, 32);
      if (t < T) {
        uint8_t* blk = y_q8 + ((int64_t)t * (N / 32) + nrow / 32) * kQ81Bytes;
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<uint32_t*>(blk + 4 + 8 * q + 4 * kh) = pk[q];
        if (kh == 0)
          *reinterpret_cast<uint32_t*>(blk) =
              float_to_half_bits(d) | (float_to_half_bits(fp32_barrier(d * (float)sum)) << 16);
      }
    }
  }
}

// ------------------------------------------------------------------------
// Decode-sized batches.
// ------------------------------------------------------------------------
constexpr int kSmallTok = 8;      // largest batch of the GEMV-shaped kernel
constexpr int kSmallRows = 32;    // output rows per workgroup with q8_1 output (one q8_1 block)
// With fp32 output only, a workgroup takes this many rows (at least one lane
// group): a CU keeps only so many loads in flight, so the weight stream needs
// many CUs, and D (1024 rows) would have 32 workgroups of 32 rows.
constexpr int kSmallRowsF32 = 4;
// Waves of a workgroup of ROWS rows for LPR lanes per row: enough that each
// wave has one or two rows (many loads in flight per CU: these workgroups are
// latency bound), at most 16.
constexpr int small_waves(int lpr, int rows) { return 64 / lpr * 16 <= rows ? 16 : rows / (64 / lpr); }
constexpr int small_rows_f32(int lpr) { return 64 / lpr > kSmallRowsF32 ? 64 / lpr : kSmallRowsF32; }

// 16 bytes from LDS at a 4-byte-aligned address (one ds_read_b128: gfx950
// serves unaligned LDS accesses).
__device__ __forceinline__ uint4 lds_u128_a4(const uint8_t* p) {
  struct __attribute__((packed, aligned(4))) U {
    uint32_t a, b, c, d;
  };
  const U v = *reinterpret_cast<const U*>(p);
  return uint4{v.a, v.b, v.c, v.d};
}

// Sum over the LPR lanes of each aligned lane group (LPR a power of two <= 64).
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// BPL: blocks per lane and row (the row's K/32 blocks are dealt to LPR lanes
// round-robin); LPR: lanes per row; ROWS: output rows per workgroup (32 for
// q8_1 output).  A row's value does not depend on ROWS: the same lanes fold
// the same blocks in the same order.
template <int BPL, int LPR, bool PROBE, int WFMT, int ROWS>
__global__ __launch_bounds__(64 * small_waves(LPR, ROWS)) void k_dense_small(const uint8_t* __restrict__ x,
                                                                     const uint8_t* __restrict__ w, int T, int N,
                                                                     int K, float* __restrict__ y_f32,
                                                                     uint8_t* __restrict__ y_q8, ProbeRows probe) {
  constexpr int kSmallThreads = 64 * small_waves(LPR, ROWS);
  constexpr int kRowsPerIter = 64 / LPR;
  constexpr int kRowsPerWave = ROWS / small_waves(LPR, ROWS);
  static_assert(kRowsPerWave % kRowsPerIter == 0 && kRowsPerWave >= kRowsPerIter,
                "rows of a wave come in whole iterations");
  __shared__ float ys[kSmallTok][ROWS];
  extern __shared__ __align__(16) uint8_t xraw[];  // the T activation rows as they are in memory (+16)
  const int nb = K / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = blockIdx.x * ROWS;
  const int li = lane & (LPR - 1), sub = lane / LPR;  // lane within its row group, row group
  constexpr int kWB = WFMT == kDenseQ40 ? kQ40Bytes : kQ80Bytes;  // weight block bytes
  const rsrc_t rw = make_rsrc(w, (uint32_t)((int64_t)N * nb * kWB));
  const rsrc_t rx = make_rsrc(x, (uint32_t)((int64_t)T * nb * kQ81Bytes));

  // This wave's weight blocks (row of iteration it, block li + LPR j) into
  // registers first, so their latency overlaps the activation staging below.
  constexpr int kIters = kRowsPerWave / kRowsPerIter;
  uint32_t wq[kIters][BPL][8];
  float wd[kIters][BPL];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int r = row0 + kRowsPerWave * wave + kRowsPerIter * it + sub;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int b = li + LPR * j;
      const int off = (r < N && b < nb) ? (r * nb + b) * kWB : kOutOfRange;
      if constexpr (WFMT == kDenseQ40) {
        // 16 bytes of nibbles: element i < 16 low nibble of byte i, i >= 16 high nibble of byte i - 16
        const uint4 n = buf_u128(rw, off, 2);
        const uint32_t nw[4] = {n.x, n.y, n.z, n.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          wq[it][j][k] = down_lookup<kDownQ40>(nw[k] & 0x0f0f0f0fu);
          wq[it][j][4 + k] = down_lookup<kDownQ40>((nw[k] >> 4) & 0x0f0f0f0fu);
        }
      } else {
        const uint4 w0 = buf_u128(rw, off, 2), w1 = buf_u128(rw, off, 18);
        wq[it][j][0] = w0.x; wq[it][j][1] = w0.y; wq[it][j][2] = w0.z; wq[it][j][3] = w0.w;
        wq[it][j][4] = w1.x; wq[it][j][5] = w1.y; wq[it][j][6] = w1.z; wq[it][j][7] = w1.w;
      }
      wd[it][j] = half_bits_to_float(buf_u16(rw, off, 0));
    }
  }

  // The activation rows ([T][K/32] q8_1 blocks, contiguous) into LDS once, in
  // consecutive 16-byte chunks.
  {
    const int xbytes = T * nb * kQ81Bytes;  // a multiple of 4
    const int full = xbytes / 16, tail = (xbytes - 16 * full) / 4;
    for (int c = tid; c < full; c += kSmallThreads) reinterpret_cast<uint4*>(xraw)[c] = buf_u128(rx, 16 * c, 0);
    if (tid < tail) reinterpret_cast<uint32_t*>(xraw)[4 * full + tid] = buf_u32(rx, 16 * full + 4 * tid, 0);
  }
  __syncthreads();
  uint32_t xq[kSmallTok][BPL][8];
  float xd[kSmallTok][BPL];
#pragma unroll
  for (int t = 0; t < kSmallTok; ++t) {
    if (t >= T) break;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int b = min(li + LPR * j, nb - 1);  // lanes past the row's last block compute unused values
      const uint8_t* src = xraw + (t * nb + b) * kQ81Bytes;
      xd[t][j] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(src));
      const uint32_t* cw = reinterpret_cast<const uint32_t*>(src + 4);  // 4-byte aligned
#pragma unroll
      for (int k = 0; k < 8; ++k) xq[t][j][k] = cw[k];
    }
  }

#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int rl = kRowsPerWave * wave + kRowsPerIter * it + sub;  // row within the workgroup
    const int r = row0 + rl;
    float part[kSmallTok];
#pragma unroll
    for (int t = 0; t < kSmallTok; ++t) part[t] = 0.f;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int b = li + LPR * j;
      // activation block (t, b) from LDS; lanes past the row's last block read
      // block nb - 1 and multiply it by zeros
      const uint8_t* xb = xraw + min(b, nb - 1) * kQ81Bytes;
#pragma unroll
      for (int t = 0; t < kSmallTok; ++t) {
        if (t >= T) break;
        const uint8_t* src = xb + t * nb * kQ81Bytes;
        const uint4 c0 = lds_u128_a4(src + 4), c1 = lds_u128_a4(src + 20);
        const float xdv = half_bits_to_float(*reinterpret_cast<const uint16_t*>(src));
        const uint32_t xw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        int dot = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) dot = __builtin_amdgcn_sdot4((int)wq[it][j][k], (int)xw[k], dot, false);
        part[t] = __builtin_fmaf(wd[it][j], xdv * (float)dot, part[t]);
        if (PROBE && r < N && b < nb) {
          const int pr = r - probe.row0;
          if (pr >= 0 && pr < probe.rows) probe.out[((int64_t)t * probe.rows + pr) * nb + b] = dot;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kSmallTok; ++t) {
      if (t >= T) break;
      const float v = group_sum<LPR>(part[t]);
      if (li == 0) ys[t][rl] = v;
    }
  }
  __syncthreads();

  if (y_f32) {
    for (int i = tid; i < T * ROWS; i += kSmallThreads) {
      const int t = i / ROWS, rl = i - t * ROWS;
      if (row0 + rl < N) y_f32[(int64_t)t * N + row0 + rl] = ys[t][rl];
    }
  }
  if (ROWS == kSmallRows && y_q8 && tid < 64 * ((T + 1) / 2)) {
    // q8_1 rule over the 32 rows of a token, 32 lanes per token (two tokens a wave)
#pragma clang fp contract(off)
    const int t = tid >> 5, i = tid & 31;
    const float v = ys[t < T ? t : 0][i];
    float amax = fabsf(v);
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const float d = amax / 127.0f;
    const float id = d != 0.0f ? 1.0f / d : 0.0f;
    const int q = round_half_away(v * id);
    int sum = q;
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) sum += __shfl_xor(sum, m);
    if (t < T) {
      uint8_t* blk = y_q8 + ((int64_t)t * (N / 32) + row0 / 32) * kQ81Bytes;
      blk[4 + i] = (uint8_t)(int8_t)q;
      if (i == 0)
        *reinterpret_cast<uint32_t*>(blk) =
            float_to_half_bits(d) | (float_to_half_bits(fp32_barrier(d * (float)sum)) << 16);
    }
  }
}

template <int BPL, int LPR, int WFMT, int ROWS>
void launch_small_rows(const uint8_t* x, const uint8_t* w, int T, int N, int K, float* y_f32, uint8_t* y_q8,
                       const ProbeRows* probe, hipStream_t st) {
  const dim3 grid((N + ROWS - 1) / ROWS);
  const size_t lds = (size_t)T * (K / 32) * kQ81Bytes + 16;
  const ProbeRows none = {nullptr, 0, 0};
  const dim3 block(64 * small_waves(LPR, ROWS));
  if (probe)
    hipLaunchKernelGGL((k_dense_small<BPL, LPR, true, WFMT, ROWS>), grid, block, lds, st, x, w, T, N, K, y_f32, y_q8,
                       *probe);
  else
    hipLaunchKernelGGL((k_dense_small<BPL, LPR, false, WFMT, ROWS>), grid, block, lds, st, x, w, T, N, K, y_f32, y_q8,
                       none);
}

// q8_1 output: workgroups of 32 rows, which round their rows themselves.  fp32
// output only: workgroups of small_rows_f32(LPR) rows, many more of them.
template <int BPL, int LPR, int WFMT>
void launch_small_fmt(const uint8_t* x, const uint8_t* w, int T, int N, int K, float* y_f32, uint8_t* y_q8,
                      const ProbeRows* probe, hipStream_t st) {
  if (y_q8)
    launch_small_rows<BPL, LPR, WFMT, kSmallRows>(x, w, T, N, K, y_f32, y_q8, probe, st);
  else
    launch_small_rows<BPL, LPR, WFMT, small_rows_f32(LPR)>(x, w, T, N, K, y_f32, nullptr, probe, st);
}

template <int BPL, int LPR>
void launch_small(int wfmt, const uint8_t* x, const uint8_t* w, int T, int N, int K, float* y_f32, uint8_t* y_q8,
                  const ProbeRows* probe, hipStream_t st) {
  if (wfmt == kDenseQ40)
    launch_small_fmt<BPL, LPR, kDenseQ40>(x, w, T, N, K, y_f32, y_q8, probe, st);
  else
    launch_small_fmt<BPL, LPR, kDenseQ80>(x, w, T, N, K, y_f32, y_q8, probe, st);
}

// The GEMV-shaped kernel's configuration for K/32 blocks, or false when the
// batch or K is too large for it (its activation blocks live in registers).
bool small_config(int64_t T, int nb, int* bpl, int* lpr) {
  if (T > kSmallTok) return false;
  if (nb <= 8) { *lpr = 8; *bpl = 1; return true; }
  if (nb <= 16) { *lpr = 16; *bpl = 1; return true; }
  if (nb <= 32) { *lpr = 32; *bpl = 1; return true; }
  *lpr = 64;
  if (nb <= 64) { *bpl = 1; return true; }
  if (nb <= 128) { *bpl = 2; return true; }
  if (nb <= 256 && T <= kSmallTok / 2) { *bpl = 4; return true; }
  return false;
}

}  // namespace

bool dense_shape_ok(int wfmt, int64_t T, int N, int K) {
  int bpl = 0, lpr = 0;
  return wfmt == kDenseQ80 || small_config(T, K / 32, &bpl, &lpr) || dense_ws_shape(N, K);
}

hipError_t launch_dense(const uint8_t* x, const uint8_t* w, int wfmt, int64_t T, int N, int K, float* y_f32,
                        uint8_t* y_q8, const ProbeRows* probe, int num_cus, hipStream_t st) {
  int bpl = 0, lpr = 0;
  if (small_config(T, K / 32, &bpl, &lpr)) {
    const int t = (int)T;
    // Both outputs: the fp32 rows from the many-workgroup kernel, then their
    // q8_1 rounding (the same bytes the 32-row workgroups would write).
    uint8_t* q8_direct = y_f32 ? nullptr : y_q8;
    if (lpr == 8) launch_small<1, 8>(wfmt, x, w, t, N, K, y_f32, q8_direct, probe, st);
    else if (lpr == 16) launch_small<1, 16>(wfmt, x, w, t, N, K, y_f32, q8_direct, probe, st);
    else if (lpr == 32) launch_small<1, 32>(wfmt, x, w, t, N, K, y_f32, q8_direct, probe, st);
    else if (bpl == 1) launch_small<1, 64>(wfmt, x, w, t, N, K, y_f32, q8_direct, probe, st);
    else if (bpl == 2) launch_small<2, 64>(wfmt, x, w, t, N, K, y_f32, q8_direct, probe, st);
    else launch_small<4, 64>(wfmt, x, w, t, N, K, y_f32, q8_direct, probe, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !y_q8 || q8_direct) return e;
    return launch_quantize_q8_1(y_f32, T, N, y_q8, st);
  }
  // Q4_0 weights above the GEMV sizes take the persistent kernel at any T
  // (the entry point has checked its shape rule); Q8_0 weights from T = 128.
  if (dense_ws_shape(N, K) && (wfmt == kDenseQ40 || T >= 128))
    return launch_dense_ws(x, w, wfmt, T, N, K, y_f32, y_q8, probe, num_cus, st);
  const int n_rt = (N + kRowsWG - 1) / kRowsWG;
  const int n_tt = (int)((T + kTokWG - 1) / kTokWG);
  const int items = n_rt * n_tt;
  const int group_rows = max(1, min(n_rt, (int)(kGroupBytes / ((int64_t)kRowsWG * (K / 32) * kQ80Bytes))));
  const int per_xcd = (items + kXcds - 1) / kXcds;
  const dim3 grid(per_xcd * kXcds);
  const ProbeRows none = {nullptr, 0, 0};
  if (probe)
    hipLaunchKernelGGL(k_dense_q8_0<true>, grid, dim3(kThreads), 0, st, x, w, (int)T, N, K, n_rt, n_tt, group_rows,
                       items, per_xcd, y_f32, y_q8, *probe);
  else
    hipLaunchKernelGGL(k_dense_q8_0<false>, grid, dim3(kThreads), 0, st, x, w, (int)T, N, K, n_rt, n_tt, group_rows,
                       items, per_xcd, y_f32, y_q8, none);
  return hipGetLastError();
}

}  // namespace latmoe
