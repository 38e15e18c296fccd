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
// K steps of kKB blocks, double-buffered in LDS: every thread loads one
// 16-byte half of a weight block's codes and two of activation codes
// (buffer loads; Q8_0 rows are 34-byte blocks, read unaligned), plus the fp16
// scales, and writes them to LDS as [block][half][row][16 B] so that a
// fragment read is 1 KiB contiguous.  Loads for step g + 2 are issued before
// the MFMAs of step g.
//
// Work items are dealt XCD-major: workgroup w runs on XCD w % 8 and takes
// item (w % 8) * ceil(items / 8) + w / 8, items ordered token tile major,
// so each XCD's L2 holds one contiguous range of activation rows and the
// weight rows it sweeps over.
#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsWG = 64;   // weight rows per work item
constexpr int kTokWG = 128;   // tokens per work item
constexpr int kKB = 2;        // 32-value blocks per K step
constexpr int kQ80Bytes = 34;
constexpr int kXcds = 8;

struct Smem {
  int8_t a[2][kKB][2][kRowsWG][16];  // weight codes [buf][block][half][row]
  int8_t b[2][kKB][2][kTokWG][16];   // activation codes [buf][block][half][token]
  float dw[2][kKB][kRowsWG];         // weight block scales
  float dx[2][kKB][kTokWG];          // activation block scales
};
static_assert(kRowsWG * kKB * 2 == kThreads, "one weight half-block per thread and step");
static_assert(kTokWG * kKB * 2 == 2 * kThreads, "two activation half-blocks per thread and step");

template <bool PROBE>
__global__ __launch_bounds__(kThreads) void k_dense_q8_0(const uint8_t* __restrict__ x, const uint8_t* __restrict__ w,
                                                         int T, int N, int K, int n_rt, int items, int per_xcd,
                                                         float* __restrict__ y_f32, uint8_t* __restrict__ y_q8,
                                                         ProbeRows probe) {
  __shared__ __align__(16) Smem sm;
  const int wg = blockIdx.x;
  const int item = (wg % kXcds) * per_xcd + wg / kXcds;
  if (item >= items) return;
  const int tt = item / n_rt, rt = item - tt * n_rt;
  const int row0 = rt * kRowsWG, tok0 = tt * kTokWG;
  const int nb = K / 32;
  const int n_steps = (nb + kKB - 1) / kKB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave & 1, wc = wave >> 1;

  // ---- loader: fixed per-thread roles ----
  // weight half-block: row row0 + (tid & 63), block (tid >> 7) of the step, half (tid >> 6) & 1
  const rsrc_t rw = make_rsrc(w, (uint32_t)((int64_t)N * nb * kQ80Bytes));
  const rsrc_t rx = make_rsrc(x, (uint32_t)((int64_t)T * nb * kQ81Bytes));
  const int a_row = row0 + (tid & 63), a_blk = tid >> 7, a_half = (tid >> 6) & 1;
  const int a_off = a_row < N ? (a_row * nb + a_blk) * kQ80Bytes + 2 + 16 * a_half : kOutOfRange;
  // weight scale (threads < 128): row row0 + (tid & 63), block tid >> 6
  const int s_row = row0 + (tid & 63), s_blk = (tid >> 6) & 1;
  const int sw_off = (tid < kRowsWG * kKB && s_row < N) ? (s_row * nb + s_blk) * kQ80Bytes : kOutOfRange;
  // activation half-blocks: item q = tid + 256 j -> block q >> 8, half (q >> 7) & 1, token q & 127
  int b_off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = tid + kThreads * j;
    const int t = tok0 + (q & 127);
    b_off[j] = t < T ? (t * nb + (q >> 8)) * kQ81Bytes + 4 + 16 * ((q >> 7) & 1) : kOutOfRange;
  }
  // activation scale: token tok0 + (tid & 127), block tid >> 7
  const int s_tok = tok0 + (tid & 127);
  const int sx_off = s_tok < T ? (s_tok * nb + (tid >> 7)) * kQ81Bytes : kOutOfRange;

  uint4 ra, rb[2];
  uint32_t rsw, rsx;
  int ls = 0;  // next step to load
  auto load_next = [&]() {
    // blocks past the end of K read as zeros (offset beyond the buffer)
    const int kb0 = ls * kKB;
    const bool a_in = kb0 + a_blk < nb, s_in = kb0 + s_blk < nb, x_in = kb0 + (tid >> 7) < nb;
    const int sw = __builtin_amdgcn_readfirstlane(kb0 * kQ80Bytes);
    const int sx = __builtin_amdgcn_readfirstlane(kb0 * kQ81Bytes);
    ra = buf_u128(rw, a_in ? a_off : kOutOfRange, sw);
#pragma unroll
    for (int j = 0; j < 2; ++j) rb[j] = buf_u128(rx, kb0 + ((tid + kThreads * j) >> 8) < nb ? b_off[j] : kOutOfRange, sx);
    rsw = buf_u16(rw, s_in ? sw_off : kOutOfRange, sw);
    rsx = buf_u16(rx, x_in ? sx_off : kOutOfRange, sx);
    ++ls;
  };
  auto stage = [&](int buf) {
    reinterpret_cast<uint4*>(&sm.a[buf][0][0][0][0])[tid] = ra;
#pragma unroll
    for (int j = 0; j < 2; ++j) reinterpret_cast<uint4*>(&sm.b[buf][0][0][0][0])[tid + kThreads * j] = rb[j];
    if (tid < kRowsWG * kKB) (&sm.dw[buf][0][0])[tid] = half_bits_to_float(rsw);
    (&sm.dx[buf][0][0])[tid] = half_bits_to_float(rsx);
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
      const v4i va = *reinterpret_cast<const v4i*>(&sm.a[buf][kb][kh][32 * wr + col][0]);
      const v4i vb0 = *reinterpret_cast<const v4i*>(&sm.b[buf][kb][kh][64 * wc + col][0]);
      const v4i vb1 = *reinterpret_cast<const v4i*>(&sm.b[buf][kb][kh][64 * wc + 32 + col][0]);
      const v16i r0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb0, magic, 0, 0, 0);
      const v16i r1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb1, magic, 0, 0, 0);
      const float dx0 = sm.dx[buf][kb][64 * wc + col];
      const float dx1 = sm.dx[buf][kb][64 * wc + 32 + col];
      const float m0 = -kMagic * dx0, m1 = -kMagic * dx1;
      float dwv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 d4 = *reinterpret_cast<const float4*>(&sm.dw[buf][kb][32 * wr + 8 * q + 4 * kh]);
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

  // ---- pipeline: stage g+1, load g+2, compute g, barrier ----
  load_next();
  stage(0);
  if (n_steps > 1) load_next();
  __syncthreads();
  for (int g = 0; g < n_steps; ++g) {
    if (g + 1 < n_steps) stage((g + 1) & 1);
    if (g + 2 < n_steps) load_next();
    compute(g & 1, g);
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

}  // namespace

hipError_t launch_dense_q8_0(const uint8_t* x, const uint8_t* w, int64_t T, int N, int K, float* y_f32,
                             uint8_t* y_q8, const ProbeRows* probe, hipStream_t st) {
  const int n_rt = (N + kRowsWG - 1) / kRowsWG;
  const int n_tt = (int)((T + kTokWG - 1) / kTokWG);
  const int items = n_rt * n_tt;
  const int per_xcd = (items + kXcds - 1) / kXcds;
  const dim3 grid(per_xcd * kXcds);
  const ProbeRows none = {nullptr, 0, 0};
  if (probe)
    hipLaunchKernelGGL(k_dense_q8_0<true>, grid, dim3(kThreads), 0, st, x, w, (int)T, N, K, n_rt, items, per_xcd,
                       y_f32, y_q8, *probe);
  else
    hipLaunchKernelGGL(k_dense_q8_0<false>, grid, dim3(kThreads), 0, st, x, w, (int)T, N, K, n_rt, items, per_xcd,
                       y_f32, y_q8, none);
  return hipGetLastError();
}

}  // namespace latmoe
