// Latent D / U dense projection, Q8_0 weights x q8_1 activations, for batches
// of whole token tiles: a persistent, warp-specialized kernel with the
// structure of the expert stage's down kernel (N % 128 == 0, K % 256 == 0).
//
// Page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1", the
// lat_dense_w11.cu commit message: D and U are Q8_0 x q8_1 integer dots per
// 32-value block, D stores its products as q8_1 rows (the rule of the other
// q8_1 stores):
//   y[t][n] = sum over blocks b of d_w[n][b] * d_x[t][b] * I[t][n][b].
//
// Work item: 128 weight rows x 128 tokens.  One workgroup of 12 waves per CU
// (3 per SIMD) walks its items:
//   8 consumer waves: wave c owns rows 32 (c & 3) .. +31 against tokens
//     64 (c >> 2) .. +63, two 32x32 tiles sharing the weight fragment (items
//     of at most 64 tokens: tokens 32 (c >> 2) .. +31, one tile).  Per block:
//     v_mfma_i32_32x32x32_i8 with the accumulator input at the bits of
//     1.5 * 2^23, so the result reads as the float 1.5 * 2^23 + I (|I| <=
//     2^19); t = fma(that, d_x, -1.5 * 2^23 * d_x) = fl(d_x * I) and
//     acc = fma(d_w, t, acc), d_w read as fp16: two VALU operations per
//     (row, token, block).
//   4 producer waves: producer p owns rows 32p .. +31 and tokens 32p .. +31.
//     Per K step of 8 blocks it loads its rows' and tokens' codes as 16-byte
//     block halves (buffer loads at the blocks' unaligned code offsets: Q8_0
//     blocks are 34 bytes, q8_1 blocks 36; the lanes of one load walk four
//     contiguous row segments), the fp16 scales, and writes them to LDS.
//     Q8_0 codes are the MFMA operand as they are: no expansion step.  Q4_0
//     weights (18-byte blocks: fp16 d, 16 bytes of nibbles; weight = d *
//     (nibble - 8)) are loaded a whole block per lane, four per lane and
//     step, and expanded in registers into the same operand rows.
// Operand rows are 256 bytes (8 blocks) with their 16-byte chunks XOR-swizzled
// by the row's low 4 bits; operands and scales are double-buffered, one
// barrier per step; step g + 2's loads are in flight during step g.
// Items run in the grouped order of the other dense kernel (about
// kGroupBytes of weight rows swept over every token tile), dealt XCD-major:
// XCD x (workgroups w with w % 8 == x) takes a contiguous eighth of that order,
// its workgroup w / 8 every (G/8)-th item of it, so an XCD's L2 keeps the
// group's weight rows and each token tile's rows.
// Epilogue: the fp32 rows and/or the q8_1 rounding of each token's 32-row
// blocks (16 rows in lane l, 16 in lane l ^ 32).
#include <type_traits>

#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kXcds = 8;
constexpr int kCons = 8, kProd = 4;
constexpr int kThreads = 64 * (kCons + kProd);  // 768
constexpr int kLT = 128;                        // weight rows per item
constexpr int kNT = 128;                        // tokens per item
constexpr int kGroupBytes = 2 << 20;
static_assert(kLT == 32 * kProd && kNT == 32 * kProd, "a producer owns 32 rows and 32 tokens");

__device__ __forceinline__ int swz(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

// Position of row r (0..127) in the per-block d_w vector: the 16 rows a lane
// of a 32x32 tile holds (8(i/4) + 4*half + i%4) are contiguous.
__device__ __forceinline__ int dw_pos(int r) {
  const int q = (r >> 3) & 3, h = (r >> 2) & 1, m = r & 3;
  return (r & ~31) + 16 * h + 4 * q + m;
}

// Item of the grouped order -> (row tile, token tile).
__device__ __forceinline__ void item_tiles(int item, int n_rt, int n_tt, int group_rows, int& rt, int& tt) {
  const int group = item / (group_rows * n_tt);
  const int within = item - group * group_rows * n_tt;
  const int g_rows = min(group_rows, n_rt - group * group_rows);
  tt = within / g_rows;
  rt = group * group_rows + (within - tt * g_rows);
}

template <bool PROBE, int WFMT>
__global__ __launch_bounds__(kThreads) void k_dense_ws(const uint8_t* __restrict__ x, const uint8_t* __restrict__ w,
                                                       int T, int N, int K, int n_rt, int n_tt, int group_rows,
                                                       int items, float* __restrict__ y_f32,
                                                       uint8_t* __restrict__ y_q8, ProbeRows probe) {
  __shared__ __align__(16) int8_t As[2][kLT * 256];
  __shared__ __align__(16) int8_t Bs[2][kNT * 256];
  __shared__ __align__(16) _Float16 dws[2][8][kLT];  // d_w per block, rows in dw_pos order
  __shared__ __align__(16) float dxs[2][kNT][8];     // d_x per token and block

  const int xcd = (int)blockIdx.x % kXcds, G8 = gridDim.x / kXcds, wl = (int)blockIdx.x / kXcds;
  const int i0 = (int)((int64_t)items * xcd / kXcds), i1 = (int)((int64_t)items * (xcd + 1) / kXcds);
  const int x_items = i1 - i0;
  if (wl >= x_items) return;
  const int my_items = (x_items - 1 - wl) / G8 + 1;
  const int nb = K / 32, nsb = K / 256;
  const int n_steps = my_items * nsb;
  // first weight row, first token and token count of the workgroup's j-th item
  auto item_of = [&](int j, int& l0, int& n0, int& cnt) {
    int rt, tt;
    item_tiles(i0 + wl + j * G8, n_rt, n_tt, group_rows, rt, tt);
    l0 = rt * kLT;
    n0 = tt * kNT;
    cnt = min(kNT, T - n0);
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: role branches stay scalar

  if (wave >= kCons) {
    // =============================== producer ===============================
    const int p = wave - kCons;
    constexpr int kWB = WFMT == kDenseQ40 ? kQ40Bytes : kQ80Bytes;  // weight block bytes
    const rsrc_t rw = make_rsrc(w, (uint32_t)((int64_t)N * nb * kWB));
    const rsrc_t rx = make_rsrc(x, (uint32_t)((int64_t)T * nb * kQ81Bytes));
    // codes, load m < 8: row (token) 32p + 4m + (lane >> 4), chunk lane & 15 =
    // (block (lane & 15) >> 1, half lane & 1); scales, load c < 4: row (token)
    // 32p + 8c + (lane >> 3), block lane & 7.  Step s adds 8 s blocks.  Q4_0
    // weights: load c < 4 takes the whole block (row 32p + 8c + (lane >> 3),
    // block lane & 7): its d and its 16 bytes of nibbles.
    const int pc = lane & 15, pkb = pc >> 1, ph = pc & 1;
    int woff[8], xoff[8], wsoff[4], xsoff[4];
    int lj = 0, lsb = 0;
    bool need_setup = true;
    auto setup = [&](int j) {
      int l0, n0, cnt;
      item_of(j, l0, n0, cnt);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int r = l0 + 32 * p + 4 * m + (lane >> 4);  // < N: N % 128 == 0
        woff[m] = (r * nb + pkb) * kQ80Bytes + 2 + 16 * ph;
        const int n = 32 * p + 4 * m + (lane >> 4);
        xoff[m] = n < cnt ? ((n0 + n) * nb + pkb) * kQ81Bytes + 4 + 16 * ph : kOutOfRange;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = l0 + 32 * p + 8 * c + (lane >> 3);
        wsoff[c] = (r * nb + (lane & 7)) * kWB;
        const int n = 32 * p + 8 * c + (lane >> 3);
        xsoff[c] = n < cnt ? ((n0 + n) * nb + (lane & 7)) * kQ81Bytes : kOutOfRange;
      }
    };
    uint4 rq[WFMT == kDenseQ40 ? 4 : 8], rv[8];
    uint32_t rwd[4], rxd[4];
    auto load_next = [&]() {
      if (need_setup) {
        setup(lj);
        need_setup = false;
      }
      const int sw = __builtin_amdgcn_readfirstlane(lsb * 8 * kWB);  // scalar offsets stay in SGPRs
      const int sx = __builtin_amdgcn_readfirstlane(lsb * 8 * kQ81Bytes);
      if constexpr (WFMT == kDenseQ40) {
#pragma unroll
        for (int c = 0; c < 4; ++c) rq[c] = buf_u128(rw, wsoff[c] + 2, sw);
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) rq[m] = buf_u128(rw, woff[m], sw);
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) rv[m] = buf_u128(rx, xoff[m], sx);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        rwd[c] = buf_u16(rw, wsoff[c], sw);
        rxd[c] = buf_u16(rx, xsoff[c], sx);
      }
      if (++lsb == nsb) {
        lsb = 0;
        need_setup = ++lj < my_items;
      }
    };
    // registers -> LDS buffer b (free again after it: the next loads follow)
    auto stage = [&](int b) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int r = 32 * p + 4 * m + (lane >> 4);
        if constexpr (WFMT != kDenseQ40) *reinterpret_cast<uint4*>(As[b] + swz(r, pc)) = rq[m];
        *reinterpret_cast<uint4*>(Bs[b] + swz(r, pc)) = rv[m];  // token r of the item
      }
      if constexpr (WFMT == kDenseQ40) {
        // element i < 16 of a block: low nibble of byte i; i >= 16: high nibble of byte i - 16
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = 32 * p + 8 * c + (lane >> 3), kb = lane & 7;
          const uint4 n = rq[c];
          const uint4 lo = {down_lookup<kDownQ40>(n.x & 0x0f0f0f0fu), down_lookup<kDownQ40>(n.y & 0x0f0f0f0fu),
                            down_lookup<kDownQ40>(n.z & 0x0f0f0f0fu), down_lookup<kDownQ40>(n.w & 0x0f0f0f0fu)};
          const uint4 hi = {down_lookup<kDownQ40>((n.x >> 4) & 0x0f0f0f0fu),
                            down_lookup<kDownQ40>((n.y >> 4) & 0x0f0f0f0fu),
                            down_lookup<kDownQ40>((n.z >> 4) & 0x0f0f0f0fu),
                            down_lookup<kDownQ40>((n.w >> 4) & 0x0f0f0f0fu)};
          *reinterpret_cast<uint4*>(As[b] + swz(r, 2 * kb)) = lo;
          *reinterpret_cast<uint4*>(As[b] + swz(r, 2 * kb + 1)) = hi;
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 32 * p + 8 * c + (lane >> 3);
        dws[b][lane & 7][dw_pos(r)] = __builtin_bit_cast(_Float16, (uint16_t)rwd[c]);
        dxs[b][r][lane & 7] = half_bits_to_float(rxd[c] & 0xffffu);  // token r of the item
      }
    };
    load_next();
    stage(0);
    if (n_steps > 1) load_next();
    __syncthreads();
    for (int g = 0; g < n_steps; ++g) {
      if (g + 1 < n_steps) stage((g & 1) ^ 1);
      if (g + 2 < n_steps) load_next();
      __syncthreads();
    }
    return;
  }

  // =============================== consumer ===============================
  const int rs = wave & 3, th = wave >> 2;
  const int col = lane & 31, khalf = lane >> 5;
  const int xo = (khalf ^ (col & 15)) << 4;  // chunk (2kb + khalf) of a row with these low bits: 32kb ^ xo
  v16i magic;
#pragma unroll
  for (int i = 0; i < 16; ++i) magic[i] = kMagicBits;
  float acc0[16], acc1[16];
  int cj = 0, csb = 0;
  int cl0, cn0, ccnt;
  item_of(0, cl0, cn0, ccnt);
  // one K step over both token halves (TWO) or the first only
  auto mma = [&](auto two_tag, auto grp_tag, int b) {
    constexpr bool TWO = decltype(two_tag)::value;
    constexpr int GRP = decltype(grp_tag)::value;
    const int n0 = (TWO ? 64 : 32) * th + col, n1 = n0 + 32;
    const int8_t* ap = As[b] + (32 * rs + col) * 256;
    const int8_t* bp0 = Bs[b] + n0 * 256;
    const int8_t* bp1 = Bs[b] + (TWO ? n1 : n0) * 256;
    const float4 x00 = *reinterpret_cast<const float4*>(&dxs[b][n0][0]);
    const float4 x01 = *reinterpret_cast<const float4*>(&dxs[b][n0][4]);
    float4 x10 = x00, x11 = x01;
    if (TWO) {
      x10 = *reinterpret_cast<const float4*>(&dxs[b][n1][0]);
      x11 = *reinterpret_cast<const float4*>(&dxs[b][n1][4]);
    }
    const float dx0[8] = {x00.x, x00.y, x00.z, x00.w, x01.x, x01.y, x01.z, x01.w};
    const float dx1[8] = {x10.x, x10.y, x10.z, x10.w, x11.x, x11.y, x11.z, x11.w};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      // the two consumer waves of a SIMD (th = 0, 1) take turns at the higher
      // priority, two blocks each, so both finish the step together
      if (kb % 2 == 0) {
        if ((GRP ^ (kb / 2)) & 1) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
      }
      const int off = (32 * kb) ^ xo;
      const v4i va = *reinterpret_cast<const v4i*>(ap + off);
      const v4i vb0 = *reinterpret_cast<const v4i*>(bp0 + off);
      const v16i j0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb0, magic, 0, 0, 0);
      v16i j1 = magic;
      if (TWO) {
        const v4i vb1 = *reinterpret_cast<const v4i*>(bp1 + off);
        j1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb1, magic, 0, 0, 0);
      }
      // d_w of this lane's 16 rows for block kb (fp16, contiguous)
      const uint4 dq0 = *reinterpret_cast<const uint4*>(&dws[b][kb][32 * rs + 16 * khalf]);
      const uint4 dq1 = *reinterpret_cast<const uint4*>(&dws[b][kb][32 * rs + 16 * khalf + 8]);
      const uint32_t dq[8] = {dq0.x, dq0.y, dq0.z, dq0.w, dq1.x, dq1.y, dq1.z, dq1.w};
      const float c0 = -kMagic * dx0[kb], c1 = -kMagic * dx1[kb];  // exact
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float dw = half_bits_to_float((i & 1) ? (dq[i >> 1] >> 16) : (dq[i >> 1] & 0xffffu));
        acc0[i] = __builtin_fmaf(dw, __builtin_fmaf(dx0[kb], as_float(j0[i]), c0), acc0[i]);
        if (TWO) acc1[i] = __builtin_fmaf(dw, __builtin_fmaf(dx1[kb], as_float(j1[i]), c1), acc1[i]);
      }
      if (PROBE) {
#pragma unroll
        for (int t = 0; t < (TWO ? 2 : 1); ++t) {
          const int n = t ? n1 : n0;
          if (n < ccnt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int rr = cl0 + 32 * rs + 8 * (i >> 2) + 4 * khalf + (i & 3) - probe.row0;
              if (rr >= 0 && rr < probe.rows)
                probe.out[((int64_t)(cn0 + n) * probe.rows + rr) * nb + csb * 8 + kb] = (t ? j1[i] : j0[i]) - kMagicBits;
            }
          }
        }
      }
    }
  };
  // fp32 rows and / or their q8_1 blocks for the token half t
  auto store = [&](int t, bool wide) {
    // The q8_1 rule rounds every product to fp32 on its own (no FMA).
#pragma clang fp contract(off)
    const int n = (wide ? 64 : 32) * th + 32 * t + col;
    const bool live = n < ccnt;
    const int64_t tok = cn0 + n;
    const int nrow = cl0 + 32 * rs;  // first row of this wave's 32 (one q8_1 block of a token's output)
    const float* a = t ? acc1 : acc0;
    if (y_f32 && live) {
      float* dst = y_f32 + tok * N + nrow + 4 * khalf;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(dst + 8 * q) = float4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
    }
    if (y_q8) {
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(a[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const float d = amax / 127.0f;
      const float id = d != 0.0f ? 1.0f / d : 0.0f;
      uint32_t pk[4];
      int sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        pk[q] = pack_codes(round_half_away(a[4 * q] * id), round_half_away(a[4 * q + 1] * id),
                           round_half_away(a[4 * q + 2] * id), round_half_away(a[4 * q + 3] * id));
        sum = __builtin_amdgcn_sdot4((int)pk[q], 0x01010101, sum, false);
      }
      sum += __shfl_xor(sum, 32);
      if (live) {
        uint8_t* blk = y_q8 + (tok * (N / 32) + nrow / 32) * kQ81Bytes;
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<uint32_t*>(blk + 4 + 8 * q + 4 * khalf) = pk[q];
        if (khalf == 0)
          *reinterpret_cast<uint32_t*>(blk) =
              float_to_half_bits(d) | (float_to_half_bits(fp32_barrier(d * (float)sum)) << 16);
      }
    }
  };
  // one copy of the loop per token group th (the priority pattern is an immediate)
  auto consumer_loop = [&](auto grp_tag) {
    __syncthreads();
    for (int g = 0; g < n_steps; ++g) {
      const int b = g & 1;
      const bool wide = ccnt > 64;
      if (csb == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc0[i] = acc1[i] = 0.f;
      }
      if (wide) {
        if (64 * th < ccnt) mma(std::true_type{}, grp_tag, b);
      } else if (32 * th < ccnt) {
        mma(std::false_type{}, grp_tag, b);
      }
      if (++csb == nsb) {
        store(0, wide);
        if (wide) store(1, wide);
        csb = 0;
        if (++cj < my_items) item_of(cj, cl0, cn0, ccnt);
      }
      __syncthreads();
    }
  };
  if (th) consumer_loop(std::integral_constant<int, 1>{});
  else consumer_loop(std::integral_constant<int, 0>{});
}

}  // namespace

bool dense_ws_shape(int N, int K) { return N % kLT == 0 && K % 256 == 0; }

hipError_t launch_dense_ws(const uint8_t* x, const uint8_t* w, int wfmt, int64_t T, int N, int K, float* y_f32,
                           uint8_t* y_q8, const ProbeRows* probe, int num_cus, hipStream_t st) {
  // one persistent workgroup per CU, a multiple of the XCD count
  int grid = num_cus - num_cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  const int n_rt = N / kLT;
  const int n_tt = (int)((T + kNT - 1) / kNT);
  const int items = n_rt * n_tt;
  const int wb = wfmt == kDenseQ40 ? kQ40Bytes : kQ80Bytes;
  const int group_rows = max(1, min(n_rt, (int)(kGroupBytes / ((int64_t)kLT * (K / 32) * wb))));
  const ProbeRows none = {nullptr, 0, 0};
  const ProbeRows pr = probe ? *probe : none;
  if (wfmt == kDenseQ40) {
    if (probe)
      hipLaunchKernelGGL((k_dense_ws<true, kDenseQ40>), dim3(grid), dim3(kThreads), 0, st, x, w, (int)T, N, K, n_rt,
                         n_tt, group_rows, items, y_f32, y_q8, pr);
    else
      hipLaunchKernelGGL((k_dense_ws<false, kDenseQ40>), dim3(grid), dim3(kThreads), 0, st, x, w, (int)T, N, K, n_rt,
                         n_tt, group_rows, items, y_f32, y_q8, pr);
  } else {
    if (probe)
      hipLaunchKernelGGL((k_dense_ws<true, kDenseQ80>), dim3(grid), dim3(kThreads), 0, st, x, w, (int)T, N, K, n_rt,
                         n_tt, group_rows, items, y_f32, y_q8, pr);
    else
      hipLaunchKernelGGL((k_dense_ws<false, kDenseQ80>), dim3(grid), dim3(kThreads), 0, st, x, w, (int)T, N, K, n_rt,
                         n_tt, group_rows, items, y_f32, y_q8, pr);
  }
  return hipGetLastError();
}

}  // namespace latmoe
