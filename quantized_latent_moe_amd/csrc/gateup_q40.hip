// Gate/up grouped GEMM with the SwiGLU + q8_1 epilogue for Q4_0 gate/up
// weights (18-byte blocks of 32: fp16 d, 16 bytes of nibbles; weight =
// d * (nibble - 8); ggml's Q4_0, a format the PR page "Run Edge0-145B Q3_K on
// AMD HIP (Linux, gfx1100) #1" names in section "Not done").  The same stage
// as the Q3_K kernel (section "Contents": gate/up, SwiGLU, H rounded to
// q8_1), with a weight scale per 32 values instead of per 256:
//   G/U[p][r] = sum over blocks b of d_w[r][b] * d_x[t][b] * I32[p][r][b].
//
// Persistent kernel, one workgroup of 12 waves per CU, items of (token tile of
// up to 128 sorted pairs, 64 features), dealt as in the Q3_K kernel: XCD x
// takes a contiguous range of token tiles with all their feature tiles.
//   8 consumer waves: wave c owns the gate and the up 32x32 tile of features
//     f0 + 32 (c & 1) .. +31 and tokens 32 ((c >> 1) & 3) .. +31.  Per block:
//     two v_mfma_i32_32x32x32_i8 (gate, up) sharing the activation fragment,
//     accumulator input at the bits of 1.5 * 2^23; t = fma(f, d_x,
//     -1.5 * 2^23 * d_x) = fl(d_x * I) and acc = fma(d_w, t, acc), d_w read as
//     fp16: two VALU operations per (row, token, block).
//   4 producer waves: producer p owns item rows 32p .. +31 (rows 0..63 gate,
//     64..127 up) and tokens 32p .. +31.  Per K step of 8 blocks each lane
//     loads four whole weight blocks (rows 32p + 8c + (lane >> 3), block
//     lane & 7) and expands their nibbles in registers straight into the
//     operand rows; activation codes (16-byte chunks) and fp32 scales come
//     from the split activation rows through the tile's token ids.
// Operand rows are 256 bytes (8 blocks) with their 16-byte chunks XOR-swizzled
// by the row's low 4 bits; double-buffered, one barrier per step, step g + 2's
// loads in flight during step g.
#include <type_traits>

#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kXcds = 8;
constexpr int kConsumers = 8, kProducers = 4;
constexpr int kThreads = 64 * (kConsumers + kProducers);  // 768
constexpr int kFT = 64;         // features per work item
constexpr int kRows = 2 * kFT;  // weight rows per work item (gate + up)
constexpr int kNT = kTileN;     // tokens per work item
static_assert(kRows == 32 * kProducers && kNT == 32 * kProducers, "a producer owns 32 rows and 32 tokens");

__device__ __forceinline__ int swz(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

// Position of item row r (0..127) in the per-block d_w vector: the 16 rows a
// lane of a 32x32 tile holds (8(i/4) + 4*half + i%4) are contiguous.
__device__ __forceinline__ int dw_pos(int r) {
  const int q = (r >> 3) & 3, h = (r >> 2) & 1, m = r & 3;
  return (r & ~31) + 16 * h + 4 * q + m;
}

struct Item {
  int e, pos0, cnt, f0;
};

// Where item j of a workgroup sits in its XCD's list (tile major): q = wl + j
// * G8 as the tile q / nft past the range's first tile and the feature tile
// q % nft, stepped from item to item without a division.
struct ItemPos {
  int qd, qm;
};

template <bool PROBE>
__global__ __launch_bounds__(kThreads) void k_gateup_q40(const int8_t* __restrict__ xc, const float* __restrict__ xd,
                                                         const uint8_t* __restrict__ gu,
                                                         const int32_t* __restrict__ perm,
                                                         const int32_t* __restrict__ tiles,
                                                         const int32_t* __restrict__ misc, int T, int k, int L, int F,
                                                         int8_t* __restrict__ h_codes, uint32_t* __restrict__ h_ds,
                                                         ProbeRows probe) {
  __shared__ __align__(16) int8_t As[2][kRows * 256];
  __shared__ __align__(16) int8_t Bs[2][kNT * 256];
  __shared__ __align__(16) _Float16 dws[2][8][kRows];  // d_w per block, item rows in dw_pos order
  __shared__ __align__(16) float dxs[2][kNT][8];       // d_x per token and block
  __shared__ int32_t ids[2][kNT];                      // token ids (or -1) of the producers' next items

  const int nft = (F + kFT - 1) / kFT;
  const int n_tiles = misc[kMiscTiles];
  const int xcd = (int)blockIdx.x % kXcds, G8 = gridDim.x / kXcds, wl = (int)blockIdx.x / kXcds;
  const int t0 = (int)((int64_t)n_tiles * xcd / kXcds), t1 = (int)((int64_t)n_tiles * (xcd + 1) / kXcds);
  const int x_items = (t1 - t0) * nft;
  if (wl >= x_items) return;
  const int my_items = (x_items - 1 - wl) / G8 + 1;
  const int g8d = G8 / nft, g8m = G8 - g8d * nft;
  const ItemPos first_pos = {wl / nft, wl % nft};
  auto next_pos = [&](ItemPos a) {
    a.qd += g8d;
    a.qm += g8m;
    if (a.qm >= nft) {
      a.qm -= nft;
      ++a.qd;
    }
    return a;
  };
  auto item_at = [&](ItemPos a) {
    Item it;
    const int tile = t0 + a.qd;
    it.f0 = a.qm * kFT;
    it.e = tiles[kTileWords * tile];
    it.pos0 = tiles[kTileWords * tile + 1];
    it.cnt = tiles[kTileWords * tile + 2];
    return it;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: role branches stay scalar
  const int nb = L / 32, nsb = L / 256;
  const int row_bytes = nb * kQ40Bytes;
  const int n_steps = my_items * nsb;

  if (wave >= kConsumers) {
    // =============================== producer ===============================
    const int p = wave - kConsumers;
    const rsrc_t rx_src = make_rsrc(xc, (uint32_t)(T * L));
    const rsrc_t rd_src = make_rsrc(xd, (uint32_t)(T * nb * 4));
    rsrc_t rw_src;
    // weights, load c < 4: item row 32p + 8c + (lane >> 3), block lane & 7;
    // codes, load a < 8: token 32p + 4a + (lane >> 4), chunk lane & 15;
    // scales, load c < 4: token 32p + 8c + (lane >> 3), block lane & 7.
    int woff[4], xoff[8], doff[4];
    int lj = 0, lsb = 0;
    bool need_setup = true;
    // Producer p fetches the token ids of its own tokens 32p .. 32p+31, so
    // only the wave that stores an entry reads it (with one K step per item
    // the next setup can follow without a barrier between).  The pair loads
    // are issued in setup; their LDS store (flush_ids) comes at the end of
    // the step, or at the next setup if that comes first.
    int pend_pair = -1, pend_buf = 0;
    bool pend = false;
    auto fetch_ids = [&](int j, ItemPos at) {
      if (j < my_items) {
        const Item it = item_at(at);
        const int n = 32 * p + lane;
        if (lane < 32) pend_pair = n < it.cnt ? perm[it.pos0 + n] : -1;
        pend_buf = j & 1;
        pend = true;
      }
    };
    auto flush_ids = [&]() {
      if (pend) {
        if (lane < 32) ids[pend_buf][32 * p + lane] = pend_pair >= 0 ? pend_pair / k : -1;
        pend = false;
      }
    };
    ItemPos lpos = first_pos;  // item lj's position
    auto setup = [&](int j) {
      const Item it = item_at(lpos);
      const int e = __builtin_amdgcn_readfirstlane(it.e);  // uniform: the descriptor lives in SGPRs
      rw_src = make_rsrc(gu + (int64_t)e * 2 * F * row_bytes, (uint32_t)(2 * F * row_bytes));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 32 * p + 8 * c + (lane >> 3);  // item row
        const int rl = r < kFT ? r : r - kFT;
        const int row = (r < kFT ? 0 : F) + it.f0 + rl;
        woff[c] = it.f0 + rl < F ? (row * nb + (lane & 7)) * kQ40Bytes : kOutOfRange;
      }
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const int t = ids[j & 1][32 * p + 4 * a + (lane >> 4)];
        xoff[a] = t >= 0 ? t * L + 16 * (lane & 15) : kOutOfRange;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int t = ids[j & 1][32 * p + 8 * c + (lane >> 3)];
        doff[c] = t >= 0 ? (t * nb + (lane & 7)) * 4 : kOutOfRange;
      }
      lpos = next_pos(lpos);
      fetch_ids(j + 1, lpos);
    };
    uint4 rq[4], rx[8];
    uint32_t rwd[4], rd[4];
    auto load_next = [&]() {
      if (need_setup) {
        flush_ids();  // the ids this setup reads, if their store is still pending
        setup(lj);
        need_setup = false;
      }
      const int sw = __builtin_amdgcn_readfirstlane(lsb * 8 * kQ40Bytes);  // scalar offsets stay in SGPRs
      const int sx = __builtin_amdgcn_readfirstlane(lsb * 256);
      const int sd = __builtin_amdgcn_readfirstlane(lsb * 32);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        rq[c] = buf_u128(rw_src, woff[c] + 2, sw);
        rwd[c] = buf_u16(rw_src, woff[c], sw);
      }
#pragma unroll
      for (int a = 0; a < 8; ++a) rx[a] = buf_u128(rx_src, xoff[a], sx);
#pragma unroll
      for (int c = 0; c < 4; ++c) rd[c] = buf_u32(rd_src, doff[c], sd);
      if (++lsb == nsb) {
        lsb = 0;
        need_setup = ++lj < my_items;
      }
    };
    // registers -> LDS buffer b, the weights expanded on the way
    auto stage = [&](int b) {
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const int n = 32 * p + 4 * a + (lane >> 4);
        *reinterpret_cast<uint4*>(Bs[b] + swz(n, lane & 15)) = rx[a];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 32 * p + 8 * c + (lane >> 3), kb = lane & 7;
        // element i < 16 of a block: low nibble of byte i; i >= 16: high nibble of byte i - 16
        const uint4 nq = rq[c];
        const uint4 lo = {down_lookup<kDownQ40>(nq.x & 0x0f0f0f0fu), down_lookup<kDownQ40>(nq.y & 0x0f0f0f0fu),
                          down_lookup<kDownQ40>(nq.z & 0x0f0f0f0fu), down_lookup<kDownQ40>(nq.w & 0x0f0f0f0fu)};
        const uint4 hi = {down_lookup<kDownQ40>((nq.x >> 4) & 0x0f0f0f0fu),
                          down_lookup<kDownQ40>((nq.y >> 4) & 0x0f0f0f0fu),
                          down_lookup<kDownQ40>((nq.z >> 4) & 0x0f0f0f0fu),
                          down_lookup<kDownQ40>((nq.w >> 4) & 0x0f0f0f0fu)};
        *reinterpret_cast<uint4*>(As[b] + swz(r, 2 * kb)) = lo;
        *reinterpret_cast<uint4*>(As[b] + swz(r, 2 * kb + 1)) = hi;
        dws[b][kb][dw_pos(r)] = __builtin_bit_cast(_Float16, (uint16_t)rwd[c]);
        const int n = 32 * p + 8 * c + (lane >> 3);
        dxs[b][n][kb] = as_float((int)rd[c]);
      }
    };
    fetch_ids(0, first_pos);
    flush_ids();
    __syncthreads();
    load_next();
    stage(0);
    flush_ids();
    __syncthreads();
    if (n_steps > 1) load_next();
    for (int g = 0; g < n_steps; ++g) {
      if (g + 1 < n_steps) stage((g & 1) ^ 1);
      if (g + 2 < n_steps) load_next();
      flush_ids();
      __syncthreads();
    }
    return;
  }

  // =============================== consumer ===============================
  const int fsub = wave & 1, tsub = (wave >> 1) & 3;
  const int col = lane & 31, khalf = lane >> 5;
  const int xo = (khalf ^ (col & 15)) << 4;  // chunk (2kb + khalf) of a row with these low bits: 32kb ^ xo
  v16i magic;
#pragma unroll
  for (int i = 0; i < 16; ++i) magic[i] = kMagicBits;
  float accg[16], accu[16];
  int cj = 0, csb = 0;
  ItemPos cpos = first_pos;  // item cj's position
  Item cur = item_at(cpos);

  auto mfma_step = [&](auto grp_tag, int b) {
    constexpr int GRP = decltype(grp_tag)::value;
    const int n = 32 * tsub + col;
    const int8_t* ag = As[b] + (32 * fsub + col) * 256;
    const int8_t* au = As[b] + (kFT + 32 * fsub + col) * 256;
    const int8_t* bp = Bs[b] + n * 256;
    const float4 x0 = *reinterpret_cast<const float4*>(&dxs[b][n][0]);
    const float4 x1 = *reinterpret_cast<const float4*>(&dxs[b][n][4]);
    const float dxv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    int probe_pair = -1;
    if (PROBE && n < cur.cnt) probe_pair = perm[cur.pos0 + n];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      // the two consumer waves of a SIMD (groups 0 and 1) take turns at the
      // higher priority, one block each, so both finish the step together
      if ((GRP ^ kb) & 1) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
      const int off = (32 * kb) ^ xo;
      const v4i va = *reinterpret_cast<const v4i*>(ag + off);
      const v4i vu = *reinterpret_cast<const v4i*>(au + off);
      const v4i vb = *reinterpret_cast<const v4i*>(bp + off);
      const v16i jg = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb, magic, 0, 0, 0);
      const v16i ju = __builtin_amdgcn_mfma_i32_32x32x32_i8(vu, vb, magic, 0, 0, 0);
      // d_w of this lane's 16 gate rows and 16 up rows for block kb (fp16)
      const uint4 g0 = *reinterpret_cast<const uint4*>(&dws[b][kb][32 * fsub + 16 * khalf]);
      const uint4 g1 = *reinterpret_cast<const uint4*>(&dws[b][kb][32 * fsub + 16 * khalf + 8]);
      const uint4 u0 = *reinterpret_cast<const uint4*>(&dws[b][kb][kFT + 32 * fsub + 16 * khalf]);
      const uint4 u1 = *reinterpret_cast<const uint4*>(&dws[b][kb][kFT + 32 * fsub + 16 * khalf + 8]);
      const uint32_t dg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const uint32_t du[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      const float d = dxv[kb], c = -kMagic * d;  // exact
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float wg = half_bits_to_float((i & 1) ? (dg[i >> 1] >> 16) : (dg[i >> 1] & 0xffffu));
        const float wu = half_bits_to_float((i & 1) ? (du[i >> 1] >> 16) : (du[i >> 1] & 0xffffu));
        accg[i] = __builtin_fmaf(wg, __builtin_fmaf(d, as_float(jg[i]), c), accg[i]);
        accu[i] = __builtin_fmaf(wu, __builtin_fmaf(d, as_float(ju[i]), c), accu[i]);
      }
      if (PROBE && probe_pair >= 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int f = cur.f0 + 32 * fsub + 8 * (i >> 2) + 4 * khalf + (i & 3);
          const int rg = f - probe.row0, ru = F + f - probe.row0;
          const int64_t o = (int64_t)probe_pair * probe.rows;
          if (f < F && rg >= 0 && rg < probe.rows) probe.out[(o + rg) * nb + csb * 8 + kb] = jg[i] - kMagicBits;
          if (f < F && ru >= 0 && ru < probe.rows) probe.out[(o + ru) * nb + csb * 8 + kb] = ju[i] - kMagicBits;
        }
      }
    }
  };

  auto epilogue = [&]() {
    // The q8_1 rule rounds every product to fp32 on its own (no FMA, no fused
    // multiply-convert to fp16).
#pragma clang fp contract(off)
    if (32 * tsub >= cur.cnt) return;
    const int n = 32 * tsub + col;
    const int fb = cur.f0 + 32 * fsub;  // first feature of this 32-feature block
    float h[16];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float gv = accg[i];
      const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-gv));  // sigmoid (approximate reciprocal)
      h[i] = gv * sig * accu[i];
      amax = fmaxf(amax, fabsf(h[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float d = amax / 127.0f;
    const float id = d != 0.0f ? 1.0f / d : 0.0f;
    uint32_t pk[4];
    int sum = 0;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      pk[qq] = pack_codes(round_half_away(h[4 * qq] * id), round_half_away(h[4 * qq + 1] * id),
                          round_half_away(h[4 * qq + 2] * id), round_half_away(h[4 * qq + 3] * id));
      sum = __builtin_amdgcn_sdot4((int)pk[qq], 0x01010101, sum, false);  // sum of the four codes
    }
    sum += __shfl_xor(sum, 32);
    if (n < cur.cnt && fb < F) {
      const int64_t pos = cur.pos0 + n;
      int8_t* dst = h_codes + pos * F + fb + 4 * khalf;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) *reinterpret_cast<uint32_t*>(dst + 8 * qq) = pk[qq];
      if (khalf == 0)
        h_ds[pos * (F / 32) + fb / 32] =
            float_to_half_bits(d) | (float_to_half_bits(fp32_barrier(d * (float)sum)) << 16);
    }
  };

  // one copy of the loop per consumer group (wave >> 2): the group selects
  // the priority pattern, which s_setprio takes as an immediate
  auto consumer_loop = [&](auto grp_tag) {
    __syncthreads();
    __syncthreads();
    for (int g = 0; g < n_steps; ++g) {
      if (csb == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) accg[i] = accu[i] = 0.f;
      }
      if (32 * tsub < cur.cnt) mfma_step(grp_tag, g & 1);  // all 32 tokens padding: nothing to do
      if (++csb == nsb) {
        epilogue();
        csb = 0;
        if (++cj < my_items) {
          cpos = next_pos(cpos);
          cur = item_at(cpos);
        }
      }
      __syncthreads();
    }
  };
  if (wave >> 2) consumer_loop(std::integral_constant<int, 1>{});
  else consumer_loop(std::integral_constant<int, 0>{});
}

}  // namespace

hipError_t launch_gateup_q40(const Shapes& s, const Work& w, const uint8_t* gu, const ProbeRows* probe,
                             hipStream_t st) {
  // one persistent workgroup per CU, a multiple of the XCD count
  int grid = w.num_cus - w.num_cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  const ProbeRows none = {nullptr, 0, 0};
  if (probe)
    hipLaunchKernelGGL(k_gateup_q40<true>, dim3(grid), dim3(kThreads), 0, st, w.xc, w.xd, gu, w.perm, w.tiles,
                       w.misc, (int)s.T, s.k, s.L, s.F, w.h_codes, w.h_ds, *probe);
  else
    hipLaunchKernelGGL(k_gateup_q40<false>, dim3(grid), dim3(kThreads), 0, st, w.xc, w.xd, gu, w.perm, w.tiles,
                       w.misc, (int)s.T, s.k, s.L, s.F, w.h_codes, w.h_ds, none);
  return hipGetLastError();
}

}  // namespace latmoe
