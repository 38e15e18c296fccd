// Down grouped GEMM (IQ4_NL x q8_1 H) with the router-weight epilogue.
//
// Page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1", section
// "Contents": after gate/up, down reads IQ4_NL.  Both operands carry one scale
// per 32 values, so each int32 block dot J is folded as
//   O[l][p] += d_dn[l][b] * (d_H[p][b] * J)
// in fp32, the product d_H * J formed exactly rounded from the MFMA result
// without an int-to-float conversion (see the MFMA step below).
// Work item = (expert e, tile of up to kTileN = 128 sorted pairs, 128 output
// rows l0..l0+127); wave w of 16 (4 per SIMD) owns the 32x32 tile of rows
// l0 + 32*(w&3) .. +31 and tokens 32*(w>>2) .. +31 (skipped when all padding).
// K (= F) is walked 256 values (8 blocks) at a time with the next step's global
// loads issued into registers before the current step computes: IQ4_NL rows
// (16-byte loads when rows are 16-byte aligned, else 16-bit loads), H codes
// (contiguous per sorted pair) and fp16 d_H.  The 4-bit indices expand to int8
// through the 16-entry table with two v_perm_b32 lookups and a byte select.
// Epilogue: O * router_w[p] is written to the pair's slot row (pair order), so
// the combine sums each token's k slots in a fixed order; or, for the combine
// by atomic adds, added into the token's row of y with fp32 atomics.
#include <type_traits>

#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kThreads = 1024;
constexpr int kLT = 128;                   // output rows per work item
constexpr int kNT = kTileN;                // tokens per work item
constexpr int kRawStride = 8 * kIq4Bytes;  // 144 bytes: 8 IQ4_NL blocks of one row
constexpr int kOpStride = 256 + 16;        // int8 operand row in LDS (bytes)
constexpr int kRaw16 = kLT * kRawStride / 16;                  // 16-byte pieces per step (1152)
constexpr int kRaw16Per = (kRaw16 + kThreads - 1) / kThreads;  // 2
constexpr int kRawHalf = kLT * kRawStride / 2;                 // 16-bit words per step (9216)
constexpr int kRawHalfPer = kRawHalf / kThreads;               // 9
static_assert(kRawHalf % kThreads == 0, "staging split");
static_assert(kNT * 16 == 2 * kThreads && kNT * 8 == kThreads && kLT * 8 == kThreads, "staging split");

// Four consecutive floats of an output row: a 16-byte store into a slot row,
// or four fp32 atomic adds into y (global_atomic_add_f32, no return value).
template <bool ATOMIC>
__device__ __forceinline__ void store_or_add(float* dst, float4 v) {
  if constexpr (ATOMIC) {
    unsafeAtomicAdd(dst + 0, v.x);
    unsafeAtomicAdd(dst + 1, v.y);
    unsafeAtomicAdd(dst + 2, v.z);
    unsafeAtomicAdd(dst + 3, v.w);
  } else {
    *reinterpret_cast<float4*>(dst) = v;
  }
}

// out: the slot rows [T*k][L] (ATOMIC false) or y [T][L] (ATOMIC true: each
// pair's weighted row is added into its token's row with fp32 atomic adds).
template <bool PROBE, bool ALIGNED16, int FMT, bool ATOMIC>
__global__ __launch_bounds__(kThreads) void k_down_generic(const uint8_t* __restrict__ dn, const float* __restrict__ router_w,
                                                   const int32_t* __restrict__ perm,
                                                   const int32_t* __restrict__ tiles,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ misc, int L, int F, int k,
                                                   const int8_t* __restrict__ h_codes,
                                                   const uint32_t* __restrict__ h_ds, float* __restrict__ out,
                                                   ProbeRows probe) {
  __shared__ __align__(16) uint8_t raw[kLT * kRawStride];
  __shared__ __align__(16) int8_t As[kLT * kOpStride];
  __shared__ __align__(16) int8_t Bs[kNT * kOpStride];
  __shared__ __align__(16) float dds[8][kLT];  // d_dn per block and row
  __shared__ float dhs[8][kNT];                // d_H per block and token
  __shared__ int32_t pid[kNT];

  const int tile = blockIdx.x;
  if (tile >= misc[kMiscTiles]) return;
  const int e = tiles[kTileWords * tile];
  const int pos0 = tiles[kTileWords * tile + 1];
  const int cnt = tiles[kTileWords * tile + 2];  // at most kTileN == kNT
  const int l0 = blockIdx.y * kLT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lsub = wave & 3, tsub = wave >> 2;
  const int nfb = F / 32;
  const int64_t row_bytes = (int64_t)nfb * kIq4Bytes;
  const uint8_t* dn_e = dn + ((int64_t)e * L + l0) * row_bytes;

  if (tid < kNT) pid[tid] = tid < cnt ? perm[pos0 + tid] : -1;

  uint4 r16[ALIGNED16 ? kRaw16Per : 1];
  uint32_t rh[ALIGNED16 ? 1 : kRawHalfPer];
  // load() only moves bits into registers (no arithmetic on loaded values, or
  // the compiler must wait for them right away); store() converts and writes.
  uint4 rhc[2];
  uint32_t rdh;
  const int hn0 = tid >> 4, hn1 = (tid + kThreads) >> 4, hc16 = tid & 15;

  // Stage step kc: the rows' 8-block chunk (bytes kc*144 .. +nb*18 of each row),
  // the tile's H codes and d_H.
  auto load = [&](int kc) {
    const int nb = min(8, nfb - kc * 8);
    if (ALIGNED16) {
#pragma unroll
      for (int m = 0; m < kRaw16Per; ++m) {
        const int i = tid + kThreads * m, r = i / 9, c = i - r * 9;
        r16[m] = uint4{0, 0, 0, 0};
        if (i < kRaw16) r16[m] = *reinterpret_cast<const uint4*>(dn_e + r * row_bytes + kc * kRawStride + c * 16);
      }
    } else {
#pragma unroll
      for (int m = 0; m < kRawHalfPer; ++m) {
        const int i = tid + kThreads * m, r = i / 72, hw = i - r * 72;
        rh[m] = 0;
        if (hw < nb * 9) rh[m] = reinterpret_cast<const uint16_t*>(dn_e + r * row_bytes + kc * kRawStride)[hw];
      }
    }
    rhc[0] = (hn0 < cnt && hc16 < nb * 2)
                 ? *reinterpret_cast<const uint4*>(h_codes + (int64_t)(pos0 + hn0) * F + kc * 256 + hc16 * 16)
                 : uint4{0, 0, 0, 0};
    rhc[1] = (hn1 < cnt && hc16 < nb * 2)
                 ? *reinterpret_cast<const uint4*>(h_codes + (int64_t)(pos0 + hn1) * F + kc * 256 + hc16 * 16)
                 : uint4{0, 0, 0, 0};
    const int dn_ = tid >> 3, db = tid & 7;
    rdh = (dn_ < cnt && db < nb) ? h_ds[(int64_t)(pos0 + dn_) * nfb + kc * 8 + db] : 0u;
  };
  auto store = [&]() {
    if (ALIGNED16) {
#pragma unroll
      for (int m = 0; m < kRaw16Per; ++m) {
        const int i = tid + kThreads * m;
        if (i < kRaw16) *reinterpret_cast<uint4*>(raw + (i / 9) * kRawStride + (i % 9) * 16) = r16[m];
      }
    } else {
#pragma unroll
      for (int m = 0; m < kRawHalfPer; ++m) {
        const int i = tid + kThreads * m;
        reinterpret_cast<uint16_t*>(raw)[(i / 72) * (kRawStride / 2) + i % 72] = (uint16_t)rh[m];
      }
    }
    *reinterpret_cast<uint4*>(Bs + hn0 * kOpStride + hc16 * 16) = rhc[0];
    *reinterpret_cast<uint4*>(Bs + hn1 * kOpStride + hc16 * 16) = rhc[1];
    dhs[tid & 7][tid >> 3] = half_bits_to_float(rdh & 0xffffu);
  };

  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  v16i magic;
#pragma unroll
  for (int i = 0; i < 16; ++i) magic[i] = kMagicBits;

  const bool active = 32 * tsub < cnt;
  const int col = lane & 31, khalf = lane >> 5;
  const int8_t* ap = As + (32 * lsub + col) * kOpStride + 16 * khalf;
  const int8_t* bp = Bs + (32 * tsub + col) * kOpStride + 16 * khalf;

  const int nkc = (nfb + 7) / 8;  // steps of 8 blocks
  load(0);
  for (int kc = 0; kc < nkc; ++kc) {
    const int nb = min(8, nfb - kc * 8);
    store();
    __syncthreads();
    if (kc + 1 < nkc) load(kc + 1);
    // ---- unpack: thread -> (row r, block b); consecutive lanes take consecutive rows
    {
      const int r = tid & (kLT - 1), b = tid >> 7;
      const uint8_t* blk = raw + r * kRawStride + b * kIq4Bytes;
      uint4* dst = reinterpret_cast<uint4*>(As + r * kOpStride + b * 32);
      if (b < nb) {
        const uint16_t* h16 = reinterpret_cast<const uint16_t*>(blk);
        uint32_t qw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) qw[w] = (uint32_t)h16[1 + 2 * w] | ((uint32_t)h16[2 + 2 * w] << 16);
        uint32_t o[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          o[w] = down_lookup<FMT>(qw[w] & 0x0f0f0f0fu);             // values 4w .. 4w+3
          o[4 + w] = down_lookup<FMT>((qw[w] >> 4) & 0x0f0f0f0fu);  // values 16+4w ..
        }
        dst[0] = uint4{o[0], o[1], o[2], o[3]};
        dst[1] = uint4{o[4], o[5], o[6], o[7]};
        dds[b][r] = half_bits_to_float(h16[0]);
      } else {
        dst[0] = uint4{0, 0, 0, 0};
        dst[1] = uint4{0, 0, 0, 0};
        dds[b][r] = 0.f;
      }
    }
    __syncthreads();
    // ---- MFMA per block (accumulator initialised to the bits of 1.5 * 2^23, so
    // the int32 result reads as the float 1.5 * 2^23 + J), fold with both scales:
    // t = fma(d_H, f, -1.5 * 2^23 * d_H) is exactly fl(d_H * J), acc += d_dn * t.
    if (active) {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        if (!ALIGNED16 && b >= nb) break;  // 16-byte-aligned rows imply F % 256 == 0: every step has 8 blocks
        const v4i va = *reinterpret_cast<const v4i*>(ap + 32 * b);
        const v4i vb = *reinterpret_cast<const v4i*>(bp + 32 * b);
        const v16i j = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb, magic, 0, 0, 0);
        const float dh = dhs[b][32 * tsub + col];
        const float ch = -kMagic * dh;  // exact
        const float4* ddp = reinterpret_cast<const float4*>(&dds[b][32 * lsub + 4 * khalf]);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float4 dd = ddp[2 * qq];  // rows 8qq + 4khalf + 0..3
          acc[4 * qq + 0] = __builtin_fmaf(dd.x, __builtin_fmaf(dh, as_float(j[4 * qq + 0]), ch), acc[4 * qq + 0]);
          acc[4 * qq + 1] = __builtin_fmaf(dd.y, __builtin_fmaf(dh, as_float(j[4 * qq + 1]), ch), acc[4 * qq + 1]);
          acc[4 * qq + 2] = __builtin_fmaf(dd.z, __builtin_fmaf(dh, as_float(j[4 * qq + 2]), ch), acc[4 * qq + 2]);
          acc[4 * qq + 3] = __builtin_fmaf(dd.w, __builtin_fmaf(dh, as_float(j[4 * qq + 3]), ch), acc[4 * qq + 3]);
        }
        if (PROBE) {
          const int p = pid[32 * tsub + col];
          if (p >= 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int l = l0 + 32 * lsub + 8 * (i >> 2) + 4 * khalf + (i & 3);
              const int rr = l - probe.row0;
              if (rr >= 0 && rr < probe.rows)
                probe.out[((int64_t)p * probe.rows + rr) * nfb + kc * 8 + b] = j[i] - kMagicBits;
            }
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: weighted output rows into the pair's slot (or y)
  if (!active) return;
  const int n = 32 * tsub + col;
  const int p = pid[n];
  if (p >= 0) {
    const float wgt = router_w[p];
    float* dst = out + (int64_t)(ATOMIC ? p / k : p) * L + l0 + 32 * lsub + 4 * khalf;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      float4 v;
      v.x = acc[4 * qq + 0] * wgt;
      v.y = acc[4 * qq + 1] * wgt;
      v.z = acc[4 * qq + 2] * wgt;
      v.w = acc[4 * qq + 3] * wgt;
      store_or_add<ATOMIC>(dst + 8 * qq, v);
    }
  }
}


// ---------------------------------------------------------------------------
// Main path (F % 256 == 0, so every 8-block K step of a row is 144 contiguous,
// 16-byte-aligned bytes): a persistent, warp-specialized kernel.
//
// One workgroup of 12 waves per CU walks the items (expert, tile of up to 128
// sorted pairs, 128 output rows): each XCD takes a contiguous range of token
// tiles with all their row tiles, so the H tile of an item is fetched from
// memory once and shared in that XCD's L2 by the workgroups working on its
// row tiles, and an expert's rows stay there across its consecutive tiles
// (dealing a fixed row tile to each XCD instead made every XCD read every H
// tile: 0.97 GB per launch at 5268 tokens).
//   8 consumer waves: wave c owns rows 32*(c&3) .. +31 against tokens
//     64*(c>>2) .. +63 (two 32x32 tiles sharing the weight fragment).  Per
//     block: J = v_mfma_i32_32x32x32_i8 with the accumulator initialised to
//     the bits of 1.5 * 2^23, so the result reads as the float 1.5 * 2^23 + J;
//     t = fma(d_H, f, -1.5 * 2^23 * d_H) is exactly fl(d_H * J) (d_H is the
//     lane's token), acc = fma(d_dn, t, acc) (d_dn per row, from fp16).
//   4 producer waves: producer p owns rows 32p .. +31 and tokens 32p .. +31.
//     Per step it loads its rows' 144-byte chunks (16-byte buffer loads), its
//     tokens' H codes and fp16 d_H (out-of-range offsets give zeros for
//     padding), writes them to LDS, and expands its rows' IQ4_NL blocks: two
//     lanes per row, each reading 72 bytes (4 blocks) and turning 4 indices
//     into 4 table bytes with two v_perm_b32 and a select.
//     The next step's loads are issued between the LDS writes and the
//     expansion, so their latency overlaps the expansion.
// Operand rows are 256 bytes with their 16-byte chunks XOR-swizzled by the
// row's low 4 bits (conflict-free 16-byte reads without padding); operands
// and scales are double-buffered, one barrier per step.
constexpr int kXcds = 8;  // workgroups are dealt to the XCDs round-robin
constexpr int kWsConsumers = 8, kWsProducers = 4;
constexpr int kWsThreads = 64 * (kWsConsumers + kWsProducers);  // 768
constexpr int kWsLT = 128;                                      // output rows per item
constexpr int kWsNT = kTileN;                                   // tokens per item
constexpr int kWsStep = 8 * kIq4Bytes;                          // 144 raw bytes per row and step
static_assert(kWsLT == 32 * kWsProducers && kWsNT == 32 * kWsProducers, "a producer owns 32 rows and 32 tokens");

__device__ __forceinline__ int swz(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

// Position of row r (0..127) in the per-block d_dn vector: the 16 rows a lane
// of a 32x32 tile holds (8(i/4) + 4*half + i%4) are contiguous.
__device__ __forceinline__ int dd_pos(int r) {
  const int q = (r >> 3) & 3, h = (r >> 2) & 1, m = r & 3;
  return (r & ~31) + 16 * h + 4 * q + m;
}

struct DItem {
  int e, pos0, cnt, l0;
};

// Where item j of a workgroup sits in its XCD's list (tile major): q = wl + j
// * G8 as the tile q / nlt past the range's first tile and the row tile
// q % nlt, stepped from item to item without a division.
struct DItemPos {
  int qd, qm;
};

template <bool PROBE, int FMT, bool ATOMIC>
__global__ __launch_bounds__(kWsThreads) void k_down(const uint8_t* __restrict__ dn, const float* __restrict__ router_w,
                                                     const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ tiles,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ misc, int pairs, int L, int F, int k,
                                                     const int8_t* __restrict__ h_codes,
                                                     const uint32_t* __restrict__ h_ds, float* __restrict__ out,
                                                     ProbeRows probe) {
  __shared__ __align__(16) uint8_t raw[kWsLT * kWsStep];
  __shared__ __align__(16) int8_t As[2][kWsLT * 256];
  __shared__ __align__(16) int8_t Bs[2][kWsNT * 256];
  // d_dn in fp32, d_H in fp16: a consumer lane folds 16 rows' d_dn per block
  // (fp32 there keeps that a full-rate v_fma_f32; a mixed fp16 operand makes
  // it a v_fma_mix_f32, which issues at about 0.6 of the rate) and one or two
  // tokens' d_H, which it converts itself.
  __shared__ __align__(16) float dds[2][8][kWsLT];          // d_dn per block, rows in dd_pos order
  __shared__ __align__(16) _Float16 dhs[2][kWsNT][8];       // d_H per token and block

  const int nlt = L / kWsLT;
  // XCD x (workgroups w with w % 8 == x) takes token tiles [t0, t1), all their
  // row tiles; its workgroup l = w / 8 takes items l, l + G/8, ... of that
  // list (tile major), so the XCD's workgroups share each H tile in L2 and
  // an expert's consecutive tiles reuse its rows there.
  const int n_tiles = misc[kMiscTiles];
  const int xcd = (int)blockIdx.x % kXcds, G8 = gridDim.x / kXcds, wl = (int)blockIdx.x / kXcds;
  const int t0 = (int)((int64_t)n_tiles * xcd / kXcds), t1 = (int)((int64_t)n_tiles * (xcd + 1) / kXcds);
  const int x_items = (t1 - t0) * nlt;
  if (wl >= x_items) return;
  const int my_items = (x_items - 1 - wl) / G8 + 1;
  const int g8d = G8 / nlt, g8m = G8 - g8d * nlt;
  const DItemPos first_pos = {wl / nlt, wl % nlt};
  auto next_pos = [&](DItemPos a) {
    a.qd += g8d;
    a.qm += g8m;
    if (a.qm >= nlt) {
      a.qm -= nlt;
      ++a.qd;
    }
    return a;
  };
  auto item_at = [&](DItemPos a) {
    DItem it;
    const int tile = t0 + a.qd;
    it.l0 = a.qm * kWsLT;
    it.e = tiles[kTileWords * tile];
    it.pos0 = tiles[kTileWords * tile + 1];
    it.cnt = tiles[kTileWords * tile + 2];  // at most kTileN == kWsNT
    return it;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: role branches stay scalar
  const int nfb = F / 32, nsb = F / 256;
  const int row_bytes = nfb * kIq4Bytes;
  const int n_steps = my_items * nsb;

  if (wave >= kWsConsumers) {
    // =============================== producer ===============================
    const int p = wave - kWsConsumers;
    const rsrc_t rh_src = make_rsrc(h_codes, (uint32_t)(pairs * F));
    const rsrc_t rs_src = make_rsrc(h_ds, (uint32_t)(pairs * nfb * 4));
    rsrc_t rw_src;
    // raw: piece i = lane + 64m (m < 5, i < 288) of this producer's 32 rows x
    // 9 pieces; H codes: token 32p + 4a + (lane >> 4), chunk lane & 15; d_H:
    // token 32p + 8c + (lane >> 3), block lane & 7.
    int qoff[5], hoff[8], soff[4];
    int lj = 0, lsb = 0, ql0 = -1;
    bool need_setup = true;
    // whether this producer's 32 tokens of the item being loaded hold a pair
    // (else their H loads and LDS stores are skipped: no consumer reads those
    // rows), for the item set up and for the data in registers
    bool h_live_item = true, h_live_regs = true;
    DItemPos lpos = first_pos;  // item lj's position
    auto setup = [&]() {
      const DItem it = item_at(lpos);
      lpos = next_pos(lpos);
      const int e = __builtin_amdgcn_readfirstlane(it.e);
      rw_src = make_rsrc(dn + (int64_t)e * L * row_bytes, (uint32_t)(L * row_bytes));
      if (it.l0 != ql0) {  // once per workgroup when the grid is a multiple of nlt
        ql0 = it.l0;
#pragma unroll
        for (int m = 0; m < 5; ++m) {
          const int i = lane + 64 * m, r = i / 9, c = i - 9 * r;
          const int row = it.l0 + 32 * p + r;
          qoff[m] = (i < 288 && row < L) ? row * row_bytes + 16 * c : kOutOfRange;
        }
      }
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const int n = 32 * p + 4 * a + (lane >> 4);
        hoff[a] = n < it.cnt ? (it.pos0 + n) * F + 16 * (lane & 15) : kOutOfRange;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int n = 32 * p + 8 * c + (lane >> 3);
        soff[c] = n < it.cnt ? ((it.pos0 + n) * nfb + (lane & 7)) * 4 : kOutOfRange;
      }
      h_live_item = 32 * p < it.cnt;
    };
    uint4 rq[5], rx[8];
    uint32_t rd[4];
    auto load_next = [&]() {
      if (need_setup) {
        setup();
        need_setup = false;
      }
      const int sq = __builtin_amdgcn_readfirstlane(lsb * kWsStep);  // scalar offsets stay in SGPRs
      const int sx = __builtin_amdgcn_readfirstlane(lsb * 256);
      const int sd = __builtin_amdgcn_readfirstlane(lsb * 32);
#pragma unroll
      for (int m = 0; m < 5; ++m) rq[m] = buf_u128(rw_src, qoff[m], sq);
      h_live_regs = h_live_item;
      if (h_live_regs) {
#pragma unroll
        for (int a = 0; a < 8; ++a) rx[a] = buf_u128(rh_src, hoff[a], sx);
#pragma unroll
        for (int c = 0; c < 4; ++c) rd[c] = buf_u32(rs_src, soff[c], sd);
      }
      if (++lsb == nsb) {
        lsb = 0;
        need_setup = ++lj < my_items;
      }
    };
    // S: registers -> LDS buffer b.  The registers are free again after it,
    // so the next step's loads are issued before the expansion (U) and their
    // latency overlaps it.
    auto stage = [&](int b) {
      uint4* raw16 = reinterpret_cast<uint4*>(raw + 32 * p * kWsStep);
#pragma unroll
      for (int m = 0; m < 5; ++m)
        if (m < 4 || lane < 32) raw16[lane + 64 * m] = rq[m];
      if (h_live_regs) {
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          const int n = 32 * p + 4 * a + (lane >> 4);
          *reinterpret_cast<uint4*>(Bs[b] + swz(n, lane & 15)) = rx[a];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
          dhs[b][32 * p + 8 * c + (lane >> 3)][lane & 7] = __builtin_bit_cast(_Float16, (uint16_t)(rd[c] & 0xffffu));
      }
    };
    auto unpack = [&](int b) {
      // expand: row 32p + (lane & 31), blocks 4*(lane >> 5) .. +3 from the 72
      // bytes at 72*(lane >> 5) of the row's chunk
      const int r = 32 * p + (lane & 31), hb = lane >> 5;
      const uint2* src = reinterpret_cast<const uint2*>(raw + r * kWsStep + 72 * hb);
      uint32_t w[18];
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        const uint2 v = src[i];
        w[2 * i] = v.x;
        w[2 * i + 1] = v.y;
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int o = 18 * kk;  // block kk: d at bytes o..o+1, indices at o+2..o+17
        const uint32_t dbits = (o & 2) ? (w[o >> 2] >> 16) : (w[o >> 2] & 0xffffu);
        uint32_t nib[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int ob = o + 2 + 4 * jj;
          nib[jj] = (ob & 3) ? __builtin_amdgcn_alignbyte(w[(ob >> 2) + 1], w[ob >> 2], ob & 3) : w[ob >> 2];
        }
        // element l < 16: low nibble of byte l; element l + 16: high nibble
        const uint4 lo = {down_lookup<FMT>(nib[0] & 0x0f0f0f0fu), down_lookup<FMT>(nib[1] & 0x0f0f0f0fu),
                          down_lookup<FMT>(nib[2] & 0x0f0f0f0fu), down_lookup<FMT>(nib[3] & 0x0f0f0f0fu)};
        const uint4 hi = {down_lookup<FMT>((nib[0] >> 4) & 0x0f0f0f0fu), down_lookup<FMT>((nib[1] >> 4) & 0x0f0f0f0fu),
                          down_lookup<FMT>((nib[2] >> 4) & 0x0f0f0f0fu), down_lookup<FMT>((nib[3] >> 4) & 0x0f0f0f0fu)};
        const int kg = 4 * hb + kk;
        *reinterpret_cast<uint4*>(As[b] + swz(r, 2 * kg)) = lo;
        *reinterpret_cast<uint4*>(As[b] + swz(r, 2 * kg + 1)) = hi;
        dds[b][kg][dd_pos(r)] = half_bits_to_float(dbits);
      }
    };

    load_next();
    stage(0);
    if (n_steps > 1) load_next();
    unpack(0);
    __syncthreads();
    for (int g = 0; g < n_steps; ++g) {
      if (g + 1 < n_steps) stage((g & 1) ^ 1);
      if (g + 2 < n_steps) load_next();
      if (g + 1 < n_steps) unpack((g & 1) ^ 1);
      __syncthreads();
    }
    return;
  }

  // =============================== consumer ===============================
  // Wide items (more than 64 tokens): wave (rs, th) owns rows 32 rs .. +31 and
  // tokens 64 th .. +63 as two 32-token halves.  Narrow items (at most 64
  // tokens): it owns tokens 32 th .. +31 only, so all 8 waves (2 per SIMD)
  // share the work; one wave per SIMD issues VALU at well under full rate.
  const int rs = wave & 3, th = wave >> 2;
  const int col = lane & 31, khalf = lane >> 5;
  const int xo = (khalf ^ (col & 15)) << 4;  // chunk (2kb + khalf) of a row with these low bits: 32kb ^ xo
  v16i magic;
#pragma unroll
  for (int i = 0; i < 16; ++i) magic[i] = kMagicBits;
  float acc0[16], acc1[16];
  int cj = 0, csb = 0;
  DItemPos cpos = first_pos;  // item cj's position
  DItem cur = item_at(cpos);
  int pair0 = -1, pair1 = -1;
  float w0 = 0.f, w1 = 0.f;
  // one K step over both halves (TWO) or the first only; WIDE: this wave's
  // tokens start at 64 th (a wide item), else at 32 th
  auto mma = [&](auto two_tag, auto wide_tag, auto grp_tag, int b) {
    constexpr bool TWO = decltype(two_tag)::value;
    constexpr bool WIDE = decltype(wide_tag)::value;
    constexpr int GRP = decltype(grp_tag)::value;
    const int n0 = (WIDE ? 64 : 32) * th + col, n1 = n0 + 32;
    const int8_t* ap = As[b] + (32 * rs + col) * 256;
    const int8_t* bp0 = Bs[b] + n0 * 256;
    const int8_t* bp1 = Bs[b] + (TWO ? n1 : n0) * 256;
    const uint4 hq0 = *reinterpret_cast<const uint4*>(&dhs[b][n0][0]);
    const uint4 hq1 = TWO ? *reinterpret_cast<const uint4*>(&dhs[b][n1][0]) : hq0;
    const uint32_t hw0[4] = {hq0.x, hq0.y, hq0.z, hq0.w}, hw1[4] = {hq1.x, hq1.y, hq1.z, hq1.w};
    // converted once per step; the empty asm keeps the compiler from folding
    // the conversion into every fma of the block as a v_fma_mix_f32
    float dh0[8], dh1[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      dh0[q] = half_bits_to_float((q & 1) ? hw0[q >> 1] >> 16 : hw0[q >> 1] & 0xffffu);
      dh1[q] = TWO ? half_bits_to_float((q & 1) ? hw1[q >> 1] >> 16 : hw1[q >> 1] & 0xffffu) : dh0[q];
      asm volatile("" : "+v"(dh0[q]), "+v"(dh1[q]));
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      // The two consumer waves of a SIMD (th = 0, 1) take turns at the higher
      // priority, two blocks each, so both finish the step together.
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
      // d_dn of this lane's 16 rows for block kb (fp16, contiguous)
      const float4* dqp = reinterpret_cast<const float4*>(&dds[b][kb][32 * rs + 16 * khalf]);
      const float4 dq0 = dqp[0], dq1 = dqp[1], dq2 = dqp[2], dq3 = dqp[3];
      const float ddv[16] = {dq0.x, dq0.y, dq0.z, dq0.w, dq1.x, dq1.y, dq1.z, dq1.w,
                             dq2.x, dq2.y, dq2.z, dq2.w, dq3.x, dq3.y, dq3.z, dq3.w};
      const float c0 = -kMagic * dh0[kb], c1 = -kMagic * dh1[kb];  // exact
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc0[i] = __builtin_fmaf(ddv[i], __builtin_fmaf(dh0[kb], as_float(j0[i]), c0), acc0[i]);
        if (TWO) acc1[i] = __builtin_fmaf(ddv[i], __builtin_fmaf(dh1[kb], as_float(j1[i]), c1), acc1[i]);
      }
      if (PROBE) {
#pragma unroll
        for (int t = 0; t < (TWO ? 2 : 1); ++t) {
          const int pr = t ? pair1 : pair0;
          if (pr >= 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int l = cur.l0 + 32 * rs + 8 * (i >> 2) + 4 * khalf + (i & 3);
              const int rr = l - probe.row0;
              if (rr >= 0 && rr < probe.rows)
                probe.out[((int64_t)pr * probe.rows + rr) * nfb + csb * 8 + kb] = (t ? j1[i] : j0[i]) - kMagicBits;
            }
          }
        }
      }
    }
  };
  // one copy of the loop per token group th (the priority pattern is an immediate)
  auto consumer_loop = [&](auto grp_tag) {
    __syncthreads();
    DItem nxt = cur;
    for (int g = 0; g < n_steps; ++g) {
      const int b = g & 1;
      const bool wide = cur.cnt > 64;
      // Loads whose results wait: the next item's tile entry at the start of
      // the item's last step (the barrier that ends a step waits for all
      // scalar loads), the pairs at the item's first step and their router
      // weights one step later (the weight's address needs the pair).
      if (csb == nsb - 1 && cj + 1 < my_items) {
        cpos = next_pos(cpos);
        nxt = item_at(cpos);
      }
      if (csb == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc0[i] = acc1[i] = 0.f;
        const int n0 = (wide ? 64 : 32) * th + col, n1 = n0 + 32;
        pair0 = n0 < cur.cnt ? perm[cur.pos0 + n0] : -1;
        pair1 = wide && n1 < cur.cnt ? perm[cur.pos0 + n1] : -1;
      }
      if (csb == (nsb > 1 ? 1 : 0)) {
        w0 = pair0 >= 0 ? router_w[pair0] : 0.f;
        w1 = pair1 >= 0 ? router_w[pair1] : 0.f;
      }
      if (wide) {
        // the second half only when it holds a token (an item of 65..96
        // tokens leaves the upper wave's second half all padding)
        if (64 * th + 32 < cur.cnt) mma(std::true_type{}, std::true_type{}, grp_tag, b);
        else if (64 * th < cur.cnt) mma(std::false_type{}, std::true_type{}, grp_tag, b);
      } else if (32 * th < cur.cnt) {
        mma(std::false_type{}, std::false_type{}, grp_tag, b);
      }
      if (++csb == nsb) {
        // ---- weighted output rows into the pairs' slots (or added into y)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int pr = t ? pair1 : pair0;
          const float wgt = t ? w1 : w0;
          if (pr >= 0) {
            float* dst = out + (int64_t)(ATOMIC ? pr / k : pr) * L + cur.l0 + 32 * rs + 4 * khalf;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const float* a = t ? acc1 : acc0;
              float4 v;
              v.x = a[4 * qq + 0] * wgt;
              v.y = a[4 * qq + 1] * wgt;
              v.z = a[4 * qq + 2] * wgt;
              v.w = a[4 * qq + 3] * wgt;
              store_or_add<ATOMIC>(dst + 8 * qq, v);
            }
          }
        }
        csb = 0;
        if (++cj < my_items) cur = nxt;
      }
      __syncthreads();
    }
  };
  if (th) consumer_loop(std::integral_constant<int, 1>{});
  else consumer_loop(std::integral_constant<int, 0>{});
}

template <bool PROBE, int FMT, bool ATOMIC>
void launch_variant(bool aligned, dim3 grid, hipStream_t st, const uint8_t* dn, const float* router_w,
                    const Shapes& s, const Work& w, float* out, ProbeRows probe) {
  if (aligned)
    hipLaunchKernelGGL((k_down_generic<PROBE, true, FMT, ATOMIC>), grid, dim3(kThreads), 0, st, dn, router_w, w.perm,
                       w.tiles, w.offsets, w.misc, s.L, s.F, s.k, w.h_codes, w.h_ds, out, probe);
  else
    hipLaunchKernelGGL((k_down_generic<PROBE, false, FMT, ATOMIC>), grid, dim3(kThreads), 0, st, dn, router_w, w.perm,
                       w.tiles, w.offsets, w.misc, s.L, s.F, s.k, w.h_codes, w.h_ds, out, probe);
}

template <int FMT, bool ATOMIC>
void launch_fmt(const uint8_t* dn, const float* router_w, const Shapes& s, const Work& w, float* out,
                const ProbeRows* probe, hipStream_t st) {
  const ProbeRows none = {nullptr, 0, 0};
  if (s.F % 256 == 0 && ((uintptr_t)dn & 15u) == 0) {
    // one persistent workgroup per CU, a multiple of the XCD count
    int grid = w.num_cus - w.num_cus % kXcds;
    if (grid < kXcds) grid = kXcds;
    const int pairs = (int)s.pairs();
    if (probe)
      hipLaunchKernelGGL((k_down<true, FMT, ATOMIC>), dim3(grid), dim3(kWsThreads), 0, st, dn, router_w, w.perm,
                         w.tiles, w.offsets, w.misc, pairs, s.L, s.F, s.k, w.h_codes, w.h_ds, out, *probe);
    else
      hipLaunchKernelGGL((k_down<false, FMT, ATOMIC>), dim3(grid), dim3(kWsThreads), 0, st, dn, router_w, w.perm,
                         w.tiles, w.offsets, w.misc, pairs, s.L, s.F, s.k, w.h_codes, w.h_ds, out, none);
    return;
  }
  const dim3 grid(w.max_tiles, s.L / kLT);
  // 16-byte staging needs every row (and so every 8-block step) 16-byte aligned;
  // that also means F is a multiple of 256, so every step is a full 144-byte chunk.
  const bool aligned = ((int64_t)(s.F / 32) * kIq4Bytes) % 16 == 0 && ((uintptr_t)dn & 15u) == 0;
  if (probe)
    launch_variant<true, FMT, ATOMIC>(aligned, grid, st, dn, router_w, s, w, out, *probe);
  else
    launch_variant<false, FMT, ATOMIC>(aligned, grid, st, dn, router_w, s, w, out, none);
}

}  // namespace

hipError_t launch_down(const uint8_t* dn, int fmt, const float* router_w, const Shapes& s, const Work& w,
                       float* y_atomic, const ProbeRows* probe, hipStream_t st) {
  if (y_atomic) {
    if (fmt == kDownQ40)
      launch_fmt<kDownQ40, true>(dn, router_w, s, w, y_atomic, probe, st);
    else
      launch_fmt<kDownIq4Nl, true>(dn, router_w, s, w, y_atomic, probe, st);
  } else {
    if (fmt == kDownQ40)
      launch_fmt<kDownQ40, false>(dn, router_w, s, w, w.slots, probe, st);
    else
      launch_fmt<kDownIq4Nl, false>(dn, router_w, s, w, w.slots, probe, st);
  }
  return hipGetLastError();
}

}  // namespace latmoe
