// Gate/up grouped GEMM with the SwiGLU + q8_1 epilogue.
//
// Page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1": gate/up reads
// Q3_K, applies SwiGLU and rounds H to q8_1 (section "Contents"); the 6-bit
// sub-block scale is multiplied into the int8 operand as (4 - code)(scale - 32)
// in [-128, 124], so one integer dot covers a whole 32-value activation block
// (lat_q3k_w11.cu commit message).
//
// Persistent kernel: one workgroup per CU walks the work items (token tile of
// up to kTileN = 128 sorted pairs, 64 features): each XCD takes a contiguous
// range of token tiles with all their feature tiles, so a tile's gathered
// activation rows are fetched from memory once and shared in that XCD's L2,
// and an expert's rows stay there across its consecutive tiles.
//
// The workgroup's 12 waves have two roles (3 waves per SIMD):
//   8 consumer waves: wave c owns the gate and the up 32x32 tile of features
//     f0 + 32*(c&1) .. +31 and tokens 32*(c>>1) .. +31 (both MFMAs share the
//     activation fragment; gate and up of a (feature, token) meet in one lane
//     for SwiGLU).  Per K step of 256 values: v_mfma_i32_32x32x32_i8 per
//     32-value block with the float bits of M = 1.5 * 2^23 as accumulator
//     input, so the result read as a float is M - I32 exactly (the operand is
//     -w, |I32| < 2^20); fma(-d_x, M - I32, d_x * M) is d_x * I32 rounded
//     once, added into acc_sb; once per step acc += d_w[row][sb] * acc_sb.
//     A wave whose 32 tokens are all padding skips its MFMAs.
//   4 producer waves: producer p owns weight rows 32p .. 32p+31 of the item
//     (gate rows, then up rows) and tokens 32p .. 32p+31.  Per K step it loads
//     into registers, through buffer loads whose out-of-range offset returns
//     zeros for padding, its rows' Q3_K blocks as dwords (blocks are only
//     2-byte aligned: unaligned dword loads, 28 lanes a row), its tokens'
//     int8 codes (16-byte loads) and fp32 block scales; writes them to LDS;
//     and unpacks its rows from LDS: per (row, half, j) 32 codes become
//     (4 - c) * sigma with one v_perm_b32 per 4 values against the 8-entry
//     table of the sub-block scale (one 8-byte LDS read from the 64 tables
//     the workgroup builds at its start).  Only the producer itself reads
//     its raw rows, so no barrier separates its stores from its unpack.
// Step g: producers stage the loaded data of step g+1 in the other LDS buffer,
// issue the global loads of step g+2, then unpack step g+1's weights;
// consumers run the MFMAs of step g; one barrier.
// Epilogue (after an item's last step, consumers): H = G * sigmoid(G) * U,
// then per 32 features of a token (16 in this lane, 16 in lane ^ 32) the q8_1
// rule: amax, d = amax/127, id = 1/d, q = round-half-away(H * id) with IEEE
// divisions (the codes' sum by v_dot4 on the packed codes); codes and fp16
// (d, s) go to the workspace in sorted order.
#include <type_traits>

#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kXcds = 8;  // workgroups are dealt to the XCDs round-robin
constexpr int kConsumers = 8, kProducers = 4;
constexpr int kThreads = 64 * (kConsumers + kProducers);  // 768
constexpr int kFT = 64;              // features per work item
constexpr int kRows = 2 * kFT;       // weight rows per work item (gate + up)
constexpr int kNT = kTileN;          // tokens per work item
constexpr int kRawStride = 112;      // staged Q3_K block, bytes (110 rounded up to 16)
constexpr int kOpStride = 256 + 16;  // int8 operand row in LDS (bytes); 16 mod 256: conflict-free b128
// The pad bytes of operand rows are never read as operands.  Those of rows
// 0..63 of As[0] hold the Q3_K operand table of each 6-bit scale sc (byte c =
// (4 - c)(sc - 32), c = 0..7), written once per workgroup.
constexpr int kTabOff = 256;
static_assert(kRows == 32 * kProducers && kNT == 32 * kProducers, "a producer owns 32 rows and 32 tokens");
static_assert(kNT == 4 * 32 && kFT == 2 * 32, "8 consumers = 2 feature halves x 4 token slices");

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
__global__ __launch_bounds__(kThreads) void k_gateup(const int8_t* __restrict__ xc, const float* __restrict__ xd,
                                                     const uint8_t* __restrict__ gu, const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ tiles,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ misc, int T, int k, int L, int F,
                                                     int8_t* __restrict__ h_codes, uint32_t* __restrict__ h_ds,
                                                     ProbeRows probe) {
  __shared__ __align__(16) uint8_t raw[kRows * kRawStride];
  __shared__ __align__(16) int8_t As[2][kRows * kOpStride];
  __shared__ __align__(16) int8_t Bs[2][kNT * kOpStride];
  __shared__ __align__(16) float dxs[2][kNT * 8];  // [token][block], negated
  __shared__ __align__(16) float dws[2][kRows];
  __shared__ int32_t ids[2][kNT];  // token ids (or -1) of the producers' next items

  const int nft = (F + kFT - 1) / kFT;
  // XCD x (workgroups w with w % 8 == x) takes token tiles [t0, t1), all their
  // feature tiles; its workgroup l = w / 8 takes items l, l + G/8, ... of that
  // list (tile major), so the XCD's workgroups share each tile's activation
  // rows in L2 and an expert's rows stay there across its consecutive tiles.
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
    it.cnt = tiles[kTileWords * tile + 2];  // at most kTileN == kNT
    return it;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: role branches stay scalar
  const bool producer = wave >= kConsumers;
  const int nsb = L / 256, nxb = L / 32;
  const int row_bytes = nsb * kQ3kBytes;
  const int n_steps = my_items * nsb;

  // =========================== producer state ===========================
  const int p = wave - kConsumers;  // producer index (meaningful for producers)
  const int ptid = tid - 64 * kConsumers;  // 0 .. 255 for producers
  const rsrc_t rx_src = make_rsrc(xc, (uint32_t)(T * L));
  const rsrc_t rd_src = make_rsrc(xd, (uint32_t)(T * nxb * 4));
  rsrc_t rw_src;
  // raw: dword w = lane & 31 of rows 32p + 2i + (lane >> 5), i < 16 (w < 27:
  // block bytes 4w .. 4w+3; w = 27: bytes 106 .. 109, so d lands in the high
  // half of staged dword 27 and no load reaches past the block; w > 27 load
  // nothing).  The blocks are only 2-byte aligned, so these are unaligned
  // dword loads: two rows a load instead of 16 bytes of eight, which keeps
  // the CU's address unit from queueing the four producers' loads.  codes:
  // tokens 32p + 4a + (lane >> 4), 16-byte chunk lane & 15.  scales: tokens
  // 32p + 8c + (lane >> 3), block lane & 7.
  int qoff = kOutOfRange, xoff[8], doff[4];
  int lj = 0, lsb = 0, qf0 = -1;
  // whether this producer's 32 tokens of the item being loaded hold a pair
  // (else its activation loads and LDS stores are skipped: no consumer reads
  // those rows), for the item set up and for the data in registers
  bool x_live_item = true, x_live_regs = true;
  bool need_setup = true;
  // The next item's token ids: producer p fetches those of its own tokens
  // 32p .. 32p+31 (lanes 0..31), so only the wave that writes an entry reads
  // it and no barrier has to separate the two (with one K step per item the
  // next setup can follow in the same step).  The pair loads are issued in
  // setup; their LDS store (flush_ids) comes at the end of the step, or at
  // the next setup if that comes first.
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
    if (it.f0 != qf0) {  // once per workgroup when the grid is a multiple of nft
      qf0 = it.f0;
      // this producer's 32 rows: gate (p < 2) or up rows f0 + 32 (p & 1) ..,
      // all inside F or all past it (F % 32 == 0)
      const int rl0 = 32 * (p & 1), w = lane & 31;
      const int row = (p < 2 ? 0 : F) + it.f0 + rl0 + (lane >> 5);
      qoff = (it.f0 + rl0 < F && w < 28) ? row * row_bytes + (w < 27 ? 4 * w : 106) : kOutOfRange;
    }
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int t = ids[j & 1][32 * p + 4 * a + (lane >> 4)];
      xoff[a] = t >= 0 ? t * L + 16 * (lane & 15) : kOutOfRange;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = ids[j & 1][32 * p + 8 * c + (lane >> 3)];
      doff[c] = t >= 0 ? (t * nxb + (lane & 7)) * 4 : kOutOfRange;
    }
    x_live_item = 32 * p < it.cnt;
    lpos = next_pos(lpos);
    fetch_ids(j + 1, lpos);
  };
  uint32_t rq[16];
  uint4 rx[8];
  uint32_t rd[4];
  // L: sets up a new item when the loader enters one (reading the ids this
  // wave stored for it), then only moves bits into registers and advances
  // the loader.
  auto load_next = [&]() {
    if (need_setup) {
      flush_ids();  // the ids this setup reads, if their store is still pending
      setup(lj);
      need_setup = false;
    }
    const int sq = __builtin_amdgcn_readfirstlane(lsb * kQ3kBytes);  // scalar offsets stay in SGPRs
    const int sx = __builtin_amdgcn_readfirstlane(lsb * 256);
    const int sd = __builtin_amdgcn_readfirstlane(lsb * 32);
#pragma unroll
    for (int i = 0; i < 16; ++i) rq[i] = buf_u32(rw_src, qoff, sq + 2 * i * row_bytes);
    x_live_regs = x_live_item;
    if (x_live_regs) {
#pragma unroll
      for (int a = 0; a < 8; ++a) rx[a] = buf_u128(rx_src, xoff[a], sx);
#pragma unroll
      for (int c = 0; c < 4; ++c) rd[c] = buf_u32(rd_src, doff[c], sd);
    }
    if (++lsb == nsb) {
      lsb = 0;
      need_setup = ++lj < my_items;
    }
  };
  // S: registers -> LDS buffer b (raw rows, operand B, scales).  The
  // registers are free again after it, so the next step's loads are issued
  // before the unpack and their latency overlaps it.
  auto stage = [&](int b) {
    uint32_t* raw32 = reinterpret_cast<uint32_t*>(raw) + (32 * p + (lane >> 5)) * (kRawStride / 4) + (lane & 31);
    if ((lane & 31) < 28) {
#pragma unroll
      for (int i = 0; i < 16; ++i) raw32[2 * i * (kRawStride / 4)] = rq[i];
    }
    if (x_live_regs) {
#pragma unroll
      for (int a = 0; a < 8; ++a)
        *reinterpret_cast<uint4*>(Bs[b] + (32 * p + 4 * a + (lane >> 4)) * kOpStride + 16 * (lane & 15)) = rx[a];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        dxs[b][(32 * p + 8 * c + (lane >> 3)) * 8 + (lane & 7)] = -as_float((int)rd[c]);  // minus: operand A is -w
    }
  };
  // U: the producer's own staged rows unpacked into operand A of buffer b.
  auto unpack = [&](int b) {
    // this lane's row ur, tasks (un, uj) = (u >> 1, 2 (u & 1) + (lane >> 5))
    const int ur = 32 * p + (lane & 31);
    const uint8_t* ublk = raw + ur * kRawStride;
    const uint4 h0 = *reinterpret_cast<const uint4*>(ublk);
    const uint4 h1 = *reinterpret_cast<const uint4*>(ublk + 16);
    const uint4 scw = *reinterpret_cast<const uint4*>(ublk + 96);  // scales[12] | scales[10..11] | d
    const uint32_t hm[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
    const uint32_t scb[3] = {scw.x, scw.y, scw.z};
    if (lane < 32) dws[b][ur] = half_bits_to_float(scw.w >> 16);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int un = u >> 1, uj = 2 * (u & 1) + (lane >> 5);
      const uint4 q0 = *reinterpret_cast<const uint4*>(ublk + 32 + 32 * un);
      const uint4 q1 = *reinterpret_cast<const uint4*>(ublk + 48 + 32 * un);
      const uint32_t qs[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      uint32_t tlo[2], thi[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int s = 8 * un + 2 * uj + t;  // sub-block of 16 values
        const int sl = s & 7;
        const int lo = (int)((scb[sl >> 2] >> (8 * (sl & 3) + (s < 8 ? 0 : 4))) & 15u);
        const int hi = (int)((scb[2] >> (8 * (s & 3) + 2 * (s >> 2))) & 3u);
        const uint2 tb = *reinterpret_cast<const uint2*>(As[0] + (lo | (hi << 4)) * kOpStride + kTabOff);
        tlo[t] = tb.x;
        thi[t] = tb.y;
      }
      const int qshift = 2 * uj;       // low two bits of element 128un + 32uj + l: bit 2uj of qs[l]
      const int hs = 4 * un + uj - 2;  // its high bit (bit 4un + uj of hmask[l]) moves to bit 2
      // Two words at a time through 64-bit shifts: the bits a shift moves
      // across the word boundary (at most 6 at the top of the low word, 2 at
      // the bottom of the high word) fall outside the masks.
      uint32_t o[8];
#pragma unroll
      for (int g = 0; g < 8; g += 2) {
        const uint64_t h64 = ((uint64_t)hm[g + 1] << 32) | hm[g];
        const uint64_t q64 = ((uint64_t)qs[g + 1] << 32) | qs[g];
        const uint64_t hsh = hs >= 0 ? (h64 >> hs) : (h64 << -hs);
        const uint64_t qsh = q64 >> qshift;
        const uint32_t c0 = ((uint32_t)qsh & 0x03030303u) | ((uint32_t)hsh & 0x04040404u);
        const uint32_t c1 = ((uint32_t)(qsh >> 32) & 0x03030303u) | ((uint32_t)(hsh >> 32) & 0x04040404u);
        o[g] = __builtin_amdgcn_perm(thi[g >> 2], tlo[g >> 2], c0);
        o[g + 1] = __builtin_amdgcn_perm(thi[g >> 2], tlo[g >> 2], c1);
      }
      uint4* udst = reinterpret_cast<uint4*>(As[b] + ur * kOpStride + 128 * un + 32 * uj);
      udst[0] = uint4{o[0], o[1], o[2], o[3]};
      udst[1] = uint4{o[4], o[5], o[6], o[7]};
    }
  };

  // =========================== consumer state ===========================
  const int fsub = wave & 1, tsub = (wave >> 1) & 3;
  const int col = lane & 31, khalf = lane >> 5;
  // MFMA accumulator input: the float bits of 1.5 * 2^23 in every element, so
  // an MFMA returns those bits plus the int32 block dot, which read as a float
  // is 1.5 * 2^23 + dot exactly (|dot| < 2^22): the conversion costs no VALU
  // instruction.  Built by opaque moves: with a visible splat constant as the
  // accumulator input, this compiler treats all 16 results as equal.
  v16i magic;
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("v_mov_b32 %0, 0x4b400000" : "=v"(magic[i]));
  float accg[16], accu[16];
  int cj = 0, csb = 0;  // item index and super-block of the MFMA step
  ItemPos cpos = first_pos;  // item cj's position
  Item cur = item_at(cpos);

  auto mfma_step = [&](auto grp_tag, int b) {
    constexpr int GRP = decltype(grp_tag)::value;
    const bool active = 32 * tsub < cur.cnt;
    if (csb == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) accg[i] = accu[i] = 0.f;
    }
    if (!active) return;
    const int8_t* ag = As[b] + (32 * fsub + col) * kOpStride + 16 * khalf;
    const int8_t* au = As[b] + (kFT + 32 * fsub + col) * kOpStride + 16 * khalf;
    const int8_t* bp = Bs[b] + (32 * tsub + col) * kOpStride + 16 * khalf;
    const float4 dx0 = *reinterpret_cast<const float4*>(&dxs[b][(32 * tsub + col) * 8]);
    const float4 dx1 = *reinterpret_cast<const float4*>(&dxs[b][(32 * tsub + col) * 8 + 4]);
    const float dxv[8] = {dx0.x, dx0.y, dx0.z, dx0.w, dx1.x, dx1.y, dx1.z, dx1.w};  // -d_x
    int probe_pair = -1;
    if (PROBE) {
      const int n = 32 * tsub + col;
      if (n < cur.cnt) probe_pair = perm[cur.pos0 + n];
    }
    float sbg[16], sbu[16];
    v4i va = *reinterpret_cast<const v4i*>(ag);
    v4i vu = *reinterpret_cast<const v4i*>(au);
    v4i vb = *reinterpret_cast<const v4i*>(bp);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      // The two consumer waves of a SIMD (groups 0 and 1) take turns at the
      // higher priority, one block each, so both finish the step together
      // (oldest-first issue alone lets one run ahead and the other finish
      // alone at a fraction of the VALU rate).
      if ((GRP ^ kb) & 1) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
      const v16i ig = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb, magic, 0, 0, 0);  // M - I32
      const v16i iu = __builtin_amdgcn_mfma_i32_32x32x32_i8(vu, vb, magic, 0, 0, 0);
      if (kb < 7) {  // next block's operands
        va = *reinterpret_cast<const v4i*>(ag + 32 * (kb + 1));
        vu = *reinterpret_cast<const v4i*>(au + 32 * (kb + 1));
        vb = *reinterpret_cast<const v4i*>(bp + 32 * (kb + 1));
      }
      const float d = dxv[kb];  // -d_x
      const float cm = -d * kMagic;  // exact: d has at most 11 significant bits
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // d * (M - I) - d * M, rounded once: d_x * I rounded
        const float tg = __builtin_fmaf(d, as_float(ig[i]), cm);
        const float tu = __builtin_fmaf(d, as_float(iu[i]), cm);
        sbg[i] = kb == 0 ? tg : sbg[i] + tg;
        sbu[i] = kb == 0 ? tu : sbu[i] + tu;
      }
      if (PROBE && probe_pair >= 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int f = cur.f0 + 32 * fsub + 8 * (i >> 2) + 4 * khalf + (i & 3);
          const int rg = f - probe.row0, ru = F + f - probe.row0;
          const int64_t o = (int64_t)probe_pair * probe.rows;
          if (f < F && rg >= 0 && rg < probe.rows) probe.out[(o + rg) * nxb + csb * 8 + kb] = kMagicBits - ig[i];
          if (f < F && ru >= 0 && ru < probe.rows) probe.out[(o + ru) * nxb + csb * 8 + kb] = kMagicBits - iu[i];
        }
      }
    }
    const float4* dgp = reinterpret_cast<const float4*>(dws[b] + 32 * fsub + 4 * khalf);
    const float4* dup = reinterpret_cast<const float4*>(dws[b] + kFT + 32 * fsub + 4 * khalf);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const float4 wg = dgp[2 * qq], wu = dup[2 * qq];  // rows 8qq + 4khalf + 0..3
      accg[4 * qq + 0] = __builtin_fmaf(wg.x, sbg[4 * qq + 0], accg[4 * qq + 0]);
      accg[4 * qq + 1] = __builtin_fmaf(wg.y, sbg[4 * qq + 1], accg[4 * qq + 1]);
      accg[4 * qq + 2] = __builtin_fmaf(wg.z, sbg[4 * qq + 2], accg[4 * qq + 2]);
      accg[4 * qq + 3] = __builtin_fmaf(wg.w, sbg[4 * qq + 3], accg[4 * qq + 3]);
      accu[4 * qq + 0] = __builtin_fmaf(wu.x, sbu[4 * qq + 0], accu[4 * qq + 0]);
      accu[4 * qq + 1] = __builtin_fmaf(wu.y, sbu[4 * qq + 1], accu[4 * qq + 1]);
      accu[4 * qq + 2] = __builtin_fmaf(wu.z, sbu[4 * qq + 2], accu[4 * qq + 2]);
      accu[4 * qq + 3] = __builtin_fmaf(wu.w, sbu[4 * qq + 3], accu[4 * qq + 3]);
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

  // The two roles run separate loops (so their registers are not live at the
  // same time) with the same barriers: two in the prologue, one per step.
  if (producer) {
    // Producers issue first when both roles have VALU work: their chain of
    // loads, LDS staging and unpack gates the next step of all waves.
    __builtin_amdgcn_s_setprio(2);
    // prologue: the scale tables, operands of step 0 in buffer 0, loads of
    // step 1 in flight
    if (ptid < 64) {
      uint32_t tlo, thi;
      q3_tables(ptid - 32, tlo, thi);
      *reinterpret_cast<uint2*>(As[0] + ptid * kOpStride + kTabOff) = uint2{tlo, thi};
    }
    fetch_ids(0, first_pos);
    flush_ids();
    __syncthreads();
    load_next();
    stage(0);
    unpack(0);
    flush_ids();
    __syncthreads();
    if (n_steps > 1) load_next();
    for (int g = 0; g < n_steps; ++g) {
      if (g + 1 < n_steps) stage((g & 1) ^ 1);
      if (g + 2 < n_steps) load_next();
      if (g + 1 < n_steps) unpack((g & 1) ^ 1);
      flush_ids();
      __syncthreads();
    }
  } else {
    // one copy of the loop per consumer group (wave >> 2): the group selects
    // the priority pattern, which s_setprio takes as an immediate
    auto consumer_loop = [&](auto grp_tag) {
      __syncthreads();
      __syncthreads();
      Item nxt = cur;
      for (int g = 0; g < n_steps; ++g) {
        // the next item's tile entry is read at the start of the item's last
        // step, so the barrier that ends the step (which waits for all scalar
        // loads) does not wait for it
        if (csb == nsb - 1 && cj + 1 < my_items) {
          cpos = next_pos(cpos);
          nxt = item_at(cpos);
        }
        mfma_step(grp_tag, g & 1);
        if (++csb == nsb) {
          epilogue();
          csb = 0;
          if (++cj < my_items) cur = nxt;
        }
        __syncthreads();
      }
    };
    if (wave >> 2) consumer_loop(std::integral_constant<int, 1>{});
    else consumer_loop(std::integral_constant<int, 0>{});
  }
}

}  // namespace

hipError_t launch_gateup(const Shapes& s, const Work& w, const uint8_t* gu, const ProbeRows* probe, hipStream_t st) {
  // One persistent workgroup per CU, rounded down to a multiple of the XCD count.
  int grid = w.num_cus - w.num_cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  const ProbeRows none = {nullptr, 0, 0};
  if (probe)
    hipLaunchKernelGGL(k_gateup<true>, dim3(grid), dim3(kThreads), 0, st, w.xc, w.xd, gu, w.perm, w.tiles, w.offsets,
                       w.misc, (int)s.T, s.k, s.L, s.F, w.h_codes, w.h_ds, *probe);
  else
    hipLaunchKernelGGL(k_gateup<false>, dim3(grid), dim3(kThreads), 0, st, w.xc, w.xd, gu, w.perm, w.tiles, w.offsets,
                       w.misc, (int)s.T, s.k, s.L, s.F, w.h_codes, w.h_ds, none);
  return hipGetLastError();
}

}  // namespace latmoe
