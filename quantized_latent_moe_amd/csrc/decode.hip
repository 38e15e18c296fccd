// Gate/up and down for decode-sized batches: two launches that read the
// routing directly (no sort, no gather, no combine kernel).
//
// Same computation as the grouped GEMMs (page "Run Edge0-145B Q3_K on AMD HIP
// (Linux, gfx1100) #1", section "Contents": gate/up on Q3_K with SwiGLU and
// the q8_1 rounding of H, down on IQ4_NL), for batches of at most
// kDecodeMaxPairs routed pairs with L <= 1024 and F <= 2048, where each
// active expert holds a handful of tokens and the stage is the stream of the
// active experts' weights: every byte of them should be in flight as soon as
// the routing is known.
//
// Gate/up, workgroup (pair slot p, 32 features f0..): each wave loads all
// router ids at once (one load, a lane per pair), so the workgroup knows its
// expert e = idx[p] and whether p is the first slot routed to e; only the
// first one works, for every pair of e (a ballot gives them, in pair order).
// Its threads then issue the loads of the expert's 64 weight rows (gate
// f0.., up F+f0..; a thread takes one 110-byte super-block of one row, or
// half of one, straight into registers), and the pairs' q8_1 activation
// rows go to LDS in batches of up to 8.  H is written in pair order.  A wave
// issues an instruction only every few cycles, so few items (few experts)
// are finished sooner by two threads per super-block, while many items keep
// more of themselves resident with one; the host picks the layout that
// needs fewer rounds of resident workgroups.
//
// Q3_K dots: the int8 operand is the 3-bit code c = low2 | hbit << 2 itself
// ((qs >> 2j) & 3 and bit (4n + j) of hmask moved to bit 2), so v = c - 4
// and, with the per-16 sums of x, sigma * sum v x = sigma * (sum c x -
// 4 sum x): the scale-folded 32-value block dot I32 of the large kernels, its
// two products in 24-bit multiplies (|sum c x - 4 sum x| < 2^15); then
// acc_sb += d_x * I32 per block and acc += d_w * acc_sb per super-block.
// Q4_0 gate/up: I32 = sum nibble * x - 8 sum x, acc += d_w * fl(d_x * I32).
// The 32 features are one q8_1 block of H, so SwiGLU and the requant finish
// inside a half wave.
//
// Down, workgroup (token t, R output rows l0..): its 512 threads are (slot
// j, row, slice of 4 blocks), a wave per slot; per pass of 8 slots each
// thread loads the 72 contiguous bytes of its row's slice for expert
// idx[t][j] while the token's H rows (pair order, no dependence on the
// routing) go to LDS; block dots J32 by v_dot4 against the table-expanded
// indices, acc += fl(d_dn * d_H) * J32, a sum over the row's slices, and
// y[t][l] = sum over j of w[t][j] * O_j taken in slot order: the combine
// happens here, deterministically.  Slices of 4 blocks (rather than 8) give
// twice the waves, each with half the instructions to issue.
#include <mutex>
#include <type_traits>

#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kTok = 2;                 // tokens per dot pass of the gate/up kernel (an expert holds 1-2 at decode)
constexpr int kBatch = 8;               // tokens whose activations the gate/up kernel stages at once
constexpr int kGuMaxThreads = 512;      // 64 weight rows x up to 8 parts (two per super-block)
constexpr int kDnSlots = 8;             // pairs of the token per pass of the down kernel
constexpr int kDnThreads = 64 * kDnSlots;  // a wave per slot: rows x 4-block slices = 64
constexpr int kDnMaxK = kDecodeMaxPairs;  // experts per token (T >= 1)
static_assert(kDnThreads == 512 && kDecodeMaxPairs <= 64, "one lane per pair in a wave");

// Router ids of the batch in the lanes of the calling wave: lane p < P holds
// router_idx[p], the others -1 (one buffer load, no branch around it).
__device__ __forceinline__ int load_ids(const int32_t* __restrict__ idx, int P) {
  const int lane = threadIdx.x & 63;
  const rsrc_t r = make_rsrc(idx, (uint32_t)P * 4u);
  const int v = (int)buf_u32(r, lane < P ? lane * 4 : kOutOfRange, 0);
  return lane < P ? v : -1;
}

// (x >> s) moved so that bit s of every byte lands on bit 2, other bits 0.
template <int S>
__device__ __forceinline__ uint32_t bit_to_2(uint32_t x) {
  if constexpr (S >= 2)
    return (x >> (S - 2)) & 0x04040404u;
  else
    return (x << (2 - S)) & 0x04040404u;
}

// ---------------------------------------------------------------------------
// Thread (row r, part) of a gate/up workgroup: r < 64 the item's weight row
// (gate f0 + r, then up F + f0 + r - 32), part < tpr its share of the row.
// PARTS = 1: the whole super-block (or 8-block Q4_0 slice) sb = part;
// PARTS = 2: sb = part / 2 and its half n = part % 2 -- blocks 4n .. 4n + 3,
// values 128n .. 128n + 127.  Parts with sb >= L / 256 stay idle.  A wave
// issues one instruction at a time, several cycles apart, so when the batch
// has few items (few experts, few feature blocks) two threads per
// super-block finish each item sooner; with many items one thread per
// super-block keeps more items resident at once (the host picks).
template <bool PROBE, int GFMT, int PARTS>
__global__ __launch_bounds__(kGuMaxThreads) void k_dec_gateup(const uint8_t* __restrict__ x,
                                                            const int32_t* __restrict__ idx,
                                                            const uint8_t* __restrict__ gu, int T, int P, int k, int L,
                                                            int F, int E, int tpr_log2, int8_t* __restrict__ h_codes,
                                                            uint32_t* __restrict__ h_ds, ProbeRows probe) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int p = blockIdx.x;
  const int f0 = blockIdx.y * 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int ids = load_ids(idx, P);
  const int e = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(ids, p));
  if ((unsigned)e >= (unsigned)E) return;
  const uint64_t same = __ballot(ids == e);  // the pairs routed to e (lanes >= P hold -1)
  if (same & ((1ull << p) - 1)) return;      // an earlier slot has this expert

  constexpr bool kQ40 = GFMT == LAT_MOE_GATEUP_Q4_0;
  const int nsb = L / 256, nxb = L / 32, nsub = L / 16, nfb = F / 32;
  const int row_bytes = nsb * (kQ40 ? 8 * kQ40Bytes : kQ3kBytes);
  const int tpr = 1 << tpr_log2, nthr = 64 << tpr_log2;
  static_assert(PARTS == 1 || PARTS == 2, "one or two parts per super-block");
  constexpr int kBpt = 8 / PARTS;  // blocks per thread
  const int r = tid >> tpr_log2, part = tid & (tpr - 1);
  const int sb = PARTS == 2 ? part >> 1 : part, n = PARTS == 2 ? part & 1 : 0;
  const bool act = sb < nsb;
  const int wrow = r < 32 ? f0 + r : F + f0 + r - 32;  // weight row of the expert
  const rsrc_t rw = make_rsrc(gu + (int64_t)e * 2 * F * row_bytes, (uint32_t)(2 * F * row_bytes));
  // This thread's blocks straight into registers (buffer loads at
  // 2-byte-aligned offsets return the bytes there).  Q3_K: hmask (bytes
  // 0..31, all of it: every block takes a bit of each byte), the qs of its
  // half(s) (bytes 32 + 32n ..), the scales (96..107) and d (108).  Q4_0:
  // blocks 4n .. 4n + 3 of the slice (72 bytes at 144 sb + 72 n), or all 8.
  constexpr int kQsWords = 8 * (kBpt / 4);             // qs words held (8 per half)
  constexpr int kScW = 8 + kQsWords, kDW = kScW + 3;   // scale words, d word (Q3_K)
  uint32_t blk[kQ40 ? (PARTS == 2 ? 18 : 36) : kDW + 1];
  if constexpr (kQ40 && PARTS == 1) {
    const int boff = act ? wrow * row_bytes + sb * 8 * kQ40Bytes : kOutOfRange;
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      const uint4 v = buf_u128(rw, boff, 16 * c);
      blk[4 * c] = v.x, blk[4 * c + 1] = v.y, blk[4 * c + 2] = v.z, blk[4 * c + 3] = v.w;
    }
  } else if constexpr (kQ40) {
    const int boff = act ? wrow * row_bytes + sb * 8 * kQ40Bytes + 72 * n : kOutOfRange;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 v = buf_u128(rw, boff, 16 * c);
      blk[4 * c] = v.x, blk[4 * c + 1] = v.y, blk[4 * c + 2] = v.z, blk[4 * c + 3] = v.w;
    }
    const auto t2 = __builtin_amdgcn_raw_buffer_load_b64(rw, boff, 64, 0);
    blk[16] = t2[0], blk[17] = t2[1];
  } else {
    const int boff = act ? wrow * row_bytes + sb * kQ3kBytes : kOutOfRange;
    const int qoff = act ? boff + 32 + 32 * n : kOutOfRange;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint4 h = buf_u128(rw, boff, 16 * c);
      blk[4 * c] = h.x, blk[4 * c + 1] = h.y, blk[4 * c + 2] = h.z, blk[4 * c + 3] = h.w;
    }
#pragma unroll
    for (int c = 0; c < kQsWords / 4; ++c) {
      const uint4 q = buf_u128(rw, qoff, 16 * c);
      blk[8 + 4 * c] = q.x, blk[9 + 4 * c] = q.y, blk[10 + 4 * c] = q.z, blk[11 + 4 * c] = q.w;
    }
    const auto t3 = __builtin_amdgcn_raw_buffer_load_b96(rw, boff, 96, 0);
    blk[kScW] = t3[0], blk[kScW + 1] = t3[1], blk[kScW + 2] = t3[2];
    blk[kDW] = buf_u16(rw, boff, 108);
  }
  // LDS: xs[kBatch][L] | xds[kBatch][nxb] | xsum[kBatch][nsub] | gus[64][kBatch] | pairs[64]
  int8_t* xs = reinterpret_cast<int8_t*>(smem);
  float* xds = reinterpret_cast<float*>(xs + kBatch * L);
  int* xsum = reinterpret_cast<int*>(xds + kBatch * nxb);
  float* gus = reinterpret_cast<float*>(xsum + kBatch * nsub);
  int* s_pb = reinterpret_cast<int*>(gus + 64 * kBatch);
  const rsrc_t rx = make_rsrc(x, (uint32_t)(T * nxb * kQ81Bytes));

  // The expert's pairs in pair order (wave 0, one lane per pair).
  if (tid < 64 && ((same >> tid) & 1)) s_pb[__popcll(same & ((1ull << tid) - 1))] = tid;
  __syncthreads();
  const int cnt = __popcll(same);
  const int tk = tid / nxb, b = tid - tk * nxb;  // a batch's token and q8_1 block of this thread
  // Batches of up to kBatch of the pairs: thread (tk, b) loads one activation
  // block.  The first batch's loads follow the weight loads at once, so the
  // two are in flight together.
  for (int bt = 0; bt < cnt; bt += kBatch) {
    const int nb = min(kBatch, cnt - bt);
    if (bt > 0) __syncthreads();  // the previous batch's reads of xs / gus are done
    {
      const int tok = tk < nb ? s_pb[bt + tk] / k : -1;
      const int xoff = tok >= 0 ? (int)__umul24((unsigned)__umul24(tok, nxb) + b, kQ81Bytes) : kOutOfRange;
      const uint32_t dv = buf_u32(rx, xoff, 0);
      const uint4 xlo = buf_u128(rx, xoff, 4), xhi = buf_u128(rx, xoff, 20);
      if (tk < nb) {
        uint4* dst = reinterpret_cast<uint4*>(xs + tk * L + 32 * b);
        dst[0] = xlo;
        dst[1] = xhi;
        xds[tk * nxb + b] = half_bits_to_float(dv & 0xffffu);
        int s0 = __builtin_amdgcn_sdot4((int)xlo.x, 0x01010101, 0, false);
        s0 = __builtin_amdgcn_sdot4((int)xlo.y, 0x01010101, s0, false);
        s0 = __builtin_amdgcn_sdot4((int)xlo.z, 0x01010101, s0, false);
        s0 = __builtin_amdgcn_sdot4((int)xlo.w, 0x01010101, s0, false);
        int s1 = __builtin_amdgcn_sdot4((int)xhi.x, 0x01010101, 0, false);
        s1 = __builtin_amdgcn_sdot4((int)xhi.y, 0x01010101, s1, false);
        s1 = __builtin_amdgcn_sdot4((int)xhi.z, 0x01010101, s1, false);
        s1 = __builtin_amdgcn_sdot4((int)xhi.w, 0x01010101, s1, false);
        xsum[tk * nsub + 2 * b] = s0;  // sum of the 16 codes of each half
        xsum[tk * nsub + 2 * b + 1] = s1;
      }
    }
    __syncthreads();
    for (int t0 = 0; t0 < nb; t0 += kTok) {
    const int nt = min(kTok, nb - t0);
    int pr[kTok];  // the pass's pairs
#pragma unroll
    for (int i = 0; i < kTok; ++i) pr[i] = s_pb[bt + t0 + min(i, nt - 1)];
    // The weight words are re-read each pass (an empty asm marks them as
    // changed), so the unpack below stays inside the pass, one block at a
    // time, instead of being hoisted whole in front of the loop.
#pragma unroll
    for (int w = 0; w < (int)(sizeof(blk) / 4); ++w) asm volatile("" : "+v"(blk[w]));

    float acc[kTok];
#pragma unroll
    for (int t = 0; t < kTok; ++t) acc[t] = 0.f;
    // this thread's activations: row t of the pass at xq + t L (block jb of
    // the half at byte 32 jb), its 16-value sums and its block scales
    const int8_t* xq = xs + t0 * L + sb * 256 + 128 * n;
    const int* xsq = xsum + t0 * nsub + sb * 16 + 8 * n;
    const float* xdq = xds + t0 * nxb + sb * 8 + 4 * n;
    const int bq = sb * 8 + 4 * n;  // block index (of L / 32) of the half's first block
    // The pass's dots for NT tokens (a compile-time count: no branch inside
    // the blocks, so each block's operands die with it).
    auto dots = [&](auto nt_tag) {
      constexpr int NT = decltype(nt_tag)::value;
      if constexpr (kQ40) {
        if (act) {
#pragma unroll
        for (int jb = 0; jb < kBpt; ++jb) {
          // block jb at byte 18 jb of the thread's bytes: d, then 16 nibble bytes
          const int base = 18 * jb, wi = base >> 2;
          uint32_t nw[4], d16;
          if ((base & 3) == 0) {
            d16 = blk[wi] & 0xffffu;
#pragma unroll
            for (int w = 0; w < 4; ++w) nw[w] = __builtin_amdgcn_alignbyte(blk[wi + w + 1], blk[wi + w], 2);
          } else {
            d16 = blk[wi] >> 16;
#pragma unroll
            for (int w = 0; w < 4; ++w) nw[w] = blk[wi + 1 + w];
          }
          const float dwb = half_bits_to_float(d16);
          uint32_t lo[4], hi[4];  // values 0..15 (low nibbles) and 16..31 (high nibbles)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            lo[w] = nw[w] & 0x0f0f0f0fu;
            hi[w] = (nw[w] >> 4) & 0x0f0f0f0fu;
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const uint4* xp = reinterpret_cast<const uint4*>(xq + t * L + 32 * jb);
            const uint4 x0 = xp[0], x1 = xp[1];
            int dn = __builtin_amdgcn_sdot4((int)lo[0], (int)x0.x, 0, false);
            dn = __builtin_amdgcn_sdot4((int)lo[1], (int)x0.y, dn, false);
            dn = __builtin_amdgcn_sdot4((int)lo[2], (int)x0.z, dn, false);
            dn = __builtin_amdgcn_sdot4((int)lo[3], (int)x0.w, dn, false);
            dn = __builtin_amdgcn_sdot4((int)hi[0], (int)x1.x, dn, false);
            dn = __builtin_amdgcn_sdot4((int)hi[1], (int)x1.y, dn, false);
            dn = __builtin_amdgcn_sdot4((int)hi[2], (int)x1.z, dn, false);
            dn = __builtin_amdgcn_sdot4((int)hi[3], (int)x1.w, dn, false);
            const int2 sx = *reinterpret_cast<const int2*>(&xsq[t * nsub + 2 * jb]);
            const int I = dn - 8 * (sx.x + sx.y);  // sum (nibble - 8) x
            const float tt = xdq[t * nxb + jb] * (float)I;
            acc[t] = __builtin_fmaf(dwb, tt, acc[t]);
            if (PROBE) {
              const int rr = wrow - probe.row0;
              if (rr >= 0 && rr < probe.rows) probe.out[((int64_t)pr[t] * probe.rows + rr) * nxb + bq + jb] = I;
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        }
      } else if (act) {
        const float dw = half_bits_to_float(blk[kDW] & 0xffffu);
        // The thread's 6-bit sub-block scales (8n .. 8n + 7, or all 16) as
        // bytes, bit 5 flipped so that a signed 6-bit field extract gives
        // sigma = sc6 - 32: the low nibbles of bytes 0..7 for the first half,
        // their high nibbles for the second, the two high bits from bytes 8..11.
        const uint32_t c0 = blk[kScW], c1 = blk[kScW + 1], c2 = blk[kScW + 2];
        uint32_t xsc[kBpt / 2];
        if constexpr (PARTS == 2) {
          xsc[0] = (((c0 >> (4 * n)) & 0x0f0f0f0fu) | ((n ? c2 : c2 << 4) & 0x30303030u)) ^ 0x20202020u;
          xsc[1] = (((c1 >> (4 * n)) & 0x0f0f0f0fu) | ((n ? c2 >> 2 : c2 << 2) & 0x30303030u)) ^ 0x20202020u;
        } else {
          xsc[0] = ((c0 & 0x0f0f0f0fu) | ((c2 << 4) & 0x30303030u)) ^ 0x20202020u;
          xsc[1] = ((c1 & 0x0f0f0f0fu) | ((c2 << 2) & 0x30303030u)) ^ 0x20202020u;
          xsc[2] = (((c0 >> 4) & 0x0f0f0f0fu) | (c2 & 0x30303030u)) ^ 0x20202020u;
          xsc[3] = (((c1 >> 4) & 0x0f0f0f0fu) | ((c2 >> 2) & 0x30303030u)) ^ 0x20202020u;
        }
        // hmask with bit 4n of every byte moved to bit 0 (PARTS = 2): block jb
        // takes bit jb
        uint32_t hm[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) hm[w] = PARTS == 2 ? blk[w] >> (4 * n) : blk[w];
        float asb[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) asb[t] = 0.f;
        auto block = [&](auto jb_tag) {
          constexpr int jb = decltype(jb_tag)::value;
          const int sg0 = __builtin_amdgcn_sbfe((int)xsc[jb >> 1], 16 * (jb & 1), 6);
          const int sg1 = __builtin_amdgcn_sbfe((int)xsc[jb >> 1], 16 * (jb & 1) + 8, 6);
          uint32_t op[8];  // c per byte, elements 32 jb + 4w .. of the half
#pragma unroll
          for (int w = 0; w < 8; ++w)
            op[w] = ((blk[8 + 8 * (jb >> 2) + w] >> (2 * (jb & 3))) & 0x03030303u) | bit_to_2<jb>(hm[w]);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const uint4* xp = reinterpret_cast<const uint4*>(xq + t * L + 32 * jb);
            const uint4 x0 = xp[0], x1 = xp[1];
            int da = __builtin_amdgcn_sdot4((int)op[0], (int)x0.x, 0, false);
            da = __builtin_amdgcn_sdot4((int)op[1], (int)x0.y, da, false);
            da = __builtin_amdgcn_sdot4((int)op[2], (int)x0.z, da, false);
            da = __builtin_amdgcn_sdot4((int)op[3], (int)x0.w, da, false);
            int db = __builtin_amdgcn_sdot4((int)op[4], (int)x1.x, 0, false);
            db = __builtin_amdgcn_sdot4((int)op[5], (int)x1.y, db, false);
            db = __builtin_amdgcn_sdot4((int)op[6], (int)x1.z, db, false);
            db = __builtin_amdgcn_sdot4((int)op[7], (int)x1.w, db, false);
            const int2 sx = *reinterpret_cast<const int2*>(&xsq[t * nsub + 2 * jb]);
            // I32 = sum over the block of sigma * v * x, with v * x = c x - 4 x
            const int I = __mul24(sg0, da - 4 * sx.x) + __mul24(sg1, db - 4 * sx.y);
            asb[t] = __builtin_fmaf(xdq[t * nxb + jb], (float)I, asb[t]);
            if (PROBE) {
              const int rr = wrow - probe.row0;
              if (rr >= 0 && rr < probe.rows) probe.out[((int64_t)pr[t] * probe.rows + rr) * nxb + bq + jb] = I;
            }
          }
          // one block's operands live at a time
          __builtin_amdgcn_sched_barrier(0);
        };
        block(std::integral_constant<int, 0>{});
        block(std::integral_constant<int, 1>{});
        block(std::integral_constant<int, 2>{});
        block(std::integral_constant<int, 3>{});
        if constexpr (kBpt == 8) {
          block(std::integral_constant<int, 4>{});
          block(std::integral_constant<int, 5>{});
          block(std::integral_constant<int, 6>{});
          block(std::integral_constant<int, 7>{});
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(dw, asb[t], acc[t]);
      }
    };
    static_assert(kTok == 2, "passes of one or two tokens");
    if (nt == 1)
      dots(std::integral_constant<int, 1>{});
    else
      dots(std::integral_constant<int, 2>{});
    // sum the row's parts (lanes tpr r .. tpr r + tpr - 1)
#pragma unroll
    for (int t = 0; t < kTok; ++t)
      for (int o = 1; o < tpr; o <<= 1) acc[t] += __shfl_xor(acc[t], o);
    if (part == 0) {
      gus[r * kBatch + t0] = acc[0];
      if (nt > 1) gus[r * kBatch + t0 + 1] = acc[1];
    }
    }
    __syncthreads();
    // ---- SwiGLU + q8_1 of H: half wave h of the workgroup takes token h
    for (int t = tid >> 5; t < nb; t += nthr / 32) {
      // The q8_1 rule rounds every product to fp32 on its own.
#pragma clang fp contract(off)
      const int f = lane & 31;
      const float gv = gus[f * kBatch + t], uv = gus[(32 + f) * kBatch + t];
      const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-gv));
      const float h = gv * sig * uv;
      float amax = fabsf(h);
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
      const float d = amax / 127.0f;
      const float id = d != 0.0f ? 1.0f / d : 0.0f;
      const int qv = round_half_away(h * id);
      int sum = qv;
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 32);
      const int pt = s_pb[bt + t];
      h_codes[(int64_t)pt * F + f0 + f] = (int8_t)qv;
      if (f == 0)
        h_ds[(int64_t)pt * nfb + f0 / 32] =
            float_to_half_bits(d) | (float_to_half_bits(fp32_barrier(d * (float)sum)) << 16);
    }
  }
}

// ---------------------------------------------------------------------------
// Thread (slot, row, slice) of a down workgroup: a wave is one slot's 64
// lanes, rows x slices = 64 with a slice of 4 blocks (72 bytes) of the row;
// S = slices per row (a power of two, >= F / 128), R = 64 / S rows per
// workgroup.  WHOLE: F % 128 == 0, so every slice is 4 whole blocks inside
// its row, loaded as four 16-byte pieces and 8 bytes; otherwise each block is
// loaded on its own (d, then the 16 index bytes), so no load reaches past its
// row (a load partly past the end of the buffer would come back zero).
template <bool PROBE, int FMT, bool WHOLE>
__global__ __launch_bounds__(kDnThreads) void k_dec_down(const uint8_t* __restrict__ dn, const int32_t* __restrict__ idx,
                                                       const float* __restrict__ router_w, int P, int k, int L, int F,
                                                       int E, int s_log2, const int8_t* __restrict__ h_codes,
                                                       const uint32_t* __restrict__ h_ds, float* __restrict__ y,
                                                       ProbeRows probe) {
  __shared__ __align__(16) int8_t hs[kDnSlots][2048];  // the pass's H codes (F <= 2048)
  __shared__ float hds[kDnSlots][64];                   // and their fp32 d_H
  __shared__ float osum[kDnMaxK][64];                   // O of each slot and row
  const int S = 1 << s_log2, R = 64 >> s_log2;
  const int t = blockIdx.x, l0 = blockIdx.y * R;
  const int tid = threadIdx.x;
  // a wave = one slot's R rows; slot is read as wave-uniform, so the expert's
  // buffer descriptor stays scalar (a per-lane one makes every weight load a
  // readfirstlane loop)
  const int slice = tid & (S - 1), row = (tid & 63) >> s_log2, slot = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nfb = F / 32, row_bytes = nfb * kIq4Bytes;
  const int l = l0 + row;
  const rsrc_t rh = make_rsrc(h_codes, (uint32_t)(P * F));
  const rsrc_t rs = make_rsrc(h_ds, (uint32_t)(P * nfb * 4));
  const rsrc_t ri = make_rsrc(idx, (uint32_t)P * 4u);

  for (int j0 = 0; j0 < k; j0 += kDnSlots) {
    const int j = j0 + slot;
    const int pair = t * k + j;  // uniform per wave
    // this slot's expert (one load per wave, uniform)
    const int e = __builtin_amdgcn_readfirstlane((int)buf_u32(ri, j < k ? pair * 4 : kOutOfRange, 0));
    const bool valid = j < k && (unsigned)e < (unsigned)E;
    // H of the pass's pairs, pair order (independent of the routing): codes
    // as 16-byte pieces i = tid, tid + 512 of 8 x 128, scales one per thread
    uint4 hv[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int i = tid + kDnThreads * m, s = i >> 7, c = i & 127;
      const bool ok = j0 + s < k && 16 * c < F;
      hv[m] = buf_u128(rh, ok ? (t * k + j0 + s) * F + 16 * c : kOutOfRange, 0);
    }
    const int ds_s = tid >> 6, ds_b = tid & 63;
    const uint32_t dv = buf_u32(rs, (j0 + ds_s < k && ds_b < nfb) ? ((t * k + j0 + ds_s) * nfb + ds_b) * 4 : kOutOfRange,
                                0);
    // this thread's slice: bytes 72 slice .. +71 of row l of expert e
    const rsrc_t rw = make_rsrc(dn + (int64_t)(valid ? e : 0) * L * row_bytes, (uint32_t)(L * row_bytes));
    const int woff = valid && 4 * slice < nfb ? l * row_bytes + 72 * slice : kOutOfRange;
    uint32_t wb[18];
    if constexpr (WHOLE) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 v = buf_u128(rw, woff, 16 * c);
        wb[4 * c] = v.x, wb[4 * c + 1] = v.y, wb[4 * c + 2] = v.z, wb[4 * c + 3] = v.w;
      }
      const auto t2 = __builtin_amdgcn_raw_buffer_load_b64(rw, woff, 64, 0);
      wb[16] = t2[0], wb[17] = t2[1];
    } else {
      // block m: d into the 16-bit half at byte 18 m, indices at 18 m + 2 (the
      // layout of the 72-byte piece, as the unpack below reads it)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int bo = 4 * slice + m < nfb ? woff + 18 * m : kOutOfRange;
        const uint32_t d16 = buf_u16(rw, bo, 0);
        const uint4 v = buf_u128(rw, bo, 2);
        const int wi = (18 * m) >> 2;
        if ((18 * m) & 3) {  // d in the high half of word wi (its low half: block m - 1's last two
                             // index bytes), indices from word wi + 1 on
          wb[wi] |= d16 << 16;
          wb[wi + 1] = v.x, wb[wi + 2] = v.y, wb[wi + 3] = v.z, wb[wi + 4] = v.w;
        } else {  // d in the low half of word wi, indices from byte 2 of it
          wb[wi] = d16 | (v.x << 16);
          wb[wi + 1] = (v.x >> 16) | (v.y << 16);
          wb[wi + 2] = (v.y >> 16) | (v.z << 16);
          wb[wi + 3] = (v.z >> 16) | (v.w << 16);
          wb[wi + 4] = v.w >> 16;
        }
      }
    }
    if (j0 > 0) __syncthreads();  // the previous pass's reads of hs / hds are done
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int i = tid + kDnThreads * m;
      *reinterpret_cast<uint4*>(&hs[i >> 7][16 * (i & 127)]) = hv[m];
    }
    hds[ds_s][ds_b] = half_bits_to_float(dv & 0xffffu);
    __syncthreads();

    float acc = 0.f;
    if (valid) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int b = 4 * slice + m;
        if (b < nfb) {
          // block m at byte 18 m of the slice: d, then 16 index bytes
          const int base = 18 * m, wi = base >> 2;
          uint32_t nw[4], d16;
          if ((base & 3) == 0) {
            d16 = wb[wi] & 0xffffu;
#pragma unroll
            for (int w = 0; w < 4; ++w) nw[w] = __builtin_amdgcn_alignbyte(wb[wi + w + 1], wb[wi + w], 2);
          } else {
            d16 = wb[wi] >> 16;
#pragma unroll
            for (int w = 0; w < 4; ++w) nw[w] = wb[wi + 1 + w];
          }
          const uint4* hp = reinterpret_cast<const uint4*>(&hs[slot][32 * b]);
          const uint4 h0 = hp[0], h1 = hp[1];
          const uint32_t hw[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
          int J = 0;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            J = __builtin_amdgcn_sdot4((int)down_lookup<FMT>(nw[w] & 0x0f0f0f0fu), (int)hw[w], J, false);
            J = __builtin_amdgcn_sdot4((int)down_lookup<FMT>((nw[w] >> 4) & 0x0f0f0f0fu), (int)hw[4 + w], J, false);
          }
          acc = __builtin_fmaf(half_bits_to_float(d16) * hds[slot][b], (float)J, acc);
          if (PROBE) {
            const int rr = l - probe.row0;
            if (rr >= 0 && rr < probe.rows) probe.out[((int64_t)pair * probe.rows + rr) * nfb + b] = J;
          }
        }
      }
    }
    // sum the row's S slices (adjacent lanes of the wave)
    for (int o = 1; o < S; o <<= 1) acc += __shfl_xor(acc, o);
    if (slice == 0 && j < k) osum[j][row] = valid ? acc : 0.f;
  }
  __syncthreads();
  // combine: y[t][l] = sum over the slots, in order, of w[t][j] * O_j[l]
  if (tid < R) {
    float v = 0.f;
    for (int j = 0; j < k; ++j) v = __builtin_fmaf(router_w[t * k + j], osum[j][tid], v);
    y[(int64_t)t * L + l0 + tid] = v;
  }
}

// H of pair p in ggml q8_1 blocks (pairs with an invalid id: zero blocks).
__global__ __launch_bounds__(256) void k_export_h_pairs(const int32_t* __restrict__ idx, int E, int64_t nblocks, int nfb,
                                                       const int8_t* __restrict__ h_codes,
                                                       const uint32_t* __restrict__ h_ds, uint8_t* __restrict__ h_out) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one q8_1 block
  if (q >= nblocks) return;
  const int64_t p = q / nfb;
  const int e = idx[p];
  uint32_t* dst = reinterpret_cast<uint32_t*>(h_out + q * kQ81Bytes);
  const bool ok = (unsigned)e < (unsigned)E;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(h_codes + q * 32);
  dst[0] = ok ? h_ds[q] : 0u;
#pragma unroll
  for (int w = 0; w < 8; ++w) dst[1 + w] = ok ? src[w] : 0u;
}

typedef void (*GateupKernel)(const uint8_t*, const int32_t*, const uint8_t*, int, int, int, int, int, int, int, int8_t*,
                             uint32_t*, ProbeRows);

// Resident workgroups per CU of a gate/up kernel at a block size and dynamic
// LDS size, cached per device.
int blocks_per_cu(GateupKernel kern, int threads, size_t lds) {
  static std::mutex mu;
  struct Entry {
    int dev;
    GateupKernel kern;
    int threads;
    size_t lds;
    int n;
  };
  static Entry cache[64];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  std::lock_guard<std::mutex> g(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].dev == dev && cache[i].kern == kern && cache[i].threads == threads && cache[i].lds == lds)
      return cache[i].n;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(kern), threads, lds) !=
          hipSuccess ||
      n < 1)
    n = 1;
  if (used < 64) cache[used++] = Entry{dev, kern, threads, lds, n};
  return n;
}

}  // namespace

bool decode_path(const Shapes& s) { return s.pairs() <= kDecodeMaxPairs && s.L <= 1024 && s.F <= 2048; }

hipError_t launch_decode(const Shapes& s, const Work& w, const uint8_t* x, const int32_t* idx, const float* router_w,
                         const uint8_t* gu, int gu_fmt, const uint8_t* dn, int dn_fmt, float* y,
                         const ProbeRows* probe_gu, const ProbeRows* probe_dn, hipStream_t st,
                         hipEvent_t after_gateup) {
  const int P = (int)s.pairs();
  const ProbeRows none = {nullptr, 0, 0};
  {
    const int nxb = s.L / 32;
    const size_t lds = kBatch * s.L + 4 * kBatch * nxb + 4 * kBatch * (s.L / 16) + 4 * 64 * kBatch + 4 * 64;
    const dim3 grid((unsigned)P, s.F / 32);
    const bool q40 = gu_fmt == LAT_MOE_GATEUP_Q4_0;
    const bool pr = probe_gu != nullptr;
    auto pick = [&](bool probe, auto parts_tag) -> GateupKernel {
      constexpr int PARTS = decltype(parts_tag)::value;
      return probe ? (q40 ? k_dec_gateup<true, LAT_MOE_GATEUP_Q4_0, PARTS> : k_dec_gateup<true, LAT_MOE_GATEUP_Q3_K, PARTS>)
                   : (q40 ? k_dec_gateup<false, LAT_MOE_GATEUP_Q4_0, PARTS> : k_dec_gateup<false, LAT_MOE_GATEUP_Q3_K, PARTS>);
    };
    // threads per row: parts per super-block x super-blocks (a power of two)
    const int nsb = s.L / 256, sb_log2 = nsb == 1 ? 0 : nsb == 2 ? 1 : 2;
    // The items that can be active (distinct experts x feature blocks) over the
    // workgroups resident at once: the layout that needs fewer rounds of
    // workgroups, two parts per super-block on a tie.  Decided from the plain
    // kernels, so that a call with probes sums in the same order as without.
    const int64_t items = (int64_t)(P < s.E ? P : s.E) * (s.F / 32);
    const int cus = w.num_cus > 0 ? w.num_cus : 1;
    const int64_t cap1 =
        (int64_t)blocks_per_cu(pick(false, std::integral_constant<int, 1>{}), 64 << sb_log2, lds) * cus;
    const int64_t cap2 =
        (int64_t)blocks_per_cu(pick(false, std::integral_constant<int, 2>{}), 128 << sb_log2, lds) * cus;
    const bool two = (items + cap2 - 1) / cap2 <= (items + cap1 - 1) / cap1;
    const int tpr_log2 = sb_log2 + (two ? 1 : 0);
    const GateupKernel kern = two ? pick(pr, std::integral_constant<int, 2>{}) : pick(pr, std::integral_constant<int, 1>{});
    hipLaunchKernelGGL(kern, grid, dim3(64u << tpr_log2), lds, st, x, idx, gu, (int)s.T, P, s.k, s.L, s.F,
                       s.E, tpr_log2, w.h_codes, w.h_ds, probe_gu ? *probe_gu : none);
  }
  if (after_gateup && hipEventRecord(after_gateup, st) != hipSuccess) return hipErrorUnknown;
  {
    // slices of 4 blocks per row: a power of two covering F / 128, rows = 64 / slices
    const int nsl = (s.F / 32 + 3) / 4;
    const int s_log2 = nsl <= 1 ? 0 : nsl <= 2 ? 1 : nsl <= 4 ? 2 : nsl <= 8 ? 3 : 4;
    const dim3 grid((unsigned)s.T, s.L >> (6 - s_log2));
    const bool q40 = dn_fmt == kDownQ40;
    auto kern = s.F % 128 == 0
                    ? (probe_dn ? (q40 ? k_dec_down<true, kDownQ40, true> : k_dec_down<true, kDownIq4Nl, true>)
                                : (q40 ? k_dec_down<false, kDownQ40, true> : k_dec_down<false, kDownIq4Nl, true>))
                    : (probe_dn ? (q40 ? k_dec_down<true, kDownQ40, false> : k_dec_down<true, kDownIq4Nl, false>)
                                : (q40 ? k_dec_down<false, kDownQ40, false> : k_dec_down<false, kDownIq4Nl, false>));
    hipLaunchKernelGGL(kern, grid, dim3(kDnThreads), 0, st, dn, idx, router_w, P, s.k, s.L, s.F, s.E, s_log2,
                       w.h_codes, w.h_ds, y, probe_dn ? *probe_dn : none);
  }
  return hipGetLastError();
}

hipError_t launch_export_h_pairs(const int32_t* idx, const Shapes& s, const Work& w, uint8_t* h_out, hipStream_t st) {
  const int nfb = s.F / 32;
  const int64_t n = s.pairs() * nfb;
  hipLaunchKernelGGL(k_export_h_pairs, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, idx, s.E, n, nfb,
                     w.h_codes, w.h_ds, h_out);
  return hipGetLastError();
}

}  // namespace latmoe
