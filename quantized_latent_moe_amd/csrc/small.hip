// Gate/up and down for small batches (decode): GEMV-shaped kernels.
//
// Same computation as the grouped GEMMs (page "Run Edge0-145B Q3_K on AMD HIP
// (Linux, gfx1100) #1", section "Contents": gate/up on Q3_K with SwiGLU and the
// q8_1 rounding of H, down on IQ4_NL), for batches of at most kSmallMaxPairs
// routed pairs, where every expert holds a handful of tokens and the stage
// streams the active experts' weights once.  One workgroup per (active
// expert, 32 features) for gate/up and per (active expert, 32 output rows)
// for down: it issues the loads of its rows (contiguous in memory, 16-byte
// coalesced buffer loads) and of its tokens' rows together (gate/up reads the
// rows the route pass gathered in sorted order, down the H rows, both found
// from the tile entry alone), stages them in LDS, then each thread takes a K slice of one row and forms the 32-value
// block dots with v_dot4 against up to kSmallTok tokens at a time; lane
// shuffles sum the row's slices.  2-byte-aligned blocks are realigned with
// v_alignbyte.
//
// Gate/up works on the code c = low2 + 4 * hbit directly: the int8 operand is
// 7 - c = 3 - v (v = c - 4 the Q3_K value; a byte-wise XOR, no per-sub-block
// table), the 16-value dots are taken apart and the sub-block scale applied to
// them: sum sigma * v * x = sigma * (3 * sum x - sum (7 - c) x), with sum x per
// token and 16 values formed once per workgroup.  The result is the same
// scale-folded 32-value integer dot I32 as in the large kernel, then
// acc_sb += d_x * I32 per block and acc += d_w * acc_sb per super-block; down
// folds acc += (d_dn * d_H) * J32 per block.  32 features are one q8_1 block
// of H, so SwiGLU and the requant finish inside a half wave.
//
// Gate/up weights in Q4_0 take the same workgroups: a thread's K slice is 8
// whole 18-byte blocks (144 contiguous bytes, 16-byte aligned), the nibbles
// are split into low and high halves by masks, and the block dot is
// I32 = sum nib * x - 8 * sum x (the same per-16 code sums), folded as
// acc += d_w * fl(d_x * I32) per block.
#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kSmallTok = 4;  // tokens per pass
constexpr int kSmallThreads = 256;

// ---------------------------------------------------------------------------
// Gate/up: workgroup (tile j of the route table -> expert, 32 features f0).
// Threads: row r = t >> 2 of 64 (32 gate rows f0.., 32 up rows F+f0..), K
// slice q = t & 3 (super-blocks q, q + 4, ...).
template <bool PROBE, int GFMT>
__global__ __launch_bounds__(kSmallThreads) void k_gateup_small(
    const int8_t* __restrict__ xg, const float* __restrict__ xgd, const uint8_t* __restrict__ gu,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles, const int32_t* __restrict__ misc, int L,
    int F, int8_t* __restrict__ h_codes, uint32_t* __restrict__ h_ds, ProbeRows probe) {
  extern __shared__ __align__(16) uint8_t smem[];
  if ((int)blockIdx.x >= misc[kMiscTiles]) return;
  const int4 te = *reinterpret_cast<const int4*>(tiles + kTileWords * blockIdx.x);
  const int e = te.x, pos0 = te.y, cnt = te.z;  // cnt <= kGatherRows
  const int f0 = blockIdx.y * 32;
  const int tid = threadIdx.x, lane = tid & 63;
  constexpr bool kQ40 = GFMT == LAT_MOE_GATEUP_Q4_0;
  const int nsb = L / 256, nxb = L / 32, nsub = L / 16, row_bytes = nsb * (kQ40 ? 8 * kQ40Bytes : kQ3kBytes);
  // LDS: xs[kSmallTok][L] | xds[kSmallTok][nxb] | xsum[kSmallTok][nsub] | gus[64][kSmallTok]
  int8_t* xs = reinterpret_cast<int8_t*>(smem);
  float* xds = reinterpret_cast<float*>(xs + kSmallTok * L);
  int* xsum = reinterpret_cast<int*>(xds + kSmallTok * nxb);
  float* gus = reinterpret_cast<float*>(xsum + kSmallTok * nsub);

  const rsrc_t rw = make_rsrc(gu + (int64_t)e * 2 * F * row_bytes, (uint32_t)(2 * F * row_bytes));
  // the gathered rows: sorted position pos at xg + pos * L, xgd + pos * nxb
  const rsrc_t rx = make_rsrc(xg, (uint32_t)(kGatherRows * L));
  const rsrc_t rd = make_rsrc(xgd, (uint32_t)(kGatherRows * nxb * 4));
  constexpr int kXPer = kSmallTok * 1024 / 16 / kSmallThreads;  // 2
  const int r = tid >> 2, q = tid & 3;
  const int wrow = r < 32 ? f0 + r : F + f0 + r - 32;  // weight row of the expert
  // This thread's super-block (L <= 1024: at most one, sb = q) straight into
  // registers: bytes 0..107 as 16-byte pieces and a 12-byte tail (buffer loads
  // at 2-byte-aligned offsets return the bytes there), d as a 16-bit load.
  // Adjacent threads read adjacent blocks, a wave 16 whole rows.
  // Q4_0: the slice's 8 blocks (144 bytes) as nine 16-byte loads.
  uint32_t blk[kQ40 ? 36 : 28];
  if constexpr (kQ40) {
    const int boff = q < nsb ? wrow * row_bytes + q * 8 * kQ40Bytes : kOutOfRange;
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      const uint4 v = buf_u128(rw, boff, 16 * c);
      blk[4 * c] = v.x, blk[4 * c + 1] = v.y, blk[4 * c + 2] = v.z, blk[4 * c + 3] = v.w;
    }
  } else {
    const int boff = q < nsb ? wrow * row_bytes + q * kQ3kBytes : kOutOfRange;
#pragma unroll
    for (int c = 0; c < 6; ++c) {
      const uint4 v = buf_u128(rw, boff, 16 * c);
      blk[4 * c] = v.x, blk[4 * c + 1] = v.y, blk[4 * c + 2] = v.z, blk[4 * c + 3] = v.w;
    }
    const auto t = __builtin_amdgcn_raw_buffer_load_b96(rw, boff, 96, 0);
    blk[24] = t[0], blk[25] = t[1], blk[26] = t[2];
    blk[27] = buf_u16(rw, boff, 108);
  }
  for (int g0 = 0; g0 < cnt; g0 += kSmallTok) {
    const int nt = min(kSmallTok, cnt - g0);
    // ---- the group's token rows, at their sorted positions
    uint4 xv[kXPer];
    uint32_t dv;
#pragma unroll
    for (int m = 0; m < kXPer; ++m) {
      const int i = tid + kSmallThreads * m;
      const int tk = i / (L / 16), c = i - tk * (L / 16);
      const bool ok = tk < nt && i < kSmallTok * (L / 16);
      xv[m] = buf_u128(rx, ok ? (pos0 + g0 + tk) * L + 16 * c : kOutOfRange, 0);
    }
    {
      const int tk = tid / nxb, b = tid - tk * nxb;
      const bool ok = tk < nt && tid < kSmallTok * nxb;
      dv = buf_u32(rd, ok ? ((pos0 + g0 + tk) * nxb + b) * 4 : kOutOfRange, 0);
    }
    if (g0 > 0) __syncthreads();  // the previous group's reads of xs / gus are done
#pragma unroll
    for (int m = 0; m < kXPer; ++m) {
      const int i = tid + kSmallThreads * m;
      if (i < kSmallTok * (L / 16)) {
        reinterpret_cast<uint4*>(xs)[i] = xv[m];
        // sum of the 16 codes of (token, sub-block)
        int s = __builtin_amdgcn_sdot4((int)xv[m].x, 0x01010101, 0, false);
        s = __builtin_amdgcn_sdot4((int)xv[m].y, 0x01010101, s, false);
        s = __builtin_amdgcn_sdot4((int)xv[m].z, 0x01010101, s, false);
        s = __builtin_amdgcn_sdot4((int)xv[m].w, 0x01010101, s, false);
        xsum[i] = s;  // i = tk * nsub + sub-block
      }
    }
    if (tid < kSmallTok * nxb) xds[tid] = as_float((int)dv);
    __syncthreads();

    float acc[kSmallTok];
#pragma unroll
    for (int tk = 0; tk < kSmallTok; ++tk) acc[tk] = 0.f;
    if (kQ40 && q < nsb) {
      const int sb = q;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        // block kb at byte 18 kb of the slice: d, then 16 nibble bytes
        const int base = 18 * kb, wi = base >> 2;
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
        for (int tk = 0; tk < kSmallTok; ++tk) {
          if (tk < nt) {
            const uint4* xp = reinterpret_cast<const uint4*>(xs + tk * L + sb * 256 + 32 * kb);
            const uint4 x0 = xp[0], x1 = xp[1];
            int dn = __builtin_amdgcn_sdot4((int)lo[0], (int)x0.x, 0, false);
            dn = __builtin_amdgcn_sdot4((int)lo[1], (int)x0.y, dn, false);
            dn = __builtin_amdgcn_sdot4((int)lo[2], (int)x0.z, dn, false);
            dn = __builtin_amdgcn_sdot4((int)lo[3], (int)x0.w, dn, false);
            dn = __builtin_amdgcn_sdot4((int)hi[0], (int)x1.x, dn, false);
            dn = __builtin_amdgcn_sdot4((int)hi[1], (int)x1.y, dn, false);
            dn = __builtin_amdgcn_sdot4((int)hi[2], (int)x1.z, dn, false);
            dn = __builtin_amdgcn_sdot4((int)hi[3], (int)x1.w, dn, false);
            const int2 sx = *reinterpret_cast<const int2*>(&xsum[tk * nsub + sb * 16 + 2 * kb]);
            const int I = dn - 8 * (sx.x + sx.y);  // sum (nib - 8) x
            const float t = xds[tk * nxb + sb * 8 + kb] * (float)I;
            acc[tk] = __builtin_fmaf(dwb, t, acc[tk]);
            if (PROBE) {
              const int rr = wrow - probe.row0;
              if (rr >= 0 && rr < probe.rows)
                probe.out[((int64_t)perm[pos0 + g0 + tk] * probe.rows + rr) * nxb + sb * 8 + kb] = I;
            }
          }
        }
      }
    }
    if (!kQ40 && q < nsb) {
      const int sb = q;
      const float dw = half_bits_to_float(blk[27] & 0xffffu);
      float asb[kSmallTok];
#pragma unroll
      for (int tk = 0; tk < kSmallTok; ++tk) asb[tk] = 0.f;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const int n = kb >> 2, j = kb & 3;
        int sg[2];  // sub-block scales sc6 - 32
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int s = 8 * n + 2 * j + t;
          const int sl = s & 7;
          const int lo = (int)((blk[24 + (sl >> 2)] >> (8 * (sl & 3) + (s < 8 ? 0 : 4))) & 15u);
          const int hi = (int)((blk[26] >> (8 * (s & 3) + 2 * (s >> 2))) & 3u);
          sg[t] = (lo | (hi << 4)) - 32;
        }
        uint32_t op[8];  // 7 - c per byte
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const uint32_t hb = ((blk[w] >> (4 * n + j)) << 2) & 0x04040404u;
          const uint32_t c = ((blk[8 + 8 * n + w] >> (2 * j)) & 0x03030303u) | hb;
          op[w] = c ^ 0x07070707u;
        }
#pragma unroll
        for (int tk = 0; tk < kSmallTok; ++tk) {
          if (tk < nt) {
            const uint4* xp = reinterpret_cast<const uint4*>(xs + tk * L + sb * 256 + 32 * kb);
            const uint4 x0 = xp[0], x1 = xp[1];
            int da = __builtin_amdgcn_sdot4((int)op[0], (int)x0.x, 0, false);
            da = __builtin_amdgcn_sdot4((int)op[1], (int)x0.y, da, false);
            da = __builtin_amdgcn_sdot4((int)op[2], (int)x0.z, da, false);
            da = __builtin_amdgcn_sdot4((int)op[3], (int)x0.w, da, false);
            int db = __builtin_amdgcn_sdot4((int)op[4], (int)x1.x, 0, false);
            db = __builtin_amdgcn_sdot4((int)op[5], (int)x1.y, db, false);
            db = __builtin_amdgcn_sdot4((int)op[6], (int)x1.z, db, false);
            db = __builtin_amdgcn_sdot4((int)op[7], (int)x1.w, db, false);
            const int2 sx = *reinterpret_cast<const int2*>(&xsum[tk * nsub + sb * 16 + 2 * kb]);
            // I32 = sum over the block of sigma * v * x, with v * x = 3x - (7 - c) x
            const int I = sg[0] * (3 * sx.x - da) + sg[1] * (3 * sx.y - db);
            asb[tk] = __builtin_fmaf(xds[tk * nxb + sb * 8 + kb], (float)I, asb[tk]);
            if (PROBE) {
              const int rr = wrow - probe.row0;
              if (rr >= 0 && rr < probe.rows)
                probe.out[((int64_t)perm[pos0 + g0 + tk] * probe.rows + rr) * nxb + sb * 8 + kb] = I;
            }
          }
        }
      }
#pragma unroll
      for (int tk = 0; tk < kSmallTok; ++tk) acc[tk] = __builtin_fmaf(dw, asb[tk], acc[tk]);
    }
    // sum the row's 4 K slices (lanes 4r .. 4r+3)
#pragma unroll
    for (int tk = 0; tk < kSmallTok; ++tk) {
      acc[tk] += __shfl_xor(acc[tk], 1);
      acc[tk] += __shfl_xor(acc[tk], 2);
    }
    if (q == 0) {
#pragma unroll
      for (int tk = 0; tk < kSmallTok; ++tk) gus[r * kSmallTok + tk] = acc[tk];
    }
    __syncthreads();
    // ---- SwiGLU + q8_1 of H: half wave h of the workgroup takes token h
    for (int tk = tid >> 5; tk < nt; tk += kSmallThreads / 32) {
      // The q8_1 rule rounds every product to fp32 on its own.
#pragma clang fp contract(off)
      const int f = lane & 31;
      const float gv = gus[f * kSmallTok + tk], uv = gus[(32 + f) * kSmallTok + tk];
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
      const int64_t pos = pos0 + g0 + tk;
      h_codes[pos * F + f0 + f] = (int8_t)qv;
      if (f == 0)
        h_ds[pos * (F / 32) + f0 / 32] =
            float_to_half_bits(d) | (float_to_half_bits(fp32_barrier(d * (float)sum)) << 16);
    }
  }
}

// ---------------------------------------------------------------------------
// Down: workgroup (tile j -> expert, 32 output rows l0).  Threads: row r = t
// >> 3, K slice q = t & 7 (blocks q, q + 8, ...).
template <bool PROBE, int FMT>
__global__ __launch_bounds__(kSmallThreads) void k_down_small(
    const uint8_t* __restrict__ dn, const float* __restrict__ router_w, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ misc,
    int pairs, int L, int F, const int8_t* __restrict__ h_codes, const uint32_t* __restrict__ h_ds,
    float* __restrict__ slots, ProbeRows probe) {
  extern __shared__ __align__(16) uint8_t smem[];
  if ((int)blockIdx.x >= misc[kMiscTiles]) return;
  const int4 te = *reinterpret_cast<const int4*>(tiles + kTileWords * blockIdx.x);
  const int e = te.x, pos0 = te.y, cnt = te.z;  // cnt <= kSmallMaxPairs
  const int l0 = blockIdx.y * 32;
  const int tid = threadIdx.x;
  const int nfb = F / 32, row_bytes = nfb * kIq4Bytes;
  int8_t* hs = reinterpret_cast<int8_t*>(smem);                // [kSmallTok][F]
  float* hds = reinterpret_cast<float*>(hs + kSmallTok * F);    // [kSmallTok][nfb]

  const rsrc_t rw = make_rsrc(dn + (int64_t)e * L * row_bytes, (uint32_t)(L * row_bytes));
  const rsrc_t rh = make_rsrc(h_codes, (uint32_t)(pairs * F));
  const rsrc_t rs = make_rsrc(h_ds, (uint32_t)(pairs * nfb * 4));
  constexpr int kHPer = kSmallTok * 2048 / 16 / kSmallThreads;  // 4
  constexpr int kDPer = kSmallTok * 64 / kSmallThreads;         // 2
  constexpr int kBPer = 2048 / 32 / 8;                          // blocks per thread (F <= 2048): 8
  const int r = tid >> 3, q = tid & 7;
  // This thread's blocks q, q + 8, ... of row l0 + r straight into registers:
  // d as a 16-bit load, the 16 index bytes as one 16-byte load at the block's
  // byte 2 (buffer loads at 2-byte-aligned offsets return the bytes there).
  uint32_t bd[kBPer];
  uint4 bi[kBPer];
#pragma unroll
  for (int m = 0; m < kBPer; ++m) {
    const int kb = q + 8 * m;
    const int boff = kb < nfb ? (l0 + r) * row_bytes + kb * kIq4Bytes : kOutOfRange;
    bd[m] = buf_u16(rw, boff, 0);
    bi[m] = buf_u128(rw, boff, 2);
  }
  for (int g0 = 0; g0 < cnt; g0 += kSmallTok) {
    const int nt = min(kSmallTok, cnt - g0);
    uint4 hv[kHPer];
    uint32_t dv[kDPer];
#pragma unroll
    for (int m = 0; m < kHPer; ++m) {
      const int i = tid + kSmallThreads * m;
      const int tk = i / (F / 16), c = i - tk * (F / 16);
      hv[m] = buf_u128(rh, (tk < nt && i < kSmallTok * (F / 16)) ? (pos0 + g0 + tk) * F + 16 * c : kOutOfRange, 0);
    }
#pragma unroll
    for (int m = 0; m < kDPer; ++m) {
      const int i = tid + kSmallThreads * m;
      const int tk = i / nfb, bb = i - tk * nfb;
      dv[m] = buf_u32(rs, (tk < nt && i < kSmallTok * nfb) ? ((pos0 + g0 + tk) * nfb + bb) * 4 : kOutOfRange, 0);
    }
    if (g0 > 0) __syncthreads();
#pragma unroll
    for (int m = 0; m < kHPer; ++m) {
      const int i = tid + kSmallThreads * m;
      if (i < kSmallTok * (F / 16)) reinterpret_cast<uint4*>(hs)[i] = hv[m];
    }
#pragma unroll
    for (int m = 0; m < kDPer; ++m) {
      const int i = tid + kSmallThreads * m;
      if (i < kSmallTok * nfb) hds[i] = half_bits_to_float(dv[m] & 0xffffu);
    }
    __syncthreads();

    float acc[kSmallTok];
#pragma unroll
    for (int tk = 0; tk < kSmallTok; ++tk) acc[tk] = 0.f;
#pragma unroll
    for (int m = 0; m < kBPer; ++m) {
      const int kb = q + 8 * m;
      if (kb >= nfb) break;
      const float dd = half_bits_to_float(bd[m] & 0xffffu);
      const uint32_t nibs[4] = {bi[m].x, bi[m].y, bi[m].z, bi[m].w};  // index bytes 4w .. 4w+3
      uint32_t op[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        op[w] = down_lookup<FMT>(nibs[w] & 0x0f0f0f0fu);             // elements 4w .. 4w+3
        op[4 + w] = down_lookup<FMT>((nibs[w] >> 4) & 0x0f0f0f0fu);  // elements 16+4w ..
      }
#pragma unroll
      for (int tk = 0; tk < kSmallTok; ++tk) {
        if (tk < nt) {
          const uint4* hp = reinterpret_cast<const uint4*>(hs + tk * F + 32 * kb);
          const uint4 h0 = hp[0], h1 = hp[1];
          const uint32_t hw[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
          int J = 0;
#pragma unroll
          for (int w = 0; w < 8; ++w) J = __builtin_amdgcn_sdot4((int)op[w], (int)hw[w], J, false);
          acc[tk] = __builtin_fmaf(dd * hds[tk * nfb + kb], (float)J, acc[tk]);
          if (PROBE) {
            const int rr = l0 + r - probe.row0;
            if (rr >= 0 && rr < probe.rows)
              probe.out[((int64_t)perm[pos0 + g0 + tk] * probe.rows + rr) * nfb + kb] = J;
          }
        }
      }
    }
#pragma unroll
    for (int tk = 0; tk < kSmallTok; ++tk) {
      acc[tk] += __shfl_xor(acc[tk], 1);
      acc[tk] += __shfl_xor(acc[tk], 2);
      acc[tk] += __shfl_xor(acc[tk], 4);
    }
    if (q < nt) {  // lane q of the row writes token q
      float v = acc[0];
#pragma unroll
      for (int tk = 1; tk < kSmallTok; ++tk)
        if (q == tk) v = acc[tk];
      const int p = perm[pos0 + g0 + q];
      slots[(int64_t)p * L + l0 + r] = v * router_w[p];
    }
  }
}

}  // namespace

bool small_path(const Shapes& s) {
  return s.pairs() <= kSmallMaxPairs && s.L <= 1024 && s.F <= 2048;
}

hipError_t launch_gateup_small(const Shapes& s, const Work& w, const uint8_t* gu, int fmt, const ProbeRows* probe,
                               hipStream_t st) {
  const int nxb = s.L / 32;
  const size_t lds = kSmallTok * s.L + 4 * kSmallTok * nxb + 4 * kSmallTok * (s.L / 16) + 4 * 64 * kSmallTok;
  const dim3 grid((unsigned)(s.pairs() < s.E ? s.pairs() : s.E), s.F / 32);
  const ProbeRows none = {nullptr, 0, 0};
  const ProbeRows pr = probe ? *probe : none;
  const bool q40 = fmt == LAT_MOE_GATEUP_Q4_0;
  auto kern = probe ? (q40 ? k_gateup_small<true, LAT_MOE_GATEUP_Q4_0> : k_gateup_small<true, LAT_MOE_GATEUP_Q3_K>)
                    : (q40 ? k_gateup_small<false, LAT_MOE_GATEUP_Q4_0> : k_gateup_small<false, LAT_MOE_GATEUP_Q3_K>);
  hipLaunchKernelGGL(kern, grid, dim3(kSmallThreads), lds, st, w.xg, w.xgd, gu, w.perm, w.tiles, w.misc, s.L, s.F,
                     w.h_codes, w.h_ds, pr);
  return hipGetLastError();
}

namespace {

template <int FMT>
void launch_down_small_fmt(const uint8_t* dn, const float* router_w, const Shapes& s, const Work& w,
                           const ProbeRows* probe, hipStream_t st) {
  const int nfb = s.F / 32;
  const size_t lds = kSmallTok * s.F + 4 * kSmallTok * nfb;
  const dim3 grid((unsigned)(s.pairs() < s.E ? s.pairs() : s.E), s.L / 32);
  const ProbeRows none = {nullptr, 0, 0};
  if (probe)
    hipLaunchKernelGGL((k_down_small<true, FMT>), grid, dim3(kSmallThreads), lds, st, dn, router_w, w.perm, w.tiles,
                       w.misc, (int)s.pairs(), s.L, s.F, w.h_codes, w.h_ds, w.slots, *probe);
  else
    hipLaunchKernelGGL((k_down_small<false, FMT>), grid, dim3(kSmallThreads), lds, st, dn, router_w, w.perm, w.tiles,
                       w.misc, (int)s.pairs(), s.L, s.F, w.h_codes, w.h_ds, w.slots, none);
}

}  // namespace

hipError_t launch_down_small(const uint8_t* dn, int fmt, const float* router_w, const Shapes& s, const Work& w,
                             const ProbeRows* probe, hipStream_t st) {
  if (fmt == kDownQ40)
    launch_down_small_fmt<kDownQ40>(dn, router_w, s, w, probe, st);
  else
    launch_down_small_fmt<kDownIq4Nl>(dn, router_w, s, w, probe, st);
  return hipGetLastError();
}

}  // namespace latmoe
