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
// the combine sums each token's k slots in a fixed order.
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

// The IQ4_NL non-linear table (ggml), packed as four little-endian words.
constexpr int kIq4Table[16] = {-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113};
constexpr uint32_t tab_word(int w) {
  return (uint32_t)(kIq4Table[4 * w] & 0xff) | ((uint32_t)(kIq4Table[4 * w + 1] & 0xff) << 8) |
         ((uint32_t)(kIq4Table[4 * w + 2] & 0xff) << 16) | ((uint32_t)(kIq4Table[4 * w + 3] & 0xff) << 24);
}
constexpr uint32_t kTab0 = tab_word(0), kTab1 = tab_word(1), kTab2 = tab_word(2), kTab3 = tab_word(3);
static_assert(kTab0 == 0xBFAD9881u && kTab3 == 0x71594535u, "IQ4_NL table packing");

// 4 nibble indices (one per byte) -> 4 table bytes.
__device__ __forceinline__ uint32_t iq4_lookup(uint32_t nib) {
  const uint32_t sel = nib & 0x07070707u;
  const uint32_t lo = __builtin_amdgcn_perm(kTab1, kTab0, sel);
  const uint32_t hi = __builtin_amdgcn_perm(kTab3, kTab2, sel);
  const uint32_t m = ((nib >> 3) & 0x01010101u) * 0xffu;
  return (lo & ~m) | (hi & m);
}

template <bool PROBE, bool ALIGNED16>
__global__ __launch_bounds__(kThreads) void k_down(const uint8_t* __restrict__ dn, const float* __restrict__ router_w,
                                                   const int32_t* __restrict__ perm,
                                                   const int32_t* __restrict__ tiles,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ misc, int L, int F,
                                                   const int8_t* __restrict__ h_codes,
                                                   const uint32_t* __restrict__ h_ds, float* __restrict__ slots,
                                                   ProbeRows probe) {
  __shared__ __align__(16) uint8_t raw[kLT * kRawStride];
  __shared__ __align__(16) int8_t As[kLT * kOpStride];
  __shared__ __align__(16) int8_t Bs[kNT * kOpStride];
  __shared__ __align__(16) float dds[8][kLT];  // d_dn per block and row
  __shared__ float dhs[8][kNT];                // d_H per block and token
  __shared__ int32_t pid[kNT];

  const int tile = blockIdx.x;
  if (tile >= misc[kMiscTiles]) return;
  const int e = tiles[2 * tile];
  const int pos0 = tiles[2 * tile + 1];
  const int cnt = min(kNT, offsets[e + 1] - pos0);
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
          o[w] = iq4_lookup(qw[w] & 0x0f0f0f0fu);             // values 4w .. 4w+3
          o[4 + w] = iq4_lookup((qw[w] >> 4) & 0x0f0f0f0fu);  // values 16+4w ..
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

  // ---- epilogue: weighted output rows into the pair's slot
  if (!active) return;
  const int n = 32 * tsub + col;
  const int p = pid[n];
  if (p >= 0) {
    const float wgt = router_w[p];
    float* dst = slots + (int64_t)p * L + l0 + 32 * lsub + 4 * khalf;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      float4 v;
      v.x = acc[4 * qq + 0] * wgt;
      v.y = acc[4 * qq + 1] * wgt;
      v.z = acc[4 * qq + 2] * wgt;
      v.w = acc[4 * qq + 3] * wgt;
      *reinterpret_cast<float4*>(dst + 8 * qq) = v;
    }
  }
}

template <bool PROBE>
void launch_variant(bool aligned, dim3 grid, hipStream_t st, const uint8_t* dn, const float* router_w,
                    const Shapes& s, const Work& w, ProbeRows probe) {
  if (aligned)
    hipLaunchKernelGGL((k_down<PROBE, true>), grid, dim3(kThreads), 0, st, dn, router_w, w.perm, w.tiles, w.offsets,
                       w.misc, s.L, s.F, w.h_codes, w.h_ds, w.slots, probe);
  else
    hipLaunchKernelGGL((k_down<PROBE, false>), grid, dim3(kThreads), 0, st, dn, router_w, w.perm, w.tiles, w.offsets,
                       w.misc, s.L, s.F, w.h_codes, w.h_ds, w.slots, probe);
}

}  // namespace

hipError_t launch_down(const uint8_t* dn, const float* router_w, const Shapes& s, const Work& w,
                       const ProbeRows* probe, hipStream_t st) {
  const dim3 grid(w.max_tiles, s.L / kLT);
  // 16-byte staging needs every row (and so every 8-block step) 16-byte aligned;
  // that also means F is a multiple of 256, so every step is a full 144-byte chunk.
  const bool aligned = ((int64_t)(s.F / 32) * kIq4Bytes) % 16 == 0 && ((uintptr_t)dn & 15u) == 0;
  if (probe)
    launch_variant<true>(aligned, grid, st, dn, router_w, s, w, *probe);
  else
    launch_variant<false>(aligned, grid, st, dn, router_w, s, w, ProbeRows{nullptr, 0, 0});
  return hipGetLastError();
}

}  // namespace latmoe
