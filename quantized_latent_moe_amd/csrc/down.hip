// Down grouped GEMM (IQ4_NL x q8_1 H) with the router-weight epilogue.
//
// Page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1", section
// "Contents": after gate/up, down reads IQ4_NL.  Both operands carry one scale
// per 32 values, so each int32 block dot J is folded as
//   O[l][p] += d_dn[l][b] * (d_H[p][b] * float(J)).
// Work item = (expert e, tile of kTileN sorted pairs, 64 output rows l0..l0+63);
// wave w owns rows l0 + 32*(w&1) .. +31 and tokens 32*(w>>1) .. +31.  K (= F)
// is walked 256 values (8 blocks) at a time: IQ4_NL rows are staged into LDS
// with 16-bit loads (18-byte blocks are 2-byte aligned) and expanded to int8
// through the 16-entry table with two v_perm_b32 lookups and a byte select;
// H codes (contiguous per sorted pair) and fp16 d_H are staged alongside.
// Epilogue: O * router_w[p] is written to the pair's slot row (pair order), so
// the combine can sum each token's k slots in a fixed order.
#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kLT = 64;              // output rows per work item
constexpr int kRawStride = 8 * kIq4Bytes;  // 144 bytes: 8 IQ4_NL blocks of one row
constexpr int kOpStride = 256 + 16;  // int8 operand row in LDS (bytes)

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

template <bool PROBE>
__global__ __launch_bounds__(256) void k_down(const uint8_t* __restrict__ dn, const float* __restrict__ router_w,
                                              const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles,
                                              const int32_t* __restrict__ offsets,
                                              const int32_t* __restrict__ misc, int L, int F,
                                              const int8_t* __restrict__ h_codes,
                                              const uint32_t* __restrict__ h_ds, float* __restrict__ slots,
                                              ProbeRows probe) {
  __shared__ __align__(16) uint8_t raw[kLT * kRawStride];
  __shared__ __align__(16) int8_t As[kLT * kOpStride];
  __shared__ __align__(16) int8_t Bs[kTileN * kOpStride];
  __shared__ __align__(16) float dds[8][kLT];  // d_dn per block and row
  __shared__ float dhs[8][kTileN];             // d_H per block and token
  __shared__ int32_t pid[kTileN];

  const int tile = blockIdx.x;
  if (tile >= misc[kMiscTiles]) return;
  const int e = tiles[2 * tile];
  const int pos0 = tiles[2 * tile + 1];
  const int cnt = min(kTileN, offsets[e + 1] - pos0);
  const int l0 = blockIdx.y * kLT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lsub = wave & 1, tsub = wave >> 1;
  const int nfb = F / 32;
  const int64_t row_bytes = (int64_t)nfb * kIq4Bytes;
  const uint8_t* dn_e = dn + (int64_t)e * L * row_bytes;

  if (tid < kTileN) pid[tid] = tid < cnt ? perm[pos0 + tid] : -1;

  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  const int col = lane & 31, khalf = lane >> 5;
  const int8_t* ap = As + (32 * lsub + col) * kOpStride + 16 * khalf;
  const int8_t* bp = Bs + (32 * tsub + col) * kOpStride + 16 * khalf;

  const int nkc = (nfb + 7) / 8;  // chunks of 8 blocks
  for (int kc = 0; kc < nkc; ++kc) {
    const int nb = min(8, nfb - kc * 8);  // blocks in this chunk
    // ---- stage IQ4_NL: 64 rows x nb blocks x 9 halfwords
    for (int i = tid; i < kLT * 72; i += 256) {
      const int r = i / 72, hw = i - r * 72;
      uint16_t v = 0;
      if (hw < nb * 9) v = reinterpret_cast<const uint16_t*>(dn_e + (l0 + r) * row_bytes + kc * 8 * kIq4Bytes)[hw];
      reinterpret_cast<uint16_t*>(raw + r * kRawStride)[hw] = v;
    }
    // ---- stage H codes (16 bytes per thread-step) and d_H
    for (int i = tid; i < kTileN * 16; i += 256) {
      const int n = i >> 4, c16 = i & 15;  // 16-byte piece c16 of 256 codes
      uint4 v = {0, 0, 0, 0};
      if (n < cnt && c16 < nb * 2)
        v = *reinterpret_cast<const uint4*>(h_codes + (int64_t)(pos0 + n) * F + kc * 256 + c16 * 16);
      *reinterpret_cast<uint4*>(Bs + n * kOpStride + c16 * 16) = v;
    }
    for (int i = tid; i < kTileN * 8; i += 256) {
      const int n = i >> 3, b = i & 7;
      float dh = 0.f;
      if (n < cnt && b < nb) dh = half_bits_to_float(h_ds[(int64_t)(pos0 + n) * nfb + kc * 8 + b] & 0xffffu);
      dhs[b][n] = dh;
    }
    __syncthreads();
    // ---- unpack: thread -> (row r, block pair) ; 64 rows x 8 blocks = 512 blocks, 2 per thread
    for (int i = tid; i < kLT * 8; i += 256) {
      const int r = i >> 3, b = i & 7;
      const uint8_t* blk = raw + r * kRawStride + b * kIq4Bytes;
      uint32_t* dst = reinterpret_cast<uint32_t*>(As + r * kOpStride + b * 32);
      if (b < nb) {
        const uint16_t* h16 = reinterpret_cast<const uint16_t*>(blk);
        // 16 code bytes at blk+2 .. blk+17 (2-byte aligned): gather as 4 words
        uint32_t qw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) qw[w] = (uint32_t)h16[1 + 2 * w] | ((uint32_t)h16[2 + 2 * w] << 16);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          dst[w] = iq4_lookup(qw[w] & 0x0f0f0f0fu);             // values 4w .. 4w+3
          dst[4 + w] = iq4_lookup((qw[w] >> 4) & 0x0f0f0f0fu);  // values 16+4w ..
        }
        dds[b][r] = half_bits_to_float(h16[0]);
      } else {
#pragma unroll
        for (int w = 0; w < 8; ++w) dst[w] = 0;
        dds[b][r] = 0.f;
      }
    }
    __syncthreads();
    // ---- MFMA per block, fold with both scales
    for (int b = 0; b < nb; ++b) {
      const v4i va = *reinterpret_cast<const v4i*>(ap + 32 * b);
      const v4i vb = *reinterpret_cast<const v4i*>(bp + 32 * b);
      const v16i zero = {};
      const v16i j = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb, zero, 0, 0, 0);
      const float dh = dhs[b][32 * tsub + col];
      const float4* ddp = reinterpret_cast<const float4*>(&dds[b][32 * lsub + 4 * khalf]);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const float4 dd = ddp[2 * qq];  // rows 8qq + 4khalf + 0..3
        acc[4 * qq + 0] = __builtin_fmaf(dd.x, dh * (float)j[4 * qq + 0], acc[4 * qq + 0]);
        acc[4 * qq + 1] = __builtin_fmaf(dd.y, dh * (float)j[4 * qq + 1], acc[4 * qq + 1]);
        acc[4 * qq + 2] = __builtin_fmaf(dd.z, dh * (float)j[4 * qq + 2], acc[4 * qq + 2]);
        acc[4 * qq + 3] = __builtin_fmaf(dd.w, dh * (float)j[4 * qq + 3], acc[4 * qq + 3]);
      }
      if (PROBE) {
        const int p = pid[32 * tsub + col];
        if (p >= 0) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int l = l0 + 32 * lsub + 8 * (i >> 2) + 4 * khalf + (i & 3);
            const int rr = l - probe.row0;
            if (rr >= 0 && rr < probe.rows) probe.out[((int64_t)p * probe.rows + rr) * nfb + kc * 8 + b] = j[i];
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: weighted output rows into the pair's slot
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

}  // namespace

hipError_t launch_down(const uint8_t* dn, const float* router_w, const Shapes& s, const Work& w,
                       const ProbeRows* probe, hipStream_t st) {
  const dim3 grid(w.max_tiles, s.L / kLT);
  if (probe) {
    hipLaunchKernelGGL(k_down<true>, grid, dim3(256), 0, st, dn, router_w, w.perm, w.tiles, w.offsets, w.misc, s.L,
                       s.F, w.h_codes, w.h_ds, w.slots, *probe);
  } else {
    const ProbeRows none = {nullptr, 0, 0};
    hipLaunchKernelGGL(k_down<false>, grid, dim3(256), 0, st, dn, router_w, w.perm, w.tiles, w.offsets, w.misc, s.L,
                       s.F, w.h_codes, w.h_ds, w.slots, none);
  }
  return hipGetLastError();
}

}  // namespace latmoe
