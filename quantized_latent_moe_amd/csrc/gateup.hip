// Gate/up grouped GEMM with the SwiGLU + q8_1 epilogue.
//
// Page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1": gate/up reads
// Q3_K, applies SwiGLU and rounds H to q8_1 (section "Contents"); the 6-bit
// sub-block scale is multiplied into the int8 operand as (4 - code)(scale - 32)
// in [-128, 124], so one integer dot covers a whole 32-value activation block
// (lat_q3k_w11.cu commit message).
//
// Work item = (expert e, tile of up to kTileN = 128 sorted pairs, 64 features).
// A workgroup of 8 waves computes gate rows f0..f0+63 and the matching up rows
// F+f0.. against the tile's token rows; wave w owns features f0 + 32*(w&1)
// .. +31 (gate and up) and tokens 32*(w>>1) .. +31, so gate and up of each
// (feature, token) land in the same lane for SwiGLU.  A wave whose 32 tokens
// are all padding skips its MFMAs and fold.
// K (= L) is walked one Q3_K super-block (256 values) at a time, with the
// global loads of step sb+1 issued into registers before step sb computes:
//   stage   Q3_K blocks (16-bit loads: rows are only 2-byte aligned) and the
//           tokens' int8 codes (16-byte loads) and block scales into LDS;
//   unpack  2-bit + high-bit codes -> (4 - c) * sigma with one v_perm_b32 per
//           4 values against an 8-entry table built from the sub-block scale;
//   MFMA    v_mfma_i32_32x32x32_i8, one per 32-value activation block: the
//           int32 result is minus the block dot sum sigma * v * q;
//   fold    acc_sb += (-d_x[token][b]) * float(I)   (fp32, per block),
//           acc    += d_w[row][sb] * acc_sb          (once per super-block).
// Epilogue: H = G * sigmoid(G) * U, then per 32 features of a token (16 in this
// lane, 16 in lane ^ 32) the q8_1 rule: amax, d = amax/127, id = 1/d,
// q = round-half-away(H * id); codes and fp16 (d, s) go to the workspace in
// sorted order.
#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kThreads = 512;
constexpr int kFT = 64;                 // features per work item
constexpr int kRows = 2 * kFT;          // weight rows per work item (gate + up)
constexpr int kNT = kTileN;             // tokens per work item
constexpr int kRawStride = 112;         // staged Q3_K block, bytes (110 rounded up)
constexpr int kOpStride = 256 + 16;     // int8 operand row in LDS, bytes (padded)
constexpr int kRawHalf = kRows * (kQ3kBytes / 2);              // 16-bit words per step
constexpr int kRawPer = (kRawHalf + kThreads - 1) / kThreads;  // per thread
constexpr int kXPer = kNT * 16 / kThreads;                     // 16-byte code pieces per thread
constexpr int kDPer = kNT * 8 / kThreads;                      // block scales per thread
static_assert(kNT * 16 % kThreads == 0 && kNT * 8 % kThreads == 0, "staging split");
static_assert(kNT == 4 * 32, "8 waves = 2 feature halves x 4 token slices");

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(d & 0xff) << 24);
}

template <bool PROBE>
__global__ __launch_bounds__(kThreads) void k_gateup(const int8_t* __restrict__ xc, const float* __restrict__ xd,
                                                     const uint8_t* __restrict__ gu, const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ tiles,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ misc, int k, int L, int F,
                                                     int8_t* __restrict__ h_codes, uint32_t* __restrict__ h_ds,
                                                     ProbeRows probe) {
  __shared__ __align__(16) uint8_t raw[kRows * kRawStride];
  __shared__ __align__(16) int8_t As[kRows * kOpStride];
  __shared__ __align__(16) int8_t Bs[kNT * kOpStride];
  __shared__ float dws[kRows];
  __shared__ float dxs[8][kNT];
  __shared__ int32_t tok[kNT];
  __shared__ int32_t pid[kNT];

  const int tile = blockIdx.x;
  if (tile >= misc[kMiscTiles]) return;
  const int e = tiles[2 * tile];
  const int pos0 = tiles[2 * tile + 1];
  const int cnt = min(kNT, offsets[e + 1] - pos0);
  const int f0 = blockIdx.y * kFT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fsub = wave & 1, tsub = wave >> 1;
  const int nsb = L / 256, nxb = L / 32;
  const int64_t row_bytes = (int64_t)nsb * kQ3kBytes;
  const uint8_t* gu_e = gu + (int64_t)e * 2 * F * row_bytes;

  if (tid < kNT) {
    const int p = tid < cnt ? perm[pos0 + tid] : -1;
    pid[tid] = p;
    tok[tid] = p >= 0 ? p / k : -1;
  }
  __syncthreads();

  // ---- per-thread staging descriptors (the same for every super-block)
  const uint16_t* rsrc[kRawPer];
  int rdst[kRawPer];
#pragma unroll
  for (int m = 0; m < kRawPer; ++m) {
    const int i = tid + kThreads * m;
    rsrc[m] = nullptr;
    rdst[m] = -1;
    if (i < kRawHalf) {
      const int r = i / (kQ3kBytes / 2), h = i - r * (kQ3kBytes / 2);
      const int f = f0 + (r < kFT ? r : r - kFT);
      rdst[m] = r * (kRawStride / 2) + h;
      if (f < F) rsrc[m] = reinterpret_cast<const uint16_t*>(gu_e + (r < kFT ? f : F + f) * row_bytes) + h;
    }
  }
  const int8_t* xsrc[kXPer];
#pragma unroll
  for (int m = 0; m < kXPer; ++m) {
    const int piece = tid + kThreads * m, n = piece >> 4, c16 = piece & 15;
    xsrc[m] = tok[n] >= 0 ? xc + (int64_t)tok[n] * L + c16 * 16 : nullptr;
  }
  const float* dsrc[kDPer];
#pragma unroll
  for (int m = 0; m < kDPer; ++m) {
    const int q = tid + kThreads * m, n = q >> 3, b = q & 7;
    dsrc[m] = tok[n] >= 0 ? xd + (int64_t)tok[n] * nxb + b : nullptr;
  }

  uint32_t rr[kRawPer];
  uint4 rx[kXPer];
  float rd[kDPer];
  auto load = [&](int sb) {
#pragma unroll
    for (int m = 0; m < kRawPer; ++m) rr[m] = rsrc[m] ? (uint32_t)rsrc[m][sb * (kQ3kBytes / 2)] : 0u;
#pragma unroll
    for (int m = 0; m < kXPer; ++m)
      rx[m] = xsrc[m] ? *reinterpret_cast<const uint4*>(xsrc[m] + sb * 256) : uint4{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < kDPer; ++m) rd[m] = dsrc[m] ? -dsrc[m][sb * 8] : 0.f;
  };
  auto store = [&]() {
#pragma unroll
    for (int m = 0; m < kRawPer; ++m)
      if (rdst[m] >= 0) reinterpret_cast<uint16_t*>(raw)[rdst[m]] = (uint16_t)rr[m];
#pragma unroll
    for (int m = 0; m < kXPer; ++m) {
      const int piece = tid + kThreads * m, n = piece >> 4, c16 = piece & 15;
      *reinterpret_cast<uint4*>(Bs + n * kOpStride + c16 * 16) = rx[m];
    }
#pragma unroll
    for (int m = 0; m < kDPer; ++m) {
      const int q = tid + kThreads * m;
      dxs[q & 7][q >> 3] = rd[m];
    }
  };

  float accg[16], accu[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) accg[i] = accu[i] = 0.f;

  const bool active = 32 * tsub < cnt;
  const int col = lane & 31, khalf = lane >> 5;
  const int8_t* ag = As + (32 * fsub + col) * kOpStride + 16 * khalf;
  const int8_t* au = As + (kFT + 32 * fsub + col) * kOpStride + 16 * khalf;
  const int8_t* bp = Bs + (32 * tsub + col) * kOpStride + 16 * khalf;

  load(0);
  for (int sb = 0; sb < nsb; ++sb) {
    store();
    __syncthreads();
    if (sb + 1 < nsb) load(sb + 1);
    // ---- unpack: thread -> (row r, half n, pair of j) = 64 values
    {
      const int r = tid >> 2, n = (tid >> 1) & 1, jp = tid & 1;
      const uint8_t* blk = raw + r * kRawStride;
      const uint32_t* hm32 = reinterpret_cast<const uint32_t*>(blk);
      const uint32_t* qs32 = reinterpret_cast<const uint32_t*>(blk + 32);
      const uint8_t* sc = blk + 96;
      uint32_t tlo[4], thi[4];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int s = 8 * n + 4 * jp + t4;  // sub-blocks of j = 2jp (t4 = 0, 1) and 2jp + 1 (t4 = 2, 3)
        const int lo = s < 8 ? (sc[s] & 15) : (sc[s - 8] >> 4);
        const int hi = (sc[8 + (s & 3)] >> (2 * (s >> 2))) & 3;
        const int sg = (lo | (hi << 4)) - 32;
        tlo[t4] = pack4(4 * sg, 3 * sg, 2 * sg, sg);
        thi[t4] = pack4(0, -sg, -2 * sg, -3 * sg);
      }
      uint32_t* dst = reinterpret_cast<uint32_t*>(As + r * kOpStride + 128 * n);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * jp + jj;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const uint32_t q = qs32[8 * n + g];
          const uint32_t h = hm32[g];
          const uint32_t c = ((q >> (2 * j)) & 0x03030303u) | (((h >> (4 * n + j)) & 0x01010101u) << 2);
          const int sl = 2 * jj + (g >> 2);
          dst[8 * j + g] = __builtin_amdgcn_perm(thi[sl], tlo[sl], c);
        }
      }
      if ((tid & 3) == 0) dws[r] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(blk + 108));
    }
    __syncthreads();
    // ---- MFMA per 32-value block, fp32 fold
    if (active) {
      float sbg[16], sbu[16];
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const v4i va = *reinterpret_cast<const v4i*>(ag + 32 * b);
        const v4i vu = *reinterpret_cast<const v4i*>(au + 32 * b);
        const v4i vb = *reinterpret_cast<const v4i*>(bp + 32 * b);
        const v16i zero = {};
        const v16i ig = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb, zero, 0, 0, 0);
        const v16i iu = __builtin_amdgcn_mfma_i32_32x32x32_i8(vu, vb, zero, 0, 0, 0);
        const float d = dxs[b][32 * tsub + col];
        if (b == 0) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            sbg[i] = d * (float)ig[i];
            sbu[i] = d * (float)iu[i];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            sbg[i] = __builtin_fmaf(d, (float)ig[i], sbg[i]);
            sbu[i] = __builtin_fmaf(d, (float)iu[i], sbu[i]);
          }
        }
        if (PROBE) {
          const int p = pid[32 * tsub + col];
          if (p >= 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int m = 8 * (i >> 2) + 4 * khalf + (i & 3);
              const int f = f0 + 32 * fsub + m;
              if (f < F) {
                const int rg = f - probe.row0, ru = F + f - probe.row0;
                const int64_t o = (int64_t)p * probe.rows;
                if (rg >= 0 && rg < probe.rows) probe.out[(o + rg) * nxb + sb * 8 + b] = -ig[i];
                if (ru >= 0 && ru < probe.rows) probe.out[(o + ru) * nxb + sb * 8 + b] = -iu[i];
              }
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = 8 * (i >> 2) + 4 * khalf + (i & 3);
        accg[i] = __builtin_fmaf(dws[32 * fsub + m], sbg[i], accg[i]);
        accu[i] = __builtin_fmaf(dws[kFT + 32 * fsub + m], sbu[i], accu[i]);
      }
    }
    __syncthreads();
  }
  if (!active) return;

  // ---- epilogue: SwiGLU, q8_1 rounding of H per 32 features
  {
    // The q8_1 rule rounds every product to fp32 on its own (no FMA, no fused
    // multiply-convert to fp16).
#pragma clang fp contract(off)
    const int n = 32 * tsub + col;
    const int fb = f0 + 32 * fsub;  // first feature of this 32-feature block
    float h[16];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float g = accg[i];
      const float sig = 1.0f / (1.0f + __expf(-g));
      h[i] = g * sig * accu[i];
      amax = fmaxf(amax, fabsf(h[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float d = amax / 127.0f;
    const float id = d != 0.0f ? 1.0f / d : 0.0f;
    int q[16];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      q[i] = (int)__builtin_roundf(h[i] * id);
      sum += q[i];
    }
    sum += __shfl_xor(sum, 32);
    if (n < cnt && fb < F) {
      const int64_t pos = pos0 + n;
      int8_t* dst = h_codes + pos * F + fb + 4 * khalf;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        *reinterpret_cast<uint32_t*>(dst + 8 * qq) = pack4(q[4 * qq], q[4 * qq + 1], q[4 * qq + 2], q[4 * qq + 3]);
      if (khalf == 0)
        h_ds[pos * (F / 32) + fb / 32] =
            float_to_half_bits(d) | (float_to_half_bits(fp32_barrier(d * (float)sum)) << 16);
    }
  }
}

}  // namespace

hipError_t launch_gateup(const Shapes& s, const Work& w, const uint8_t* gu, const ProbeRows* probe, hipStream_t st) {
  const dim3 grid(w.max_tiles, (s.F + kFT - 1) / kFT);
  const ProbeRows none = {nullptr, 0, 0};
  if (probe)
    hipLaunchKernelGGL(k_gateup<true>, grid, dim3(kThreads), 0, st, w.xc, w.xd, gu, w.perm, w.tiles, w.offsets,
                       w.misc, s.k, s.L, s.F, w.h_codes, w.h_ds, *probe);
  else
    hipLaunchKernelGGL(k_gateup<false>, grid, dim3(kThreads), 0, st, w.xc, w.xd, gu, w.perm, w.tiles, w.offsets,
                       w.misc, s.k, s.L, s.F, w.h_codes, w.h_ds, none);
  return hipGetLastError();
}

}  // namespace latmoe
