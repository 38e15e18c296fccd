// Gate/up grouped GEMM with the SwiGLU + q8_1 epilogue.
//
// Page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1": gate/up reads
// Q3_K, applies SwiGLU and rounds H to q8_1 (section "Contents"); the 6-bit
// sub-block scale is multiplied into the int8 operand as (4 - code)(scale - 32)
// in [-128, 124], so one integer dot covers a whole 32-value activation block
// (lat_q3k_w11.cu commit message).
//
// Persistent kernel: one workgroup of 8 waves per CU walks the work items
// (token tile of up to kTileN = 128 sorted pairs, 64 features) round-robin:
// item i = tile * nft + feature tile, workgroup w takes w, w + G, w + 2G, ...
// With G a multiple of the feature-tile count a workgroup keeps one feature
// tile, and since workgroups are dealt to the 8 XCDs round-robin, each XCD's
// L2 serves a fixed subset of every expert's rows.
// Wave w owns the gate and the up 32x32 tile of features f0 + 32*(w&1) .. +31
// and tokens 32*(w>>1) .. +31: both MFMAs share the activation fragment, and
// gate and up of each (feature, token) meet in one lane for SwiGLU.  A wave
// whose 32 tokens are all padding skips its MFMAs and fold.
//
// K (= L) is walked one Q3_K super-block (256 values) per step; the steps of
// all the workgroup's items form one pipeline, two barriers per step:
//   L(g)  global loads of step g into registers (issued two steps ahead):
//         Q3_K blocks as 16-bit words (rows are only 2-byte aligned; lanes
//         read consecutive words, 56 per block of which the last is an
//         out-of-range load), the tokens' int8 codes (16-byte loads) and fp32
//         block scales, all through buffer loads whose out-of-range offset
//         returns zeros for padding;
//   S(g)  those registers into LDS (raw blocks, operand B, scales);
//   U(g)  unpack: per (row, half, j) 32 codes from 16-byte LDS reads,
//         (4 - c) * sigma with one v_perm_b32 per 4 values against an 8-entry
//         table built from the sub-block scale, 16-byte writes to operand A;
//   M(g)  v_mfma_i32_32x32x32_i8 per 32-value block with the accumulator
//         initialised to the bits of 1.5 * 2^23, so each result (minus the
//         block dot) reads as the float 1.5 * 2^23 - I32 with no conversion;
//         t = fma(-d_x, f, 1.5 * 2^23 * d_x) is exactly fl(d_x * I32) (the
//         constant has at most 13 significant bits), acc_sb += t, and once per
//         super-block acc += d_w[row][sb] * acc_sb.
// Step g's iteration runs S(g+1) | barrier | L(g+2), U(g+1), M(g) | barrier,
// with operands A and B double-buffered, so the unpack of the next step and
// this step's MFMA + fold interleave.
// Epilogue (after an item's last step): H = G * sigmoid(G) * U, then per 32
// features of a token (16 in this lane, 16 in lane ^ 32) the q8_1 rule: amax,
// d = amax/127, id = 1/d, q = round-half-away(H * id) with IEEE divisions;
// codes and fp16 (d, s) go to the workspace in sorted order.
#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kThreads = 512;
constexpr int kFT = 64;              // features per work item
constexpr int kRows = 2 * kFT;       // weight rows per work item (gate + up)
constexpr int kNT = kTileN;          // tokens per work item
constexpr int kRawStride = 112;      // staged Q3_K block, bytes (110 rounded up to 16)
constexpr int kOpStride = 256 + 16;  // int8 operand row in LDS (bytes); 16 mod 256: conflict-free b128
constexpr int kWords = kQ3kBytes / 2;               // 55 16-bit words per block
constexpr int kSlots = kRawStride / 2;              // 56 staged words per block (the last one reads as 0)
constexpr int kRawPer = kRows * kSlots / kThreads;  // 14
static_assert(kRows * kSlots % kThreads == 0, "raw staging split");
constexpr int kXPer = kNT * 16 / kThreads;                      // 16-byte code pieces per thread (4)
constexpr int kDPer = kNT * 8 / kThreads;                       // block scales per thread (2)
static_assert(kNT * 16 % kThreads == 0 && kNT * 8 % kThreads == 0, "staging split");
static_assert(kRows * 8 == 2 * kThreads, "unpack split: two (row, half, j) tasks per thread");
static_assert(kNT == 4 * 32 && kFT == 2 * 32, "8 waves = 2 feature halves x 4 token slices");

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(d & 0xff) << 24);
}

struct Item {
  int e, pos0, cnt, f0;
};

__device__ __forceinline__ Item item_info(int i, int nft, const int32_t* tiles, const int32_t* offsets) {
  Item it;
  const int tile = i / nft;
  it.f0 = (i - tile * nft) * kFT;
  it.e = tiles[2 * tile];
  it.pos0 = tiles[2 * tile + 1];
  it.cnt = min(kNT, offsets[it.e + 1] - it.pos0);
  return it;
}

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
  __shared__ int32_t ids[2][kNT];  // pair ids (or -1) of the loader's next items

  const int nft = (F + kFT - 1) / kFT;
  const int n_items = misc[kMiscTiles] * nft;
  const int G = gridDim.x;
  if ((int)blockIdx.x >= n_items) return;
  const int my_items = (n_items - 1 - (int)blockIdx.x) / G + 1;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fsub = wave & 1, tsub = wave >> 1;
  const int nsb = L / 256, nxb = L / 32;
  const int row_bytes = nsb * kQ3kBytes;
  const int n_steps = my_items * nsb;
  const int col = lane & 31, khalf = lane >> 5;

  // ---- loader: walks (item, super-block) two steps ahead of the MFMAs.
  // Offsets are fixed per item (the super-block goes into the scalar offset);
  // rows past F and padding tokens get an out-of-range offset.  The pair ids
  // of the loader's next item are fetched into LDS one item ahead (read after
  // at least one barrier).
  const rsrc_t rx_src = make_rsrc(xc, (uint32_t)(T * L));
  const rsrc_t rd_src = make_rsrc(xd, (uint32_t)(T * nxb * 4));
  rsrc_t rw_src;
  int qoff[kRawPer], xoff[kXPer], doff[kDPer];
  int lj = 0, lsb = 0;
  auto fetch_ids = [&](int j) {
    if (j < my_items) {
      const Item it = item_info((int)blockIdx.x + j * G, nft, tiles, offsets);
      if (tid < kNT) ids[j & 1][tid] = tid < it.cnt ? perm[it.pos0 + tid] : -1;
    }
  };
  auto setup = [&](int j) {
    const Item it = item_info((int)blockIdx.x + j * G, nft, tiles, offsets);
    const int e = __builtin_amdgcn_readfirstlane(it.e);  // uniform: the descriptor lives in SGPRs
    rw_src = make_rsrc(gu + (int64_t)e * 2 * F * row_bytes, (uint32_t)(2 * F * row_bytes));
#pragma unroll
    for (int m = 0; m < kRawPer; ++m) {
      const int i = tid + kThreads * m;
      const int r = i / kSlots, w = i - r * kSlots;
      const int rl = r < kFT ? r : r - kFT;
      const int row = (r < kFT ? 0 : F) + it.f0 + rl;
      qoff[m] = (w < kWords && it.f0 + rl < F) ? row * row_bytes + 2 * w : kOutOfRange;
    }
#pragma unroll
    for (int m = 0; m < kXPer; ++m) {
      const int p = ids[j & 1][(tid + kThreads * m) >> 4];
      xoff[m] = p >= 0 ? (p / k) * L + (tid & 15) * 16 : kOutOfRange;
    }
#pragma unroll
    for (int m = 0; m < kDPer; ++m) {
      const int p = ids[j & 1][(tid + kThreads * m) >> 3];
      doff[m] = p >= 0 ? ((p / k) * nxb + (tid & 7)) * 4 : kOutOfRange;
    }
    fetch_ids(j + 1);
  };
  uint32_t rq[kRawPer];
  uint4 rx[kXPer];
  uint32_t rd[kDPer];
  // L: sets up a new item when the loader enters one, then only moves bits
  // into registers (arithmetic on a loaded value would make the compiler wait
  // for it) and advances the loader.
  bool need_setup = true;
  auto load_next = [&]() {
    if (need_setup) {
      setup(lj);  // reads the ids fetch_ids(lj) wrote at least one barrier ago
      need_setup = false;
    }
    // scalar offsets (readfirstlane keeps them in SGPRs, as the buffer loads need)
    const int sq = __builtin_amdgcn_readfirstlane(lsb * kQ3kBytes);
    const int sx = __builtin_amdgcn_readfirstlane(lsb * 256);
    const int sd = __builtin_amdgcn_readfirstlane(lsb * 32);
#pragma unroll
    for (int m = 0; m < kRawPer; ++m) rq[m] = buf_u16(rw_src, qoff[m], sq);
#pragma unroll
    for (int m = 0; m < kXPer; ++m) rx[m] = buf_u128(rx_src, xoff[m], sx);
#pragma unroll
    for (int m = 0; m < kDPer; ++m) rd[m] = buf_u32(rd_src, doff[m], sd);
    if (++lsb == nsb) {
      lsb = 0;
      need_setup = ++lj < my_items;
    }
  };
  // S: registers -> LDS buffer b.
  auto store = [&](int b) {
#pragma unroll
    for (int m = 0; m < kRawPer; ++m) reinterpret_cast<uint16_t*>(raw)[tid + kThreads * m] = (uint16_t)rq[m];
#pragma unroll
    for (int m = 0; m < kXPer; ++m) {
      const int piece = tid + kThreads * m;
      *reinterpret_cast<uint4*>(Bs[b] + (piece >> 4) * kOpStride + (piece & 15) * 16) = rx[m];
    }
#pragma unroll
    for (int m = 0; m < kDPer; ++m) dxs[b][tid + kThreads * m] = -as_float((int)rd[m]);  // minus: operand A is -w
  };
  // U: raw -> operand A of buffer b, row scales -> dws[b].
  auto unpack = [&](int b) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int task = tid + kThreads * u;
      const int ur = task & (kRows - 1), uq = task >> 7, un = uq >> 2, uj = uq & 3;
      const uint8_t* ublk = raw + ur * kRawStride;
      const uint4 h0 = *reinterpret_cast<const uint4*>(ublk);
      const uint4 h1 = *reinterpret_cast<const uint4*>(ublk + 16);
      const uint4 q0 = *reinterpret_cast<const uint4*>(ublk + 32 + 32 * un);
      const uint4 q1 = *reinterpret_cast<const uint4*>(ublk + 48 + 32 * un);
      const uint4 scw = *reinterpret_cast<const uint4*>(ublk + 96);  // scales[12] | d | pad
      const uint32_t hm[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
      const uint32_t qs[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const uint32_t scb[3] = {scw.x, scw.y, scw.z};
      uint32_t tlo[2], thi[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int s = 8 * un + 2 * uj + t;
        const int sl = s & 7;
        const int lo = (int)((scb[sl >> 2] >> (8 * (sl & 3) + (s < 8 ? 0 : 4))) & 15u);
        const int hi = (int)((scb[2] >> (8 * (s & 3) + 2 * (s >> 2))) & 3u);
        const int sg = (lo | (hi << 4)) - 32;
        tlo[t] = pack4(4 * sg, 3 * sg, 2 * sg, sg);
        thi[t] = pack4(0, -sg, -2 * sg, -3 * sg);
      }
      const int qshift = 2 * uj;       // low two bits of element 128un + 32uj + l: bit 2uj of qs[l]
      const int hs = 4 * un + uj - 2;  // its high bit (bit 4un + uj of hmask[l]) moves to bit 2
      uint32_t o[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const uint32_t hb = (hs >= 0 ? (hm[g] >> hs) : (hm[g] << -hs)) & 0x04040404u;
        const uint32_t c = ((qs[g] >> qshift) & 0x03030303u) | hb;
        o[g] = __builtin_amdgcn_perm(thi[g >> 2], tlo[g >> 2], c);
      }
      uint4* udst = reinterpret_cast<uint4*>(As[b] + ur * kOpStride + 128 * un + 32 * uj);
      udst[0] = uint4{o[0], o[1], o[2], o[3]};
      udst[1] = uint4{o[4], o[5], o[6], o[7]};
      if (uq == 0) dws[b][ur] = half_bits_to_float(scw.w & 0xffffu);
    }
  };

  v16i magic;
#pragma unroll
  for (int i = 0; i < 16; ++i) magic[i] = kMagicBits;
  float accg[16], accu[16];

  // ---- prologue: L(0), S(0), U(0), L(1)
  fetch_ids(0);
  __syncthreads();
  load_next();
  store(0);
  __syncthreads();
  if (n_steps > 1) load_next();
  unpack(0);
  __syncthreads();

  int cj = 0, csb = 0;  // item index and super-block of the MFMA step
  Item cur = item_info((int)blockIdx.x, nft, tiles, offsets);
  for (int g = 0; g < n_steps; ++g) {
    const int b = g & 1;
    if (g + 1 < n_steps) store(b ^ 1);
    __syncthreads();
    if (g + 2 < n_steps) load_next();
    if (g + 1 < n_steps) unpack(b ^ 1);

    // ---- M(g): MFMA per 32-value block, fp32 fold
    const bool active = 32 * tsub < cur.cnt;
    if (csb == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) accg[i] = accu[i] = 0.f;
    }
    if (active) {
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
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const v4i va = *reinterpret_cast<const v4i*>(ag + 32 * kb);
        const v4i vu = *reinterpret_cast<const v4i*>(au + 32 * kb);
        const v4i vb = *reinterpret_cast<const v4i*>(bp + 32 * kb);
        const v16i ig = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, vb, magic, 0, 0, 0);
        const v16i iu = __builtin_amdgcn_mfma_i32_32x32x32_i8(vu, vb, magic, 0, 0, 0);
        const float d = dxv[kb];
        const float c = -kMagic * d;  // exact
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float tg = __builtin_fmaf(d, as_float(ig[i]), c);  // fl(d_x * I32)
          const float tu = __builtin_fmaf(d, as_float(iu[i]), c);
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
    }

    if (++csb == nsb) {
      // ---- epilogue of item cj: SwiGLU, q8_1 rounding of H per 32 features
      if (active) {
        // The q8_1 rule rounds every product to fp32 on its own (no FMA, no
        // fused multiply-convert to fp16).
#pragma clang fp contract(off)
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
        int q[16];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          q[i] = (int)__builtin_roundf(h[i] * id);
          sum += q[i];
        }
        sum += __shfl_xor(sum, 32);
        if (n < cur.cnt && fb < F) {
          const int64_t pos = cur.pos0 + n;
          int8_t* dst = h_codes + pos * F + fb + 4 * khalf;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            *reinterpret_cast<uint32_t*>(dst + 8 * qq) =
                pack4(q[4 * qq], q[4 * qq + 1], q[4 * qq + 2], q[4 * qq + 3]);
          if (khalf == 0)
            h_ds[pos * (F / 32) + fb / 32] =
                float_to_half_bits(d) | (float_to_half_bits(fp32_barrier(d * (float)sum)) << 16);
        }
      }
      csb = 0;
      if (++cj < my_items) cur = item_info((int)blockIdx.x + cj * G, nft, tiles, offsets);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_gateup(const Shapes& s, const Work& w, const uint8_t* gu, const ProbeRows* probe, hipStream_t st) {
  // One persistent workgroup per CU, rounded down to a multiple of the feature
  // tile count (so each workgroup keeps one feature tile) when that is possible.
  const int nft = (s.F + kFT - 1) / kFT;
  int grid = w.num_cus;
  if (grid >= nft) grid -= grid % nft;
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
