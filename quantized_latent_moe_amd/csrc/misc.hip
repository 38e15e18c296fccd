// Combine, q8_1 rounding of fp32 rows, and debug exports.
#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kCombineUnroll = 8;  // slots per token whose loads are all issued up front

// y[t][l] = sum_{j=0..k-1, id valid} slot[t*k + j][l], slots taken in order.
// Each slot already holds router_w[t][j] * O (down epilogue).
// NT: non-temporal slot loads, for slot buffers larger than the 256 MB
// memory-side cache (measured: 147 -> 117 us at 21000 tokens, 688 MB of slots;
// with 173 MB of slots, 5268 tokens, plain loads are 1.3 us faster).
template <bool NT>
__global__ __launch_bounds__(256) void k_combine(const int32_t* __restrict__ idx, const float* __restrict__ slots,
                                                 int64_t T, int L, int E, int k, float* __restrict__ y) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one float4 of y
  const int l4 = L / 4;
  if (q >= T * l4) return;
  const int64_t t = q / l4;
  const int l = (int)(q - t * l4) * 4;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  if (k <= kCombineUnroll) {
    // All ids first, then every slot load with no branch between them (a load
    // guarded by its id would wait for that id before the next one issues):
    // a slot that is not summed loads slot row 0 instead and is dropped by
    // the select.
    typedef float v4f __attribute__((ext_vector_type(4)));
    int e[kCombineUnroll];
#pragma unroll
    for (int j = 0; j < kCombineUnroll; ++j) {
      const int v = idx[t * k + (j < k ? j : 0)];  // a load on every path: no branch
      e[j] = j < k ? v : -1;
    }
    v4f v[kCombineUnroll];
#pragma unroll
    for (int j = 0; j < kCombineUnroll; ++j) {
      const bool ok = (unsigned)e[j] < (unsigned)E;
      const v4f* src = reinterpret_cast<const v4f*>(slots + (ok ? (t * k + j) * L : 0) + l);
      v[j] = NT ? __builtin_nontemporal_load(src) : *src;
    }
#pragma unroll
    for (int j = 0; j < kCombineUnroll; ++j) {  // in slot order
      if ((unsigned)e[j] < (unsigned)E) {
        acc.x += v[j][0];
        acc.y += v[j][1];
        acc.z += v[j][2];
        acc.w += v[j][3];
      }
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if ((unsigned)e >= (unsigned)E) continue;
      const float4 v = *reinterpret_cast<const float4*>(slots + (t * k + j) * L + l);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
  }
  *reinterpret_cast<float4*>(y + t * L + l) = acc;
}

// One thread per 32-value block: amax, d = amax/127, id = 1/d, q = round(v*id)
// (half away from zero), d and s = d*sum(q) stored as fp16 (IEEE fp32 ops).
__global__ __launch_bounds__(256) void k_quantize_q8_1(const float* __restrict__ x, int64_t nblocks,
                                                       uint8_t* __restrict__ out) {
  // Every product here is rounded to fp32 on its own: no fusing into an FMA or
  // into a mixed-precision multiply-convert (fp16(d*sum) must round twice).
#pragma clang fp contract(off)
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const float4* src = reinterpret_cast<const float4*>(x + b * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 f = src[i];
    v[4 * i] = f.x;
    v[4 * i + 1] = f.y;
    v[4 * i + 2] = f.z;
    v[4 * i + 3] = f.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float d = amax / 127.0f;
  const float id = d != 0.0f ? 1.0f / d : 0.0f;
  uint32_t* dst = reinterpret_cast<uint32_t*>(out + b * kQ81Bytes);
  int sum = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const uint32_t word = pack_codes(round_half_away(v[4 * w] * id), round_half_away(v[4 * w + 1] * id),
                                     round_half_away(v[4 * w + 2] * id), round_half_away(v[4 * w + 3] * id));
    sum = __builtin_amdgcn_sdot4((int)word, 0x01010101, sum, false);
    dst[1 + w] = word;
  }
  dst[0] = float_to_half_bits(d) | (float_to_half_bits(fp32_barrier(d * (float)sum)) << 16);
}

// H from sorted order to q8_1 blocks in pair order; pairs with an invalid id
// (no sorted position) were zero-filled beforehand.
__global__ __launch_bounds__(256) void k_export_h(const int32_t* __restrict__ perm, const int32_t* __restrict__ misc,
                                                  const int8_t* __restrict__ h_codes,
                                                  const uint32_t* __restrict__ h_ds, int F,
                                                  uint8_t* __restrict__ h_out) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one block of one sorted position
  const int nfb = F / 32;
  const int64_t pos = q / nfb;
  if (pos >= misc[kMiscValid]) return;
  const int b = (int)(q - pos * nfb);
  const int64_t p = perm[pos];
  uint32_t* dst = reinterpret_cast<uint32_t*>(h_out + (p * nfb + b) * kQ81Bytes);
  const uint32_t* src = reinterpret_cast<const uint32_t*>(h_codes + pos * F + b * 32);
  dst[0] = h_ds[pos * nfb + b];
#pragma unroll
  for (int w = 0; w < 8; ++w) dst[1 + w] = src[w];
}

__global__ __launch_bounds__(256) void k_fill_zero(uint32_t* __restrict__ p, int64_t nwords) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nwords) p[i] = 0u;
}

__global__ __launch_bounds__(256) void k_copy_i32(const int32_t* __restrict__ s, int32_t* __restrict__ d, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) d[i] = s[i];
}

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_combine(const int32_t* idx, const Shapes& s, const Work& w, float* y, hipStream_t st) {
  const int64_t n = s.T * (s.L / 4);
  const bool nt = s.T * s.k * (int64_t)s.L * 4 > (int64_t(256) << 20);
  if (nt)
    hipLaunchKernelGGL(k_combine<true>, dim3(blocks_for(n)), dim3(256), 0, st, idx, w.slots, s.T, s.L, s.E, s.k, y);
  else
    hipLaunchKernelGGL(k_combine<false>, dim3(blocks_for(n)), dim3(256), 0, st, idx, w.slots, s.T, s.L, s.E, s.k, y);
  return hipGetLastError();
}

hipError_t launch_quantize_q8_1(const float* x, int64_t rows, int cols, uint8_t* out, hipStream_t st) {
  const int64_t nb = rows * (cols / 32);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_q8_1, dim3(blocks_for(nb)), dim3(256), 0, st, x, nb, out);
  return hipGetLastError();
}

hipError_t launch_export_h(const Shapes& s, const Work& w, uint8_t* h_out, hipStream_t st) {
  const int nfb = s.F / 32;
  const int64_t nwords = s.pairs() * nfb * (kQ81Bytes / 4);
  hipLaunchKernelGGL(k_fill_zero, dim3(blocks_for(nwords)), dim3(256), 0, st, reinterpret_cast<uint32_t*>(h_out),
                     nwords);
  const int64_t n = s.pairs() * nfb;
  hipLaunchKernelGGL(k_export_h, dim3(blocks_for(n)), dim3(256), 0, st, w.perm, w.misc, w.h_codes, w.h_ds, s.F,
                     h_out);
  return hipGetLastError();
}

hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_i32, dim3(blocks_for(n)), dim3(256), 0, st, src, dst, n);
  return hipGetLastError();
}

}  // namespace latmoe
