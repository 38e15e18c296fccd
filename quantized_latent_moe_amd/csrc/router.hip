// Router: softmax over the experts, top-k, weights renormalised over the picks.
//
// Page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1", section
// "Contents", and the HIP backend page: the MoE router picks each token's top
// experts and the stage combines their outputs with the router's weights; the
// rule is softmax over E, the k largest probabilities, renormalised.
//
// The weights renormalised over the picks are the softmax of the k picked
// logits alone (the full denominator cancels), and softmax ranks experts as
// their logits do, so no exp over all E is needed:
//   picks: the k largest logits, equal logits in ascending expert order;
//   w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max) over the picks (fp32).
//
// Up to 256 experts and 16 picks, from 256 tokens: a 16-lane row per token,
// four tokens a wave (k_router_topk16, below).  Otherwise one wave per token
// (at a few tokens the rounds' latency, not the wave count, sets the time,
// and a wave per token has the shorter chain).  Lane l
// holds logits l, l + 64, ... in registers (as
// many slots as E needs, by instantiation).  Each
// of the k rounds takes every lane's best remaining logit (ascending index,
// strict compare, so ties keep the lower expert), reduces (value, index)
// across the wave with the same tie rule (DPP steps in the VALU, not LDS
// permutes), and the owning lane marks its entry taken.  Lane j keeps pick
// j; the k exponentials are summed across the wave and every lane divides by
// lane 0's sum.
#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kRouterWaves = 4;  // tokens per workgroup

// (value, index) of the better of two candidates: larger value, then lower index.
__device__ __forceinline__ void better(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

// One DPP step of the wave reduction: combine with the lane the control word
// selects (rows outside row_mask keep their own pair).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_step(float& v, int& i) {
  const int vb = __builtin_bit_cast(int, v);
  const float ov = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(vb, vb, CTRL, ROW_MASK, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROW_MASK, 0xF, false);
  better(v, i, ov, oi);
}

// Wave-wide best (value, index), returned to every lane: DPP within the VALU
// (quad swaps, half-row and row mirrors, row broadcasts 15 and 31) leaves the
// result in lane 63, read back as a scalar.
__device__ __forceinline__ void wave_best(float& v, int& i) {
  dpp_step<0xB1, 0xF>(v, i);   // quad_perm [1,0,3,2]
  dpp_step<0x4E, 0xF>(v, i);   // quad_perm [2,3,0,1]
  dpp_step<0x141, 0xF>(v, i);  // row_half_mirror
  dpp_step<0x140, 0xF>(v, i);  // row_mirror
  dpp_step<0x142, 0xA>(v, i);  // row_bcast:15 into rows 1 and 3
  dpp_step<0x143, 0xC>(v, i);  // row_bcast:31 into rows 2 and 3
  v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

// P: logits per lane (E <= 64 P).
template <int P>
__global__ __launch_bounds__(64 * kRouterWaves) void k_router_topk(const float* __restrict__ logits, int64_t T,
                                                                    int E, int k, int32_t* __restrict__ idx,
                                                                    float* __restrict__ w) {
  constexpr int kPerLane = P;
  const int lane = threadIdx.x & 63;
  // the wave's token, read as wave-uniform so that its buffer descriptor is scalar
  const int64_t t = (int64_t)blockIdx.x * kRouterWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;
  const rsrc_t rl = make_rsrc(logits + t * E, (uint32_t)E * 4);
  float v[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = lane + 64 * i;
    const float x = as_float((int)buf_u32(rl, e < E ? 4 * e : kOutOfRange, 0));
    v[i] = e < E ? x : -INFINITY;
  }
  uint32_t taken = 0;  // bit i: entry i of this lane already picked (or past E)
#pragma unroll
  for (int i = 0; i < kPerLane; ++i)
    if (lane + 64 * i >= E) taken |= 1u << i;

  int my_idx = 0;
  float my_val = -INFINITY;
  for (int j = 0; j < k; ++j) {
    // this lane's best remaining entry (ascending index, strict compare)
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const bool free_i = !((taken >> i) & 1u);
      if (free_i && (v[i] > bv || bi == 0x7fffffff)) {
        bv = v[i];
        bi = lane + 64 * i;
      }
    }
    // wave argmax with the same tie rule (bi, bv now wave-uniform)
    wave_best(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) {
      my_idx = bi;
      my_val = bv;
    }
  }
  // weights: softmax of the picked logits (lane 0 holds the largest)
  const float top = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_val), 0));
  float ex = lane < k ? expf(my_val - top) : 0.f;
  float sum = ex;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) sum += __shfl_xor(sum, m);
  sum = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum), 0));  // one sum for all
  if (lane < k) {
    idx[t * k + lane] = my_idx;
    w[t * k + lane] = ex / sum;
  }
}

// The same rule for E <= 256 and k <= 16 with a 16-lane row (a DPP row) per
// token, four tokens a wave: lane l of a row holds logits l, l + 16, ...; the
// row's best (value, index) comes from four DPP steps that leave it in every
// lane of the row (quad swaps, half-row and row mirrors), so a round needs no
// readlane, and a wave's rounds serve four tokens.  Lane j of a row keeps pick
// j; the k exponentials are summed by the same four steps (every lane of the
// row ends with the same sum, bit for bit).
template <int P>
__global__ __launch_bounds__(64 * kRouterWaves) void k_router_topk16(const float* __restrict__ logits, int64_t T,
                                                                      int E, int k, int32_t* __restrict__ idx,
                                                                      float* __restrict__ w) {
  const int lane = threadIdx.x & 63, rl = lane & 15;
  const int64_t t0 = ((int64_t)blockIdx.x * kRouterWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * 4;
  if (t0 >= T) return;
  const int64_t t = t0 + (lane >> 4);
  const bool live = t < T;
  // one descriptor for the wave's (up to) four logit rows, so that it is
  // scalar; a row past T lies beyond num_records and loads zeros
  const int nlive = T - t0 < 4 ? (int)(T - t0) : 4;
  const rsrc_t rlg = make_rsrc(logits + t0 * E, (uint32_t)(nlive * E) * 4u);
  const int row0 = (lane >> 4) * E;
  float v[P];
  uint32_t taken = 0;  // bit i: entry i of this lane already picked (or past E)
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int e = rl + 16 * i;
    v[i] = as_float((int)buf_u32(rlg, e < E ? 4 * (row0 + e) : kOutOfRange, 0));
    if (e >= E) {
      v[i] = -INFINITY;
      taken |= 1u << i;
    }
  }
  int my_idx = 0;
  float my_val = -INFINITY, top = -INFINITY;
  for (int j = 0; j < k; ++j) {
    // this lane's best remaining entry (ascending index, strict compare)
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const bool free_i = !((taken >> i) & 1u);
      if (free_i && (v[i] > bv || bi == 0x7fffffff)) {
        bv = v[i];
        bi = rl + 16 * i;
      }
    }
    dpp_step<0xB1, 0xF>(bv, bi);   // quad_perm [1,0,3,2]
    dpp_step<0x4E, 0xF>(bv, bi);   // quad_perm [2,3,0,1]
    dpp_step<0x141, 0xF>(bv, bi);  // row_half_mirror
    dpp_step<0x140, 0xF>(bv, bi);  // row_mirror: every lane of the row holds the row's best
    if ((bi & 15) == rl) taken |= 1u << (bi >> 4);
    if (j == 0) top = bv;
    if (rl == j) {
      my_idx = bi;
      my_val = bv;
    }
  }
  // weights: softmax of the picked logits (pick 0 is the largest)
  float ex = rl < k ? expf(my_val - top) : 0.f;
  float sum = ex;
  sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, sum), __builtin_bit_cast(int, sum), 0xB1, 0xF, 0xF, false));
  sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, sum), __builtin_bit_cast(int, sum), 0x4E, 0xF, 0xF, false));
  sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, sum), __builtin_bit_cast(int, sum), 0x141, 0xF, 0xF, false));
  sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, sum), __builtin_bit_cast(int, sum), 0x140, 0xF, 0xF, false));
  if (live && rl < k) {
    idx[t * k + rl] = my_idx;
    w[t * k + rl] = ex / sum;
  }
}

}  // namespace

hipError_t launch_router_topk(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w, hipStream_t st) {
  const dim3 block(64 * kRouterWaves);
  if (E <= 256 && k <= 16 && T >= 256) {  // four tokens a wave (fewer tokens: more waves, each with a shorter chain)
    const dim3 grid16((unsigned)((T + 4 * kRouterWaves - 1) / (4 * kRouterWaves)));
    if (E <= 16) hipLaunchKernelGGL(k_router_topk16<1>, grid16, block, 0, st, logits, T, E, k, idx, w);
    else if (E <= 32) hipLaunchKernelGGL(k_router_topk16<2>, grid16, block, 0, st, logits, T, E, k, idx, w);
    else if (E <= 64) hipLaunchKernelGGL(k_router_topk16<4>, grid16, block, 0, st, logits, T, E, k, idx, w);
    else if (E <= 128) hipLaunchKernelGGL(k_router_topk16<8>, grid16, block, 0, st, logits, T, E, k, idx, w);
    else hipLaunchKernelGGL(k_router_topk16<16>, grid16, block, 0, st, logits, T, E, k, idx, w);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((T + kRouterWaves - 1) / kRouterWaves));
  if (E <= 64) hipLaunchKernelGGL(k_router_topk<1>, grid, block, 0, st, logits, T, E, k, idx, w);
  else if (E <= 128) hipLaunchKernelGGL(k_router_topk<2>, grid, block, 0, st, logits, T, E, k, idx, w);
  else if (E <= 256) hipLaunchKernelGGL(k_router_topk<4>, grid, block, 0, st, logits, T, E, k, idx, w);
  else if (E <= 512) hipLaunchKernelGGL(k_router_topk<8>, grid, block, 0, st, logits, T, E, k, idx, w);
  else hipLaunchKernelGGL(k_router_topk<16>, grid, block, 0, st, logits, T, E, k, idx, w);
  static_assert(LAT_MOE_ROUTER_MAX_E <= 64 * 16, "the largest instantiation covers the router's E");
  return hipGetLastError();
}

}  // namespace latmoe
