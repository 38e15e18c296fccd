// Counting sort of routed pairs by expert, on the device.
//
// The grouped GEMMs read every expert's weights in place and need the pairs
// routed to each expert together ("each expert read where it is", page "Run
// Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1", lat_q3k_w11.cu commit).
// Three passes, no host synchronisation:
//   1. per chunk of kRouteChunk pairs: LDS histogram of expert ids;
//   2. one workgroup: per-expert exclusive prefix over chunks, expert offsets,
//      and the table of (expert, token tile) work items for the GEMMs;
//   3. per chunk: stable scatter of pair ids (ascending within an expert),
//      ranks inside a wave from ballots over the id bits.
#include "lat_moe_internal.h"

namespace latmoe {
namespace {

__global__ __launch_bounds__(256) void k_route_hist(const int32_t* __restrict__ idx, int64_t n_pairs, int E,
                                                    int32_t* __restrict__ chunk_hist,
                                                    int32_t* __restrict__ chunk_bad) {
  extern __shared__ int32_t hist[];  // [E]
  __shared__ int32_t bad;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kRouteChunk;
  const int64_t end = base + kRouteChunk < n_pairs ? base + kRouteChunk : n_pairs;
  for (int64_t p = base + threadIdx.x; p < end; p += blockDim.x) {
    const int e = idx[p];
    if ((unsigned)e < (unsigned)E)
      atomicAdd(&hist[e], 1);
    else
      atomicAdd(&bad, 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_hist[(int64_t)blockIdx.x * E + e] = hist[e];
  if (threadIdx.x == 0) chunk_bad[blockIdx.x] = bad;
}

__global__ __launch_bounds__(1024) void k_route_scan(int32_t* __restrict__ chunk_hist,
                                                     const int32_t* __restrict__ chunk_bad, int nchunk, int E,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ tiles,
                                                     int32_t* __restrict__ misc) {
  __shared__ int32_t s_cnt[1024];
  __shared__ int32_t s_off[1024];
  __shared__ int32_t s_toff[1024];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int c = 0; c < nchunk; ++c) {
      const int v = chunk_hist[(int64_t)c * E + e];
      chunk_hist[(int64_t)c * E + e] = run;
      run += v;
    }
    s_cnt[e] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int off = 0, toff = 0;
    for (int e = 0; e < E; ++e) {
      s_off[e] = off;
      s_toff[e] = toff;
      offsets[e] = off;
      off += s_cnt[e];
      toff += (s_cnt[e] + kTileN - 1) / kTileN;
    }
    offsets[E] = off;
    int bad = 0;
    for (int c = 0; c < nchunk; ++c) bad += chunk_bad[c];
    misc[kMiscTiles] = toff;
    misc[kMiscDropped] = bad;
    misc[kMiscValid] = off;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int nt = (s_cnt[e] + kTileN - 1) / kTileN;
    for (int i = 0; i < nt; ++i) {
      const int slot = s_toff[e] + i;
      tiles[2 * slot] = e;
      tiles[2 * slot + 1] = s_off[e] + i * kTileN;
    }
  }
}

__global__ __launch_bounds__(256) void k_route_scatter(const int32_t* __restrict__ idx, int64_t n_pairs, int E,
                                                       int nbits, const int32_t* __restrict__ chunk_prefix,
                                                       const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm) {
  extern __shared__ int32_t sm[];  // base[E] | wave_count[4][E]
  int32_t* base = sm;
  int32_t* wcnt = sm + E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    base[e] = offsets[e] + chunk_prefix[(int64_t)blockIdx.x * E + e];
    for (int w = 0; w < 4; ++w) wcnt[w * E + e] = 0;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t cbase = (int64_t)blockIdx.x * kRouteChunk;
  for (int r = 0; r < kRouteChunk / 256; ++r) {
    const int64_t p = cbase + r * 256 + threadIdx.x;
    const int e = p < n_pairs ? idx[p] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & below);
    const int cnt = __popcll(same);
    const bool leader = valid && rank == 0;
    if (leader) wcnt[wave * E + e] = cnt;
    __syncthreads();
    if (valid) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += wcnt[w * E + e];
      perm[base[e] + before + rank] = (int32_t)p;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&base[e], cnt);
      wcnt[wave * E + e] = 0;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_route(const int32_t* idx, const Shapes& s, const Work& w, hipStream_t st) {
  const int64_t n = s.pairs();
  int nbits = 0;
  while ((1 << nbits) < s.E) ++nbits;
  hipLaunchKernelGGL(k_route_hist, dim3(w.nchunk), dim3(256), s.E * sizeof(int32_t), st, idx, n, s.E,
                     w.chunk_hist, w.chunk_bad);
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, st, w.chunk_hist, w.chunk_bad, w.nchunk, s.E, w.offsets,
                     w.tiles, w.misc);
  hipLaunchKernelGGL(k_route_scatter, dim3(w.nchunk), dim3(256), 5 * s.E * sizeof(int32_t), st, idx, n, s.E, nbits,
                     w.chunk_hist, w.offsets, w.perm);
  return hipGetLastError();
}

}  // namespace latmoe
