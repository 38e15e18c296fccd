// Counting sort of routed pairs by expert, on the device.
//
// The grouped GEMMs read each expert's weights in place (page "Run
// Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1", lat_q3k_w11.cu commit
// message), so the pairs routed to one expert have to sit together.
// Result: perm (pair ids grouped by expert, ascending within an expert),
// offsets[E+1], the table of (expert, first position, pairs) token tiles of
// kTileN pairs, and the dropped / valid / tile counts.  No host
// synchronisation.
//
// Up to kSmallPairs pairs: one workgroup does everything (per-wave running
// counts by expert, block scan, tile table, stable scatter).  Larger: three
// passes over chunks of kRouteChunk pairs (per-chunk histograms; one
// workgroup scanning chunks and experts; per-chunk stable scatter).  In both
// the first launch carries extra workgroups that split the q8_1 activations
// into int8 codes and fp32 scales (independent work, one launch fewer), and,
// for the combine by atomic adds, workgroups that zero y.
// Stable ranks inside a wave come from ballots over the bits of the id.
#include "lat_moe_internal.h"

namespace latmoe {
namespace {

constexpr int kSmallPairs = 4096;
constexpr int kScanStage = 32768;  // chunk-histogram entries the scan stages in LDS (128 KB)
constexpr int kSplitPerBlock = 1024;  // q8_1 blocks split per extra workgroup
constexpr int kRouteThreads = 256;    // threads of the histogram and scatter workgroups

// q8_1 block sb -> 32 codes at xc + 32 db and the fp32 scale xd[db].
// Split in two halves, so a thread can have several blocks' loads in flight
// before it stores any of them.
struct Q81Words {
  uint32_t w[kQ81Bytes / 4];
};
__device__ __forceinline__ Q81Words load_q81(const uint8_t* __restrict__ x, int64_t sb) {
  const uint32_t* src = reinterpret_cast<const uint32_t*>(x + sb * kQ81Bytes);
  Q81Words r;
#pragma unroll
  for (int i = 0; i < kQ81Bytes / 4; ++i) r.w[i] = src[i];
  return r;
}
__device__ __forceinline__ void store_split(const Q81Words& r, int64_t db, int8_t* __restrict__ xc,
                                            float* __restrict__ xd) {
  uint4* dst = reinterpret_cast<uint4*>(xc + db * 32);
  dst[0] = uint4{r.w[1], r.w[2], r.w[3], r.w[4]};
  dst[1] = uint4{r.w[5], r.w[6], r.w[7], r.w[8]};
  xd[db] = half_bits_to_float(r.w[0] & 0xffffu);
}

// Zeroes floats [i0, i0 + kZeroPerBlock) of y (clipped to n): the extra
// workgroups of the first route launch clear y for the down kernel's atomic
// adds.  float4 stores; n is a multiple of 4 (L % 256 == 0).
constexpr int kZeroPerBlock = 16384;
__device__ __forceinline__ void zero_chunk(float* __restrict__ y, int64_t n, int64_t i0) {
  for (int64_t i = i0 + 4 * (int64_t)threadIdx.x; i < i0 + kZeroPerBlock && i < n; i += 4 * (int64_t)blockDim.x)
    *reinterpret_cast<float4*>(y + i) = float4{0.f, 0.f, 0.f, 0.f};
}

// Exclusive prefix sum over the workgroup (blockDim.x a multiple of 64, at
// most 1024); *total receives the sum.  scratch: 16 ints of LDS.
__device__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int s = lane < nw ? scratch[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int y = __shfl_up(s, d);
      if (lane >= d) s += y;
    }
    if (lane < nw) scratch[lane] = s;
  }
  __syncthreads();
  const int before = wave > 0 ? scratch[wave - 1] : 0;
  *total = scratch[nw - 1];
  __syncthreads();  // scratch may be reused right after
  return before + x - v;
}

// Offsets, tile table and counts from per-expert totals cnt[e] (e < E <=
// blockDim.x = 1024, in LDS); leaves each expert's first position in
// first[e] and its first tile in tstart[e].  Every thread of the workgroup
// calls it.  The tile table is written by all threads, a tile each in turn
// (a busy expert has hundreds of tiles: one thread would issue them all).
__device__ void finish_offsets(const int* cnt, int* first, int* tstart, int E, int bad, int32_t* __restrict__ offsets,
                               int32_t* __restrict__ tiles, int32_t* __restrict__ misc, int* scratch) {
  const int e = threadIdx.x;
  const int c = e < E ? cnt[e] : 0;
  const int nt = (c + kTileN - 1) / kTileN;
  int total, ttotal;
  const int off = block_exclusive_scan(c, scratch, &total);
  const int toff = block_exclusive_scan(nt, scratch, &ttotal);
  if (e < E) {
    first[e] = off;
    tstart[e] = toff;
    offsets[e] = off;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < ttotal; q += blockDim.x) {
    // the tile's expert: the last e with tstart[e] <= q (experts without
    // tiles share their start with the next one, so the last has tiles)
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tstart[mid] <= q) lo = mid; else hi = mid - 1;
    }
    const int i = q - tstart[lo];
    int32_t* te = tiles + kTileWords * q;
    te[0] = lo;
    te[1] = first[lo] + i * kTileN;
    te[2] = min(kTileN, cnt[lo] - i * kTileN);
    te[3] = 0;
  }
  if (threadIdx.x == 0) {
    offsets[E] = total;
    misc[kMiscTiles] = ttotal;
    misc[kMiscDropped] = bad;
    misc[kMiscValid] = total;
  }
}

// Stable ranks of this wave's lanes among lanes with the same id; returns
// the rank and sets *cnt to the number of such lanes (0 for invalid ids).
__device__ __forceinline__ int wave_rank(int e, bool valid, int nbits, int* cnt) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  uint64_t same = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(bit);
    same &= bit ? m : ~m;
  }
  *cnt = valid ? __popcll(same) : 0;
  return __popcll(same & below);
}

// ---- small batches: everything in workgroup 0; workgroups 1 .. xblocks
// split x, the ones after them zero y (atomic combine).
//
// Wave w takes pairs [256 w, 256 w + 256) in 4 rounds of 64: the stable rank
// of a pair among the earlier pairs of its expert inside its wave's range is
// the wave's running count of that expert (wcnt[w][e], in LDS, touched only
// by wave w) plus its rank by ballot in the round.  After one barrier, one
// thread per expert turns the 16 running counts into the first position of
// each wave's run (expert offset + counts of the earlier waves), and each
// pair lands at that position plus its rank.  6 barriers in all.
constexpr int kSmallWaves = 16, kSmallRounds = kSmallPairs / (64 * kSmallWaves);  // 4 rounds of 64 per wave
static_assert(kSmallRounds * 64 * kSmallWaves == kSmallPairs, "small route split");

// Offsets, tile table and counts from per-expert totals c (thread e < E <=
// blockDim.x): finish_offsets with one block scan over (count | tiles << 16),
// which cannot carry at n <= kSmallPairs.  Returns expert e's first position.
__device__ int finish_offsets_small(int c, int E, int bad, int32_t* __restrict__ offsets, int32_t* __restrict__ tiles,
                                    int32_t* __restrict__ misc, int* scratch) {
  static_assert(kSmallPairs < (1 << 16) && 1024 + kSmallPairs / kTileN < (1 << 15), "packed scan without carries");
  const int e = threadIdx.x;
  const int nt = (c + kTileN - 1) / kTileN;
  int total;
  const int packed = block_exclusive_scan(c | (nt << 16), scratch, &total);
  const int off = packed & 0xffff, toff = packed >> 16;
  if (e < E) {
    offsets[e] = off;
    for (int i = 0; i < nt; ++i) {
      int32_t* te = tiles + kTileWords * (toff + i);
      te[0] = e;
      te[1] = off + i * kTileN;
      te[2] = min(kTileN, c - i * kTileN);
      te[3] = 0;
    }
  }
  if (threadIdx.x == 0) {
    offsets[E] = total & 0xffff;
    misc[kMiscTiles] = total >> 16;
    misc[kMiscDropped] = bad;
    misc[kMiscValid] = total & 0xffff;
  }
  return off;
}

__global__ __launch_bounds__(1024) void k_route_small(const int32_t* __restrict__ idx, int n, int E, int nbits,
                                                      int32_t* __restrict__ offsets, int32_t* __restrict__ tiles,
                                                      int32_t* __restrict__ misc, int32_t* __restrict__ perm,
                                                      const uint8_t* __restrict__ x, int64_t nxb,
                                                      int8_t* __restrict__ xc, float* __restrict__ xd, int xblocks,
                                                      float* __restrict__ yzero, int64_t ny) {
  if (blockIdx.x > 0) {
    if ((int)blockIdx.x > xblocks) {  // y for the atomic combine
      zero_chunk(yzero, ny, (int64_t)(blockIdx.x - 1 - xblocks) * kZeroPerBlock);
      return;
    }
    const int64_t b = (int64_t)(blockIdx.x - 1) * kSplitPerBlock + threadIdx.x;
    if (b < nxb) store_split(load_q81(x, b), b, xc, xd);
    return;
  }
  extern __shared__ int32_t wcnt[];  // [kSmallWaves][E]: running counts, then each wave's first positions
  __shared__ int scratch[16];
  __shared__ int bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the wave's ids first (their loads overlap the clearing of the counts)
  int ev[kSmallRounds];
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    const int p = 64 * (kSmallRounds * wave + r) + lane;
    ev[r] = p < n ? idx[p] : -1;
  }
  for (int i = tid; i < kSmallWaves * E; i += blockDim.x) wcnt[i] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  int* my = wcnt + wave * E;
  int rk[kSmallRounds];
  int nbad = 0;
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    const int p = 64 * (kSmallRounds * wave + r) + lane;
    const bool valid = (unsigned)ev[r] < (unsigned)E;
    nbad += __popcll(__ballot(p < n && !valid));
    int c;
    const int rank = wave_rank(ev[r], valid, nbits, &c);
    // this wave alone reads and updates its counts: the read of every lane
    // with id e is one instruction, the leader's update comes after it
    const int base = valid ? my[ev[r]] : 0;
    rk[r] = base + rank;
    if (valid && rank == 0) my[ev[r]] = base + c;
  }
  if (lane == 0 && nbad) atomicAdd(&bad, nbad);
  __syncthreads();
  // per expert: exclusive sums over the waves, the expert's total, its offset
  int c = 0;
  if (tid < E)
    for (int w = 0; w < kSmallWaves; ++w) {
      const int v = wcnt[w * E + tid];
      wcnt[w * E + tid] = c;
      c += v;
    }
  const int first = finish_offsets_small(tid < E ? c : 0, E, bad, offsets, tiles, misc, scratch);
  if (tid < E)
    for (int w = 0; w < kSmallWaves; ++w) wcnt[w * E + tid] += first;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    const int p = 64 * (kSmallRounds * wave + r) + lane;
    if ((unsigned)ev[r] < (unsigned)E) perm[my[ev[r]] + rk[r]] = p;
  }
}

// ---- large batches, pass 1: per-chunk histograms; workgroups past the
// chunks split x.
__global__ __launch_bounds__(kRouteThreads) void k_route_hist(const int32_t* __restrict__ idx, int64_t n_pairs, int E,
                                                    int nchunk, int32_t* __restrict__ chunk_hist,
                                                    int32_t* __restrict__ chunk_bad, const uint8_t* __restrict__ x,
                                                    int64_t nxb, int8_t* __restrict__ xc,
                                                    float* __restrict__ xd, int xblocks, float* __restrict__ yzero,
                                                    int64_t ny) {
  if ((int)blockIdx.x >= nchunk + xblocks) {  // y for the atomic combine
    zero_chunk(yzero, ny, (int64_t)(blockIdx.x - nchunk - xblocks) * kZeroPerBlock);
    return;
  }
  // Each thread's loads are all issued before any of their results is used
  // (a loop of load-then-use waits out one memory round trip per iteration);
  // a thread past the end loads the workgroup's first item instead and drops
  // it.
  constexpr int kPer = kSplitPerBlock / kRouteThreads;
  static_assert(kPer * kRouteThreads == kSplitPerBlock && kPer * kRouteThreads == kRouteChunk, "four per thread");
  if ((int)blockIdx.x >= nchunk) {
    const int64_t b0 = (int64_t)(blockIdx.x - nchunk) * kSplitPerBlock;
    Q81Words r[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t b = b0 + threadIdx.x + kRouteThreads * i;
      r[i] = load_q81(x, b < nxb ? b : b0);
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t b = b0 + threadIdx.x + kRouteThreads * i;
      if (b < nxb) store_split(r[i], b, xc, xd);
    }
    return;
  }
  extern __shared__ int32_t hist[];  // [E]
  __shared__ int32_t bad;
  const int64_t base = (int64_t)blockIdx.x * kRouteChunk;
  int ev[kPer];  // loaded before the counts are cleared, so the two overlap
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t p = base + threadIdx.x + kRouteThreads * i;
    ev[i] = idx[p < n_pairs ? p : base];
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t p = base + threadIdx.x + kRouteThreads * i;
    if (p < n_pairs) {
      if ((unsigned)ev[i] < (unsigned)E)
        atomicAdd(&hist[ev[i]], 1);
      else
        atomicAdd(&bad, 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_hist[(int64_t)blockIdx.x * E + e] = hist[e];
  if (threadIdx.x == 0) chunk_bad[blockIdx.x] = bad;
}

// Pass 2 (one workgroup): chunk prefixes per expert (in place), offsets,
// tiles, counts.
__global__ __launch_bounds__(1024) void k_route_scan(int32_t* __restrict__ chunk_hist,
                                                     const int32_t* __restrict__ chunk_bad, int nchunk, int E,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ tiles,
                                                     int32_t* __restrict__ misc) {
  __shared__ int32_t cnt[1024];
  __shared__ int32_t first[1024];
  __shared__ int32_t tstart[1024];
  __shared__ int scratch[16];
  __shared__ int bad;
  extern __shared__ int32_t stage[];  // the chunk histograms, when they fit (sized by the launch)
  const int64_t nh = (int64_t)nchunk * E;
  if (nh <= kScanStage) {
    // coalesced copy to LDS; per expert, G threads (adjacent lanes) each take
    // a contiguous run of chunks: their sums, an exclusive scan of those over
    // the G lanes, then the running prefixes written back; prefixes back out
    // eight loads in flight per thread before their stores (a load waited for
    // one at a time would cost a memory round trip per 1024 entries)
    for (int64_t i0 = 0; i0 < nh; i0 += 8 * (int64_t)blockDim.x) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t i = i0 + u * (int64_t)blockDim.x + threadIdx.x;
        v[u] = i < nh ? chunk_hist[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t i = i0 + u * (int64_t)blockDim.x + threadIdx.x;
        if (i < nh) stage[i] = v[u];
      }
    }
    __syncthreads();
    int G = 1;
    while (G < 64 && G * 2 * E <= (int)blockDim.x) G *= 2;
    const int e = threadIdx.x / G, g = threadIdx.x % G;
    const int per = (nchunk + G - 1) / G, c0 = g * per, c1 = min(nchunk, c0 + per);
    int part = 0;
    if (e < E) {
#pragma unroll 8
      for (int c = c0; c < c1; ++c) part += stage[c * E + e];
    }
    // inclusive scan over the group's lanes (G a power of two, groups aligned)
    int inc = part;
    for (int d = 1; d < G; d <<= 1) {
      const int y = __shfl_up(inc, d, G);
      if (g >= d) inc += y;
    }
    if (e < E) {
      int run = inc - part;
#pragma unroll 8
      for (int c = c0; c < c1; ++c) {
        const int v = stage[c * E + e];
        stage[c * E + e] = run;
        run += v;
      }
      if (g == G - 1) cnt[e] = inc;
    }
    __syncthreads();
    for (int64_t i0 = 0; i0 < nh; i0 += 8 * (int64_t)blockDim.x) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t i = i0 + u * (int64_t)blockDim.x + threadIdx.x;
        v[u] = i < nh ? stage[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t i = i0 + u * (int64_t)blockDim.x + threadIdx.x;
        if (i < nh) chunk_hist[i] = v[u];
      }
    }
  } else {
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      int run = 0;
      for (int c = 0; c < nchunk; ++c) {
        const int v = chunk_hist[(int64_t)c * E + e];
        chunk_hist[(int64_t)c * E + e] = run;
        run += v;
      }
      cnt[e] = run;
    }
  }
  int b = 0;
  for (int c = threadIdx.x; c < nchunk; c += blockDim.x) b += chunk_bad[c];
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  if (b) atomicAdd(&bad, b);
  __syncthreads();
  finish_offsets(cnt, first, tstart, E, bad, offsets, tiles, misc, scratch);
}

// Pass 3: per chunk, stable scatter of pair ids.
__global__ __launch_bounds__(kRouteThreads) void k_route_scatter(const int32_t* __restrict__ idx, int64_t n_pairs, int E,
                                                       int nbits, const int32_t* __restrict__ chunk_prefix,
                                                       const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm) {
  extern __shared__ int32_t sm[];  // base[E] | wave_count[4][E]
  int32_t* base = sm;
  int32_t* wcnt = sm + E;
  const int64_t cbase = (int64_t)blockIdx.x * kRouteChunk;
  constexpr int kRounds = kRouteChunk / kRouteThreads;
  int ev[kRounds];  // all of this thread's ids first (past the end: -1, from a load of the chunk's first id)
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t p = cbase + r * kRouteThreads + threadIdx.x;
    const int v = idx[p < n_pairs ? p : cbase];
    ev[r] = p < n_pairs ? v : -1;
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    base[e] = offsets[e] + chunk_prefix[(int64_t)blockIdx.x * E + e];
    for (int w = 0; w < 4; ++w) wcnt[w * E + e] = 0;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t p = cbase + r * kRouteThreads + threadIdx.x;
    const int e = ev[r];
    const bool valid = (unsigned)e < (unsigned)E;
    int c;
    const int rank = wave_rank(e, valid, nbits, &c);
    const bool leader = valid && rank == 0;
    if (leader) wcnt[wave * E + e] = c;
    __syncthreads();
    if (valid) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += wcnt[w * E + e];
      perm[base[e] + before + rank] = (int32_t)p;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&base[e], c);
      wcnt[wave * E + e] = 0;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_route(const int32_t* idx, const uint8_t* x, const Shapes& s, const Work& w, float* yzero,
                        hipStream_t st) {
  const int64_t n = s.pairs();
  int nbits = 0;
  while ((1 << nbits) < s.E) ++nbits;
  const int64_t nxb = s.T * (s.L / 32);
  const unsigned xblocks = (unsigned)((nxb + kSplitPerBlock - 1) / kSplitPerBlock);
  const int64_t ny = yzero ? s.T * s.L : 0;
  const unsigned zblocks = (unsigned)((ny + kZeroPerBlock - 1) / kZeroPerBlock);
  if (n <= kSmallPairs && s.E <= 512) {  // kSmallWaves * E ints of LDS
    hipLaunchKernelGGL(k_route_small, dim3(1 + xblocks + zblocks), dim3(64 * kSmallWaves),
                       kSmallWaves * s.E * sizeof(int32_t), st,
                       idx, (int)n, s.E, nbits, w.offsets, w.tiles, w.misc, w.perm, x, nxb, w.xc, w.xd, (int)xblocks,
                       yzero, ny);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_route_hist, dim3(w.nchunk + xblocks + zblocks), dim3(kRouteThreads), s.E * sizeof(int32_t), st, idx, n,
                     s.E, w.nchunk, w.chunk_hist, w.chunk_bad, x, nxb, w.xc, w.xd, (int)xblocks, yzero, ny);
  const int64_t nh = (int64_t)w.nchunk * s.E;
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), nh <= kScanStage ? nh * sizeof(int32_t) : 0, st, w.chunk_hist,
                     w.chunk_bad, w.nchunk, s.E, w.offsets, w.tiles, w.misc);
  hipLaunchKernelGGL(k_route_scatter, dim3(w.nchunk), dim3(kRouteThreads), 5 * s.E * sizeof(int32_t), st, idx, n, s.E, nbits,
                     w.chunk_hist, w.offsets, w.perm);
  return hipGetLastError();
}

}  // namespace latmoe
