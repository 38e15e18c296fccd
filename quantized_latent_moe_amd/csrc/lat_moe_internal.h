// Internal declarations of the gfx950 expert-stage kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace latmoe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Block formats (ggml GGUF layouts).
constexpr int kQ3kBytes = 110;   // 256 weights
constexpr int kIq4Bytes = 18;    // 32 weights
constexpr int kQ81Bytes = 36;    // 32 values

// Pair ids are grouped per route chunk of this many pairs (one workgroup each).
constexpr int kRouteChunk = 4096;
// Token (sorted pair) tile of the grouped GEMMs.
constexpr int kTileN = 128;

// Slots of the small device status array written by the route scan.
constexpr int kMiscTiles = 0;    // number of (expert, token tile) work items
constexpr int kMiscDropped = 1;  // pairs with an expert id outside [0, E)
constexpr int kMiscValid = 2;    // pairs with a valid id
constexpr int kMiscWords = 16;

// Row ranges whose integer block dots the debug build of a kernel stores.
struct ProbeRows {
  int32_t* out;  // [T*k][rows][blocks] int32, pair order
  int32_t row0, rows;
};

// Device views of the workspace.
struct Work {
  int32_t* chunk_hist;  // [nchunk][E]
  int32_t* chunk_bad;   // [nchunk]
  int32_t* offsets;     // [E+1]
  int32_t* misc;        // [kMiscWords]
  int32_t* tiles;       // [max_tiles][2] (expert, first sorted position)
  int32_t* perm;        // [T*k] pair ids grouped by expert
  int8_t* h_codes;      // [T*k][F] H codes in sorted order
  uint32_t* h_ds;       // [T*k][F/32] fp16 d | fp16 s << 16
  float* slots;         // [T*k][L] weighted expert outputs in pair order
  int8_t* xc;           // [T][L] activation codes (q8_1 blocks split into codes ...)
  float* xd;            // [T][L/32] ... and fp32 block scales)
  int nchunk, max_tiles;
};

struct Shapes {
  int64_t T;
  int L, F, E, k;
  int64_t pairs() const { return T * k; }
};

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}
__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32, nearest-even
}

// Materialises v as an fp32 register value: the optimizer cannot fuse the
// operation that produced it into what consumes it (for instance fp32 multiply
// then fp16 conversion into one singly-rounded v_fma_mix).
__device__ __forceinline__ float fp32_barrier(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Kernel launchers (each returns hipGetLastError() after the enqueue).
hipError_t launch_route(const int32_t* idx, const Shapes& s, const Work& w, hipStream_t st);
hipError_t launch_x_split(const uint8_t* x, const Shapes& s, const Work& w, hipStream_t st);
hipError_t launch_gateup(const Shapes& s, const Work& w, const uint8_t* gu, const ProbeRows* probe, hipStream_t st);
hipError_t launch_down(const uint8_t* dn, const float* router_w, const Shapes& s, const Work& w,
                       const ProbeRows* probe, hipStream_t st);
hipError_t launch_combine(const int32_t* idx, const Shapes& s, const Work& w, float* y, hipStream_t st);
hipError_t launch_quantize_q8_1(const float* x, int64_t rows, int cols, uint8_t* out, hipStream_t st);
hipError_t launch_export_h(const Shapes& s, const Work& w, uint8_t* h_out, hipStream_t st);
hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int64_t n, hipStream_t st);

}  // namespace latmoe
