// Internal declarations of the gfx950 expert-stage kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lat_moe.h"

namespace latmoe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Block formats (ggml GGUF layouts).
constexpr int kQ3kBytes = 110;   // 256 weights
constexpr int kIq4Bytes = 18;    // 32 weights
constexpr int kQ81Bytes = 36;    // 32 values

// Pair ids are grouped per route chunk of this many pairs (one workgroup each).
constexpr int kRouteChunk = 1024;
// Token (sorted pair) tile of the grouped GEMMs.
constexpr int kTileN = 128;
// Tile table entry: (expert, first sorted position, pairs in the tile, 0).
constexpr int kTileWords = 4;
// Batches of at most this many routed pairs (with L <= 1024, F <= 2048) take
// the two decode kernels, which read the routing as given (no sort).
constexpr int kDecodeMaxPairs = 64;

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
  int32_t* tiles;       // [max_tiles][kTileWords] (expert, first sorted position, pairs, 0)
  int32_t* perm;        // [T*k] pair ids grouped by expert
  int8_t* h_codes;      // [T*k][F] H codes in sorted order
  uint32_t* h_ds;       // [T*k][F/32] fp16 d | fp16 s << 16
  float* slots;         // [T*k][L] weighted expert outputs in pair order
  int8_t* xc;           // [T][L] activation codes (q8_1 blocks split into codes ...)
  float* xd;            // [T][L/32] ... and fp32 block scales)
  int nchunk, max_tiles;
  int num_cus;          // compute units of the current device (persistent grids)
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

// MFMA accumulator init that makes an int32 result readable as fp32: the bit
// pattern 0x4B400000 is 1.5 * 2^23, and adding an int32 I with |I| < 2^22 to
// those bits gives exactly the float 1.5 * 2^23 + I.
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;

// Reinterprets an int32 MFMA result element as fp32 (through a union:
// __builtin_bit_cast on an extracted vector element miscompiles here).
__device__ __forceinline__ float as_float(int v) {
  union {
    int i;
    float f;
  } u;
  u.i = v;
  return u.f;
}

// Materialises v as an fp32 register value: the optimizer cannot fuse the
// operation that produced it into what consumes it (for instance fp32 multiply
// then fp16 conversion into one singly-rounded v_fma_mix).
__device__ __forceinline__ float fp32_barrier(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// The q8_1 rule's round half away from zero, to int: adding the largest float
// below one half with v's sign and truncating (v_cvt_i32_f32) gives roundf's
// integer for every float |v| < 2^31 (an exhaustive host check over all fp32
// values confirms it), in three VALU operations.  Callers keep FMA
// contraction off so the add is not fused with the product that made v.
__device__ __forceinline__ int round_half_away(float v) {
  return (int)(v + __builtin_copysignf(0x1.fffffep-2f, v));
}

// Low bytes of four int32 codes as one word, byte i = code i (three v_perm_b32).
__device__ __forceinline__ uint32_t pack_codes(int a, int b, int c, int d) {
  const uint32_t lo = __builtin_amdgcn_perm((uint32_t)b, (uint32_t)a, 0x0C0C0400u);
  const uint32_t hi = __builtin_amdgcn_perm((uint32_t)d, (uint32_t)c, 0x0C0C0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Operand table of a Q3_K sub-block with signed scale sg = sc6 - 32: byte c
// of (thi:tlo) is (4 - c) * sg for the 3-bit code c, so v_perm_b32(thi, tlo,
// codes) expands four codes at once.  Products are formed two at a time in
// 16-bit halves (their low bytes are the int8 values) and gathered by v_perm.
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void q3_tables(int sg, uint32_t& tlo, uint32_t& thi) {
  const s16x2 v = {(short)sg, (short)sg};
  const s16x2 a = v * (s16x2){4, 3};
  const s16x2 b = v * (s16x2){2, 1};
  const s16x2 c = v * (s16x2){-1, -2};
  const s16x2 d = v * (s16x2){-3, 0};
  tlo = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a), 0x06040200u);
  thi = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, d), __builtin_bit_cast(uint32_t, c), 0x0402000Cu);
}

// IQ4_NL: the 16-entry non-linear table (ggml) packed as four little-endian
// words, and a lookup of 4 indices (one per byte, 0..15) -> 4 table bytes:
// two v_perm_b32 look up the low 3 bits in both 8-entry halves, a third picks
// byte b of the low half or byte b of the high half by bit 3 of index b.
constexpr int kIq4Table[16] = {-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113};
constexpr uint32_t iq4_tab_word(int w) {
  return (uint32_t)(kIq4Table[4 * w] & 0xff) | ((uint32_t)(kIq4Table[4 * w + 1] & 0xff) << 8) |
         ((uint32_t)(kIq4Table[4 * w + 2] & 0xff) << 16) | ((uint32_t)(kIq4Table[4 * w + 3] & 0xff) << 24);
}
constexpr uint32_t kIq4Tab0 = iq4_tab_word(0), kIq4Tab1 = iq4_tab_word(1), kIq4Tab2 = iq4_tab_word(2),
                   kIq4Tab3 = iq4_tab_word(3);
static_assert(kIq4Tab0 == 0xBFAD9881u && kIq4Tab3 == 0x71594535u, "IQ4_NL table packing");
__device__ __forceinline__ uint32_t iq4_lookup(uint32_t nib) {
  const uint32_t sel = nib & 0x07070707u;
  const uint32_t lo = __builtin_amdgcn_perm(kIq4Tab1, kIq4Tab0, sel);
  const uint32_t hi = __builtin_amdgcn_perm(kIq4Tab3, kIq4Tab2, sel);
  // selector byte b: b (from lo) or 4 + b (from hi); bit 3 of the index moves to bit 2
  const uint32_t pick = ((nib >> 1) & 0x04040404u) | 0x03020100u;
  return __builtin_amdgcn_perm(hi, lo, pick);
}

// Down weight formats.  Both are 18-byte blocks of 32 weights: fp16 d, then 16
// bytes of 4-bit indices (element i < 16 in the low nibble of byte i, element
// i >= 16 in the high nibble of byte i - 16); they differ in what an index is
// worth: IQ4_NL's non-linear table, or Q4_0's index - 8 (ggml's block
// formats; Q4_0 is one of the weight formats named in section "Not done" of
// the PR page "Run Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1").
enum DownFormat : int { kDownIq4Nl = 0, kDownQ40 = 1 };
// 4 indices (one per byte, each 0..15) -> their 4 int8 weights.
template <int FMT>
__device__ __forceinline__ uint32_t down_lookup(uint32_t nib) {
  if constexpr (FMT == kDownQ40)
    return (nib + 0x78787878u) ^ 0x80808080u;  // index - 8 per byte (index + 0x78 <= 0x87: no carry out)
  else
    return iq4_lookup(nib);
}

// Raw buffer loads (gfx9 buffer resource, stride 0).  A load whose 32-bit
// offset is at or past num_records returns zero without touching memory, so
// padding lanes load from kOutOfRange instead of branching around the load.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kOutOfRange = (int)0x80000000u;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buf_u16(rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf_u32(rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint4 buf_u128(rsrc_t r, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return uint4{v[0], v[1], v[2], v[3]};
}

// The expert stage (Q3_K gate/up, IQ4_NL down, ordered combine) on a given
// workspace: lat_moe_expert_forward's checks and launches.
int stage_forward(const void* x, const int32_t* idx, const float* w, const void* gu, const void* dn,
                  const lat_moe_shapes* s, float* y, void* ws, size_t ws_bytes, void* stream);
// LAT_MOE_OK if the current device is a gfx950 with 64-wide wavefronts (and
// its CU count in *num_cus if not null); cached per device.
int device_check(int* num_cus);

// Kernel launchers (each returns hipGetLastError() after the enqueue).
// Sorts pairs by expert and splits the q8_1 activations x into codes and
// scales.  yzero: y [T][L] to fill with zeros for the down kernel's atomic
// adds, or null.
hipError_t launch_route(const int32_t* idx, const uint8_t* x, const Shapes& s, const Work& w, float* yzero,
                        hipStream_t st);
hipError_t launch_gateup(const Shapes& s, const Work& w, const uint8_t* gu, const ProbeRows* probe, hipStream_t st);
// Gate/up weights in Q4_0 (18-byte blocks, a scale per 32 values), batches beyond small_path.
hipError_t launch_gateup_q40(const Shapes& s, const Work& w, const uint8_t* gu, const ProbeRows* probe,
                             hipStream_t st);
// y_atomic null: each pair's weighted row goes to its slot; otherwise it is
// added into y_atomic [T][L] (zeroed beforehand) with fp32 atomic adds.
hipError_t launch_down(const uint8_t* dn, int fmt, const float* router_w, const Shapes& s, const Work& w,
                       float* y_atomic, const ProbeRows* probe, hipStream_t st);
// Decode-sized batches: gate/up with SwiGLU and the q8_1 requant (H in pair
// order), then down with the combine in slot order straight into y.  When
// after_gateup is not null it is recorded between the two launches.
bool decode_path(const Shapes& s);
hipError_t launch_decode(const Shapes& s, const Work& w, const uint8_t* x, const int32_t* idx, const float* router_w,
                         const uint8_t* gu, int gu_fmt, const uint8_t* dn, int dn_fmt, float* y,
                         const ProbeRows* probe_gu, const ProbeRows* probe_dn, hipStream_t st, hipEvent_t after_gateup);
// H of the decode path (pair order) as q8_1 blocks, zero for invalid ids.
hipError_t launch_export_h_pairs(const int32_t* idx, const Shapes& s, const Work& w, uint8_t* h_out, hipStream_t st);
hipError_t launch_combine(const int32_t* idx, const Shapes& s, const Work& w, float* y, hipStream_t st);
hipError_t launch_quantize_q8_1(const float* x, int64_t rows, int cols, uint8_t* out, hipStream_t st);
hipError_t launch_export_h(const Shapes& s, const Work& w, uint8_t* h_out, hipStream_t st);
hipError_t launch_copy_i32(const int32_t* src, int32_t* dst, int64_t n, hipStream_t st);
// Router: fp32 logits [T][E] -> top-k ids and renormalised softmax weights.
hipError_t launch_router_topk(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w, hipStream_t st);
// Latent D / U dense projection, Q8_0 weights [N][K/32] x q8_1 rows [T][K/32]
// -> fp32 [T][N] and/or q8_1 [T][N/32] (either output may be null).
// Weight formats of the projections: Q8_0 (34-byte blocks) and Q4_0 (18-byte
// blocks, the layout of IQ4_NL with weight = d * (nibble - 8)).
enum DenseFormat : int { kDenseQ80 = 0, kDenseQ40 = 1 };
constexpr int kQ80Bytes = 34, kQ40Bytes = 18;
hipError_t launch_dense(const uint8_t* x, const uint8_t* w, int wfmt, int64_t T, int N, int K, float* y_f32,
                        uint8_t* y_q8, const ProbeRows* probe, int num_cus, hipStream_t st);
// Shapes a format's kernels take (Q8_0: all; Q4_0: the GEMV kernel's batches,
// or N % 128 == 0 and K % 256 == 0).
bool dense_shape_ok(int wfmt, int64_t T, int N, int K);
// The persistent warp-specialized form (any T >= 1), for N % 128 == 0 and K % 256 == 0.
bool dense_ws_shape(int N, int K);
hipError_t launch_dense_ws(const uint8_t* x, const uint8_t* w, int wfmt, int64_t T, int N, int K, float* y_f32,
                           uint8_t* y_q8, const ProbeRows* probe, int num_cus, hipStream_t st);

}  // namespace latmoe
