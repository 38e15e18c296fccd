// C ABI of the expert stage: argument checks, workspace layout, launches.
#include <mutex>
#include <string.h>

#include "../../include/lat_moe.h"
#include "lat_moe_internal.h"

using namespace latmoe;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool shapes_ok(const lat_moe_shapes* s) {
  if (!s) return false;
  if (s->T < 0 || s->L < 256 || s->L > 65536 || s->L % 256) return false;
  if (s->F < 32 || s->F > 65536 || s->F % 32) return false;
  if (s->E < 1 || s->E > LAT_MOE_MAX_E || s->k < 1 || s->k > s->E) return false;
  if (s->T * (int64_t)s->k >= (int64_t)1 << 31) return false;
  // one expert's gate/up rows stay below 2 GiB (kernels address within an expert with 32-bit offsets)
  if ((int64_t)2 * s->F * (s->L / 256) * 110 >= (int64_t)1 << 31) return false;
  // the activation codes, H codes and one expert's down weights too (32-bit offsets)
  if (s->T * (int64_t)s->L >= (int64_t)1 << 31) return false;
  if (s->T * (int64_t)s->k * s->F >= (int64_t)1 << 31) return false;
  if ((int64_t)s->L * (s->F / 32) * 18 >= (int64_t)1 << 31) return false;
  return true;
}

struct Layout {
  size_t chunk_hist, chunk_bad, offsets, misc, tiles, perm, h_codes, h_ds, slots, xc, xd, total;
  int nchunk, max_tiles;
};

Layout layout(const lat_moe_shapes* s) {
  Layout L{};
  const int64_t P = s->T * s->k;
  L.nchunk = (int)((P + kRouteChunk - 1) / kRouteChunk);
  L.max_tiles = (int)((P + kTileN - 1) / kTileN + s->E);
  size_t o = 0;
  L.chunk_hist = o; o = align_up(o + sizeof(int32_t) * (size_t)L.nchunk * s->E);
  L.chunk_bad = o;  o = align_up(o + sizeof(int32_t) * (size_t)L.nchunk);
  L.offsets = o;    o = align_up(o + sizeof(int32_t) * (size_t)(s->E + 1));
  L.misc = o;       o = align_up(o + sizeof(int32_t) * kMiscWords);
  L.tiles = o;      o = align_up(o + sizeof(int32_t) * kTileWords * (size_t)L.max_tiles);
  L.perm = o;       o = align_up(o + sizeof(int32_t) * (size_t)P);
  L.h_codes = o;    o = align_up(o + (size_t)P * s->F);
  L.h_ds = o;       o = align_up(o + sizeof(uint32_t) * (size_t)P * (s->F / 32));
  L.slots = o;      o = align_up(o + sizeof(float) * (size_t)P * s->L);
  L.xc = o;         o = align_up(o + (size_t)s->T * s->L);
  L.xd = o;         o = align_up(o + sizeof(float) * (size_t)s->T * (s->L / 32));
  L.total = o;
  return L;
}

Work carve(const Layout& L, void* ws) {
  char* b = static_cast<char*>(ws);
  Work w;
  w.chunk_hist = reinterpret_cast<int32_t*>(b + L.chunk_hist);
  w.chunk_bad = reinterpret_cast<int32_t*>(b + L.chunk_bad);
  w.offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  w.misc = reinterpret_cast<int32_t*>(b + L.misc);
  w.tiles = reinterpret_cast<int32_t*>(b + L.tiles);
  w.perm = reinterpret_cast<int32_t*>(b + L.perm);
  w.h_codes = reinterpret_cast<int8_t*>(b + L.h_codes);
  w.h_ds = reinterpret_cast<uint32_t*>(b + L.h_ds);
  w.slots = reinterpret_cast<float*>(b + L.slots);
  w.xc = reinterpret_cast<int8_t*>(b + L.xc);
  w.xd = reinterpret_cast<float*>(b + L.xd);
  w.nchunk = L.nchunk;
  w.max_tiles = L.max_tiles;
  w.num_cus = 1;
  return w;
}

// Once per device: is it a gfx950 with 64-wide wavefronts, and how many CUs?
int check_device(int* num_cus) {
  static std::mutex mu;
  static signed char state[64];  // 0 unknown, 1 ok, -1 unsupported
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return LAT_MOE_EDEVICE;
  std::lock_guard<std::mutex> g(mu);
  if (state[dev] == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return LAT_MOE_EDEVICE;
    state[dev] = (strncmp(p.gcnArchName, "gfx950", 6) == 0 && p.warpSize == 64) ? 1 : -1;
    cus[dev] = p.multiProcessorCount > 0 ? p.multiProcessorCount : 1;
  }
  if (num_cus) *num_cus = cus[dev];
  return state[dev] == 1 ? LAT_MOE_OK : LAT_MOE_EDEVICE;
}

int forward_impl(const void* x, const int32_t* idx, const float* w, const void* gu, int gu_fmt, const void* dn,
                 int down_fmt, const lat_moe_shapes* s, float* y, void* ws, size_t ws_bytes, void* stream,
                 const lat_moe_debug* dbg) {
  // the slot buffer and ordered combine unless the caller asks for atomic adds
  const bool deterministic = dbg ? dbg->deterministic != 0 : true;
  if (!shapes_ok(s)) return LAT_MOE_EINVAL;
  if (down_fmt != LAT_MOE_DOWN_IQ4_NL && down_fmt != LAT_MOE_DOWN_Q4_0) return LAT_MOE_EINVAL;
  if (gu_fmt != LAT_MOE_GATEUP_Q3_K && gu_fmt != LAT_MOE_GATEUP_Q4_0) return LAT_MOE_EINVAL;
  // one expert's Q4_0 gate/up weights below 2 GiB too (32-bit offsets)
  if (gu_fmt == LAT_MOE_GATEUP_Q4_0 && (int64_t)2 * s->F * (s->L / 32) * 18 >= (int64_t)1 << 31) return LAT_MOE_EINVAL;
  if (s->T > 0) {
    const void* ptrs[] = {x, idx, w, gu, dn, y, ws};
    for (const void* p : ptrs)
      if (!p || !aligned16(p)) return LAT_MOE_EINVAL;
  }
  if (dbg) {
    if (dbg->stage_events)
      for (int i = 0; i < 5; ++i)
        if (!dbg->stage_events[i]) return LAT_MOE_EINVAL;
    if (dbg->gateup_i32 && (dbg->gu_rows < 1 || dbg->gu_row0 < 0 || dbg->gu_row0 + (int64_t)dbg->gu_rows > 2 * (int64_t)s->F))
      return LAT_MOE_EINVAL;
    if (dbg->down_i32 && (dbg->dn_rows < 1 || dbg->dn_row0 < 0 || dbg->dn_row0 + (int64_t)dbg->dn_rows > s->L))
      return LAT_MOE_EINVAL;
  }
  const Layout L = layout(s);
  if (s->T == 0) return LAT_MOE_OK;
  if (ws_bytes < L.total) return LAT_MOE_EWORKSPACE;
  int num_cus = 1;
  int rc = check_device(&num_cus);
  if (rc != LAT_MOE_OK) return rc;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const Shapes sh{s->T, s->L, s->F, s->E, s->k};
  Work wk = carve(L, ws);
  wk.num_cus = num_cus;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  hipEvent_t const* ev = (dbg && dbg->stage_events) ? reinterpret_cast<hipEvent_t const*>(dbg->stage_events) : nullptr;
  auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], st) : hipSuccess; };
  if (mark(0) != hipSuccess) return LAT_MOE_ELAUNCH;
  const bool small = decode_path(sh);  // decode-sized batch: two launches on the routing as given
  ProbeRows pg{nullptr, 0, 0}, pd{nullptr, 0, 0};
  if (dbg && dbg->gateup_i32) pg = ProbeRows{dbg->gateup_i32, dbg->gu_row0, dbg->gu_rows};
  if (dbg && dbg->down_i32) pd = ProbeRows{dbg->down_i32, dbg->dn_row0, dbg->dn_rows};
  const uint8_t* gub = static_cast<const uint8_t*>(gu);
  const uint8_t* dnb = static_cast<const uint8_t*>(dn);
  const int fmt = down_fmt == LAT_MOE_DOWN_Q4_0 ? kDownQ40 : kDownIq4Nl;
  if (small) {
    // The sort runs only when its outputs are asked for (debug): the decode
    // kernels group the pairs themselves.
    if (dbg && (dbg->perm || dbg->offsets || dbg->dropped) &&
        launch_route(idx, xb, sh, wk, nullptr, st) != hipSuccess)
      return LAT_MOE_ELAUNCH;
    if (mark(1) != hipSuccess) return LAT_MOE_ELAUNCH;
    if (launch_decode(sh, wk, xb, idx, w, gub, gu_fmt, dnb, fmt, y, pg.out ? &pg : nullptr, pd.out ? &pd : nullptr,
                      st, ev ? ev[2] : nullptr) != hipSuccess)
      return LAT_MOE_ELAUNCH;
    if (mark(3) != hipSuccess || mark(4) != hipSuccess) return LAT_MOE_ELAUNCH;
    if (dbg && dbg->h_q8_1 &&
        launch_export_h_pairs(idx, sh, wk, static_cast<uint8_t*>(dbg->h_q8_1), st) != hipSuccess)
      return LAT_MOE_ELAUNCH;
  } else {
    // atomic combine: the route pass zeroes y, down adds into it, no combine kernel
    const bool atomic = !deterministic;
    if (launch_route(idx, xb, sh, wk, atomic ? y : nullptr, st) != hipSuccess) return LAT_MOE_ELAUNCH;
    if (mark(1) != hipSuccess) return LAT_MOE_ELAUNCH;
    if ((gu_fmt == LAT_MOE_GATEUP_Q4_0 ? launch_gateup_q40(sh, wk, gub, pg.out ? &pg : nullptr, st)
                                       : launch_gateup(sh, wk, gub, pg.out ? &pg : nullptr, st)) != hipSuccess)
      return LAT_MOE_ELAUNCH;
    if (mark(2) != hipSuccess) return LAT_MOE_ELAUNCH;
    if (launch_down(dnb, fmt, w, sh, wk, atomic ? y : nullptr, pd.out ? &pd : nullptr, st) != hipSuccess)
      return LAT_MOE_ELAUNCH;
    if (mark(3) != hipSuccess) return LAT_MOE_ELAUNCH;
    if (!atomic && launch_combine(idx, sh, wk, y, st) != hipSuccess) return LAT_MOE_ELAUNCH;
    if (mark(4) != hipSuccess) return LAT_MOE_ELAUNCH;
    if (dbg && dbg->h_q8_1 && launch_export_h(sh, wk, static_cast<uint8_t*>(dbg->h_q8_1), st) != hipSuccess)
      return LAT_MOE_ELAUNCH;
  }
  if (dbg) {
    if (dbg->perm && launch_copy_i32(wk.perm, dbg->perm, sh.pairs(), st) != hipSuccess) return LAT_MOE_ELAUNCH;
    if (dbg->offsets && launch_copy_i32(wk.offsets, dbg->offsets, s->E + 1, st) != hipSuccess) return LAT_MOE_ELAUNCH;
    if (dbg->dropped && launch_copy_i32(wk.misc + kMiscDropped, dbg->dropped, 1, st) != hipSuccess)
      return LAT_MOE_ELAUNCH;
  }
  return LAT_MOE_OK;
}

int dense_impl(int wfmt, const void* x_q8_1, const void* w, int64_t T, int32_t N, int32_t K, float* y_f32,
               void* y_q8_1, void* stream, int32_t* dots_i32, int32_t row0, int32_t rows) {
  if (T < 0 || K < 32 || K > 65536 || K % 32 || N < 32 || N > 65536 || N % 32) return LAT_MOE_EINVAL;
  const int wb = wfmt == kDenseQ40 ? kQ40Bytes : kQ80Bytes;
  if ((int64_t)N * (K / 32) * wb >= (int64_t)1 << 31 || T * (K / 32) * 36 >= (int64_t)1 << 31) return LAT_MOE_EINVAL;
  if (!dense_shape_ok(wfmt, T, N, K)) return LAT_MOE_EINVAL;
  if (!y_f32 && !y_q8_1) return LAT_MOE_EINVAL;
  if (dots_i32 && (row0 < 0 || rows < 1 || (int64_t)row0 + rows > N)) return LAT_MOE_EINVAL;
  if (T == 0) return LAT_MOE_OK;
  const void* need[] = {x_q8_1, w};
  for (const void* p : need)
    if (!p || !aligned16(p)) return LAT_MOE_EINVAL;
  if ((y_f32 && !aligned16(y_f32)) || (y_q8_1 && !aligned16(y_q8_1)) || (dots_i32 && !aligned16(dots_i32)))
    return LAT_MOE_EINVAL;
  int num_cus = 1;
  int rc = check_device(&num_cus);
  if (rc != LAT_MOE_OK) return rc;
  const ProbeRows probe{dots_i32, row0, rows};
  if (launch_dense(static_cast<const uint8_t*>(x_q8_1), static_cast<const uint8_t*>(w), wfmt, T, N, K, y_f32,
                   static_cast<uint8_t*>(y_q8_1), dots_i32 ? &probe : nullptr, num_cus,
                   static_cast<hipStream_t>(stream)) != hipSuccess)
    return LAT_MOE_ELAUNCH;
  return LAT_MOE_OK;
}


}  // namespace

namespace latmoe {

int stage_forward(const void* x, const int32_t* idx, const float* w, const void* gu, const void* dn,
                  const lat_moe_shapes* s, float* y, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(x, idx, w, gu, LAT_MOE_GATEUP_Q3_K, dn, LAT_MOE_DOWN_IQ4_NL, s, y, ws, ws_bytes, stream,
                      nullptr);
}

int device_check(int* num_cus) { return check_device(num_cus); }

}  // namespace latmoe

extern "C" {

size_t lat_moe_workspace_size(const lat_moe_shapes* shapes) {
  if (!shapes_ok(shapes)) return 0;
  return layout(shapes).total;
}

int lat_moe_expert_forward(const void* x_q8_1, const int32_t* router_idx, const float* router_w,
                           const void* gateup_q3k, const void* down_iq4nl, const lat_moe_shapes* shapes, float* y,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(x_q8_1, router_idx, router_w, gateup_q3k, LAT_MOE_GATEUP_Q3_K, down_iq4nl, LAT_MOE_DOWN_IQ4_NL,
                      shapes, y, workspace, workspace_bytes, stream, nullptr);
}

int lat_moe_expert_forward_ex(const void* x_q8_1, const int32_t* router_idx, const float* router_w,
                              const void* gateup_q3k, const void* down_iq4nl, const lat_moe_shapes* shapes, float* y,
                              void* workspace, size_t workspace_bytes, void* stream, const lat_moe_debug* dbg) {
  return forward_impl(x_q8_1, router_idx, router_w, gateup_q3k, LAT_MOE_GATEUP_Q3_K, down_iq4nl, LAT_MOE_DOWN_IQ4_NL,
                      shapes, y, workspace, workspace_bytes, stream, dbg);
}

int lat_moe_expert_forward_fmt(const void* x_q8_1, const int32_t* router_idx, const float* router_w,
                               const void* gateup, int32_t gateup_format, const void* down, int32_t down_format,
                               const lat_moe_shapes* shapes, float* y, void* workspace, size_t workspace_bytes,
                               void* stream, const lat_moe_debug* dbg) {
  return forward_impl(x_q8_1, router_idx, router_w, gateup, gateup_format, down, down_format, shapes, y, workspace,
                      workspace_bytes, stream, dbg);
}

int lat_moe_quantize_q8_1(const float* x, int64_t rows, int32_t cols, void* out_q8_1, void* stream) {
  if (rows < 0 || cols < 32 || cols % 32) return LAT_MOE_EINVAL;
  if (rows == 0) return LAT_MOE_OK;
  if (!x || !out_q8_1 || !aligned16(x) || !aligned16(out_q8_1)) return LAT_MOE_EINVAL;
  int rc = check_device(nullptr);
  if (rc != LAT_MOE_OK) return rc;
  if (launch_quantize_q8_1(x, rows, cols, static_cast<uint8_t*>(out_q8_1), static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return LAT_MOE_ELAUNCH;
  return LAT_MOE_OK;
}


int lat_moe_dense_q8_0_debug(const void* x_q8_1, const void* w_q8_0, int64_t T, int32_t N, int32_t K,
                             float* y_f32, void* y_q8_1, void* stream, int32_t* dots_i32, int32_t row0,
                             int32_t rows) {
  return dense_impl(kDenseQ80, x_q8_1, w_q8_0, T, N, K, y_f32, y_q8_1, stream, dots_i32, row0, rows);
}

int lat_moe_dense_q8_0(const void* x_q8_1, const void* w_q8_0, int64_t T, int32_t N, int32_t K, float* y_f32,
                       void* y_q8_1, void* stream) {
  return dense_impl(kDenseQ80, x_q8_1, w_q8_0, T, N, K, y_f32, y_q8_1, stream, nullptr, 0, 0);
}

int lat_moe_dense_q4_0_debug(const void* x_q8_1, const void* w_q4_0, int64_t T, int32_t N, int32_t K,
                             float* y_f32, void* y_q8_1, void* stream, int32_t* dots_i32, int32_t row0,
                             int32_t rows) {
  return dense_impl(kDenseQ40, x_q8_1, w_q4_0, T, N, K, y_f32, y_q8_1, stream, dots_i32, row0, rows);
}

int lat_moe_dense_q4_0(const void* x_q8_1, const void* w_q4_0, int64_t T, int32_t N, int32_t K, float* y_f32,
                       void* y_q8_1, void* stream) {
  return dense_impl(kDenseQ40, x_q8_1, w_q4_0, T, N, K, y_f32, y_q8_1, stream, nullptr, 0, 0);
}

int lat_moe_router_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* router_idx, float* router_w,
                        void* stream) {
  if (T < 0 || E < 1 || E > LAT_MOE_ROUTER_MAX_E || k < 1 || k > E || k > LAT_MOE_ROUTER_MAX_K) return LAT_MOE_EINVAL;
  if (T == 0) return LAT_MOE_OK;
  const void* ptrs[] = {logits, router_idx, router_w};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return LAT_MOE_EINVAL;
  int rc = check_device(nullptr);
  if (rc != LAT_MOE_OK) return rc;
  if (launch_router_topk(logits, T, E, k, router_idx, router_w, static_cast<hipStream_t>(stream)) != hipSuccess)
    return LAT_MOE_ELAUNCH;
  return LAT_MOE_OK;
}

const char* lat_moe_strerror(int code) {
  switch (code) {
    case LAT_MOE_OK: return "ok";
    case LAT_MOE_EINVAL: return "invalid argument (null or misaligned pointer, or unsupported shape)";
    case LAT_MOE_EWORKSPACE: return "workspace smaller than lat_moe_workspace_size()";
    case LAT_MOE_EDEVICE: return "current device is not a gfx950 with 64-wide wavefronts";
    case LAT_MOE_ELAUNCH: return "kernel launch failed";
    case LAT_MOE_ESCRATCH: return "shapes need more workspace than the no-allocation entry point's fixed scratch";
    default: return "unknown error";
  }
}

int lat_moe_version(void) { return 100; }

}  // extern "C"
