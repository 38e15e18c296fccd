"""Quantized latent-MoE expert stage on MI355X (gfx950): Python binding.

Thin ctypes marshalling over ``liblatmoe.so`` (the C ABI in
``include/lat_moe.h``).  Every step of the stage runs in the library's HIP
kernels; torch tensors only provide device memory and the current stream.
There is no fallback: if the library is not built, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblatmoe.so")

LAT_MOE_MAX_E = 1024
# down-weight formats of lat_moe_expert_forward_fmt (both 18-byte blocks of 32)
DOWN_IQ4_NL = 0
DOWN_Q4_0 = 1
# gate/up-weight formats of lat_moe_expert_forward_fmt
GATEUP_Q3_K = 0
GATEUP_Q4_0 = 1

# Symbols the C header declares (checked by the CPU test suite).
EXPORTED = (
    "lat_moe_workspace_size",
    "lat_moe_expert_forward",
    "lat_moe_expert_forward_ex",
    "lat_moe_expert_forward_fmt",
    "lat_moe_expert_forward_noalloc",
    "lat_moe_quantize_q8_1",
    "lat_moe_dense_q8_0",
    "lat_moe_dense_q8_0_debug",
    "lat_moe_dense_q4_0",
    "lat_moe_dense_q4_0_debug",
    "lat_moe_router_topk",
    "lat_moe_strerror",
    "lat_moe_version",
)


class Shapes(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("L", ctypes.c_int32), ("F", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32)]


class Debug(ctypes.Structure):
    _fields_ = [
        ("h_q8_1", ctypes.c_void_p),
        ("perm", ctypes.c_void_p),
        ("offsets", ctypes.c_void_p),
        ("dropped", ctypes.c_void_p),
        ("gateup_i32", ctypes.c_void_p),
        ("gu_row0", ctypes.c_int32),
        ("gu_rows", ctypes.c_int32),
        ("down_i32", ctypes.c_void_p),
        ("dn_row0", ctypes.c_int32),
        ("dn_rows", ctypes.c_int32),
        ("stage_events", ctypes.POINTER(ctypes.c_void_p)),
        ("deterministic", ctypes.c_int32),
    ]


class LatMoeError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Load liblatmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LatMoeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(or python quantized_latent_moe_amd/build.py)")
        c = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        c.lat_moe_workspace_size.argtypes = [ctypes.POINTER(Shapes)]
        c.lat_moe_workspace_size.restype = ctypes.c_size_t
        c.lat_moe_expert_forward.argtypes = [P, P, P, P, P, ctypes.POINTER(Shapes), P, P, ctypes.c_size_t, P]
        c.lat_moe_expert_forward.restype = ctypes.c_int
        c.lat_moe_expert_forward_ex.argtypes = [P, P, P, P, P, ctypes.POINTER(Shapes), P, P, ctypes.c_size_t, P,
                                                ctypes.POINTER(Debug)]
        c.lat_moe_expert_forward_ex.restype = ctypes.c_int
        c.lat_moe_expert_forward_fmt.argtypes = [P, P, P, P, ctypes.c_int32, P, ctypes.c_int32,
                                                 ctypes.POINTER(Shapes), P, P, ctypes.c_size_t, P,
                                                 ctypes.POINTER(Debug)]
        c.lat_moe_expert_forward_fmt.restype = ctypes.c_int
        c.lat_moe_expert_forward_noalloc.argtypes = [P, P, P, P, P, ctypes.POINTER(Shapes), P, P]
        c.lat_moe_expert_forward_noalloc.restype = ctypes.c_int
        c.lat_moe_quantize_q8_1.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P]
        c.lat_moe_quantize_q8_1.restype = ctypes.c_int
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        c.lat_moe_dense_q8_0.argtypes = [P, P, i64, i32, i32, P, P, P]
        c.lat_moe_dense_q8_0.restype = ctypes.c_int
        c.lat_moe_dense_q8_0_debug.argtypes = [P, P, i64, i32, i32, P, P, P, P, i32, i32]
        c.lat_moe_dense_q8_0_debug.restype = ctypes.c_int
        c.lat_moe_dense_q4_0.argtypes = [P, P, i64, i32, i32, P, P, P]
        c.lat_moe_dense_q4_0.restype = ctypes.c_int
        c.lat_moe_dense_q4_0_debug.argtypes = [P, P, i64, i32, i32, P, P, P, P, i32, i32]
        c.lat_moe_dense_q4_0_debug.restype = ctypes.c_int
        c.lat_moe_router_topk.argtypes = [P, i64, i32, i32, P, P, P]
        c.lat_moe_router_topk.restype = ctypes.c_int
        c.lat_moe_strerror.argtypes = [ctypes.c_int]
        c.lat_moe_strerror.restype = ctypes.c_char_p
        c.lat_moe_version.restype = ctypes.c_int
        _lib = c
    return _lib


def strerror(code: int) -> str:
    return lib().lat_moe_strerror(int(code)).decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise LatMoeError(f"lat_moe error {rc}: {strerror(rc)}")


def shapes(T: int, L: int, F: int, E: int, k: int) -> Shapes:
    return Shapes(int(T), int(L), int(F), int(E), int(k))


def workspace_size(s: Shapes) -> int:
    return int(lib().lat_moe_workspace_size(ctypes.byref(s)))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def expert_forward(x_q8_1, router_idx, router_w, gateup_q3k, down_iq4nl, s: Shapes, y, workspace,
                   stream=None) -> None:
    """Enqueue the expert stage; all tensors on the current GPU (uint8 blocks,
    int32 ids, fp32 weights, fp32 y [T, L], uint8 workspace)."""
    rc = lib().lat_moe_expert_forward(_ptr(x_q8_1), _ptr(router_idx), _ptr(router_w), _ptr(gateup_q3k),
                                      _ptr(down_iq4nl), ctypes.byref(s), _ptr(y), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc)


NOALLOC_SCRATCH_BYTES = 64 << 20
ESCRATCH = 5


def expert_forward_noalloc(x_q8_1, router_idx, router_w, gateup_q3k, down_iq4nl, s: Shapes, y, stream=None) -> None:
    """As expert_forward without a workspace: the library's fixed per-GPU
    scratch (NOALLOC_SCRATCH_BYTES) is used, and nothing is allocated."""
    rc = lib().lat_moe_expert_forward_noalloc(_ptr(x_q8_1), _ptr(router_idx), _ptr(router_w), _ptr(gateup_q3k),
                                              _ptr(down_iq4nl), ctypes.byref(s), _ptr(y), _stream(stream))
    _check(rc)


def _debug(h_q8_1, perm, offsets, dropped, gateup_i32, gu_row0, down_i32, dn_row0, stage_events, deterministic):
    ev = None
    if stage_events is not None:
        if len(stage_events) != 5:
            raise ValueError("stage_events needs 5 events")
        ev = (ctypes.c_void_p * 5)(*[int(e.cuda_event) for e in stage_events])
    d = Debug(_ptr(h_q8_1), _ptr(perm), _ptr(offsets), _ptr(dropped), _ptr(gateup_i32), int(gu_row0),
              0 if gateup_i32 is None else int(gateup_i32.shape[1]), _ptr(down_i32), int(dn_row0),
              0 if down_i32 is None else int(down_i32.shape[1]),
              ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)) if ev is not None else None,
              1 if deterministic else 0)
    return d, ev


def expert_forward_ex(x_q8_1, router_idx, router_w, gateup_q3k, down_iq4nl, s: Shapes, y, workspace, *,
                      deterministic: bool = True, h_q8_1=None, perm=None, offsets=None, dropped=None, gateup_i32=None,
                      gu_row0=0, down_i32=None, dn_row0=0, stage_events=None, stream=None) -> None:
    """As expert_forward, with the options and optional debug outputs of
    lat_moe_debug: deterministic=False sums each token's experts into y by
    fp32 atomic adds (no slot buffer, no combine kernel); gateup_i32 is
    [T*k, rows, L/32] int32 and down_i32 [T*k, rows, F/32]; stage_events is a
    list of five recorded torch.cuda.Event(enable_timing=True)."""
    d, ev = _debug(h_q8_1, perm, offsets, dropped, gateup_i32, gu_row0, down_i32, dn_row0, stage_events,
                   deterministic)
    rc = lib().lat_moe_expert_forward_ex(_ptr(x_q8_1), _ptr(router_idx), _ptr(router_w), _ptr(gateup_q3k),
                                         _ptr(down_iq4nl), ctypes.byref(s), _ptr(y), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream),
                                         ctypes.byref(d))
    _check(rc)


def expert_forward_fmt(x_q8_1, router_idx, router_w, gateup, down, down_format: int, s: Shapes, y, workspace, *,
                       gateup_format: int = GATEUP_Q3_K, debug: bool = False, deterministic: bool = True,
                       h_q8_1=None, perm=None, offsets=None, dropped=None, gateup_i32=None, gu_row0=0, down_i32=None,
                       dn_row0=0, stage_events=None, stream=None) -> None:
    """The expert stage with gate/up weights in gateup_format (GATEUP_Q3_K:
    [E, 2F, L/256, 110]; GATEUP_Q4_0: [E, 2F, L/32, 18]) and down weights in
    down_format (DOWN_IQ4_NL or DOWN_Q4_0, both [E, L, F/32, 18] uint8); with
    debug=True (or deterministic=False) the options and optional outputs of
    expert_forward_ex are passed, otherwise no debug struct is."""
    d = None
    if debug or not deterministic:
        d, ev = _debug(h_q8_1, perm, offsets, dropped, gateup_i32, gu_row0, down_i32, dn_row0, stage_events,
                       deterministic)
    rc = lib().lat_moe_expert_forward_fmt(_ptr(x_q8_1), _ptr(router_idx), _ptr(router_w), _ptr(gateup),
                                          int(gateup_format), _ptr(down), int(down_format), ctypes.byref(s), _ptr(y),
                                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(stream), ctypes.byref(d) if d is not None else None)
    _check(rc)


def quantize_q8_1(x, out, stream=None) -> None:
    """fp32 [rows, cols] -> q8_1 blocks (uint8 [rows, cols/32, 36])."""
    rows, cols = x.shape
    _check(lib().lat_moe_quantize_q8_1(_ptr(x), int(rows), int(cols), _ptr(out), _stream(stream)))


def dense_q8_0(x_q8_1, w_q8_0, T: int, N: int, K: int, y_f32=None, y_q8_1=None, *, dots_i32=None, row0: int = 0,
               stream=None) -> None:
    """Latent D / U projection: q8_1 rows x_q8_1 (uint8 [T, K/32, 36]) against
    Q8_0 weights (uint8 [N, K/32, 34]) -> y_f32 (fp32 [T, N]) and/or y_q8_1
    (uint8 [T, N/32, 36]); dots_i32 (int32 [T, rows, K/32]) takes the block
    dots of weight rows row0 .. row0+rows-1."""
    rows = 0 if dots_i32 is None else int(dots_i32.shape[1])
    _check(lib().lat_moe_dense_q8_0_debug(_ptr(x_q8_1), _ptr(w_q8_0), int(T), int(N), int(K), _ptr(y_f32),
                                          _ptr(y_q8_1), _stream(stream), _ptr(dots_i32), int(row0), rows))


def dense_q4_0(x_q8_1, w_q4_0, T: int, N: int, K: int, y_f32=None, y_q8_1=None, *, dots_i32=None, row0: int = 0,
               stream=None) -> None:
    """As dense_q8_0 with Q4_0 weights (uint8 [N, K/32, 18])."""
    rows = 0 if dots_i32 is None else int(dots_i32.shape[1])
    _check(lib().lat_moe_dense_q4_0_debug(_ptr(x_q8_1), _ptr(w_q4_0), int(T), int(N), int(K), _ptr(y_f32),
                                          _ptr(y_q8_1), _stream(stream), _ptr(dots_i32), int(row0), rows))


def router_topk(logits, k: int, router_idx, router_w, stream=None) -> None:
    """fp32 logits [T, E] -> top-k expert ids (int32 [T, k]) and renormalised
    softmax weights (fp32 [T, k]), the expert stage's routing inputs."""
    T, E = logits.shape
    _check(lib().lat_moe_router_topk(_ptr(logits), int(T), int(E), int(k), _ptr(router_idx), _ptr(router_w),
                                     _stream(stream)))


def version() -> int:
    return int(lib().lat_moe_version())
