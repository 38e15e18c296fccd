"""CPU oracle of the quantized latent-MoE expert stage (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``lat_moe_oracle.c`` (plain C,
OpenMP, fp64 folds) through ctypes and shares nothing with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lat_moe_oracle.c")
_LIB = os.path.join(_HERE, "liblatmoe_oracle.so")

# -ffp-contract=off: no fused multiply-add anywhere (the q8_1 rule must see
# separately rounded fp32 products); portable ISA so the library built here
# also runs on other x86-64 hosts.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=gnu11"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (always when ``force``)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        c = _lib
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        c.orc_half_to_double.argtypes = [ctypes.c_uint16]
        c.orc_half_to_double.restype = ctypes.c_double
        c.orc_float_to_half.argtypes = [ctypes.c_float]
        c.orc_float_to_half.restype = ctypes.c_uint16
        c.orc_quantize_q8_1.argtypes = [P, i64, i32, P]
        for f in (c.orc_dequant_q3k, c.orc_dequant_iq4nl, c.orc_dequant_q4_0, c.orc_dequant_q8_1):
            f.argtypes = [P, i64, P]
        c.orc_q3k_fields.argtypes = [P, i64, P, P, P]
        c.orc_iq4nl_fields.argtypes = [P, i64, P, P]
        c.orc_forward.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i32, P, i64, P, P, P]
        c.orc_forward.restype = i64
        c.orc_forward_fmt.argtypes = [P, P, P, P, i32, P, i32, i64, i32, i32, i32, i32, P, i64, P, P, P]
        c.orc_probe_gateup_fmt.argtypes = [P, P, P, i32, i64, i32, i32, i32, i32, i64, P, P, P, P]
        c.orc_forward_fmt.restype = i64
        c.orc_down_combine.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, P, i64, P]
        c.orc_h_blocks_fmt.argtypes = [P, P, P, i32, i64, i32, i32, i32, i32, i64, P, P, P]
        c.orc_down_combine_fmt.argtypes = [P, P, P, P, i32, i64, i32, i32, i32, i32, P, i64, P]
        c.orc_probe_down_fmt.argtypes = [P, P, P, i32, i64, i32, i32, i32, i32, i64, P, P, P]
        c.orc_probe_gateup.argtypes = [P, P, P, i64, i32, i32, i32, i32, i64, P, P, P, P]
        c.orc_probe_down.argtypes = [P, P, P, i64, i32, i32, i32, i32, i64, P, P, P]
        c.orc_dequant_q8_0.argtypes = [P, i64, P]
        c.orc_dense_q8_0.argtypes = [P, i64, P, i32, i32, P, i64, P]
        c.orc_probe_dense.argtypes = [P, i64, P, i32, i32, i64, P, P, P]
        c.orc_dense_fmt.argtypes = [P, i64, P, i32, i32, i32, P, i64, P]
        c.orc_probe_dense_fmt.argtypes = [P, i64, P, i32, i32, i32, i64, P, P, P]
        c.orc_router_topk.argtypes = [P, i64, i32, i32, P, P]
        c.orc_num_threads.restype = ctypes.c_int
        c.orc_set_num_threads.argtypes = [ctypes.c_int]
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


def half_to_double(bits: int) -> float:
    return lib().orc_half_to_double(int(bits))


def float_to_half(f: float) -> int:
    return lib().orc_float_to_half(float(f))


def quantize_q8_1(x: np.ndarray) -> np.ndarray:
    """fp32 [rows, cols] -> q8_1 bytes [rows, cols/32, 36]."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    out = np.zeros((rows, cols // 32, 36), np.uint8)
    lib().orc_quantize_q8_1(_p(x), rows, cols, _p(out))
    return out


def dequant_q3k(blocks: np.ndarray) -> np.ndarray:
    b = _c(blocks, np.uint8)
    n = b.size // 110
    out = np.empty(n * 256, np.float64)
    lib().orc_dequant_q3k(_p(b), n, _p(out))
    return out.reshape(b.shape[:-1] + (256,))


def dequant_iq4nl(blocks: np.ndarray) -> np.ndarray:
    b = _c(blocks, np.uint8)
    n = b.size // 18
    out = np.empty(n * 32, np.float64)
    lib().orc_dequant_iq4nl(_p(b), n, _p(out))
    return out.reshape(b.shape[:-1] + (32,))


def dequant_q4_0(blocks: np.ndarray) -> np.ndarray:
    """Q4_0 blocks (18 B: fp16 d | 16 nibble bytes) -> d * (nibble - 8)."""
    b = _c(blocks, np.uint8)
    n = b.size // 18
    out = np.empty(n * 32, np.float64)
    lib().orc_dequant_q4_0(_p(b), n, _p(out))
    return out.reshape(b.shape[:-1] + (32,))


# Formats of the down weights (both 18 bytes per 32 weights, the same layout)
# and of the gate/up weights (Q3_K super-blocks, or Q4_0 blocks).
DOWN_FORMATS = {"iq4_nl": 0, "q4_0": 1}
GATEUP_FORMATS = {"q3_k": 0, "q4_0": 1}


def dequant_q8_1(blocks: np.ndarray) -> np.ndarray:
    b = _c(blocks, np.uint8)
    n = b.size // 36
    out = np.empty(n * 32, np.float64)
    lib().orc_dequant_q8_1(_p(b), n, _p(out))
    return out.reshape(b.shape[:-1] + (32,))


def q3k_fields(blocks: np.ndarray):
    """-> (v [n,256] in -4..3, sigma [n,16] in -32..31, d [n])."""
    b = _c(blocks, np.uint8).reshape(-1, 110)
    n = b.shape[0]
    v = np.empty((n, 256), np.int8)
    s = np.empty((n, 16), np.int8)
    d = np.empty(n, np.float64)
    lib().orc_q3k_fields(_p(b), n, _p(v), _p(s), _p(d))
    return v, s, d


def iq4nl_fields(blocks: np.ndarray):
    """-> (table values [n,32], d [n])."""
    b = _c(blocks, np.uint8).reshape(-1, 18)
    n = b.shape[0]
    kv = np.empty((n, 32), np.int8)
    d = np.empty(n, np.float64)
    lib().orc_iq4nl_fields(_p(b), n, _p(kv), _p(d))
    return kv, d


class Result:
    def __init__(self, y, h, gu, dropped):
        self.y, self.h, self.gu, self.dropped = y, h, gu, dropped


def forward(x_q8: np.ndarray, router_idx: np.ndarray, router_w: np.ndarray, gateup: np.ndarray,
            down: np.ndarray, L: int, F: int, E: int, tokens: Optional[Sequence[int]] = None,
            want_h: bool = True, want_gu: bool = False, down_format: str = "iq4_nl",
            gateup_format: str = "q3_k") -> Result:
    """Whole stage.  y is fp64 [n_tok, L]; h is q8_1 [n_tok*k, F/32, 36] in
    pair order of the evaluated tokens; gu is fp64 [n_tok*k, 2F].  The down
    weights are IQ4_NL or (down_format "q4_0") Q4_0 blocks; the gate/up
    weights Q3_K or (gateup_format "q4_0") Q4_0 blocks [E, 2F, L/32, 18]."""
    x_q8 = _c(x_q8, np.uint8)
    idx = _c(router_idx, np.int32)
    w = _c(router_w, np.float32)
    T, k = idx.shape
    gateup = _c(gateup, np.uint8)
    down = _c(down, np.uint8)
    tok = None if tokens is None else _c(tokens, np.int64)
    n_tok = T if tok is None else tok.size
    y = np.zeros((n_tok, L), np.float64)
    h = np.zeros((n_tok * k, F // 32, 36), np.uint8) if want_h else None
    gu = np.zeros((n_tok * k, 2 * F), np.float64) if want_gu else None
    dropped = lib().orc_forward_fmt(_p(x_q8), _p(idx), _p(w), _p(gateup), GATEUP_FORMATS[gateup_format], _p(down),
                                    DOWN_FORMATS[down_format], T, L, F, E, k, _p(tok), n_tok, _p(y), _p(h), _p(gu))
    return Result(y, h, gu, int(dropped))


def down_combine(h_q8: np.ndarray, router_idx: np.ndarray, router_w: np.ndarray, down: np.ndarray, L: int, F: int,
                 E: int, tokens: Optional[Sequence[int]] = None, down_format: str = "iq4_nl") -> np.ndarray:
    """y from given H (q8_1 [T*k, F/32, 36], pair order over ALL T tokens)."""
    h = _c(h_q8, np.uint8)
    idx = _c(router_idx, np.int32)
    w = _c(router_w, np.float32)
    T, k = idx.shape
    tok = None if tokens is None else _c(tokens, np.int64)
    n_tok = T if tok is None else tok.size
    y = np.zeros((n_tok, L), np.float64)
    lib().orc_down_combine_fmt(_p(h), _p(idx), _p(w), _p(_c(down, np.uint8)), DOWN_FORMATS[down_format], T, L, F, E,
                               k, _p(tok), n_tok, _p(y))
    return y


def h_blocks(x_q8, router_idx, gateup, L, F, E, pairs, fblocks, gateup_format="q3_k"):
    """H q8_1 blocks of chosen (pair, 32-feature block) entries -> uint8 [n, 36]:
    the forward's G/U rows of those features, SwiGLU and the q8_1 rounding."""
    idx = _c(router_idx, np.int32)
    T, k = idx.shape
    pairs = _c(pairs, np.int64)
    fb = _c(fblocks, np.int32)
    assert pairs.size == fb.size and (fb.size == 0 or (fb.min() >= 0 and fb.max() < F // 32))
    assert pairs.size == 0 or (pairs.min() >= 0 and pairs.max() < T * k)
    out = np.zeros((pairs.size, 36), np.uint8)
    lib().orc_h_blocks_fmt(_p(_c(x_q8, np.uint8)), _p(idx), _p(_c(gateup, np.uint8)), GATEUP_FORMATS[gateup_format],
                           T, L, F, E, k, pairs.size, _p(pairs), _p(fb), _p(out))
    return out


def probe_gateup(x_q8, router_idx, gateup, L, F, E, pairs, rows, want_i16=False, gateup_format="q3_k"):
    idx = _c(router_idx, np.int32)
    T, k = idx.shape
    pairs = _c(pairs, np.int64)
    rows = _c(rows, np.int32)
    n = pairs.size
    o32 = np.zeros((n, L // 32), np.int32)
    o16 = np.zeros((n, L // 16), np.int32) if want_i16 else None
    lib().orc_probe_gateup_fmt(_p(_c(x_q8, np.uint8)), _p(idx), _p(_c(gateup, np.uint8)),
                               GATEUP_FORMATS[gateup_format], T, L, F, E, k, n, _p(pairs), _p(rows), _p(o32), _p(o16))
    return (o32, o16) if want_i16 else o32


def probe_down(h_q8, router_idx, down, L, F, E, pairs, rows, down_format="iq4_nl"):
    idx = _c(router_idx, np.int32)
    T, k = idx.shape
    pairs = _c(pairs, np.int64)
    rows = _c(rows, np.int32)
    n = pairs.size
    out = np.zeros((n, F // 32), np.int32)
    lib().orc_probe_down_fmt(_p(_c(h_q8, np.uint8)), _p(idx), _p(_c(down, np.uint8)), DOWN_FORMATS[down_format], T, L,
                             F, E, k, n, _p(pairs), _p(rows), _p(out))
    return out


def dequant_q8_0(blocks: np.ndarray) -> np.ndarray:
    b = _c(blocks, np.uint8)
    n = b.size // 34
    out = np.empty(n * 32, np.float64)
    lib().orc_dequant_q8_0(_p(b), n, _p(out))
    return out.reshape(b.shape[:-1] + (32,))


DENSE_FORMATS = {"q8_0": 0, "q4_0": 1}


def dense_q8_0(x_q8: np.ndarray, w_q8_0: np.ndarray, N: int, K: int,
               tokens: Optional[Sequence[int]] = None, w_format: str = "q8_0") -> np.ndarray:
    """Latent D / U projection: x q8_1 [T, K/32, 36] against Q8_0 weights
    [N, K/32, 34] (or, w_format "q4_0", Q4_0 weights [N, K/32, 18]) -> fp64
    [n_tok, N] (block dots folded in fp64)."""
    x = _c(x_q8, np.uint8)
    T = x.size // ((K // 32) * 36)
    tok = None if tokens is None else _c(tokens, np.int64)
    n_tok = T if tok is None else tok.size
    y = np.zeros((n_tok, N), np.float64)
    lib().orc_dense_fmt(_p(x), T, _p(_c(w_q8_0, np.uint8)), DENSE_FORMATS[w_format], N, K, _p(tok), n_tok, _p(y))
    return y


def probe_dense(x_q8, w_q8_0, N, K, tokens, rows, w_format="q8_0"):
    """Integer block dots of (token, weight row) probes -> int32 [n, K/32]."""
    x = _c(x_q8, np.uint8)
    T = x.size // ((K // 32) * 36)
    tok = _c(tokens, np.int64)
    rows = _c(rows, np.int32)
    assert tok.size == rows.size and (tok.size == 0 or (tok.min() >= 0 and tok.max() < T))
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < N)
    out = np.zeros((tok.size, K // 32), np.int32)
    lib().orc_probe_dense_fmt(_p(x), T, _p(_c(w_q8_0, np.uint8)), DENSE_FORMATS[w_format], N, K, tok.size, _p(tok),
                              _p(rows), _p(out))
    return out


def router_topk(logits: np.ndarray, k: int):
    """fp32 logits [T, E] -> (ids int32 [T, k], weights fp32 [T, k]): softmax,
    top-k (ties to the lower expert), weights renormalised over the picks."""
    l = _c(logits, np.float32)
    T, E = l.shape
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float32)
    lib().orc_router_topk(_p(l), T, E, k, _p(idx), _p(w))
    return idx, w
