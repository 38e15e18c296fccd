"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, sizes its workspace, and rejects bad arguments before making
any HIP call."""
import ctypes
import os
import re

import pytest

import quantized_latent_moe_amd as lm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "lat_moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lat_moe_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert names == sorted(lm.EXPORTED)
    lib = lm.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert lm.version() >= 100


def test_boundary_entry_points_and_debug_struct():
    """The boundary's calls (workspace size, the stage, the stage with the
    debug struct, error strings) are exported, and the binding's debug struct
    has the header's fields in the header's order, the deterministic flag
    last."""
    for n in ("lat_moe_workspace_size", "lat_moe_expert_forward", "lat_moe_expert_forward_ex", "lat_moe_strerror"):
        assert n in _declared()
    src = open(os.path.join(ROOT, "include", "lat_moe.h")).read()
    body = re.search(r"typedef struct lat_moe_debug \{(.*?)\} lat_moe_debug;", src, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if decl:
            fields += [re.sub(r"[^\w]", "", n.split()[-1]) for n in decl.split(",")]
    assert fields == [f[0] for f in lm.Debug._fields_]
    assert fields[-1] == "deterministic"


def test_workspace_size():
    ok = lm.shapes(5268, 1024, 2048, 128, 8)
    ws = lm.workspace_size(ok)
    P = 5268 * 8
    # H codes + H scales + weighted slots + split activation rows dominate
    main = P * 2048 + P * 64 * 4 + P * 1024 * 4 + 5268 * 1024 + 5268 * 32 * 4
    assert main <= ws < main + (1 << 22)
    for bad in [(1, 100, 512, 8, 2), (1, 256, 40, 8, 2), (1, 256, 512, 0, 1), (1, 256, 512, 8, 9), (-1, 256, 512, 8, 2),
                (1, 256, 512, 2000, 2), (1 << 29, 256, 512, 8, 8)]:
        assert lm.workspace_size(lm.shapes(*bad)) == 0, bad


def _fwd(ptrs, s, ws_bytes):
    x, idx, w, gu, dn, y, ws = ptrs
    return lm.lib().lat_moe_expert_forward(x, idx, w, gu, dn, ctypes.byref(s), y, ws, ws_bytes, None)


def test_argument_errors_before_any_hip_call():
    s = lm.shapes(4, 256, 512, 8, 2)
    need = lm.workspace_size(s)
    good = [0x10000 * (i + 1) for i in range(7)]  # aligned, never dereferenced on these paths
    for i in range(7):
        p = list(good)
        p[i] = None
        assert _fwd(p, s, need) == 1
        p[i] = good[i] + 4
        assert _fwd(p, s, need) == 1
    assert _fwd(good, s, need - 1) == 2
    assert _fwd(good, lm.shapes(4, 200, 512, 8, 2), need) == 1
    # T = 0 is a no-op that touches nothing
    assert _fwd([None] * 7, lm.shapes(0, 256, 512, 8, 2), 0) == 0
    # debug row ranges are validated too
    fx = lm.lib().lat_moe_expert_forward_ex
    for det in (0, 1):
        d = lm.Debug(None, None, None, None, 0x1000, 1000, 40, None, 0, 0, None, det)
        assert fx(*good[:5], ctypes.byref(s), good[5], good[6], need, None, ctypes.byref(d)) == 1
        d = lm.Debug(None, None, None, None, None, 0, 0, 0x1000, 250, 7, None, det)
        assert fx(*good[:5], ctypes.byref(s), good[5], good[6], need, None, ctypes.byref(d)) == 1
    # _ex with no debug struct is the plain call: same argument checks
    for i in range(7):
        p = list(good)
        p[i] = None
        assert fx(*p[:5], ctypes.byref(s), p[5], p[6], need, None, None) == 1
    assert fx(*good[:5], ctypes.byref(s), good[5], good[6], need - 1, None, None) == 2
    assert fx(None, None, None, None, None, ctypes.byref(lm.shapes(0, 256, 512, 8, 2)), None, None, 0, None,
              None) == 0
    # the format entry point: its format argument is checked first, then as above
    ex = lm.lib().lat_moe_expert_forward_fmt
    s0 = ctypes.byref(lm.shapes(0, 256, 512, 8, 2))
    for gfmt, dfmt, rc in ((lm.GATEUP_Q3_K, lm.DOWN_IQ4_NL, 0), (lm.GATEUP_Q4_0, lm.DOWN_Q4_0, 0),
                           (lm.GATEUP_Q3_K, 2, 1), (lm.GATEUP_Q3_K, -1, 1), (2, lm.DOWN_IQ4_NL, 1)):
        assert ex(None, None, None, None, gfmt, None, dfmt, s0, None, None, 0, None, None) == rc, (gfmt, dfmt)
    g5 = good[:4] + [lm.GATEUP_Q3_K, good[4]]
    assert ex(*g5, 7, ctypes.byref(s), good[5], good[6], need, None, None) == 1
    assert ex(*good[:4], lm.GATEUP_Q4_0, None, lm.DOWN_Q4_0, ctypes.byref(s), good[5], good[6], need, None, None) == 1
    assert ex(*g5, lm.DOWN_Q4_0, ctypes.byref(s), good[5], good[6], need - 1, None, None) == 2
    # one expert's Q4_0 gate/up rows past 2 GiB (Q3_K rows of the same shape fit)
    big = lm.shapes(1, 65536, 32768, 1, 1)
    assert ex(*good[:4], lm.GATEUP_Q4_0, good[4], lm.DOWN_Q4_0, ctypes.byref(big), good[5], good[6], 1 << 40, None,
              None) == 1
    assert lm.lib().lat_moe_quantize_q8_1(0x1000, 4, 40, 0x2000, None) == 1
    assert lm.lib().lat_moe_quantize_q8_1(0x1004, 4, 64, 0x2000, None) == 1
    assert lm.lib().lat_moe_quantize_q8_1(None, 0, 64, None, None) == 0


def test_noalloc_argument_errors_before_any_hip_call():
    """The no-allocation entry point checks its arguments, and the fixed
    scratch against the shapes' workspace, before any HIP call."""
    f = lm.lib().lat_moe_expert_forward_noalloc
    good = [0x10000 * (i + 1) for i in range(6)]  # aligned, never dereferenced on these paths
    s = lm.shapes(4, 1024, 2048, 128, 8)
    assert lm.workspace_size(s) <= lm.NOALLOC_SCRATCH_BYTES
    for i in range(6):
        p = list(good)
        p[i] = None
        assert f(*p[:5], ctypes.byref(s), p[5], None) == 1
        p[i] = good[i] + 4
        assert f(*p[:5], ctypes.byref(s), p[5], None) == 1
    assert f(*good[:5], ctypes.byref(lm.shapes(4, 200, 2048, 128, 8)), good[5], None) == 1
    big = lm.shapes(5268, 1024, 2048, 128, 8)
    assert lm.workspace_size(big) > lm.NOALLOC_SCRATCH_BYTES
    assert f(*good[:5], ctypes.byref(big), good[5], None) == lm.ESCRATCH
    assert "scratch" in lm.strerror(lm.ESCRATCH)
    assert f(None, None, None, None, None, ctypes.byref(lm.shapes(0, 1024, 2048, 128, 8)), None, None) == 0


def test_strerror():
    for c in range(6):
        assert lm.strerror(c)
    assert "unknown" in lm.strerror(99)


def test_dense_argument_errors_before_any_hip_call():
    f = lm.lib().lat_moe_dense_q8_0
    fd = lm.lib().lat_moe_dense_q8_0_debug
    x, w, y, q = 0x10000, 0x20000, 0x30000, 0x40000  # aligned, never dereferenced on these paths
    for T, N, K in [(4, 40, 64), (4, 64, 40), (4, 0, 64), (4, 64, 0), (-1, 64, 64), (4, 64, 1 << 17),
                    (1 << 30, 64, 64), (4, 65536, 65536)]:
        assert f(x, w, T, N, K, y, q, None) == 1, (T, N, K)
    assert f(x, w, 4, 64, 64, None, None, None) == 1           # no output
    assert f(x + 4, w, 4, 64, 64, y, None, None) == 1          # misaligned
    assert f(x, w + 2, 4, 64, 64, y, None, None) == 1
    assert f(x, w, 4, 64, 64, y + 8, None, None) == 1
    assert f(x, w, 4, 64, 64, None, q + 4, None) == 1
    assert f(None, w, 4, 64, 64, y, None, None) == 1
    assert fd(x, w, 4, 64, 64, y, None, None, 0x50000, 60, 8) == 1  # probe rows beyond N
    assert fd(x, w, 4, 64, 64, y, None, None, 0x50000, 0, 0) == 1
    # T = 0 is a no-op that touches nothing
    assert f(None, None, 0, 64, 64, y, None, None) == 0
    # Q4_0 weights: the same checks, plus the shape rule (T <= 8, or N % 128 == 0 and K % 256 == 0)
    f4 = lm.lib().lat_moe_dense_q4_0
    for T, N, K in [(4, 40, 64), (-1, 64, 64), (9, 96, 256), (200, 128, 288), (200, 160, 256), (8, 64, 8192),
                    (1 << 30, 128, 256)]:
        assert f4(x, w, T, N, K, y, q, None) == 1, (T, N, K)
    assert f4(x, w, 4, 64, 64, None, None, None) == 1
    assert f4(None, w, 200, 128, 256, y, None, None) == 1
    assert f4(None, None, 0, 128, 256, y, None, None) == 0


def test_router_argument_errors_before_any_hip_call():
    f = lm.lib().lat_moe_router_topk
    l, i, w = 0x10000, 0x20000, 0x30000
    for T, E, k in [(-1, 8, 2), (4, 0, 1), (4, 1025, 2), (4, 8, 0), (4, 8, 9), (4, 128, 65)]:
        assert f(l, T, E, k, i, w, None) == 1, (T, E, k)
    assert f(l + 4, 4, 8, 2, i, w, None) == 1
    assert f(l, 4, 8, 2, None, w, None) == 1
    assert f(None, 0, 8, 2, None, None, None) == 0   # T = 0: no-op
