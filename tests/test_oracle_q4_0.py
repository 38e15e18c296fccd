"""Pins for the oracle's Q4_0 down-weight format.

Q4_0 (ggml's public GGUF block, one of the weight formats the PR page of "Run
Edge0-145B Q3_K on AMD HIP (Linux, gfx1100) #1" names in section "Not done"):
32 weights in 18 bytes, fp16 d then 16 bytes of nibbles in IQ4_NL's places
(element i < 16: low nibble of byte i; i >= 16: high nibble of byte i - 16),
weight = d * (nibble - 8).  Pinned by:
* the decode against nibbles unpacked here with numpy, and a hand block whose
  values follow by eye;
* the stage with Q4_0 down weights against a dense fp64 evaluation on exactly
  dequantized tensors, and its integer block dots against numpy integer sums;
* the down format leaves gate/up and H unchanged, and y is linear in the
  down weights' d.
"""
import numpy as np
import pytest

import oracle
from quantized_latent_moe_amd.inputs import Workload, make_inputs
from tests._packers import pack_iq4nl


def _nibbles(blocks):
    qs = blocks[..., 2:18].astype(np.int64)
    return np.concatenate([qs & 15, qs >> 4], axis=-1)  # [..., 32] in element order


def _d(blocks):
    return blocks[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)


def test_q4_0_decode():
    rng = np.random.default_rng(5)
    nib = rng.integers(0, 16, (400, 32))
    d = rng.uniform(-2, 2, 400).astype(np.float16)
    b = pack_iq4nl(nib, d)                     # the same byte layout
    assert np.array_equal(_nibbles(b), nib)
    out = oracle.dequant_q4_0(b)
    assert np.array_equal(out, d.astype(np.float64)[:, None] * (nib - 8))
    # hand block: low nibbles 0..15, high nibbles 15..0, d = 0.5
    h = np.zeros(18, np.uint8)
    h[0:2] = np.array([0.5], np.float16).view(np.uint8)
    h[2:18] = np.arange(16) | ((15 - np.arange(16)) << 4)
    vals = list(range(-8, 8))
    assert oracle.dequant_q4_0(h[None])[0].tolist() == [0.5 * v for v in vals + vals[::-1]]


def _case(T, L, F, E, k, seed):
    I = make_inputs(Workload("q40", T=T, L=L, F=F, E=E, k=k, seed=seed))
    return I, oracle.quantize_q8_1(I.x)


def _silu(g):
    return g / (1.0 + np.exp(-g))


@pytest.mark.parametrize("L,F,E,k", [(256, 64, 3, 2), (512, 96, 4, 3)])
def test_stage_with_q4_0_down_bruteforce(L, F, E, k):
    T = 5
    I, xq = _case(T, L, F, E, k, seed=L + 7 * F)
    dn = I.down_iq4nl                           # random bytes: read as Q4_0 blocks
    r = oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, dn, L, F, E, down_format="q4_0")
    xd = oracle.dequant_q8_1(xq).reshape(T, L)
    Wgu = oracle.dequant_q3k(I.gateup_q3k).reshape(E, 2 * F, L)
    Wd = (_d(dn)[..., None] * (_nibbles(dn) - 8)).reshape(E, L, F)
    for t in range(T):
        y = np.zeros(L)
        for j in range(k):
            e, p = I.router_idx[t, j], t * k + j
            gu = Wgu[e] @ xd[t]
            hq = oracle.quantize_q8_1((_silu(gu[:F]) * gu[F:]).astype(np.float32)[None, :])[0]
            assert np.array_equal(hq, r.h[p])
            y += np.float64(I.router_w[t, j]) * (Wd[e] @ oracle.dequant_q8_1(r.h[p]).reshape(F))
        assert np.abs(r.y[t] - y).max() <= 1e-12 * np.abs(y).max()


def test_q4_0_block_dots_bruteforce():
    L, F, E, k = 256, 96, 3, 2
    I, xq = _case(4, L, F, E, k, seed=21)
    r = oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, I.down_iq4nl, L, F, E, down_format="q4_0")
    rng = np.random.default_rng(1)
    pairs = rng.integers(0, 4 * k, 30)
    rows = rng.integers(0, L, 30).astype(np.int32)
    j32 = oracle.probe_down(r.h, I.router_idx, I.down_iq4nl, L, F, E, pairs, rows, down_format="q4_0")
    qh = r.h[..., 4:].view(np.int8).reshape(4 * k, F).astype(np.int64)
    for n, (p, ll) in enumerate(zip(pairs, rows)):
        e = I.router_idx.reshape(-1)[p]
        v = (_nibbles(I.down_iq4nl[e, ll]) - 8).reshape(-1)
        assert np.array_equal(j32[n], (v * qh[p]).reshape(F // 32, 32).sum(-1))


def test_down_format_leaves_h_and_scales_linearly():
    L, F, E, k = 256, 64, 4, 2
    I, xq = _case(6, L, F, E, k, seed=3)
    a = oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, I.down_iq4nl, L, F, E)
    b = oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, I.down_iq4nl, L, F, E, down_format="q4_0")
    assert np.array_equal(a.h, b.h)
    # doubling every down block's d (exact in fp16) doubles y exactly
    dn2 = I.down_iq4nl.copy()
    d = dn2[..., 0:2].copy().view(np.float16)
    dn2[..., 0:2] = (d * np.float16(2)).view(np.uint8)
    c = oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, dn2, L, F, E, down_format="q4_0")
    assert np.array_equal(c.y, 2 * b.y)
    # and the down-only path agrees with the full stage
    y = oracle.down_combine(b.h, I.router_idx, I.router_w, I.down_iq4nl, L, F, E, down_format="q4_0")
    assert np.array_equal(y, b.y)


# ---- Q4_0 as the weight format of the latent D / U projections -------------

def _dense_case(T, N, K, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, K)) * np.exp(rng.uniform(-1, 1, (T, 1)))).astype(np.float32)
    xq = oracle.quantize_q8_1(x)
    nib = rng.integers(0, 16, (N, K // 32, 32))
    d = rng.uniform(0.5, 1.5, (N, K // 32)).astype(np.float16) * np.float16(2.0 ** -8)
    w = pack_iq4nl(nib.reshape(-1, 32), d.reshape(-1)).reshape(N, K // 32, 18)
    return xq, w, nib, d


@pytest.mark.parametrize("T,N,K", [(5, 96, 256), (3, 64, 1024)])
def test_dense_q4_0_bruteforce(T, N, K):
    """fp64 matmul of the exactly dequantized operands (non-square: a
    transposed operand or a wrong block index fails)."""
    xq, w, nib, d = _dense_case(T, N, K, seed=T + N)
    y = oracle.dense_q8_0(xq, w, N, K, w_format="q4_0")
    W = (d.astype(np.float64)[..., None] * (nib - 8)).reshape(N, K)
    X = oracle.dequant_q8_1(xq).reshape(T, K)
    ref = X @ W.T
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()


def test_dense_q4_0_block_dots_and_q8_0_equivalence():
    T, N, K = 4, 64, 512
    xq, w, nib, d = _dense_case(T, N, K, seed=7)
    rng = np.random.default_rng(2)
    toks = rng.integers(0, T, 40)
    rows = rng.integers(0, N, 40).astype(np.int32)
    dots = oracle.probe_dense(xq, w, N, K, toks, rows, w_format="q4_0")
    qx = xq[..., 4:].view(np.int8).reshape(T, K // 32, 32).astype(np.int64)
    for i, (t, r) in enumerate(zip(toks, rows)):
        assert np.array_equal(dots[i], ((nib[r] - 8) * qx[t]).sum(-1))
    # the same weights written as Q8_0 blocks (codes nibble - 8, the same d)
    # give the same projection, bit for bit
    w8 = np.zeros((N, K // 32, 34), np.uint8)
    w8[..., 0:2] = d.reshape(N, K // 32, 1).view(np.uint8)
    w8[..., 2:] = (nib - 8).astype(np.int8).view(np.uint8)
    assert np.array_equal(oracle.dense_q8_0(xq, w8, N, K), oracle.dense_q8_0(xq, w, N, K, w_format="q4_0"))


# ---- Q4_0 as the weight format of the expert's gate/up rows ----------------

@pytest.mark.parametrize("L,F,E,k", [(256, 64, 3, 2), (512, 96, 4, 3)])
def test_stage_with_q4_0_gateup_bruteforce(L, F, E, k):
    """Q4_0 gate/up (a weight scale per 32 values) and Q4_0 down against a
    dense fp64 evaluation on exactly dequantized tensors."""
    from quantized_latent_moe_amd.inputs import make_gateup_q4_0
    T = 5
    I, xq = _case(T, L, F, E, k, seed=3 * L + F)
    gu = make_gateup_q4_0(I.wl)
    assert gu.shape == (E, 2 * F, L // 32, 18)
    r = oracle.forward(xq, I.router_idx, I.router_w, gu, I.down_iq4nl, L, F, E, want_gu=True,
                       gateup_format="q4_0", down_format="q4_0")
    xd = oracle.dequant_q8_1(xq).reshape(T, L)
    Wgu = (_d(gu)[..., None] * (_nibbles(gu) - 8)).reshape(E, 2 * F, L)
    Wd = (_d(I.down_iq4nl)[..., None] * (_nibbles(I.down_iq4nl) - 8)).reshape(E, L, F)
    for t in range(T):
        y = np.zeros(L)
        for j in range(k):
            e, p = I.router_idx[t, j], t * k + j
            g = Wgu[e] @ xd[t]
            assert np.abs(r.gu[p] - g).max() <= 1e-12 * np.abs(g).max()
            hq = oracle.quantize_q8_1((_silu(g[:F]) * g[F:]).astype(np.float32)[None, :])[0]
            assert np.array_equal(hq, r.h[p])
            y += np.float64(I.router_w[t, j]) * (Wd[e] @ oracle.dequant_q8_1(r.h[p]).reshape(F))
        assert np.abs(r.y[t] - y).max() <= 1e-12 * np.abs(y).max()


def test_q4_0_gateup_block_dots_bruteforce():
    from quantized_latent_moe_amd.inputs import make_gateup_q4_0
    L, F, E, k = 512, 64, 3, 2
    I, xq = _case(4, L, F, E, k, seed=31)
    gu = make_gateup_q4_0(I.wl)
    rng = np.random.default_rng(5)
    pairs = rng.integers(0, 4 * k, 30)
    rows = rng.integers(0, 2 * F, 30).astype(np.int32)
    i32, i16 = oracle.probe_gateup(xq, I.router_idx, gu, L, F, E, pairs, rows, want_i16=True, gateup_format="q4_0")
    q = xq[..., 4:].view(np.int8).reshape(4, L).astype(np.int64)
    for n, (p, rr) in enumerate(zip(pairs, rows)):
        e = I.router_idx.reshape(-1)[p]
        v = (_nibbles(gu[e, rr]) - 8).reshape(-1)
        assert np.array_equal(i32[n], (v * q[p // k]).reshape(L // 32, 32).sum(-1))
        assert np.array_equal(i16[n], (v * q[p // k]).reshape(L // 16, 16).sum(-1))
