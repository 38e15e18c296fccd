"""Pins for the oracle's expert stage.

* brute force: dense fp64 matmuls on exactly dequantized weights and
  activations reproduce the oracle's per-block integer folds (G, U, O, y)
  to fp64 rounding, and numpy integer matmuls reproduce the integer block
  dots (I32, I16, J32) exactly;
* invariants: zero router weights give zero output, doubling the weights
  doubles y, permuting tokens permutes y, permuting slots or splitting a
  duplicate slot changes y only by rounding, invalid ids act as weight 0,
  experts without tokens have no effect;
* special case E = k = 1, w = 1: a textbook dense SwiGLU FFN, up to the
  bounded error of the q8_1 rounding of H.
"""
import numpy as np
import pytest

import oracle
from quantized_latent_moe_amd.inputs import Workload, make_inputs


def _case(T=6, L=512, F=96, E=3, k=2, seed=0, zipf=0.0):
    I = make_inputs(Workload("t", T=T, L=L, F=F, E=E, k=k, zipf_s=zipf, seed=seed))
    xq = oracle.quantize_q8_1(I.x)
    return I, xq


def _silu(g):
    return g / (1.0 + np.exp(-g))


@pytest.mark.parametrize("L,F,E,k", [(256, 64, 3, 2), (512, 96, 4, 3)])
def test_dense_bruteforce(L, F, E, k):
    I, xq = _case(T=5, L=L, F=F, E=E, k=k, seed=L + F)
    r = oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, I.down_iq4nl, L, F, E, want_gu=True)
    xd = oracle.dequant_q8_1(xq).reshape(5, L)
    Wgu = oracle.dequant_q3k(I.gateup_q3k).reshape(E, 2 * F, L)
    Wd = oracle.dequant_iq4nl(I.down_iq4nl).reshape(E, L, F)
    for t in range(5):
        y = np.zeros(L)
        for j in range(k):
            e, p = I.router_idx[t, j], t * k + j
            gu = Wgu[e] @ xd[t]
            scale = np.abs(gu).max()
            assert np.abs(r.gu[p] - gu).max() <= 1e-12 * scale
            hd = _silu(gu[:F]) * gu[F:]
            hq = oracle.quantize_q8_1(hd.astype(np.float32)[None, :])[0]
            assert np.array_equal(hq, r.h[p])
            o = Wd[e] @ oracle.dequant_q8_1(r.h[p]).reshape(F)
            y += np.float64(I.router_w[t, j]) * o
        assert np.abs(r.y[t] - y).max() <= 1e-12 * np.abs(y).max()


def test_integer_block_dots_bruteforce():
    L, F, E, k = 512, 64, 3, 2
    I, xq = _case(T=4, L=L, F=F, E=E, k=k, seed=9)
    r = oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, I.down_iq4nl, L, F, E)
    rng = np.random.default_rng(0)
    pairs = rng.integers(0, 4 * k, 40)
    rows = rng.integers(0, 2 * F, 40).astype(np.int32)
    i32, i16 = oracle.probe_gateup(xq, I.router_idx, I.gateup_q3k, L, F, E, pairs, rows, want_i16=True)
    q = xq[..., 4:].view(np.int8).reshape(4, L).astype(np.int64)
    for n, (p, rr) in enumerate(zip(pairs, rows)):
        e = I.router_idx.reshape(-1)[p]
        v, sg, _ = oracle.q3k_fields(I.gateup_q3k[e, rr])
        v = v.reshape(-1).astype(np.int64)
        sg = np.repeat(sg.reshape(-1).astype(np.int64), 16)
        qt = q[p // k]
        assert np.array_equal(i32[n], ((sg * v) * qt).reshape(L // 32, 32).sum(-1))
        assert np.array_equal(i16[n], (v * qt).reshape(L // 16, 16).sum(-1))
    drows = rng.integers(0, L, 40).astype(np.int32)
    j32 = oracle.probe_down(r.h, I.router_idx, I.down_iq4nl, L, F, E, pairs, drows)
    qh = r.h[..., 4:].view(np.int8).reshape(4 * k, F).astype(np.int64)
    for n, (p, ll) in enumerate(zip(pairs, drows)):
        e = I.router_idx.reshape(-1)[p]
        kv, _ = oracle.iq4nl_fields(I.down_iq4nl[e, ll])
        assert np.array_equal(j32[n], (kv.reshape(-1).astype(np.int64) * qh[p]).reshape(F // 32, 32).sum(-1))


def _fwd(I, xq, idx=None, w=None, gu=None, dn=None):
    wl = I.wl
    return oracle.forward(xq, I.router_idx if idx is None else idx, I.router_w if w is None else w,
                          I.gateup_q3k if gu is None else gu, I.down_iq4nl if dn is None else dn,
                          wl.L, wl.F, wl.E)


def test_invariants():
    I, xq = _case(T=8, L=256, F=64, E=6, k=3, seed=11)
    base = _fwd(I, xq)
    # zero router weights -> exactly zero output
    assert (_fwd(I, xq, w=np.zeros_like(I.router_w)).y == 0).all()
    # doubling the weights doubles y exactly (fp64, power of two)
    assert np.array_equal(_fwd(I, xq, w=2 * I.router_w).y, 2 * base.y)
    # token permutation permutes y exactly
    perm = np.random.default_rng(1).permutation(8)
    rp = oracle.forward(xq[perm], I.router_idx[perm], I.router_w[perm], I.gateup_q3k, I.down_iq4nl, 256, 64, 6)
    assert np.array_equal(rp.y, base.y[perm])
    # slot permutation: same y up to the order of the fp64 sums
    sp = _fwd(I, xq, idx=I.router_idx[:, ::-1].copy(), w=I.router_w[:, ::-1].copy())
    assert np.abs(sp.y - base.y).max() <= 1e-12 * np.abs(base.y).max()
    # invalid ids act as weight 0, and are counted
    bad = I.router_idx.copy()
    bad[2, 1] = -1
    bad[5, 0] = 6
    wz = I.router_w.copy()
    wz[2, 1] = 0
    wz[5, 0] = 0
    rb = _fwd(I, xq, idx=bad)
    assert rb.dropped == 2
    assert np.array_equal(rb.y, _fwd(I, xq, w=wz).y)
    # an expert with no tokens has no effect: rewrite its weights
    used = set(I.router_idx.reshape(-1).tolist())
    unused = [e for e in range(6) if e not in used]
    if unused:
        gu2 = I.gateup_q3k.copy()
        gu2[unused[0]] = 0x5A
        assert np.array_equal(_fwd(I, xq, gu=gu2).y, base.y)


def test_duplicate_slot_equals_merged_weight():
    I, xq = _case(T=4, L=256, F=64, E=4, k=2, seed=12)
    idx = np.array([[1, 1], [0, 3], [2, 2], [3, 0]], np.int32)
    w = np.array([[0.25, 0.5], [0.5, 0.5], [0.125, 0.75], [1, 0]], np.float32)
    dup = _fwd(I, xq, idx=idx, w=w)
    idx1 = idx.copy()
    w1 = w.copy()
    for t in (0, 2):
        idx1[t, 1] = -1
        w1[t, 0] = w[t, 0] + w[t, 1]
    merged = _fwd(I, xq, idx=idx1, w=w1)
    assert np.abs(dup.y - merged.y).max() <= 1e-12 * np.abs(dup.y).max()


def test_single_expert_is_dense_swiglu_ffn():
    """E = k = 1, w = 1: y = Wd @ (silu(Wg x) * (Wu x)) up to the q8_1 rounding of H,
    whose per-element error is bounded by d_H/2 + 127 |d_H - fp16(d_H)| (+ fp32 cast)."""
    L, F = 512, 128
    I, xq = _case(T=6, L=L, F=F, E=1, k=1, seed=13)
    w = np.ones((6, 1), np.float32)
    r = oracle.forward(xq, I.router_idx, w, I.gateup_q3k, I.down_iq4nl, L, F, 1)
    xd = oracle.dequant_q8_1(xq).reshape(6, L)
    Wgu = oracle.dequant_q3k(I.gateup_q3k[0]).reshape(2 * F, L)
    Wd = oracle.dequant_iq4nl(I.down_iq4nl[0]).reshape(L, F)
    for t in range(6):
        g, u = Wgu[:F] @ xd[t], Wgu[F:] @ xd[t]
        h = g / (1 + np.exp(-g)) * u
        y = Wd @ h
        hb = np.abs(h).reshape(F // 32, 32).max(-1)
        d = hb / 127
        d16 = d.astype(np.float16).astype(np.float64)
        per = (d / 2 + 127 * np.abs(d - d16) + 1e-6 * hb)
        bound = np.abs(Wd) @ np.repeat(per, 32)
        assert (np.abs(r.y[t] - y) <= bound).all()
        # and the bound is not vacuous: the requant error is a small part of y
        assert np.abs(r.y[t] - y).max() < 0.02 * np.abs(y).max()


FORMATS = [("q3_k", "iq4_nl"), ("q4_0", "q4_0"), ("q3_k", "q4_0"), ("q4_0", "iq4_nl")]


def _gateup(I, gfmt):
    from quantized_latent_moe_amd.inputs import make_gateup_q4_0
    return I.gateup_q3k if gfmt == "q3_k" else make_gateup_q4_0(I.wl)


@pytest.mark.parametrize("gfmt,dfmt", FORMATS)
def test_token_subset_equals_rows_of_full_run(gfmt, dfmt):
    """The token-subset mode (what the full-size GPU checks use) evaluates
    exactly the rows of the full run: y, H, G/U and the dropped count of the
    chosen tokens, byte for byte, in the order the tokens are given (repeats
    and an invalid id included), for both stage entry points."""
    T, L, F, E, k = 12, 256, 96, 5, 3
    I, xq = _case(T=T, L=L, F=F, E=E, k=k, seed=31, zipf=1.1)
    idx = I.router_idx.copy()
    idx[4, 1] = -2          # dropped pair
    idx[7, :] = 3           # one expert in every slot
    gu = _gateup(I, gfmt)
    full = oracle.forward(xq, idx, I.router_w, gu, I.down_iq4nl, L, F, E, want_gu=True, gateup_format=gfmt,
                          down_format=dfmt)
    toks = np.array([7, 0, 4, 11, 4, 2], np.int64)
    sub = oracle.forward(xq, idx, I.router_w, gu, I.down_iq4nl, L, F, E, tokens=toks, want_gu=True,
                         gateup_format=gfmt, down_format=dfmt)
    pairs = (toks[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    assert np.array_equal(sub.y, full.y[toks])
    assert np.array_equal(sub.h, full.h[pairs])
    assert np.array_equal(sub.gu, full.gu[pairs])
    assert full.dropped == 1 and sub.dropped == 2     # token 4 is evaluated twice
    yd = oracle.down_combine(full.h, idx, I.router_w, I.down_iq4nl, L, F, E, down_format=dfmt)
    ys = oracle.down_combine(full.h, idx, I.router_w, I.down_iq4nl, L, F, E, tokens=toks, down_format=dfmt)
    assert np.array_equal(ys, yd[toks])
    # fed the oracle's own H, down + combine is the forward's y
    assert np.array_equal(yd, full.y)


@pytest.mark.parametrize("gfmt", ["q3_k", "q4_0"])
def test_h_blocks_equal_forward_blocks(gfmt):
    """h_blocks (H of single 32-feature blocks, for checks at full size)
    returns the forward's H block, byte for byte, for every (pair, block),
    in any order, zeros for a dropped pair."""
    T, L, F, E, k = 6, 512, 96, 4, 2
    I, xq = _case(T=T, L=L, F=F, E=E, k=k, seed=32)
    idx = I.router_idx.copy()
    idx[2, 0] = E      # dropped
    gu = _gateup(I, gfmt)
    full = oracle.forward(xq, idx, I.router_w, gu, I.down_iq4nl, L, F, E, gateup_format=gfmt)
    P, nfb = T * k, F // 32
    pairs = np.repeat(np.arange(P), nfb)[::-1].copy()
    fb = np.tile(np.arange(nfb), P)[::-1].copy()
    got = oracle.h_blocks(xq, idx, gu, L, F, E, pairs, fb, gateup_format=gfmt)
    assert np.array_equal(got, full.h[pairs, fb])
    assert not got[(pairs == 4) & (fb == 0)].any()
