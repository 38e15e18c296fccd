"""GPU parity of the latent D / U dense projections (Q8_0 x q8_1) against the
CPU oracle, through the C ABI.

Criteria:
  * integer block dots bit-exact (debug probes of weight rows);
  * fp32 outputs within the rounding bound of an fp32 fold of the exact
    block dots: |y_gpu - y_ref| <= (K/32 + 2) * 2^-24 * S, where S is the sum
    over blocks of |d_w * d_x * I| (each term is rounded twice, d_x * I and
    then the multiply-add, and the running sum once per block);
  * q8_1 outputs: bit for bit the q8_1 rounding of the GPU's own fp32 rows
    (the oracle's quantizer applied to them), and >= 99.99 % of the codes equal
    to the rounding of the oracle's rows with the rest within +-1 and d within
    one fp16 ulp (the pages report 99.9987 % equal codes for their D kernel
    against the earlier one, the rest differing by 1).
"""
import numpy as np
import pytest

import oracle
from quantized_latent_moe_amd.inputs import DENSE_WORKLOADS, DenseWorkload, make_dense_inputs
from tests._gpu import check_h, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import quantized_latent_moe_amd as lm  # noqa: E402


def _fold_bound(xq, w, K, toks, rows, dots):
    """(K/32 + 2) * 2^-24 * sum_b |d_w d_x I| for each (token, row) probe."""
    dx = xq[toks, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float64)    # [n, K/32]
    dw = w[rows, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    S = np.abs(dw * dx * dots.astype(np.float64)).sum(-1)
    return (K // 32 + 2) * 2.0 ** -24 * S


def _run(xq, w, T, N, K, want_f32=True, want_q8=True, probe_rows=None):
    dev = torch.device("cuda", 0)
    gx = torch.from_numpy(np.ascontiguousarray(xq)).to(dev)
    gw = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
    y = torch.full((max(T, 1), N), np.nan, dtype=torch.float32, device=dev) if want_f32 else None
    q = torch.full((max(T, 1), N // 32, 36), 0xAB, dtype=torch.uint8, device=dev) if want_q8 else None
    dots = None
    if probe_rows is not None:
        dots = torch.full((max(T, 1), probe_rows[1], K // 32), -12345, dtype=torch.int32, device=dev)
    lm.dense_q8_0(gx, gw, T, N, K, y, q, dots_i32=dots, row0=0 if probe_rows is None else probe_rows[0])
    torch.cuda.synchronize()
    out = {}
    if y is not None:
        out["y"] = y[:T].cpu().numpy()
    if q is not None:
        out["q"] = q[:T].cpu().numpy()
    if dots is not None:
        out["dots"] = dots[:T].cpu().numpy()
    return out


def _check(xq, w, T, N, K, out, toks, rows_probe, label):
    """All criteria on tokens `toks` (all rows of those tokens for y and q)."""
    r0, nr = rows_probe
    rows = np.arange(r0, r0 + nr)
    # block dots
    tt = np.repeat(toks, nr)
    rr = np.tile(rows, toks.size)
    ref_dots = oracle.probe_dense(xq, w, N, K, tt, rr).reshape(toks.size, nr, K // 32)
    assert np.array_equal(out["dots"][toks], ref_dots), f"{label}: block dots differ"
    # fp32 rows against the oracle, within the fold's rounding bound
    ref = oracle.dense_q8_0(xq, w, N, K, tokens=toks)
    yg = out["y"][toks]
    assert np.isfinite(yg).all()
    allt = np.repeat(toks, N)
    allr = np.tile(np.arange(N), toks.size)
    dots_all = oracle.probe_dense(xq, w, N, K, allt, allr)
    bound = _fold_bound(xq, w, K, allt, allr, dots_all).reshape(toks.size, N)
    err = np.abs(yg.astype(np.float64) - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    say(f"{label}: {toks.size} tokens x {N} rows, max|err| = {err.max():.3e} (rms {rms:.3e}), "
        f"max err/bound = {(err / np.maximum(bound, 1e-300)).max():.3f}")
    assert (err <= bound).all()
    # q8_1 rows: the rounding of the GPU's own fp32 rows, bit for bit ...
    qg = out["q"][toks]
    assert np.array_equal(qg, oracle.quantize_q8_1(yg)), f"{label}: q8_1 rows are not the rounding of y"
    # ... and within the criterion of the rounding of the oracle's rows
    check_h(qg.reshape(-1, N // 32, 36), oracle.quantize_q8_1(ref.astype(np.float32)).reshape(-1, N // 32, 36),
            label=f"{label} q8_1")


def _inputs(T, N, K, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, K)) * np.exp(rng.uniform(-1, 1, (T, 1)))).astype(np.float32)
    xq = oracle.quantize_q8_1(x)
    from quantized_latent_moe_amd.inputs import random_q8_0
    w = random_q8_0(rng, (N, K // 32))
    return xq, w


SMALL = [
    (37, 256, 512, 1),     # D of the tiny latent layer (hidden 512 -> latent 256)
    (37, 512, 256, 2),     # its U
    (130, 96, 96, 3),      # ragged: token tail of 2, a half row tile, an odd block count
    (1, 32, 32, 4),        # one token, one row block, one K block
    (4, 1024, 4096, 5),    # decode-sized D
    (4, 4096, 1024, 6),    # decode-sized U
    (300, 160, 1056, 7),   # several tiles, 33 blocks
    # the GEMV-shaped kernel of batches of at most 8 tokens, each lane layout
    (5, 32, 96, 8),        # 3 blocks a row: 8 lanes a row
    (3, 64, 512, 9),       # 16 blocks: 16 lanes a row
    (8, 96, 2048, 10),     # 64 blocks: 64 lanes, one block each
    (8, 64, 4096, 11),     # 128 blocks: two a lane
    (4, 64, 8192, 12),     # 256 blocks: four a lane (batches of at most 4)
    (7, 32, 1056, 13),     # 33 blocks, a partly idle lane group
    (9, 64, 256, 14),      # one token more: the MFMA kernel
    # the persistent warp-specialized kernel (T >= 128, N % 128 == 0, K % 256 == 0)
    (300, 256, 512, 15),   # two full token tiles and a 44-token tail (one 32-token half)
    (129, 128, 256, 16),   # a one-token tail tile, one K step
    (200, 384, 768, 17),   # three K steps, a 72-token tail (both halves, the second partial)
    (640, 1024, 4096, 18), # D-shaped, five full token tiles
]


@pytest.mark.parametrize("T,N,K,seed", SMALL, ids=lambda v: str(v))
def test_dense_full_compare(T, N, K, seed):
    say(f"dense case T={T} N={N} K={K}")
    xq, w = _inputs(T, N, K, seed)
    nr = min(N, 64)
    r0 = N - nr
    out = _run(xq, w, T, N, K, probe_rows=(r0, nr))
    _check(xq, w, T, N, K, out, np.arange(T), (r0, nr), f"T={T} N={N} K={K}")
    # only one output requested: the same values
    y_only = _run(xq, w, T, N, K, want_q8=False)["y"]
    q_only = _run(xq, w, T, N, K, want_f32=False)["q"]
    assert np.array_equal(y_only, out["y"]) and np.array_equal(q_only, out["q"])


def test_dense_extreme_codes():
    """Every code -128 in both operands (|I| = 2^19, the largest block dot) and
    scales from fp16's subnormal and top range."""
    T, N, K = 40, 64, 128
    xq = np.zeros((T, K // 32, 36), np.uint8)
    xq[..., 4:] = 0x80
    xq[..., 0:2] = np.array([2.0 ** -20], np.float16).view(np.uint8)   # fp16 subnormal d
    xq[1::2, :, 0:2] = np.array([1.0], np.float16).view(np.uint8)
    w = np.zeros((N, K // 32, 34), np.uint8)
    w[..., 2:] = 0x80
    w[..., 0:2] = np.array([2.0 ** -14], np.float16).view(np.uint8)
    w[5, :, 2:] = 0x7F
    w[9, 1, 2:] = 0
    out = _run(xq, w, T, N, K, probe_rows=(0, N))
    assert (np.abs(out["dots"]) <= 1 << 19).all() and (out["dots"] == 1 << 19).any()
    _check(xq, w, T, N, K, out, np.arange(T), (0, N), "extreme codes")


@pytest.mark.parametrize("proj", ["D", "U"])
def test_dense_full_size_sampled(proj):
    wl = DENSE_WORKLOADS["du_prefill_5k"]
    I = make_dense_inputs(wl)
    if proj == "D":
        xq, w, N, K = oracle.quantize_q8_1(I.x), I.d_q8_0, wl.L, wl.H
    else:
        xq, w, N, K = oracle.quantize_q8_1(I.z), I.u_q8_0, wl.H, wl.L
    say(f"{wl.name} {proj}: T={wl.T} N={N} K={K}")
    out = _run(xq, w, wl.T, N, K, probe_rows=(N - 8, 8))
    say(f"{wl.name} {proj}: GPU done")
    rng = np.random.default_rng(11)
    toks = np.unique(np.concatenate([rng.choice(wl.T, 10, replace=False), [0, 127, 128, wl.T - 1]]))
    _check(xq, w, wl.T, N, K, out, toks, (N - 8, 8), f"{wl.name} {proj}")
    # every token: the q8_1 rows are the rounding of the fp32 rows
    assert np.array_equal(out["q"], oracle.quantize_q8_1(out["y"]))
    # deterministic
    again = _run(xq, w, wl.T, N, K)
    assert np.array_equal(again["y"], out["y"]) and np.array_equal(again["q"], out["q"])


def test_dense_empty_is_noop():
    y = torch.full((1, 64), 3.0, device="cuda")
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    lm.dense_q8_0(dummy, dummy, 0, 64, 64, y, None)
    torch.cuda.synchronize()
    assert (y == 3.0).all()


def test_dense_feeds_the_expert_stage():
    """D's q8_1 output is the expert stage's input format: the stage run on
    it gives the oracle's result for the same bytes."""
    from quantized_latent_moe_amd.inputs import Workload, make_inputs
    from tests._gpu import Gpu, check_y, stagewise_y
    dw = DenseWorkload("chain", T=70, H=512, L=256, seed=3)
    DI = make_dense_inputs(dw)
    xl = _run(oracle.quantize_q8_1(DI.x), DI.d_q8_0, dw.T, dw.L, dw.H, want_f32=False)["q"]
    I = make_inputs(Workload("chain", T=dw.T, L=dw.L, F=96, E=5, k=2, seed=3))
    g = Gpu(I, xl)
    out = g.forward_debug()
    ref = oracle.forward(xl, I.router_idx, I.router_w, I.gateup_q3k, I.down_iq4nl, dw.L, 96, 5)
    check_h(out["h"], ref.h, label="chain H")
    check_y(out["y"], stagewise_y(out, I), label="chain y")
