"""GPU parity of the latent D / U projections with Q4_0 weights (18-byte
blocks, weight = d * (nibble - 8)) against the CPU oracle, through the C ABI,
on both kernels that take them: the GEMV-shaped one (at most 8 tokens) and the
persistent warp-specialized one (N % 128 == 0, K % 256 == 0, any T).

Criteria as for Q8_0 weights (tests/test_dense_gpu.py): integer block dots
bit-exact; fp32 rows within the fold's rounding bound
(K/32 + 2) * 2^-24 * sum_b |d_w d_x I|; q8_1 rows bit for bit the rounding of
the GPU's own fp32 rows, and within C2 of the rounding of the oracle's rows.
"""
import numpy as np
import pytest

import oracle
from quantized_latent_moe_amd.inputs import DENSE_WORKLOADS, make_dense_inputs, random_q4_0
from tests._gpu import check_h, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import quantized_latent_moe_amd as lm  # noqa: E402

F4 = "q4_0"


def _run(xq, w, T, N, K, probe_rows=None, want_f32=True, want_q8=True):
    dev = torch.device("cuda", 0)
    gx = torch.from_numpy(np.ascontiguousarray(xq)).to(dev)
    gw = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
    y = torch.full((max(T, 1), N), np.nan, dtype=torch.float32, device=dev) if want_f32 else None
    q = torch.full((max(T, 1), N // 32, 36), 0xAB, dtype=torch.uint8, device=dev) if want_q8 else None
    dots = None
    if probe_rows is not None:
        dots = torch.full((max(T, 1), probe_rows[1], K // 32), -12345, dtype=torch.int32, device=dev)
    lm.dense_q4_0(gx, gw, T, N, K, y, q, dots_i32=dots, row0=0 if probe_rows is None else probe_rows[0])
    torch.cuda.synchronize()
    out = {}
    if y is not None:
        out["y"] = y[:T].cpu().numpy()
    if q is not None:
        out["q"] = q[:T].cpu().numpy()
    if dots is not None:
        out["dots"] = dots[:T].cpu().numpy()
    return out


def _check(xq, w, N, K, out, toks, rows_probe, label):
    r0, nr = rows_probe
    tt = np.repeat(toks, nr)
    rr = np.tile(np.arange(r0, r0 + nr), toks.size)
    ref_dots = oracle.probe_dense(xq, w, N, K, tt, rr, w_format=F4).reshape(toks.size, nr, K // 32)
    assert np.array_equal(out["dots"][toks], ref_dots), f"{label}: block dots differ"
    ref = oracle.dense_q8_0(xq, w, N, K, tokens=toks, w_format=F4)
    yg = out["y"][toks]
    assert np.isfinite(yg).all()
    allt = np.repeat(toks, N)
    allr = np.tile(np.arange(N), toks.size)
    dots_all = oracle.probe_dense(xq, w, N, K, allt, allr, w_format=F4)
    dx = xq[allt, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    dw = w[allr, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    bound = ((K // 32 + 2) * 2.0 ** -24 * np.abs(dw * dx * dots_all).sum(-1)).reshape(toks.size, N)
    err = np.abs(yg.astype(np.float64) - ref)
    say(f"{label}: {toks.size} tokens x {N} rows, max err/bound = {(err / np.maximum(bound, 1e-300)).max():.3f}")
    assert (err <= bound).all()
    qg = out["q"][toks]
    assert np.array_equal(qg, oracle.quantize_q8_1(yg)), f"{label}: q8_1 rows are not the rounding of y"
    check_h(qg.reshape(-1, N // 32, 36), oracle.quantize_q8_1(ref.astype(np.float32)).reshape(-1, N // 32, 36),
            label=f"{label} q8_1")


def _inputs(T, N, K, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, K)) * np.exp(rng.uniform(-1, 1, (T, 1)))).astype(np.float32)
    return oracle.quantize_q8_1(x), random_q4_0(rng, (N, K // 32))


CASES = [
    (1, 32, 32, 1), (5, 32, 96, 2), (3, 64, 512, 3), (8, 96, 2048, 4), (8, 64, 4096, 5), (4, 64, 8192, 6),
    (7, 32, 1056, 7),                                   # the GEMV-shaped kernel, each lane layout
    (9, 128, 256, 8), (130, 128, 512, 9), (300, 256, 512, 10), (200, 384, 768, 11),  # the persistent kernel
]


@pytest.mark.parametrize("T,N,K,seed", CASES, ids=lambda v: str(v))
def test_dense_q4_0_full_compare(T, N, K, seed):
    say(f"dense Q4_0 case T={T} N={N} K={K}")
    xq, w = _inputs(T, N, K, seed)
    nr = min(N, 64)
    out = _run(xq, w, T, N, K, probe_rows=(N - nr, nr))
    _check(xq, w, N, K, out, np.arange(T), (N - nr, nr), f"T={T} N={N} K={K}")
    assert np.array_equal(_run(xq, w, T, N, K, want_q8=False)["y"], out["y"])


@pytest.mark.parametrize("proj", ["D", "U"])
def test_dense_q4_0_full_size_sampled(proj):
    wl = DENSE_WORKLOADS["du_prefill_5k"]
    I = make_dense_inputs(wl)
    if proj == "D":
        xq, w, N, K = oracle.quantize_q8_1(I.x), I.d_q4_0, wl.L, wl.H
    else:
        xq, w, N, K = oracle.quantize_q8_1(I.z), I.u_q4_0, wl.H, wl.L
    say(f"{wl.name} {proj} Q4_0: T={wl.T} N={N} K={K}")
    out = _run(xq, w, wl.T, N, K, probe_rows=(N - 8, 8))
    rng = np.random.default_rng(12)
    toks = np.unique(np.concatenate([rng.choice(wl.T, 8, replace=False), [0, 127, 128, wl.T - 1]]))
    _check(xq, w, N, K, out, toks, (N - 8, 8), f"{wl.name} {proj} Q4_0")
    assert np.array_equal(out["q"], oracle.quantize_q8_1(out["y"]))
