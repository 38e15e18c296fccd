"""GPU parity of the expert stage with Q4_0 down weights (lat_moe_expert_forward_fmt)
against the CPU oracle, through the C ABI, on every down kernel: the
GEMV-shaped one (at most 64 pairs), the persistent one (F % 256 == 0) and the
per-tile one (other F); and with Q4_0 gate/up weights on both gate/up kernels
that take them (the GEMV-shaped one for at most 64 pairs, k_gateup_q40
otherwise).

Criteria as for IQ4_NL (tests/_gpu.py): routing exact, gate/up and down block
dots bit-exact, H codes >= 99.99 % equal and within +-1 with d_H within one
fp16 ulp, y within 2e-3 * rms of the oracle's down + combine (Q4_0) fed the
GPU's own H, y end to end within 1e-2 * rms of the oracle's.  The down bytes are the workload's random 18-byte blocks, read as
Q4_0 (the same layout): nibbles uniform over 0..15, d ~ U(0.005, 0.015).
"""
import numpy as np
import pytest

import oracle
from quantized_latent_moe_amd.inputs import WORKLOADS, Workload, make_inputs
from tests._gpu import check_e2e, check_h, check_y, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import quantized_latent_moe_amd as lm  # noqa: E402

Q40 = "q4_0"


def _run(I, xq, dn_rows, debug=True):
    wl = I.wl
    dev = torch.device("cuda", 0)
    P = wl.T * wl.k
    x = torch.from_numpy(np.ascontiguousarray(xq)).to(dev)
    idx = torch.from_numpy(np.ascontiguousarray(I.router_idx, np.int32)).to(dev)
    w = torch.from_numpy(np.ascontiguousarray(I.router_w, np.float32)).to(dev)
    gu = torch.from_numpy(I.gateup_q3k).to(dev)
    dn = torch.from_numpy(I.down_iq4nl).to(dev)
    s = lm.shapes(wl.T, wl.L, wl.F, wl.E, wl.k)
    ws = torch.empty(max(lm.workspace_size(s), 256), dtype=torch.uint8, device=dev)
    y = torch.full((max(wl.T, 1), wl.L), np.nan, dtype=torch.float32, device=dev)
    out = {}
    if debug:
        h = torch.empty((P, wl.F // 32, 36), dtype=torch.uint8, device=dev)
        perm = torch.full((P,), -7, dtype=torch.int32, device=dev)
        offs = torch.empty((wl.E + 1,), dtype=torch.int32, device=dev)
        dropped = torch.empty((1,), dtype=torch.int32, device=dev)
        di = torch.zeros((P, dn_rows[1], wl.F // 32), dtype=torch.int32, device=dev)
        lm.expert_forward_fmt(x, idx, w, gu, dn, lm.DOWN_Q4_0, s, y, ws, debug=True, h_q8_1=h, perm=perm,
                             offsets=offs, dropped=dropped, down_i32=di, dn_row0=dn_rows[0])
        torch.cuda.synchronize()
        out.update(h=h.cpu().numpy(), perm=perm.cpu().numpy(), offsets=offs.cpu().numpy(),
                   dropped=int(dropped.item()), dn_i32=di.cpu().numpy())
    else:
        lm.expert_forward_fmt(x, idx, w, gu, dn, lm.DOWN_Q4_0, s, y, ws)
        torch.cuda.synchronize()
    out["y"] = y[: wl.T].cpu().numpy()
    return out


def _check(I, xq, out, dn_rows, toks=None):
    """Routing, the down block dots of every routed pair, y of every token
    stage-wise; H of the tokens toks (all if None) against the oracle's whole
    stage, and y end to end there."""
    wl = I.wl
    ids = I.router_idx.reshape(-1)
    valid = (ids >= 0) & (ids < wl.E)
    order = np.nonzero(valid)[0][np.argsort(ids[valid], kind="stable")]
    assert np.array_equal(out["perm"][: order.size], order.astype(np.int32))
    pairs = np.nonzero(valid)[0]
    r0, nr = dn_rows
    pp = np.repeat(pairs, nr)
    rr = np.tile(np.arange(r0, r0 + nr), pairs.size).astype(np.int32)
    ref = oracle.probe_down(out["h"], I.router_idx, I.down_iq4nl, wl.L, wl.F, wl.E, pp, rr, down_format=Q40)
    assert np.array_equal(out["dn_i32"][pairs].reshape(-1, wl.F // 32), ref), "Q4_0 down block dots differ"
    say(f"{wl.name}: {pairs.size} pairs x {nr} Q4_0 down rows of block dots bit-exact")
    ys = oracle.down_combine(out["h"], I.router_idx, I.router_w, I.down_iq4nl, wl.L, wl.F, wl.E, down_format=Q40)
    check_y(out["y"], ys, label=f"{wl.name} Q4_0 stage-wise, all {wl.T} tokens")
    if toks is None:
        toks = np.arange(wl.T)
    full = oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, I.down_iq4nl, wl.L, wl.F, wl.E,
                          tokens=toks, down_format=Q40)
    allp = (toks[:, None] * wl.k + np.arange(wl.k)[None, :]).reshape(-1)
    check_h(out["h"][allp], full.h, label=f"{wl.name} (Q4_0 down, {toks.size} tokens)")
    check_e2e(out["y"][toks], full.y, label=f"{wl.name} Q4_0 ({toks.size} tokens)")


CASES = [
    WORKLOADS["tiny"],
    # several items per persistent workgroup, each of several K steps, over full token tiles
    Workload("q40_multi_item", T=2048, L=1024, F=1024, E=8, k=4, zipf_s=1.1, seed=35),                                                           # GEMV-shaped kernels
    WORKLOADS["decode"],
    Workload("q40_few_tokens", T=6, L=768, F=160, E=5, k=4, zipf_s=1.1, seed=31),
    Workload("q40_ragged", T=200, L=512, F=288, E=6, k=3, zipf_s=1.1, seed=32),   # per-tile kernel (F % 256 != 0)
    Workload("q40_persistent", T=300, L=512, F=512, E=8, k=4, zipf_s=1.1, n_masked=1, seed=33),  # persistent kernel
    Workload("q40_wide", T=40, L=2048, F=4096, E=4, k=2, seed=34),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_q4_0_down_full_compare(wl):
    say(f"Q4_0 case {wl}")
    I = make_inputs(wl)
    xq = oracle.quantize_q8_1(I.x)
    dn_rows = (max(0, wl.L - 40), min(40, wl.L))
    out = _run(I, xq, dn_rows)
    _check(I, xq, out, dn_rows)
    # the entry point without a debug struct gives the same y, bit for bit
    assert np.array_equal(_run(I, xq, dn_rows, debug=False)["y"], out["y"])


def test_q4_0_down_full_size():
    wl = WORKLOADS["prefill_5k"]
    say(f"Q4_0 case {wl} (full size)")
    I = make_inputs(wl)
    xq = oracle.quantize_q8_1(I.x)
    dn_rows = (wl.L - 132, 8)  # across the boundary of two 128-row tiles
    out = _run(I, xq, dn_rows)
    say(f"{wl.name} Q4_0: GPU done")
    rng = np.random.default_rng(17)
    toks = np.array(sorted(set(rng.choice(wl.T, 10, replace=False).tolist()) | {0, wl.T - 1}), np.int64)
    _check(I, xq, out, dn_rows, toks=toks)


# ---- Q4_0 gate/up weights (the persistent kernel at every batch size) ------

def _run_gu(I, xq, gu, down_format, gu_rows, dn_rows):
    wl = I.wl
    dev = torch.device("cuda", 0)
    P = wl.T * wl.k
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x, idx, w = t(xq), t(I.router_idx.astype(np.int32)), t(I.router_w.astype(np.float32))
    g, dn = t(gu), t(I.down_iq4nl)
    s = lm.shapes(wl.T, wl.L, wl.F, wl.E, wl.k)
    ws = torch.empty(max(lm.workspace_size(s), 256), dtype=torch.uint8, device=dev)
    y = torch.full((max(wl.T, 1), wl.L), np.nan, dtype=torch.float32, device=dev)
    h = torch.empty((P, wl.F // 32, 36), dtype=torch.uint8, device=dev)
    perm = torch.full((P,), -7, dtype=torch.int32, device=dev)
    gi = torch.zeros((P, gu_rows[1], wl.L // 32), dtype=torch.int32, device=dev)
    di = torch.zeros((P, dn_rows[1], wl.F // 32), dtype=torch.int32, device=dev)
    lm.expert_forward_fmt(x, idx, w, g, dn, down_format, s, y, ws, gateup_format=lm.GATEUP_Q4_0, debug=True,
                         h_q8_1=h, perm=perm, gateup_i32=gi, gu_row0=gu_rows[0], down_i32=di, dn_row0=dn_rows[0])
    torch.cuda.synchronize()
    out = dict(y=y[:wl.T].cpu().numpy(), h=h.cpu().numpy(), perm=perm.cpu().numpy(), gu_i32=gi.cpu().numpy(),
               dn_i32=di.cpu().numpy())
    y2 = torch.full_like(y, np.nan)
    lm.expert_forward_fmt(x, idx, w, g, dn, down_format, s, y2, ws, gateup_format=lm.GATEUP_Q4_0)
    torch.cuda.synchronize()
    out["y_plain"] = y2[:wl.T].cpu().numpy()
    return out


def _check_gu(I, xq, gu, out, dfmt, gu_rows, dn_rows, toks=None):
    """Routing, gate/up and down block dots of every routed pair, one H block
    of every pair, y of every token stage-wise; H of the tokens toks (all if
    None) against the oracle's whole stage, and y end to end there."""
    wl = I.wl
    ids = I.router_idx.reshape(-1)
    valid = (ids >= 0) & (ids < wl.E)
    order = np.nonzero(valid)[0][np.argsort(ids[valid], kind="stable")]
    assert np.array_equal(out["perm"][: order.size], order.astype(np.int32))
    pairs = np.nonzero(valid)[0]
    r0, nr = gu_rows
    pp, rr = np.repeat(pairs, nr), np.tile(np.arange(r0, r0 + nr), pairs.size).astype(np.int32)
    ref = oracle.probe_gateup(xq, I.router_idx, gu, wl.L, wl.F, wl.E, pp, rr, gateup_format=Q40)
    assert np.array_equal(out["gu_i32"][pairs].reshape(-1, wl.L // 32), ref), "Q4_0 gate/up block dots differ"
    r0, nr = dn_rows
    pp, rr = np.repeat(pairs, nr), np.tile(np.arange(r0, r0 + nr), pairs.size).astype(np.int32)
    ref = oracle.probe_down(out["h"], I.router_idx, I.down_iq4nl, wl.L, wl.F, wl.E, pp, rr, down_format=dfmt)
    assert np.array_equal(out["dn_i32"][pairs].reshape(-1, wl.F // 32), ref), "down block dots differ"
    say(f"{wl.name}: {pairs.size} pairs of Q4_0 gate/up and {dfmt} down block dots bit-exact")
    nfb = wl.F // 32
    fb = ((7 * pairs + 3) % nfb).astype(np.int32)
    hb = oracle.h_blocks(xq, I.router_idx, gu, wl.L, wl.F, wl.E, pairs, fb, gateup_format=Q40)
    check_h(out["h"][pairs, fb][:, None, :], hb[:, None, :], label=f"{wl.name}: one Q4_0 gate/up H block per pair")
    ys = oracle.down_combine(out["h"], I.router_idx, I.router_w, I.down_iq4nl, wl.L, wl.F, wl.E, down_format=dfmt)
    check_y(out["y"], ys, label=f"{wl.name} Q4_0 gate/up stage-wise, all {wl.T} tokens")
    if toks is None:
        toks = np.arange(wl.T)
    allp = (toks[:, None] * wl.k + np.arange(wl.k)[None, :]).reshape(-1)
    full = oracle.forward(xq, I.router_idx, I.router_w, gu, I.down_iq4nl, wl.L, wl.F, wl.E, tokens=toks,
                          gateup_format=Q40, down_format=dfmt)
    check_h(out["h"][allp], full.h, label=f"{wl.name} (Q4_0 gate/up, {toks.size} tokens)")
    check_e2e(out["y"][toks], full.y, label=f"{wl.name} Q4_0 gate/up ({toks.size} tokens)")
    assert np.array_equal(out["y_plain"], out["y"])


GU_CASES = [
    (WORKLOADS["tiny"], "q4_0"),
    (WORKLOADS["decode"], "iq4_nl"),                                                     # 32 pairs: 1-token tiles
    (Workload("gu40_one_step", T=100, L=256, F=96, E=4, k=2, zipf_s=1.1, seed=41), "q4_0"),  # one K step, half tile
    (Workload("gu40_ragged", T=200, L=512, F=288, E=6, k=3, zipf_s=1.1, n_masked=1, seed=42), "iq4_nl"),
    (Workload("gu40_wide", T=300, L=1024, F=512, E=8, k=4, zipf_s=1.1, seed=43), "q4_0"),
    (Workload("gu40_few", T=6, L=768, F=160, E=5, k=4, zipf_s=1.1, seed=44), "q4_0"),
    # several items per persistent workgroup, each of several K steps, over full
    # token tiles, with both down formats
    (Workload("gu40_multi_item", T=2048, L=1024, F=1024, E=8, k=4, zipf_s=1.1, seed=46), "q4_0"),
    (Workload("gu40_multi_item", T=2048, L=1024, F=1024, E=8, k=4, zipf_s=1.1, seed=46), "iq4_nl"),
]


@pytest.mark.parametrize("wl,dfmt", GU_CASES, ids=lambda v: getattr(v, "name", v))
def test_q4_0_gateup_full_compare(wl, dfmt):
    from quantized_latent_moe_amd.inputs import make_gateup_q4_0
    say(f"Q4_0 gate/up case {wl}, down {dfmt}")
    I = make_inputs(wl)
    xq = oracle.quantize_q8_1(I.x)
    gu = make_gateup_q4_0(wl)
    gu_rows = (max(0, wl.F - 24), min(48, 2 * wl.F - max(0, wl.F - 24)))
    dn_rows = (wl.L - 32, 32)
    out = _run_gu(I, xq, gu, lm.DOWN_Q4_0 if dfmt == "q4_0" else lm.DOWN_IQ4_NL, gu_rows, dn_rows)
    _check_gu(I, xq, gu, out, dfmt, gu_rows, dn_rows)


def test_q4_0_gateup_full_size():
    from quantized_latent_moe_amd.inputs import make_gateup_q4_0
    wl = WORKLOADS["prefill_5k"]
    say(f"Q4_0 gate/up case {wl} (full size)")
    I = make_inputs(wl)
    xq = oracle.quantize_q8_1(I.x)
    gu = make_gateup_q4_0(wl)
    out = _run_gu(I, xq, gu, lm.DOWN_Q4_0, (wl.F - 4, 8), (124, 8))
    say(f"{wl.name} Q4_0 gate/up: GPU done")
    rng = np.random.default_rng(19)
    toks = np.array(sorted(set(rng.choice(wl.T, 10, replace=False).tolist()) | {0, wl.T - 1}), np.int64)
    _check_gu(I, xq, gu, out, "q4_0", (wl.F - 4, 8), (124, 8), toks=toks)


@pytest.mark.parametrize("T", [9, 100], ids=["small_kernel", "persistent_kernel"])
def test_q4_0_gateup_invalid_and_duplicate_ids(T):
    """Q4_0 gate/up with dropped and repeated ids (27 pairs take the GEMV-shaped
    kernel, 300 the persistent one): only valid pairs count; every id invalid
    gives y = 0."""
    from quantized_latent_moe_amd.inputs import make_gateup_q4_0
    wl = Workload(f"gu40_edge_{T}", T=T, L=256, F=96, E=5, k=3, zipf_s=1.1, seed=18)
    say(f"Q4_0 gate/up edge case {wl}")
    I = make_inputs(wl)
    xq = oracle.quantize_q8_1(I.x)
    gu = make_gateup_q4_0(wl)
    idx = I.router_idx.copy()
    idx[0, :] = [-1, 5, 1 << 20]
    idx[1, :] = [2, 2, 2]
    idx[4, 2] = -3
    I.router_idx[...] = idx
    rows = ((0, 2 * wl.F), (0, wl.L))
    out = _run_gu(I, xq, gu, lm.DOWN_Q4_0, *rows)
    assert (out["y"][0] == 0).all()
    _check_gu(I, xq, gu, out, "q4_0", *rows)
    I.router_idx[...] = 7
    out = _run_gu(I, xq, gu, lm.DOWN_Q4_0, *rows)
    assert (out["y"] == 0).all() and (out["y_plain"] == 0).all()


def test_q4_0_empty_batch_is_noop():
    s = lm.shapes(0, 1024, 2048, 128, 8)
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    y = torch.full((1, 1024), 3.0, device="cuda")
    lm.expert_forward_fmt(dummy, dummy, dummy, dummy, dummy, lm.DOWN_Q4_0, s, y, dummy, gateup_format=lm.GATEUP_Q4_0)
    torch.cuda.synchronize()
    assert (y == 3.0).all()


@pytest.mark.parametrize("name", ["decode", "gu40_graph"])
def test_q4_0_stage_graph_replays_exactly(name):
    """The stage with Q4_0 gate/up and down weights captured in a graph (the
    GEMV-shaped kernels at decode; the large route path and the persistent
    Q4_0 kernels at 1200 pairs): every replay, with eager work between
    replays, gives the eager call's y bit for bit."""
    from quantized_latent_moe_amd.inputs import make_gateup_q4_0
    wl = WORKLOADS["decode"] if name == "decode" else Workload("gu40_graph", T=300, L=1024, F=512, E=8, k=4,
                                                               zipf_s=1.1, seed=45)
    say(f"Q4_0 graph case {wl}")
    I = make_inputs(wl)
    xq = oracle.quantize_q8_1(I.x)
    dev = torch.device("cuda", 0)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x, idx, w = t(xq), t(I.router_idx.astype(np.int32)), t(I.router_w.astype(np.float32))
    g, dn = t(make_gateup_q4_0(wl)), t(I.down_iq4nl)
    s = lm.shapes(wl.T, wl.L, wl.F, wl.E, wl.k)
    ws = torch.empty(lm.workspace_size(s), dtype=torch.uint8, device=dev)
    y = torch.empty((wl.T, wl.L), dtype=torch.float32, device=dev)

    def step():
        lm.expert_forward_fmt(x, idx, w, g, dn, lm.DOWN_Q4_0, s, y, ws, gateup_format=lm.GATEUP_Q4_0)

    step()
    torch.cuda.synchronize()
    y_eager = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    scratch = torch.randn(1 << 20, device=dev)
    for r in range(4):
        y.fill_(float("nan"))
        ws.fill_(0x5A)                  # the workspace needs no initialisation
        graph.replay()
        scratch.mul_(1.0001)            # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r}"
    say(f"{wl.name}: 4 graph replays of the Q4_0 stage equal the eager call")
