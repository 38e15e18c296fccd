"""GPU parity of the HIP expert stage against the CPU oracle (through the C ABI).

Criteria (see tests/_gpu.py): integer block dots bit-exact; routing (perm,
offsets, dropped count) exact; H codes >= 99.99 % equal and within +-1, d_H
within one fp16 ulp; y within 2e-3 * rms of the oracle's down + combine fed
the GPU's H; y end to end within 1e-2 * rms of the oracle's.  Small cases are
compared on every output.  The full-size workloads, in the launch
configuration the benchmark times: block dots of 16 weight rows and one H
block of every routed pair, y of every token stage-wise, the whole stage end
to end on sampled tokens.
"""
import numpy as np
import pytest

import oracle
from quantized_latent_moe_amd.inputs import WORKLOADS, Workload, make_inputs
from tests._gpu import Gpu, check_e2e, check_h, check_y, say, stagewise_y

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _case(wl):
    I = make_inputs(wl)
    xq = oracle.quantize_q8_1(I.x)
    return I, xq


def _check_routing(out, I):
    wl = I.wl
    ids = I.router_idx.reshape(-1)
    valid = (ids >= 0) & (ids < wl.E)
    order = np.nonzero(valid)[0][np.argsort(ids[valid], kind="stable")]
    nv = int(valid.sum())
    assert np.array_equal(out["perm"][:nv], order.astype(np.int32))
    counts = np.bincount(ids[valid], minlength=wl.E)
    assert np.array_equal(out["offsets"], np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
    assert out["dropped"] == int((~valid).sum())


def _check_probes(out, I, xq, gu_rows, dn_rows, pairs=None):
    wl = I.wl
    P = wl.T * wl.k
    ids = I.router_idx.reshape(-1)
    if pairs is None:
        pairs = np.arange(P)
    pairs = pairs[(ids[pairs] >= 0) & (ids[pairs] < wl.E)]
    r0, nr = gu_rows
    pp = np.repeat(pairs, nr)
    rr = np.tile(np.arange(r0, r0 + nr), pairs.size).astype(np.int32)
    ref = oracle.probe_gateup(xq, I.router_idx, I.gateup_q3k, wl.L, wl.F, wl.E, pp, rr)
    got = out["gu_i32"][pairs].reshape(-1, wl.L // 32)
    assert np.array_equal(got, ref), "gate/up block dots differ"
    r0, nr = dn_rows
    pp = np.repeat(pairs, nr)
    rr = np.tile(np.arange(r0, r0 + nr), pairs.size).astype(np.int32)
    ref = oracle.probe_down(out["h"], I.router_idx, I.down_iq4nl, wl.L, wl.F, wl.E, pp, rr)
    got = out["dn_i32"][pairs].reshape(-1, wl.F // 32)
    assert np.array_equal(got, ref), "down block dots differ"
    say(f"{wl.name}: {pairs.size} pairs x ({gu_rows[1]} gate/up + {dn_rows[1]} down) rows of block dots bit-exact")


def test_quantize_q8_1_bit_exact():
    say("quantize_q8_1 vs oracle")
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((300, 1024)) * np.exp(rng.uniform(-6, 6, (300, 1)))).astype(np.float32)
    x[3] = 0.0
    x[4, :32] = 127.0 * np.array([1, 0.5, -0.5, 2.5 / 127] * 8, np.float32)
    gx = torch.from_numpy(x).cuda()
    out = torch.empty((300, 32, 36), dtype=torch.uint8, device="cuda")
    import quantized_latent_moe_amd as lm
    lm.quantize_q8_1(gx, out)
    torch.cuda.synchronize()
    ref = oracle.quantize_q8_1(x)
    got = out.cpu().numpy()
    bad = np.argwhere(got != ref)
    if bad.size:
        fields = {"d": int((bad[:, 2] < 2).sum()), "s": int(((bad[:, 2] >= 2) & (bad[:, 2] < 4)).sum()),
                  "codes": int((bad[:, 2] >= 4).sum())}
        say(f"quantize mismatches by field: {fields}; first at {bad[:3].tolist()}")
    assert bad.size == 0


SMALL = [
    WORKLOADS["tiny"],
    Workload("ragged", T=200, L=512, F=288, E=6, k=3, zipf_s=1.1, seed=3),
    Workload("ragged_masked", T=150, L=768, F=160, E=9, k=4, zipf_s=1.1, n_masked=2, seed=4),
    WORKLOADS["decode"],
    # batches of at most 64 pairs take the GEMV-shaped kernels
    Workload("few_tokens", T=6, L=768, F=160, E=5, k=4, zipf_s=1.1, seed=9),
    Workload("few_tokens_crowded", T=16, L=256, F=96, E=2, k=2, seed=10),
    # more than 8 experts per token (combine's general loop)
    Workload("wide_k", T=48, L=512, F=256, E=12, k=10, zipf_s=1.1, seed=11),
    # more than 512 experts (the chunked route passes at a small batch)
    Workload("many_experts", T=64, L=256, F=128, E=600, k=4, seed=12),
    # a small batch with more than 512 experts (routed by the chunked passes,
    # rows gathered by their own kernel)
    Workload("small_batch_many_experts", T=6, L=512, F=256, E=700, k=8, seed=17),
    # the largest expert count, one expert per token
    Workload("max_experts_k1", T=300, L=256, F=256, E=1024, k=1, seed=13),
    # one token
    Workload("one_token", T=1, L=1024, F=2048, E=16, k=4, seed=14),
    # wide latent and FFN dimensions (past the small-batch limits: L > 1024, F > 2048)
    Workload("wide_dims", T=40, L=2048, F=4096, E=4, k=2, seed=15),
    Workload("wide_dims_prefill", T=700, L=2048, F=1024, E=6, k=2, zipf_s=1.1, seed=16),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_forward_full_compare(wl):
    say(f"case {wl}")
    I, xq = _case(wl)
    ref = oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, I.down_iq4nl, wl.L, wl.F, wl.E)
    g = Gpu(I, xq)
    gu_rows = (max(0, wl.F - 24), min(48, 2 * wl.F - max(0, wl.F - 24)))
    dn_rows = (wl.L - 40, 40)
    out = g.forward_debug(gu_rows=gu_rows, dn_rows=dn_rows)
    _check_routing(out, I)
    _check_probes(out, I, xq, gu_rows, dn_rows)
    check_h(out["h"], ref.h, label=wl.name)
    check_y(out["y"], stagewise_y(out, I), label=f"{wl.name} stage-wise")
    check_e2e(out["y"], ref.y, label=wl.name)
    # the plain entry point gives the same y, bit for bit, run after run
    y1 = g.forward()
    y2 = g.forward()
    assert np.array_equal(y1, out["y"]) and np.array_equal(y1, y2)


FULL = [WORKLOADS["mid_prefill"], WORKLOADS["prefill_5k"], WORKLOADS["prefill_21k"]]


def _h_block_per_pair(out, I, xq, label, gateup=None, gateup_format="q3_k"):
    """One H q8_1 block of every routed pair against the oracle's h_blocks:
    block (7 p + 3) mod F/32 of pair p, so every feature tile of the gate/up
    kernel and every token tile is compared."""
    wl = I.wl
    P, nfb = wl.T * wl.k, wl.F // 32
    ids = I.router_idx.reshape(-1)
    pairs = np.nonzero((ids >= 0) & (ids < wl.E))[0]
    fb = ((7 * pairs + 3) % nfb).astype(np.int32)
    ref = oracle.h_blocks(xq, I.router_idx, I.gateup_q3k if gateup is None else gateup, wl.L, wl.F, wl.E, pairs, fb,
                          gateup_format=gateup_format)
    check_h(out["h"][pairs, fb][:, None, :], ref[:, None, :], label=f"{label}: one H block of each of {P} pairs")


@pytest.mark.parametrize("wl", FULL, ids=lambda w: w.name)
def test_forward_full_size(wl):
    """The full-size workloads in the launch configuration the benchmark
    times: block dots of 8 gate/up and 8 down rows for every routed pair, one
    H block of every pair, y of every token against the oracle's down +
    combine fed the GPU's H, and the whole stage on sampled tokens (H, and y
    end to end)."""
    say(f"case {wl} (full size)")
    I, xq = _case(wl)
    g = Gpu(I, xq)
    gu_rows = (wl.F - 4, 8)
    dn_rows = (124, 8)  # across the boundary of the first two 128-row tiles of the down kernel
    out = g.forward_debug(gu_rows=gu_rows, dn_rows=dn_rows)
    say(f"{wl.name}: GPU done")
    _check_routing(out, I)
    _check_probes(out, I, xq, gu_rows, dn_rows)
    _h_block_per_pair(out, I, xq, wl.name)
    check_y(out["y"], stagewise_y(out, I), label=f"{wl.name} stage-wise, all {wl.T} tokens")
    rng = np.random.default_rng(7)
    ids = I.router_idx
    # tokens: random, plus ones routed to the most and the least popular experts
    counts = np.bincount(ids.reshape(-1), minlength=wl.E)
    big, small = np.argmax(counts), np.argmin(np.where(counts > 0, counts, 1 << 30))
    toks = set(rng.choice(wl.T, 24, replace=False).tolist())
    toks |= set(np.nonzero((ids == big).any(1))[0][:4].tolist()) | set(np.nonzero((ids == small).any(1))[0][:4].tolist())
    toks = np.array(sorted(toks), np.int64)
    pairs = (toks[:, None] * wl.k + np.arange(wl.k)[None, :]).reshape(-1)
    ref = oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, I.down_iq4nl, wl.L, wl.F, wl.E, tokens=toks)
    check_h(out["h"][pairs], ref.h, label=f"{wl.name} ({toks.size} tokens, every block)")
    check_e2e(out["y"][toks], ref.y, label=f"{wl.name} ({toks.size} tokens)")
    # determinism at full size
    y1 = g.forward()
    assert np.array_equal(y1, out["y"])


# Several work items per persistent workgroup, each of several K steps, over
# full token tiles (16 experts' tiles of 128 pairs and ragged ends): item
# changes inside a workgroup's pipeline, compared on every output.
MULTI_ITEM = Workload("multi_item", T=2048, L=1024, F=1024, E=8, k=4, zipf_s=1.1, seed=19)


def test_forward_multi_item_full_compare():
    wl = MULTI_ITEM
    say(f"case {wl}")
    I, xq = _case(wl)
    ref = oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, I.down_iq4nl, wl.L, wl.F, wl.E)
    g = Gpu(I, xq)
    out = g.forward_debug(gu_rows=(wl.F - 16, 32), dn_rows=(112, 32))
    _check_routing(out, I)
    _check_probes(out, I, xq, (wl.F - 16, 32), (112, 32))
    check_h(out["h"], ref.h, label=wl.name)
    check_y(out["y"], stagewise_y(out, I), label=f"{wl.name} stage-wise")
    check_e2e(out["y"], ref.y, label=wl.name)


@pytest.mark.parametrize("wl", [SMALL[1], SMALL[2], MULTI_ITEM, WORKLOADS["prefill_5k"]], ids=lambda w: w.name)
def test_atomic_combine(wl):
    """deterministic = 0: the down kernel adds each pair's weighted row into y
    with fp32 atomics (y zeroed by the route pass).  H is the same kernel's
    output as in the deterministic mode (bit for bit), y meets the stage-wise
    criterion on every token, and y differs from the ordered combine only by
    the order of the k additions."""
    say(f"atomic combine {wl}")
    I, xq = _case(wl)
    g = Gpu(I, xq)
    det = g.forward_debug()
    g.y.fill_(12345.0)  # stale y: the route pass must clear it
    out = g.forward_debug(deterministic=False)
    assert np.array_equal(out["h"], det["h"])
    check_y(out["y"], stagewise_y(out, I), label=f"{wl.name} atomic, stage-wise")
    rms = float(np.sqrt(np.mean(det["y"].astype(np.float64) ** 2)))
    diff = float(np.abs(out["y"].astype(np.float64) - det["y"]).max())
    say(f"{wl.name} atomic vs ordered combine: max|diff|/rms = {diff / rms:.3e}")
    # k fp32 additions in another order: a few ulps of the largest partial sum
    assert diff <= 1e-5 * rms


def test_invalid_and_duplicate_ids():
    wl = Workload("edge", T=40, L=256, F=96, E=5, k=3, seed=5)
    I, xq = _case(wl)
    idx = I.router_idx.copy()
    idx[0, :] = [-1, 5, 1 << 20]     # all invalid: token 0 gets y = 0
    idx[1, :] = [2, 2, 2]            # one expert three times
    idx[2, 1] = -3
    I.router_idx[...] = idx
    ref = oracle.forward(xq, idx, I.router_w, I.gateup_q3k, I.down_iq4nl, wl.L, wl.F, wl.E)
    g = Gpu(I, xq)
    out = g.forward_debug(gu_rows=(0, 2 * wl.F), dn_rows=(0, wl.L))
    _check_routing(out, I)
    assert out["dropped"] == ref.dropped == 4
    assert (out["y"][0] == 0).all()
    _check_probes(out, I, xq, (0, 2 * wl.F), (0, wl.L))
    check_h(out["h"], ref.h, label="edge")
    check_y(out["y"], stagewise_y(out, I), label="edge stage-wise")


# The large-batch counting sort at shapes that take each branch of its chunk
# scan: several lanes per expert (E = 128), one lane per expert (E = 600),
# and chunk histograms too large for the scan's LDS stage (36 chunks x 1024
# experts); and the one-workgroup sort (at most 4096 pairs and 512 experts)
# at its limits: 4088 pairs over 512 experts (the last wave's range part
# full), 4000 over 300, 80 over 7.  With invalid ids mixed in.  Routing only:
# perm, offsets, dropped.
@pytest.mark.parametrize("T,E,k", [(4000, 128, 8), (3000, 600, 8), (9000, 1024, 4),
                                   (511, 512, 8), (1000, 300, 4), (20, 7, 4)], ids=lambda v: str(v))
def test_route_scan_branches(T, E, k):
    wl = Workload(f"route_{T}_{E}", T=T, L=256, F=128, E=E, k=k, zipf_s=1.1, seed=21)
    say(f"route case T={T} E={E} k={k}")
    I, xq = _case(wl)
    rng = np.random.default_rng(5)
    idx = I.router_idx.copy()
    bad = rng.random(idx.shape) < 0.01
    idx[bad] = rng.choice(np.array([-1, E, 1 << 20], dtype=np.int32), size=int(bad.sum()))
    I.router_idx[...] = idx
    out = Gpu(I, xq).forward_debug()
    _check_routing(out, I)
    assert out["dropped"] == int(bad.sum())


def test_small_batch_invalid_and_duplicate_ids():
    """The small-batch kernels (at most 64 pairs) with dropped and repeated ids:
    only the valid pairs' rows are gathered, in sorted order."""
    wl = Workload("edge_small", T=9, L=256, F=96, E=5, k=3, seed=18)
    I, xq = _case(wl)
    idx = I.router_idx.copy()
    idx[0, :] = [-1, 5, 1 << 20]
    idx[1, :] = [2, 2, 2]
    idx[4, 2] = -3
    I.router_idx[...] = idx
    ref = oracle.forward(xq, idx, I.router_w, I.gateup_q3k, I.down_iq4nl, wl.L, wl.F, wl.E)
    g = Gpu(I, xq)
    out = g.forward_debug(gu_rows=(0, 2 * wl.F), dn_rows=(0, wl.L))
    _check_routing(out, I)
    assert out["dropped"] == ref.dropped == 4
    assert (out["y"][0] == 0).all()
    _check_probes(out, I, xq, (0, 2 * wl.F), (0, wl.L))
    check_h(out["h"], ref.h, label="edge_small")
    check_y(out["y"], stagewise_y(out, I), label="edge_small stage-wise")
    # every id invalid: no tile, nothing gathered, y = 0
    g.set_routing(np.full((wl.T, wl.k), 7, np.int32), I.router_w)
    assert (g.forward() == 0).all()


def test_all_invalid_and_zero_weights():
    wl = Workload("none", T=33, L=256, F=64, E=4, k=2, seed=6)
    I, xq = _case(wl)
    g = Gpu(I, xq)
    g.set_routing(np.full((33, 2), 9, np.int32), I.router_w)
    y = g.forward()
    assert (y == 0).all()
    g.set_routing(I.router_idx, np.zeros_like(I.router_w))
    y = g.forward()
    assert (y == 0).all()


def test_single_expert_single_slot():
    wl = Workload("e1", T=70, L=256, F=128, E=1, k=1, seed=8)
    I, xq = _case(wl)
    ref = oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, I.down_iq4nl, wl.L, wl.F, wl.E)
    g = Gpu(I, xq)
    out = g.forward_debug(gu_rows=(0, 256), dn_rows=(0, 256))
    _check_probes(out, I, xq, (0, 256), (0, 256))
    check_h(out["h"], ref.h, label="e1")
    check_y(out["y"], stagewise_y(out, I), label="e1 stage-wise")


def test_empty_batch_is_noop():
    import quantized_latent_moe_amd as lm
    s = lm.shapes(0, 1024, 2048, 128, 8)
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    y = torch.full((1, 1024), 3.0, device="cuda")
    lm.expert_forward(dummy, dummy, dummy, dummy, dummy, s, y, dummy)
    torch.cuda.synchronize()
    assert (y == 3.0).all()


@pytest.mark.parametrize("wl", [SMALL[1], SMALL[4]], ids=lambda w: w.name)
def test_workspace_contents_do_not_matter(wl):
    """The workspace needs no initialisation: a workspace filled with garbage,
    and one left over from a call with other shapes, give the same y bit for
    bit as a fresh one."""
    say(f"poisoned workspace {wl}")
    I, xq = _case(wl)
    g = Gpu(I, xq)
    g.ws.zero_()
    clean = g.forward()
    for fill in (0xFF, 0x7F, 0x80):
        g.ws.fill_(fill)
        assert np.array_equal(g.forward(), clean), f"workspace filled with {fill:#x}"
    # a larger call through the same workspace first, then this one again
    big = Workload("big_first", T=300, L=wl.L, F=wl.F, E=wl.E + 3, k=wl.k, seed=wl.seed + 100)
    Ib, xqb = _case(big)
    gb = Gpu(Ib, xqb)
    g.ws = torch.empty(max(g.ws.numel(), gb.ws.numel()), dtype=torch.uint8, device="cuda")
    gb.ws = g.ws
    gb.forward()
    assert np.array_equal(g.forward(), clean), "after a larger call through the same workspace"
