"""GPU parity of the router (softmax, top-k, renormalised weights) against the
CPU oracle, through the C ABI, and a captured graph of router + expert stage.

Criteria: expert ids bit-exact (integers decided by comparing the same fp32
logits); weights within the rounding bound of the fp32 formula the kernel
uses, w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max) over the picks:
    |w_gpu - w_ref| <= w_ref * (8 + k + 2 * max_j |l_j - l_max|) * 2^-23
(the fp32 difference l_j - l_max is rounded once, relative 2^-24, which moves
exp by |l_j - l_max| * 2^-24 relative; exp itself, the k-term sum and the
division add a few ulps).
"""
import numpy as np
import pytest

import oracle
from quantized_latent_moe_amd.inputs import WORKLOADS, Workload, make_inputs
from tests._gpu import Gpu, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import quantized_latent_moe_amd as lm  # noqa: E402


def _gpu_router(logits, k):
    T, E = logits.shape
    gl = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    idx = torch.full((max(T, 1), k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((max(T, 1), k), np.nan, dtype=torch.float32, device="cuda")
    lm.router_topk(gl, k, idx, w)
    torch.cuda.synchronize()
    return idx[:T].cpu().numpy(), w[:T].cpu().numpy()


def _check(logits, k, label):
    idx, w = _gpu_router(logits, k)
    ridx, rw = oracle.router_topk(logits, k)
    bad = np.argwhere(idx != ridx)
    if bad.size:
        say(f"{label}: first id mismatches at {bad[:3].tolist()}")
    assert np.array_equal(idx, ridx), f"{label}: ids differ"
    top = np.take_along_axis(logits, ridx[:, :1], 1).astype(np.float64)
    picked = np.take_along_axis(logits, ridx, 1).astype(np.float64)
    spread = np.where(np.isfinite(picked), np.abs(picked - top), 0.0).max(1, keepdims=True)
    bound = rw.astype(np.float64) * (8 + k + 2 * spread) * 2.0 ** -23 + 2.0 ** -126
    err = np.abs(w.astype(np.float64) - rw.astype(np.float64))
    say(f"{label}: ids equal, max weight err / bound = {(err / bound).max():.3f}")
    assert (err <= bound).all()


# From 256 tokens, E <= 256 and k <= 16 take the four-tokens-a-wave kernel:
# (1000, 128, 8), (300, 256, 1), (401, 16, 16) (a part-full last wave), (513, 40, 5)
# and (600, 200, 16) there; the rest the wave-per-token one.
@pytest.mark.parametrize("T,E,k,seed", [(1000, 128, 8, 0), (37, 8, 2, 1), (64, 1024, 64, 2), (100, 600, 10, 3),
                                         (5, 1, 1, 4), (33, 65, 64, 5), (7, 64, 64, 6), (300, 256, 1, 7),
                                         (401, 16, 16, 8), (513, 40, 5, 9), (600, 200, 16, 10)],
                         ids=lambda v: str(v))
def test_router_matches_oracle(T, E, k, seed):
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((T, E)) * rng.uniform(0.5, 4, (T, 1))).astype(np.float32)
    _check(logits, k, f"T={T} E={E} k={k}")


# T = 200 takes the wave-per-token kernel, T = 600 the four-tokens-a-wave one
@pytest.mark.parametrize("T", [200, 600])
def test_router_ties_and_masked_experts(T):
    rng = np.random.default_rng(9)
    E, k = 96, 8
    logits = (rng.integers(0, 4, (T, E)) * 0.5).astype(np.float32)     # many exact ties
    logits[:20, 1::2] = -np.inf                                           # masked experts
    logits[20:25, :] = -np.inf
    logits[20:25, [5, 70, 90]] = [1.0, 1.0, 0.5]                          # fewer finite logits than k
    _check(logits, k, "ties and masked experts")
    idx, w = _gpu_router(logits[20:25], k)
    assert (idx[:, :3] == [5, 70, 90]).all() and (w[:, 3:] == 0).all() and (idx[:, 3:] == [0, 1, 2, 3, 4]).all()


@pytest.mark.parametrize("name", ["decode", "prefill_5k", "prefill_21k"])
def test_router_on_workload_logits(name):
    """The workloads' own logits (with the Zipf prior and masked experts)."""
    wl = WORKLOADS[name]
    I = make_inputs(wl)
    _check(I.router_logits, wl.k, name)


def test_router_empty_is_noop():
    idx = torch.full((1, 2), 5, dtype=torch.int32, device="cuda")
    w = torch.full((1, 2), 3.0, device="cuda")
    lm.router_topk(torch.empty((0, 8), device="cuda"), 2, idx, w)
    torch.cuda.synchronize()
    assert (idx == 5).all() and (w == 3.0).all()


def test_graph_of_router_and_stage_replays_exactly():
    """Router + expert stage captured in one graph (decode shape): every
    replay, with eager work between replays, gives the eager call's y bit for
    bit, and the routing the oracle's."""
    wl = WORKLOADS["decode"]
    I = make_inputs(wl)
    xq = oracle.quantize_q8_1(I.x)
    g = Gpu(I, xq)
    logits = torch.from_numpy(I.router_logits).cuda()
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")

    def step():
        lm.router_topk(logits, wl.k, idx, w)
        lm.expert_forward(g.x, idx, w, g.gu, g.dn, g.s, g.y, g.ws)

    step()
    torch.cuda.synchronize()
    y_eager = g.y.clone()
    ridx, rw = oracle.router_topk(I.router_logits, wl.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    ref = oracle.forward(xq, ridx, w.cpu().numpy(), I.gateup_q3k, I.down_iq4nl, wl.L, wl.F, wl.E)
    err = float(np.abs(y_eager.cpu().numpy() - ref.y).max() / np.sqrt(np.mean(ref.y ** 2)))
    say(f"router + stage vs oracle (end to end): max|err|/rms = {err:.3e}")
    assert err < 2e-2
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    scratch = torch.randn(1 << 20, device="cuda")
    for r in range(4):
        g.y.fill_(float("nan"))
        idx.fill_(-1)
        graph.replay()
        scratch.mul_(1.0001)            # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(g.y, y_eager), f"replay {r}"
    say("4 graph replays of router + stage equal the eager call")
