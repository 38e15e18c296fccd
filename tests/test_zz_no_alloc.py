"""The no-allocation entry point (lat_moe_expert_forward_noalloc) against the
workspace entry point (lat_moe_expert_forward), through the C ABI: the same
kernels on the library's fixed per-GPU scratch, so y must be equal bit for
bit.  Two calls in a row, the second with a smaller input (the scratch keeps
the first call's contents, which the kernels must not depend on), then the
first shape again; a shape whose workspace exceeds the scratch is refused
with nothing written."""
import numpy as np
import pytest

from quantized_latent_moe_amd.inputs import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import quantized_latent_moe_amd as lm  # noqa: E402


def _say(*a):
    print("[gpu-test]", *a, flush=True)


class _Case:
    def __init__(self, wl):
        I = make_inputs(wl)
        dev = torch.device("cuda", 0)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.wl = wl
        self.x = torch.empty((wl.T, wl.L // 32, 36), dtype=torch.uint8, device=dev)
        lm.quantize_q8_1(t(I.x), self.x)
        self.idx, self.w, self.gu, self.dn = t(I.router_idx), t(I.router_w), t(I.gateup_q3k), t(I.down_iq4nl)
        self.s = lm.shapes(wl.T, wl.L, wl.F, wl.E, wl.k)

    def with_workspace(self):
        ws = torch.empty(lm.workspace_size(self.s), dtype=torch.uint8, device="cuda")
        y = torch.full((self.wl.T, self.wl.L), float("nan"), device="cuda")
        lm.expert_forward(self.x, self.idx, self.w, self.gu, self.dn, self.s, y, ws)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    def no_alloc(self):
        y = torch.full((self.wl.T, self.wl.L), float("nan"), device="cuda")
        lm.expert_forward_noalloc(self.x, self.idx, self.w, self.gu, self.dn, self.s, y)
        torch.cuda.synchronize()
        return y.cpu().numpy()


def test_noalloc_equals_workspace_entry_point():
    big = _Case(WORKLOADS["mid_prefill"])       # 4096 pairs: the route passes and persistent kernels
    small = _Case(WORKLOADS["decode"])          # 32 pairs: the small-batch kernels
    assert lm.workspace_size(big.s) <= lm.NOALLOC_SCRATCH_BYTES
    ref_big, ref_small = big.with_workspace(), small.with_workspace()
    for label, case, ref in (("mid_prefill", big, ref_big), ("decode (smaller, second)", small, ref_small),
                             ("mid_prefill again", big, ref_big)):
        _say(f"no-alloc call: {label}, shapes T={case.wl.T} E={case.wl.E} k={case.wl.k}")
        got = case.no_alloc()
        assert np.isfinite(got).all()
        assert np.array_equal(got, ref), label
    # a ragged shape with more than 8 experts per token, after the others
    odd = _Case(Workload("noalloc_ragged", T=150, L=768, F=160, E=12, k=10, zipf_s=1.1, seed=4))
    _say("no-alloc call: ragged, k = 10")
    assert np.array_equal(odd.no_alloc(), odd.with_workspace())


def test_noalloc_refuses_shapes_beyond_the_scratch():
    wl = WORKLOADS["prefill_5k"]
    s = lm.shapes(wl.T, wl.L, wl.F, wl.E, wl.k)
    assert lm.workspace_size(s) > lm.NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(16, dtype=torch.uint8, device="cuda")
    y = torch.full((2, wl.L), 3.0, device="cuda")
    with pytest.raises(lm.LatMoeError, match="error 5"):
        lm.expert_forward_noalloc(dummy, dummy, dummy, dummy, dummy, s, y)
    torch.cuda.synchronize()
    assert (y == 3.0).all()
