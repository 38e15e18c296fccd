#!/usr/bin/env python3
"""Benchmark of the quantized latent-MoE expert stage on one MI355X.

A step is one whole expert-stage call (device routing sort, gate/up GEMM with
the SwiGLU + q8_1 epilogue, IQ4_NL down GEMM, weighted combine) over one
batch of synthetic inputs already resident in HBM.  Default workload: the
5268-token prefill (L=1024, F=2048, E=128, top-8, Zipf-skewed routing).

Prints one JSON line: whole-job tokens/s over exactly --steps timed calls, the
dominant kernel's roofline (algorithmic int8 ops per launch over its measured
launch duration, from events recorded on the kernels' own stream), a
decode-shaped bandwidth line, and the CPU oracle timed on a bounded token
sample of the same workload as a reference baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
# fp32 VALU instructions without packed math: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12   # 39.3 T lane-ops/s
METRIC = "expert-stage prefill tokens/s at T=5268; % int8 MFMA peak; HBM GB/s"


def algorithmic(wl, idx, gateup_q4_0=False):
    """Valid pairs, int8 ops per stage and algorithmic HBM bytes of one call
    (gate/up weights Q3_K, 110 B per 256 values, or Q4_0, 18 B per 32)."""
    import numpy as np
    ids = idx.reshape(-1)
    valid = (ids >= 0) & (ids < wl.E)
    pv = int(valid.sum())
    active = int(np.unique(ids[valid]).size)
    gu_bytes = 2 * wl.F * (wl.L // 32) * 18 if gateup_q4_0 else 2 * wl.F * (wl.L // 256) * 110
    dn_bytes = wl.L * (wl.F // 32) * 18
    ops_gateup = 2 * pv * 2 * wl.F * wl.L
    ops_down = 2 * pv * wl.L * wl.F
    # per-block scale folds: one (convert or scale) and one accumulate per
    # 32-value block result
    fold_gateup = 2 * pv * 2 * wl.F * (wl.L // 32)
    fold_down = 2 * pv * wl.L * (wl.F // 32)
    nbytes = (active * (gu_bytes + dn_bytes) + wl.T * (wl.L // 32) * 36 + wl.T * wl.k * 8 + wl.T * wl.L * 4)
    return dict(pairs=pv, active=active, ops_gateup=ops_gateup, ops_down=ops_down, bytes=nbytes,
                fold_gateup=fold_gateup, fold_down=fold_down,
                gu_bytes_active=active * gu_bytes, dn_bytes_active=active * dn_bytes)


class Stage:
    """One workload resident on the GPU (down weights IQ4_NL, or with
    down_format = DOWN_Q4_0 the same bytes read as Q4_0 blocks; gate/up
    weights Q3_K, or with gateup_format = GATEUP_Q4_0 Q4_0 blocks drawn for
    the workload)."""

    def __init__(self, wl, down_format=0, gateup_format=0):
        import numpy as np
        import torch
        import quantized_latent_moe_amd as lm
        from quantized_latent_moe_amd.inputs import make_inputs
        self.lm, self.torch, self.wl = lm, torch, wl
        self.down_format, self.gateup_format = down_format, gateup_format
        self.ex = bool(down_format or gateup_format)
        I = make_inputs(wl)
        self.inputs = I
        dev = torch.device("cuda", 0)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        x32 = t(I.x)
        self.x = torch.empty((wl.T, wl.L // 32, 36), dtype=torch.uint8, device=dev)
        lm.quantize_q8_1(x32, self.x)     # the producer's q8_1 rounding; not part of the stage
        del x32
        self.idx, self.w = t(I.router_idx), t(I.router_w)
        if gateup_format:
            from quantized_latent_moe_amd.inputs import make_gateup_q4_0
            self.gu = t(make_gateup_q4_0(wl))
        else:
            self.gu = t(I.gateup_q3k)
        self.dn = t(I.down_iq4nl)
        self.s = lm.shapes(wl.T, wl.L, wl.F, wl.E, wl.k)
        self.ws = torch.empty(lm.workspace_size(self.s), dtype=torch.uint8, device=dev)
        self.y = torch.empty((wl.T, wl.L), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    def step(self, deterministic=True):
        if self.ex:
            self.lm.expert_forward_fmt(self.x, self.idx, self.w, self.gu, self.dn, self.down_format, self.s, self.y,
                                       self.ws, gateup_format=self.gateup_format, deterministic=deterministic)
        elif deterministic:
            self.lm.expert_forward(self.x, self.idx, self.w, self.gu, self.dn, self.s, self.y, self.ws)
        else:
            self.lm.expert_forward_ex(self.x, self.idx, self.w, self.gu, self.dn, self.s, self.y, self.ws,
                                      deterministic=False)

    def routing_draws(self, n):
        """Device copies of the workload's routing (draw 0) and n - 1 more
        draws of activations and routing with the same weights: a list of
        (x q8_1, router_idx, router_w, algorithmic counts)."""
        import numpy as np
        torch, lm = self.torch, self.lm
        from quantized_latent_moe_amd.inputs import make_routing_draws
        out = [(self.x, self.idx, self.w, algorithmic(self.wl, self.inputs.router_idx))]
        for x, idx, w in make_routing_draws(self.wl, n - 1):
            xq = torch.empty_like(self.x)
            lm.quantize_q8_1(torch.from_numpy(x).cuda(), xq)
            out.append((xq, torch.from_numpy(np.ascontiguousarray(idx)).cuda(),
                        torch.from_numpy(np.ascontiguousarray(w)).cuda(), algorithmic(self.wl, idx)))
        torch.cuda.synchronize()
        return out

    def use(self, draw):
        self.x, self.idx, self.w = draw[0], draw[1], draw[2]

    def prime(self, seconds=0.1):
        """Part of setup, before the counted warm-up: run the stage for about
        `seconds` so that the GPU has left its idle clocks (the first tens of
        milliseconds of work in a fresh process run about 8% slower)."""
        torch = self.torch
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                self.step()
            torch.cuda.synchronize()

    def step_timed(self, events, deterministic=True):
        if self.ex:
            self.lm.expert_forward_fmt(self.x, self.idx, self.w, self.gu, self.dn, self.down_format, self.s, self.y,
                                       self.ws, gateup_format=self.gateup_format, debug=True, stage_events=events,
                                       deterministic=deterministic)
        else:
            self.lm.expert_forward_ex(self.x, self.idx, self.w, self.gu, self.dn, self.s, self.y, self.ws,
                                      stage_events=events, deterministic=deterministic)

    def time_steps(self, steps, warmup, deterministic=True):
        torch = self.torch
        for _ in range(warmup):
            self.step(deterministic)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            self.step(deterministic)
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return e0.elapsed_time(e1) / steps, wall

    def router_and_graph(self, steps):
        """µs of the router alone, and µs per step of router + stage replayed
        from one captured graph (each replay checked against the eager step)."""
        torch, lm, wl = self.torch, self.lm, self.wl
        logits = torch.from_numpy(self.inputs.router_logits).cuda()
        idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
        w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
        route = lambda: lm.router_topk(logits, wl.k, idx, w)

        def step():
            route()
            lm.expert_forward(self.x, idx, w, self.gu, self.dn, self.s, self.y, self.ws)

        for _ in range(3):
            step()
        torch.cuda.synchronize()
        ref = self.y.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g_route, g_step = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_route):
            for _ in range(10):
                route()
        with torch.cuda.graph(g_step):
            step()
        for _ in range(2):
            self.y.zero_()
            g_step.replay()
            torch.cuda.synchronize()
            if not torch.equal(self.y, ref):
                raise RuntimeError("graph replay of router + stage differs from the eager step")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(steps // 10, 2)
        e0.record()
        for _ in range(reps):
            g_route.replay()
        e1.record()
        torch.cuda.synchronize()
        router_us = e0.elapsed_time(e1) * 1e3 / (10 * reps)
        e0.record()
        for _ in range(steps):
            g_step.replay()
        e1.record()
        torch.cuda.synchronize()
        return router_us, e0.elapsed_time(e1) * 1e3 / steps

    def stage_times(self, steps, deterministic=True):
        """Mean ms of route / gate-up / down / combine over `steps` calls."""
        torch = self.torch
        evs = []
        for _ in range(steps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            for e in ev:
                e.record()          # creates the underlying hipEvent_t
            evs.append(ev)
        torch.cuda.synchronize()
        for ev in evs:
            self.step_timed(ev, deterministic)
        torch.cuda.synchronize()
        acc = [0.0] * 4
        for ev in evs:
            for i in range(4):
                acc[i] += ev[i].elapsed_time(ev[i + 1])
        return [a / steps for a in acc]


class DenseStage:
    """The latent layer's D and U projections (Q8_0 x q8_1) resident on the GPU:
    D takes the hidden rows (q8_1) to q8_1 latent rows, U takes latent rows
    (q8_1) to fp32 hidden rows."""

    def __init__(self, dwl):
        import numpy as np
        import torch
        import quantized_latent_moe_amd as lm
        from quantized_latent_moe_amd.inputs import make_dense_inputs
        self.lm, self.torch, self.wl = lm, torch, dwl
        I = make_dense_inputs(dwl)
        dev = torch.device("cuda", 0)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.xh = torch.empty((dwl.T, dwl.H // 32, 36), dtype=torch.uint8, device=dev)
        self.zl = torch.empty((dwl.T, dwl.L // 32, 36), dtype=torch.uint8, device=dev)
        lm.quantize_q8_1(t(I.x), self.xh)
        lm.quantize_q8_1(t(I.z), self.zl)
        self.dw, self.uw = t(I.d_q8_0), t(I.u_q8_0)
        self.dw4, self.uw4 = t(I.d_q4_0), t(I.u_q4_0)  # the same projections with Q4_0 weights
        self.xl = torch.empty((dwl.T, dwl.L // 32, 36), dtype=torch.uint8, device=dev)
        self.xlf = torch.empty((dwl.T, dwl.L), dtype=torch.float32, device=dev)
        self.out = torch.empty((dwl.T, dwl.H), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    def run_d(self):
        # decode-sized batches ask for the fp32 rows too: the library then
        # spreads the weight stream over many workgroups and rounds the rows
        # to q8_1 in a second kernel (q8_1 output alone keeps one workgroup
        # per 32 rows)
        w = self.wl
        self.lm.dense_q8_0(self.xh, self.dw, w.T, w.L, w.H, self.xlf if w.T <= 8 else None, self.xl)

    def run_u(self):
        w = self.wl
        self.lm.dense_q8_0(self.zl, self.uw, w.T, w.H, w.L, self.out, None)

    def run_d4(self):
        w = self.wl
        self.lm.dense_q4_0(self.xh, self.dw4, w.T, w.L, w.H, self.xlf if w.T <= 8 else None, self.xl)

    def run_u4(self):
        w = self.wl
        self.lm.dense_q4_0(self.zl, self.uw4, w.T, w.H, w.L, self.out, None)

    def time(self, fn, steps, warmup, out=None):
        """ms per call.  Decode-sized calls are replayed from a captured graph of
        10 calls (one Python call per launch would otherwise set the pace); every
        replay's output is checked against the eager call's."""
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if self.wl.T > 64 or out is None:
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps
        ref = out.clone()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(10):
                fn()
        reps = max(1, steps // 10)
        for _ in range(2):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(out, ref):
                raise RuntimeError("graph replay of the dense projection differs from the eager call")
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (10 * reps)

    def report(self, steps, warmup):
        w = self.wl
        res = {"workload": w.name, "T": w.T, "H": w.H, "L": w.L}
        for name, fn, N, K, out_bytes, out, wb in (
                ("D", self.run_d, w.L, w.H, w.T * (w.L // 32) * 36, self.xl, 34),
                ("U", self.run_u, w.H, w.L, w.T * w.H * 4, self.out, 34),
                ("D_q4_0", self.run_d4, w.L, w.H, w.T * (w.L // 32) * 36, self.xl, 18),
                ("U_q4_0", self.run_u4, w.H, w.L, w.T * w.H * 4, self.out, 18)):
            ms = self.time(fn, steps, warmup, out)
            ops = 2 * w.T * N * K
            folds = 2 * w.T * N * (K // 32)
            nbytes = N * (K // 32) * wb + w.T * (K // 32) * 36 + out_bytes
            fold_t = folds / (ms * 1e-3) / 1e12
            gbs = nbytes / (ms * 1e-3) / 1e9
            # prefill: bound by the per-block fp32 fold on the VALU (2 lane-ops per
            # block result); decode: by streaming the weights
            roof = ({"bound": "alu", "achieved": round(fold_t, 2), "peak": round(PEAK_VALU_TOPS, 1),
                     "unit": "T lane-op/s", "frac": round(fold_t / PEAK_VALU_TOPS, 4)} if w.T > 64 else
                    {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4)})
            res[name] = {"us": round(ms * 1e3, 2), "N": N, "K": K, "roofline": roof,
                         "int8_frac": round(ops / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
                         "hbm_gbs": round(gbs, 1), "alg_bytes": nbytes}
            print(f"[bench] {w.name} {name}: {ms * 1e3:.2f} us", file=sys.stderr, flush=True)
        return res


# Cold-call repetitions per workload (one call between two events, caches
# evicted before each): tiny, decode, mid_prefill 50; prefill_5k 20; prefill_21k 10.
COLD_REPS = {"tiny": 50, "decode": 50, "mid_prefill": 50, "prefill_5k": 20, "prefill_21k": 10}


class Evictor:
    """Streams a 1 GiB buffer through the caches by reading it (a sum into
    one float): larger than the 256 MB last-level cache and the L2s, and it
    leaves them holding clean lines, so the next call pays no write-back of
    the eviction's own data inside its timed window."""

    def __init__(self):
        import torch
        self.torch = torch
        self.buf = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
        self.out = torch.empty((), dtype=torch.float32, device="cuda")

    def __call__(self):
        self.torch.sum(self.buf, dim=0, out=self.out)

    def free(self):
        del self.buf, self.out
        self.torch.cuda.empty_cache()


def decode_cold(st, reps, draws=4):
    """One call at a time with the L2s and the 256 MB last-level cache evicted
    before each (a 1 GiB buffer read), rotating among `draws` routings of
    the workload (the same weights), so no call finds its experts in cache:
    median, p10 and p90 µs, and the algorithmic bytes of each call (its
    active experts' weights, x, routing, y) over its time."""
    import numpy as np
    torch = st.torch
    ds = st.routing_draws(draws)
    evict = Evictor()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times, gbs = [], []
    for i in range(reps):
        d = ds[i % len(ds)]
        st.use(d)
        evict()
        e0.record()
        st.step()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3
        times.append(us)
        gbs.append(d[3]["bytes"] / (us * 1e-6) / 1e9)
    st.use(ds[0])
    evict.free()
    med = float(np.median(times))
    return {"median_us": round(med, 2), "p10_us": round(float(np.percentile(times, 10)), 2),
            "p90_us": round(float(np.percentile(times, 90)), 2), "calls": reps, "routing_draws": len(ds),
            "active_experts": [d[3]["active"] for d in ds], "alg_bytes": [d[3]["bytes"] for d in ds],
            "hbm_gbs_median": round(float(np.median(gbs)), 1),
            "hbm_frac_median": round(float(np.median(gbs)) / PEAK_HBM_GBS, 4)}


def combine_report(names, steps, warmup):
    """The two combines at the large workloads: the slot buffer with the
    ordered combine kernel (deterministic, the default) and the fp32 atomic
    adds of the down kernel into y (deterministic = 0): ms per step back to
    back, and the route / gate-up / down / combine times by events."""
    import torch
    from quantized_latent_moe_amd.inputs import WORKLOADS
    stage = ["route", "gateup", "down", "combine"]
    rep = {}
    for name in names:
        st = Stage(WORKLOADS[name])
        st.prime()
        r = {}
        for label, det in (("slots", True), ("atomic", False)):
            ms, _ = st.time_steps(steps, warmup, deterministic=det)
            times = st.stage_times(steps, deterministic=det)
            r[label] = {"ms_per_step": round(ms, 5), "stage_ms": {k: round(v, 5) for k, v in zip(stage, times)}}
            print(f"[bench] {name} combine {label}: {ms * 1e3:.1f} us/step, route {times[0] * 1e3:.1f}, down "
                  f"{times[2] * 1e3:.1f}, combine {times[3] * 1e3:.1f} us", file=sys.stderr, flush=True)
        r["atomic_over_slots"] = round(r["atomic"]["ms_per_step"] / r["slots"]["ms_per_step"], 4)
        rep[name] = r
        del st
        torch.cuda.empty_cache()
    return rep


def device_info():
    """CU count from the device properties, and a measured plain streaming
    copy (1 GiB read and 1 GiB written per call, bytes of both counted) next
    to the nominal 8 TB/s."""
    import torch
    p = torch.cuda.get_device_properties(0)
    src = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * (1 << 30) * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "stream_copy_gbs": round(gbs, 1), "hbm_peak_gbs": PEAK_HBM_GBS}


def per_config(names):
    """Every workload timed one call at a time, with the L2s and the 256 MB
    last-level cache evicted before each call (a 1 GiB buffer read), as the
    median, p10 and p90 of the call time; and the back-to-back rate."""
    import numpy as np
    import torch
    from quantized_latent_moe_amd.inputs import WORKLOADS
    evict = Evictor()
    out = {}
    for name in names:
        wl = WORKLOADS[name]
        st = Stage(wl)
        st.prime(0.05)
        alg = algorithmic(wl, st.inputs.router_idx)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(COLD_REPS[name]):
            evict()
            e0.record()
            st.step()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        warm_ms, _ = st.time_steps(COLD_REPS[name], 3)
        med = float(np.median(times))
        ops = alg["ops_gateup"] + alg["ops_down"]
        out[name] = {"T": wl.T, "cold_us": {"median": round(med, 2), "p10": round(float(np.percentile(times, 10)), 2),
                                            "p90": round(float(np.percentile(times, 90)), 2), "calls": len(times)},
                     "warm_us": round(warm_ms * 1e3, 2),
                     "tokens_per_s_cold": round(wl.T / (med * 1e-6), 1),
                     "int8_frac_cold": round(ops / (med * 1e-6) / 1e12 / PEAK_INT8_TOPS, 4),
                     "alg_gbs_cold": round(alg["bytes"] / (med * 1e-6) / 1e9, 1)}
        print(f"[bench] {name}: cold median {med:.1f} us (p10 {out[name]['cold_us']['p10']}, "
              f"p90 {out[name]['cold_us']['p90']}), back-to-back {warm_ms * 1e3:.1f} us", file=sys.stderr, flush=True)
        del st
        torch.cuda.empty_cache()
    evict.free()
    return out


def cpu_baseline_dense(dwl, target_s):
    """The oracle's D and U projections, as they stand, on the first n tokens."""
    import oracle
    from quantized_latent_moe_amd.inputs import make_dense_inputs
    I = make_dense_inputs(dwl)
    xq, zq = oracle.quantize_q8_1(I.x), oracle.quantize_q8_1(I.z)

    def run(n):
        toks = list(range(n))
        oracle.dense_q8_0(xq, I.d_q8_0, dwl.L, dwl.H, tokens=toks)
        oracle.dense_q8_0(zq, I.u_q8_0, dwl.H, dwl.L, tokens=toks)

    cores = oracle.num_threads()
    n0 = min(dwl.T, max(cores, 8))
    t0 = time.perf_counter()
    run(n0)
    per_tok = (time.perf_counter() - t0) / n0
    n = int(min(dwl.T, max(n0, target_s / max(per_tok, 1e-9))))
    t0 = time.perf_counter()
    run(n)
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "tokens/s (D + U)", "cores": cores, "kind": "oracle",
            "sample": f"first {n} of {dwl.T} tokens of {dwl.name}, D and U, {dt:.1f} s"}


def host_cpu():
    """CPU model and the host threads this process may use."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count()}


def cpu_baseline(wl, target_s, runs=3):
    """The oracle, as it stands, on the first n tokens of the same workload:
    the median of `runs` timed runs, n chosen for about target_s / runs
    seconds each."""
    import numpy as np
    import oracle
    from quantized_latent_moe_amd.inputs import make_inputs
    I = make_inputs(wl)
    xq = oracle.quantize_q8_1(I.x)
    run = lambda n: oracle.forward(xq, I.router_idx, I.router_w, I.gateup_q3k, I.down_iq4nl, wl.L, wl.F, wl.E,
                                   tokens=np.arange(n), want_h=False)
    cores = oracle.num_threads()
    n0 = min(wl.T, max(cores, 8))
    t0 = time.perf_counter()
    run(n0)
    per_tok = (time.perf_counter() - t0) / n0
    n = int(min(wl.T, max(n0, target_s / runs / max(per_tok, 1e-9))))
    rates = []
    for _ in range(runs):
        t0 = time.perf_counter()
        run(n)
        rates.append(n / (time.perf_counter() - t0))
    med = float(np.median(rates))
    return {"value": round(med, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n} of {wl.T} tokens of {wl.name} ({n * wl.k} routed pairs), median of {runs} runs "
                      f"({', '.join(f'{r:.1f}' for r in rates)} tokens/s), {n * runs / med:.1f} s in all",
            "runs_tokens_per_s": [round(r, 3) for r in rates], **host_cpu()}


KERNEL_SOURCES = {"k_gateup": "gateup.hip", "k_down": "down.hip", "k_gateup_q40": "gateup_q40.hip"}


def kernel_source_hash(kernel):
    """sha256 over the kernel's source file, the shared internal header and the
    flags the source is compiled with."""
    import hashlib
    from quantized_latent_moe_amd import build as hipbuild
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "lat_moe_internal.h"):
        h.update(open(os.path.join(ROOT, "quantized_latent_moe_amd", "csrc", f), "rb").read())
    h.update(" ".join(hipbuild.compile_flags(KERNEL_SOURCES[kernel])).encode())
    return h.hexdigest()


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary
    (profiles/<kernel>_<workload>_traffic.txt), or None if there is none or the
    kernel's source has changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(p):
        return None
    vals = dict(line.split()[:2] for line in open(p) if line.startswith(("hbm_bytes_per_launch", "source_sha256")))
    if vals.get("source_sha256") != kernel_source_hash(kernel) or "hbm_bytes_per_launch" not in vals:
        return None
    return int(float(vals["hbm_bytes_per_launch"]))


def _pmc_rows(d):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        rows += list(csv.DictReader(open(f)))
    return rows


def pmc_summary(fetch_dir, write_dir, kernel, copy_mib):
    """HBM bytes per launch of `kernel` from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the plain copy of
    copy_mib MiB (torch.neg, one read and one write of every byte)."""
    n = copy_mib << 20
    out = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = {}
        for r in _pmc_rows(d):
            if r["Counter_Name"] != name:
                continue
            per.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), 0.0)
            per[(r["Kernel_Name"], r["Dispatch_Id"])] += float(r["Counter_Value"]) * 1024.0
        copy = [v for (k, _), v in per.items() if "elementwise" in k]
        kern = [v for (k, _), v in per.items() if re.search(r"::%s[<(]" % kernel, k)]
        if not copy or not kern:
            sys.exit(f"{name}: no copy ({len(copy)}) or {kernel} ({len(kern)}) dispatches in {d}")
        copy_b = max(copy)                    # the copy dispatches (ignore smaller elementwise kernels)
        scale = n / copy_b
        out[name] = (sum(kern) / len(kern), copy_b, scale, len(kern))
    fetch = out["FETCH_SIZE"][0] * out["FETCH_SIZE"][2]
    write = out["WRITE_SIZE"][0] * out["WRITE_SIZE"][2]
    print(f"kernel {kernel}")
    for name, (kb, cb, sc, nk) in out.items():
        print(f"{name}: {kb:.0f} B per launch (mean of {nk} dispatches); copy of {n} B reads as {cb:.0f} B; "
              f"scale {sc:.4f}")
    print(f"hbm_read_bytes_per_launch {fetch:.0f}")
    print(f"hbm_write_bytes_per_launch {write:.0f}")
    print(f"hbm_bytes_per_launch {fetch + write:.0f}")


def q4_0_report(steps, warmup, gateup_q4_0, workloads=("prefill_5k", "decode")):
    """The stage with Q4_0 weights: down weights Q4_0 (each workload's random
    down blocks read as Q4_0, the same bytes), and with gateup_q4_0 the
    gate/up weights Q4_0 too (drawn for the workload).  Time per step, stage
    times and the Q4_0 kernels against their fold roof, at prefill_5k and
    decode (or the given workloads)."""
    import torch
    import quantized_latent_moe_amd as lm
    from quantized_latent_moe_amd.inputs import WORKLOADS
    names = ["route", "gateup", "down", "combine"]
    label = "Q4_0 gate/up + down" if gateup_q4_0 else "Q4_0 down"
    rep = {}
    for name in workloads:
        wl = WORKLOADS[name]
        st = Stage(wl, down_format=lm.DOWN_Q4_0, gateup_format=lm.GATEUP_Q4_0 if gateup_q4_0 else 0)
        st.prime()
        n = steps if name != "decode" else max(steps, 50)
        ms, _ = st.time_steps(n, warmup)
        stages = st.stage_times(n)
        alg = algorithmic(wl, st.inputs.router_idx, gateup_q4_0=gateup_q4_0)
        # the decode workload runs the two-launch path: only gate/up and down are stages there
        shown = ("gateup", "down") if name == "decode" else names
        r = {"workload": name, "ms_per_step": round(ms, 5), "tokens_per_s": round(wl.T / (ms * 1e-3), 1),
             "stage_ms": {k: round(v, 5) for k, v in zip(names, stages) if k in shown}}
        if name == "prefill_5k":
            fold = alg["fold_down"] / (stages[2] * 1e-3) / 1e12
            r["down_roofline"] = {"bound": "alu", "kernel": "k_down (Q4_0)", "achieved": round(fold, 2),
                                  "peak": round(PEAK_VALU_TOPS, 1), "unit": "T lane-op/s",
                                  "frac": round(fold / PEAK_VALU_TOPS, 4)}
            if gateup_q4_0:
                fold = alg["fold_gateup"] / (stages[1] * 1e-3) / 1e12
                r["gateup_roofline"] = {"bound": "alu", "kernel": "k_gateup_q40", "achieved": round(fold, 2),
                                        "peak": round(PEAK_VALU_TOPS, 1), "unit": "T lane-op/s",
                                        "frac": round(fold / PEAK_VALU_TOPS, 4),
                                        "traffic": read_traffic("k_gateup_q40", name)}
        else:
            gbs = alg["bytes"] / (ms * 1e-3) / 1e9
            r.update(alg_bytes=alg["bytes"], hbm_gbs=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4))
        print(f"[bench] {label}, {name}: {ms * 1e3:.1f} us/step, gate/up {stages[1] * 1e3:.1f} us, "
              f"down {stages[2] * 1e3:.1f} us", file=sys.stderr, flush=True)
        rep[name] = r
        del st
        torch.cuda.empty_cache()
    return rep


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_5k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-du", action="store_true", help="skip the latent D / U projection timings")
    ap.add_argument("--du-only", action="store_true", help="time only the latent D / U projections")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the cold-cache timing of every workload (per_config)")
    ap.add_argument("--no-formats", action="store_true", help="skip the Q4_0 weight timings")
    ap.add_argument("--no-combine", action="store_true",
                    help="skip the slot-buffer vs atomic-add combine comparison at prefill_5k and prefill_21k")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode workload (cold, rotating routings; and back to back) and print it")
    ap.add_argument("--formats-only", action="store_true",
                    help="time only the stage with Q4_0 gate/up and down weights, at --workload")
    ap.add_argument("--cpu-seconds", type=float, default=18.0, help="CPU oracle time over its 3 runs")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (three times), the reference for counter scaling")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of --calibrate-copy and exit")
    ap.add_argument("--kernel", default="k_gateup", help="kernel the --pmc-summary is for")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.kernel, args.calibrate_copy or 256)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the expert stage here is built and timed on a single MI355X "
              f"(--gpus {args.gpus} is not supported: the token-parallel sharding across GPUs is not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_latent_moe_amd.inputs import WORKLOADS
    torch.cuda.set_device(0)
    wl = WORKLOADS[args.workload]
    print(f"[bench] workload {wl}", file=sys.stderr, flush=True)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)   # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        del src, dst
    if args.du_only:
        from quantized_latent_moe_amd.inputs import DENSE_WORKLOADS
        for name in ("du_prefill_5k", "du_decode"):
            ds = DenseStage(DENSE_WORKLOADS[name])
            rep = ds.report(args.steps, args.warmup)
            del ds
            if name == "du_prefill_5k" and not args.no_cpu_baseline:
                rep["cpu_baseline"] = cpu_baseline_dense(DENSE_WORKLOADS[name], 3.0)
            print(json.dumps(rep), flush=True)
        return
    if args.formats_only:
        print(json.dumps(q4_0_report(args.steps, args.warmup, gateup_q4_0=True, workloads=(wl.name,))), flush=True)
        return
    if args.decode_only:
        ds = Stage(WORKLOADS["decode"])
        ds.prime()
        dms, _ = ds.time_steps(max(args.steps, 50), args.warmup)
        cold = decode_cold(ds, max(args.steps, 50))
        print(f"[bench] decode cold {cold['median_us']:.2f} us/step ({cold['hbm_gbs_median']:.0f} GB/s), "
              f"back to back {dms * 1e3:.2f} us/step", file=sys.stderr, flush=True)
        print(json.dumps({"workload": "decode", "cold": cold, "warm_us_per_step": round(dms * 1e3, 2)}), flush=True)
        return
    st = Stage(wl)
    st.prime()
    alg = algorithmic(wl, st.inputs.router_idx)
    ms, wall_ms = st.time_steps(args.steps, args.warmup)
    print(f"[bench] {ms:.4f} ms/step (events), {wall_ms:.4f} ms/step (host clock)", file=sys.stderr, flush=True)
    stages = st.stage_times(args.steps)
    router_us, _ = st.router_and_graph(args.steps)
    names = ["route", "gateup", "down", "combine"]
    # decode-sized batches (at most 64 routed pairs, L <= 1024, F <= 2048) make
    # two launches, the GEMV-shaped gate/up and down kernels: no route or
    # combine kernel runs between their events
    small = wl.T * wl.k <= 64 and wl.L <= 1024 and wl.F <= 2048
    shown = ["gateup", "down"] if small else names
    print("[bench] stage ms: " + ", ".join(f"{n}={stages[names.index(n)]:.4f}" for n in shown), file=sys.stderr,
          flush=True)
    ops = {"gateup": alg["ops_gateup"], "down": alg["ops_down"]}
    folds = {"gateup": alg["fold_gateup"], "down": alg["fold_down"]}
    dom = max(("gateup", "down"), key=lambda n: stages[names.index(n)])
    dom_ms = stages[names.index(dom)]
    achieved = ops[dom] / (dom_ms * 1e-3) / 1e12
    kernel = ({"gateup": "k_dec_gateup", "down": "k_dec_down"} if small else {"gateup": "k_gateup", "down": "k_down"})[dom]
    fold_tops = folds[dom] / (dom_ms * 1e-3) / 1e12
    # The dominant kernel against the int8 MFMA peak (the metric's roof).  Its
    # binding limit is the per-block fp32 scale fold on the VALU (2 unpacked
    # VALU lane-ops per 32-value block result, about 4x the block's MFMA
    # time), given beside it as fold_valu.
    roofline = {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS,
                "unit": "TOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4),
                "traffic": read_traffic(kernel, wl.name), "launch_ms": round(dom_ms, 5),
                "fold_valu": {"bound": "alu", "achieved": round(fold_tops, 2), "peak": round(PEAK_VALU_TOPS, 1),
                              "unit": "T lane-op/s", "frac": round(fold_tops / PEAK_VALU_TOPS, 4)}}
    total_ops = alg["ops_gateup"] + alg["ops_down"]
    out = {
        "metric": METRIC,
        "value": round(wl.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "L": wl.L, "F": wl.F, "E": wl.E, "k": wl.k,
                   "zipf_s": wl.zipf_s, "n_masked": wl.n_masked, "seed": wl.seed, "pairs": alg["pairs"],
                   "active_experts": alg["active"]},
        "roofline": roofline,
        "stage_ms": {n: round(stages[names.index(n)], 5) for n in shown},
        "router_us": round(router_us, 2),
        "stage_int8_frac": round(total_ops / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
        "stage_hbm_gbs": round(alg["bytes"] / (ms * 1e-3) / 1e9, 1),
    }
    del st
    torch.cuda.empty_cache()
    if not args.no_decode:
        dwl = WORKLOADS["decode"]
        ds = Stage(dwl)
        ds.prime()
        dalg = algorithmic(dwl, ds.inputs.router_idx)
        dms, _ = ds.time_steps(max(args.steps, 50), args.warmup)
        dstage = ds.stage_times(max(args.steps, 50))
        gbs = dalg["bytes"] / (dms * 1e-3) / 1e9
        cold = decode_cold(ds, 100)
        r_us, g_us = ds.router_and_graph(max(args.steps, 50))
        # headline: caches evicted before every call, four routings in turn;
        # back to back (same routing, weights may stay in the last-level
        # cache between calls) beside it
        out["decode"] = {"workload": dwl.name, "us_per_step": cold["median_us"],
                         "hbm_gbs": cold["hbm_gbs_median"], "hbm_frac": cold["hbm_frac_median"],
                         "cold": cold,
                         "warm": {"us_per_step": round(dms * 1e3, 2), "alg_bytes": dalg["bytes"],
                                  "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                                  # decode-sized batches make two launches (gate/up, down): no route
                                  # or combine kernel, so only those two intervals are stage times
                                  "stage_us": {"gateup": round(dstage[1] * 1e3, 2),
                                               "down": round(dstage[2] * 1e3, 2)}},
                         "router_us": round(r_us, 2),
                         "router_and_stage_graph_us_per_step": round(g_us, 2)}
        print(f"[bench] decode router {r_us:.2f} us, router + stage from one graph {g_us:.2f} us/step",
              file=sys.stderr, flush=True)
        print(f"[bench] decode cold {cold['median_us']:.2f} us/step ({cold['hbm_gbs_median']:.0f} GB/s), "
              f"back to back {dms * 1e3:.2f} us/step ({gbs:.0f} GB/s)", file=sys.stderr, flush=True)
        del ds
    if not args.no_combine:
        out["combine"] = combine_report(["prefill_5k", "prefill_21k"], args.steps, args.warmup)
    if not args.no_formats:
        out["down_q4_0"] = q4_0_report(args.steps, args.warmup, gateup_q4_0=False)
        out["gateup_down_q4_0"] = q4_0_report(args.steps, args.warmup, gateup_q4_0=True)
    if not args.no_per_config:
        out["device"] = device_info()
        out["per_config"] = per_config(["tiny", "decode", "mid_prefill", "prefill_5k", "prefill_21k"])
    if not args.no_du:
        from quantized_latent_moe_amd.inputs import DENSE_WORKLOADS
        du = {}
        for name in ("du_prefill_5k", "du_decode"):
            ds = DenseStage(DENSE_WORKLOADS[name])
            du[name] = ds.report(args.steps if name == "du_prefill_5k" else max(args.steps, 50), args.warmup)
            del ds
            if name == "du_prefill_5k" and not args.no_cpu_baseline:
                du[name]["cpu_baseline"] = cpu_baseline_dense(DENSE_WORKLOADS[name], 3.0)
        out["latent_du"] = du
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
