"""Pins for the oracle's q8_1 rounding (used for the input rows and for H).

Checked by properties that any correct implementation of the rule must have:
the block maximum maps to +-127, the reconstruction error is bounded by half a
step (plus the fp16 rounding of the stored scale), an all-zero block stores
zeros, exact halfway cases round away from zero, and s = fp16(d * sum(q)).
"""
import numpy as np

import oracle


def _split(qb):
    d = qb[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    s = qb[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    q = qb[..., 4:36].view(np.int8).astype(np.int64)
    return d, s, q


def test_amax_maps_to_127_and_error_bound():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((400, 256)) * np.exp(rng.uniform(-8, 8, (400, 1)))).astype(np.float32)
    qb = oracle.quantize_q8_1(x)
    d16, _, q = _split(qb)
    xb = x.reshape(400, 8, 32).astype(np.float64)
    amax = np.abs(xb).max(-1)
    d = (amax.astype(np.float32) / np.float32(127)).astype(np.float64)   # unrounded scale
    i = np.abs(xb).argmax(-1)
    qa = np.take_along_axis(q, i[..., None], -1)[..., 0]
    xa = np.take_along_axis(xb, i[..., None], -1)[..., 0]
    assert np.array_equal(np.abs(qa), np.full_like(qa, 127))
    assert np.array_equal(np.sign(qa), np.sign(xa).astype(np.int64))
    assert (np.abs(q) <= 127).all()
    # |x - d16*q| <= d/2 (rounding) + 127*|d - d16| (stored-scale rounding) + slack for fp32 ops
    err = np.abs(xb - d16[..., None] * q)
    bound = d[..., None] * (0.5 + 1e-6) + 127 * np.abs(d - d16)[..., None]
    assert (err <= bound).all()
    # stored d is the fp16 rounding of the unrounded d
    assert np.array_equal(d16, d.astype(np.float16).astype(np.float64))


def test_zero_block():
    x = np.zeros((3, 64), np.float32)
    x[1, 32:] = np.linspace(-1, 1, 32)
    qb = oracle.quantize_q8_1(x)
    d, s, q = _split(qb)
    assert d[0, 0] == 0 and d[0, 1] == 0 and d[1, 0] == 0 and s[1, 0] == 0
    assert (q[0] == 0).all() and (q[1, 0] == 0).all()
    assert d[1, 1] > 0


def test_halfway_rounds_away_from_zero():
    # amax = 127 gives d = 1 and 1/d = 1 exactly, so x * (1/d) = x: the halves are exact ties
    x = np.zeros((1, 32), np.float32)
    vals = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5, -126.5, 3.4999998, -0.49999997]
    x[0, : len(vals)] = vals
    d, s, q = _split(oracle.quantize_q8_1(x))
    assert d[0, 0] == 1.0
    assert q[0, 0, : len(vals)].tolist() == [127, 3, -3, 1, -1, 2, -2, 127, -127, 3, 0]


def test_sum_field():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((50, 96)).astype(np.float32)
    qb = oracle.quantize_q8_1(x)
    d16, s16, q = _split(qb)
    amax = np.abs(x.reshape(50, 3, 32)).max(-1)
    d = amax / np.float32(127)
    expect = (d * q.sum(-1).astype(np.float32)).astype(np.float16).astype(np.float64)
    assert np.array_equal(s16, expect)
