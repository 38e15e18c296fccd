"""Pins for the oracle's block decoders and fp16 conversions.

The decoders are checked against an independent encoder (tests/_packers.py,
the inverse bit operations), against hand-derived single-field blocks, and
against the operand range the pages print for the folded Q3_K operand
(tests/golden/fold_range.txt).  fp16 conversions are checked against numpy's
IEEE binary16 conversion (a library routine).
"""
import os

import numpy as np
import pytest

import oracle
from tests._packers import IQ4NL_TABLE, pack_iq4nl, pack_q3k, pack_q8_1

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_half_to_double_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(ref) & (ref > 0))


def test_float_to_half_matches_numpy_rne():
    rng = np.random.default_rng(1)
    # every exponent that lands in or near binary16 range, random mantissas,
    # plus the exact halfway points between adjacent halves (ties to even)
    exps = rng.integers(-30, 18, size=200000)
    mant = rng.random(200000) + 1.0
    vals = (np.sign(rng.random(200000) - 0.5) * mant * np.exp2(exps)).astype(np.float32)
    h = np.arange(0, 0x7bff, dtype=np.uint16)
    mids = ((h.view(np.float16).astype(np.float64) + (h + 1).view(np.float16).astype(np.float64)) / 2).astype(np.float32)
    specials = np.array([0.0, -0.0, 65504.0, 65519.0, 65520.0, 1e9, 5.96e-8, 2.98e-8, 2.99e-8, 6.1e-5, 1e-30],
                        np.float32)
    allv = np.concatenate([vals, mids, -mids, specials])
    ref = allv.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(float(v)) for v in allv], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (allv[bad[:5]], got[bad[:5]], ref[bad[:5]])


def _random_q3k_fields(rng, n):
    return (rng.integers(0, 8, (n, 256)), rng.integers(0, 64, (n, 16)),
            rng.uniform(-2, 2, n).astype(np.float16))


def test_q3k_roundtrip_random():
    rng = np.random.default_rng(2)
    c, s, d = _random_q3k_fields(rng, 300)
    v, sg, dd = oracle.q3k_fields(pack_q3k(c, s, d))
    assert np.array_equal(v, c - 4)
    assert np.array_equal(sg, s - 32)
    assert np.array_equal(dd, d.astype(np.float64))


def test_q3k_roundtrip_every_field_value_at_every_position():
    n = 64
    b = np.arange(n)[:, None]
    codes = (np.arange(256)[None, :] + b) % 8          # every code at every element
    sc6 = (np.arange(16)[None, :] * 5 + b) % 64          # every scale at every sub-block
    d = np.full(n, 0.5, np.float16)
    v, sg, _ = oracle.q3k_fields(pack_q3k(codes, sc6, d))
    assert np.array_equal(v, codes - 4)
    assert np.array_equal(sg, sc6 - 32)
    # dequantized weight = d * sigma * v
    w = oracle.dequant_q3k(pack_q3k(codes, sc6, d))
    sub = np.repeat(sc6 - 32, 16, axis=1)
    assert np.array_equal(w, 0.5 * sub * (codes - 4))


def _blk(**fields):
    b = np.zeros(110, np.uint8)
    for off, val in fields.get("set", []):
        b[off] = val
    return b


def test_q3k_hand_blocks():
    # all-zero bytes: code 0 -> v = -4 everywhere, 6-bit scale 0 -> sigma = -32, d = 0
    v, s, d = oracle.q3k_fields(np.zeros(110, np.uint8))
    assert (v == -4).all() and (s == -32).all() and d[0] == 0.0
    # all-ones bytes except d: low bits 3, high bit 1 -> code 7 -> v = 3; scale 63 -> sigma = 31
    b = np.full(110, 0xFF, np.uint8)
    b[108:110] = np.array([1.0], np.float16).view(np.uint8)
    v, s, d = oracle.q3k_fields(b)
    assert (v == 3).all() and (s == 31).all() and d[0] == 1.0
    # one high bit: hmask[5] bit 6 = 4*1 + 2 -> element 128 + 64 + 5 = 197 gets code 4 (v = 0)
    b = np.zeros(110, np.uint8)
    b[5] = 1 << 6
    v, _, _ = oracle.q3k_fields(b)
    expect = np.full(256, -4)
    expect[197] = 0
    assert np.array_equal(v[0], expect)
    # qs[40] = 0b11_00_10_01: half 1, l = 8; j = 0..3 low bits 1, 2, 0, 3
    b = np.zeros(110, np.uint8)
    b[32 + 40] = 0b11001001
    v, _, _ = oracle.q3k_fields(b)
    expect = np.full(256, -4)
    expect[136], expect[168], expect[200], expect[232] = -3, -2, -4, -1
    assert np.array_equal(v[0], expect)
    # scales[3] = 0xA5 (nibbles of sub-blocks 3 and 11), scales[11] = 0b11_10_01_00
    # (top bits of sub-blocks 3, 7, 11, 15 = 0, 1, 2, 3)
    b = np.zeros(110, np.uint8)
    b[96 + 3] = 0xA5
    b[96 + 11] = 0b11100100
    _, s, _ = oracle.q3k_fields(b)
    expect = np.full(16, -32)
    expect[3] = 5 - 32
    expect[7] = 16 - 32
    expect[11] = (10 | 2 << 4) - 32
    expect[15] = 48 - 32
    assert np.array_equal(s[0], expect)


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    return vals


def test_folded_operand_range_matches_pages():
    # every (code, 6-bit scale) pair placed at element 0 / sub-block 0, decoded by the oracle
    cs = np.array([(c, s) for c in range(8) for s in range(64)])
    codes = np.zeros((len(cs), 256), np.int64)
    sc6 = np.zeros((len(cs), 16), np.int64)
    codes[:, 0] = cs[:, 0]
    sc6[:, 0] = cs[:, 1]
    v, sg, _ = oracle.q3k_fields(pack_q3k(codes, sc6, np.ones(len(cs), np.float16)))
    folded = -(v[:, 0].astype(int)) * sg[:, 0].astype(int)   # (4 - c) * (sc6 - 32)
    g = _golden("fold_range.txt")
    assert folded.min() == g["min"] and folded.max() == g["max"]
    # the operand is the negated weight product: the unnegated v*sigma reaches +128,
    # which int8 cannot hold, while the folded form always fits
    assert (v[:, 0].astype(int) * sg[:, 0]).max() == 128
    assert ((folded >= -128) & (folded <= 127)).all()


def test_iq4nl_roundtrip_and_table():
    rng = np.random.default_rng(3)
    nib = rng.integers(0, 16, (500, 32))
    d = rng.uniform(-1, 1, 500).astype(np.float16)
    kv, dd = oracle.iq4nl_fields(pack_iq4nl(nib, d))
    assert np.array_equal(kv, IQ4NL_TABLE[nib])
    assert np.array_equal(dd, d.astype(np.float64))
    # hand block: low nibbles 0..15, high nibbles 15..0 -> table forwards then backwards
    b = np.zeros(18, np.uint8)
    b[0:2] = np.array([2.0], np.float16).view(np.uint8)
    b[2:18] = np.arange(16) | ((15 - np.arange(16)) << 4)
    kv, dd = oracle.iq4nl_fields(b)
    table = [-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113]
    assert kv[0].tolist() == table + table[::-1]
    assert dd[0] == 2.0
    assert np.array_equal(oracle.dequant_iq4nl(b[None])[0], 2.0 * np.array(table + table[::-1]))


def test_q8_1_decode_roundtrip():
    rng = np.random.default_rng(4)
    q = rng.integers(-127, 128, (200, 32)).astype(np.int8)
    d = rng.uniform(0, 0.1, 200).astype(np.float16)
    s = rng.uniform(-5, 5, 200).astype(np.float16)
    deq = oracle.dequant_q8_1(pack_q8_1(q, d, s))
    assert np.array_equal(deq, d.astype(np.float64)[:, None] * q)
