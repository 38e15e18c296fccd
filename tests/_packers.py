"""Block *encoders* for the ggml Q3_K / IQ4_NL / q8_1 / Q8_0 layouts (test helper).

These write fields into bytes -- the inverse of the oracle's decoders -- so a
round trip (pack here, decode in the oracle) pins the decoders' bit layout
without re-typing them.  Layouts (ggml GGUF block formats):
  Q3_K   110 B: hmask[32] | qs[64] | scales[12] | d fp16    (256 weights)
  IQ4_NL  18 B: d fp16 | qs[16]                               (32 weights)
  q8_1    36 B: d fp16 | s fp16 | qs[32] int8                 (32 values)
  Q8_0    34 B: d fp16 | qs[32] int8                          (32 weights)
"""
import numpy as np

IQ4NL_TABLE = np.array([-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113], np.int64)


def pack_q3k(codes: np.ndarray, sc6: np.ndarray, d: np.ndarray) -> np.ndarray:
    """codes [n,256] in 0..7, sc6 [n,16] in 0..63, d [n] float16 -> [n,110] uint8.

    Element e = 128*h + 32*j + l keeps its low two bits in qs[32*h + l] at bit
    position 2*j and its high bit in hmask[l] at bit position 4*h + j.
    Sub-block scale s keeps its low nibble in scales[s % 8] (low nibble for
    s < 8, high nibble otherwise) and its top two bits in scales[8 + s % 4]
    at bit position 2*(s // 4)."""
    codes = np.asarray(codes, np.int64)
    sc6 = np.asarray(sc6, np.int64)
    n = codes.shape[0]
    out = np.zeros((n, 110), np.uint8)
    e = np.arange(256)
    h, j, l = e // 128, (e % 128) // 32, e % 32
    hmask = np.zeros((n, 32), np.int64)
    qs = np.zeros((n, 64), np.int64)
    for ei in range(256):
        c = codes[:, ei]
        qs[:, 32 * h[ei] + l[ei]] |= (c & 3) << (2 * j[ei])
        hmask[:, l[ei]] |= ((c >> 2) & 1) << (4 * h[ei] + j[ei])
    scales = np.zeros((n, 12), np.int64)
    for s in range(16):
        lo, hi = sc6[:, s] & 15, sc6[:, s] >> 4
        scales[:, s % 8] |= lo << (0 if s < 8 else 4)
        scales[:, 8 + s % 4] |= hi << (2 * (s // 4))
    out[:, 0:32] = hmask
    out[:, 32:96] = qs
    out[:, 96:108] = scales
    out[:, 108:110] = np.asarray(d, np.float16).view(np.uint8).reshape(n, 2)
    return out


def pack_iq4nl(nib: np.ndarray, d: np.ndarray) -> np.ndarray:
    """nib [n,32] table indices 0..15, d [n] float16 -> [n,18] uint8.
    Element i < 16 sits in the low nibble of qs[i], i >= 16 in the high
    nibble of qs[i - 16]."""
    nib = np.asarray(nib, np.int64)
    n = nib.shape[0]
    out = np.zeros((n, 18), np.uint8)
    out[:, 0:2] = np.asarray(d, np.float16).view(np.uint8).reshape(n, 2)
    out[:, 2:18] = nib[:, :16] | (nib[:, 16:] << 4)
    return out


def pack_q8_1(q: np.ndarray, d: np.ndarray, s: np.ndarray) -> np.ndarray:
    """q [n,32] int8, d/s [n] float16 -> [n,36] uint8."""
    q = np.asarray(q, np.int8)
    n = q.shape[0]
    out = np.zeros((n, 36), np.uint8)
    out[:, 0:2] = np.asarray(d, np.float16).view(np.uint8).reshape(n, 2)
    out[:, 2:4] = np.asarray(s, np.float16).view(np.uint8).reshape(n, 2)
    out[:, 4:36] = q.view(np.uint8)
    return out


def pack_q8_0(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """q [n,32] int8, d [n] float16 -> [n,34] uint8."""
    q = np.asarray(q, np.int8)
    n = q.shape[0]
    out = np.zeros((n, 34), np.uint8)
    out[:, 0:2] = np.asarray(d, np.float16).view(np.uint8).reshape(n, 2)
    out[:, 2:34] = q.view(np.uint8)
    return out
