"""Independent brute-force checkers used to pin the oracle.

Everything here is written from the mathematical definitions, without looking
at how the oracle computes the same thing: a code is the argmin over every
code's value, attention is a double loop in pure Python.  Only small inputs.
"""
from __future__ import annotations

import math

import numpy as np


def all_finite_bf16() -> np.ndarray:
    """Every finite bf16 bit pattern (uint16), as float32 values and bits."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(f)
    return bits[keep], f[keep]


def int_codes_argmin(y: np.ndarray, qmax: int) -> np.ndarray:
    """Nearest integer in [-qmax, qmax] to each y; exact ties go to the even one."""
    cands = np.arange(-qmax, qmax + 1, dtype=np.float64)
    # values beyond the grid (including +-inf) are nearest to its ends either way
    yd = np.clip(y.astype(np.float64), -qmax - 1.0, qmax + 1.0)[:, None]
    dist = np.abs(yd - cands[None, :])
    best = dist.min(axis=1, keepdims=True)
    tie = dist == best
    # among tied candidates prefer the even integer
    even = (np.abs(cands) % 2 == 0)[None, :]
    pick = np.where(tie & even, 1, 0) * 2 + np.where(tie, 1, 0)
    idx = pick.argmax(axis=1)
    return cands[idx].astype(np.int64)


def fp8_value_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes from the format definition (NaN for S.1111.111)."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * m * 2.0 ** -9
        else:
            vals[c] = s * (1 + m / 8) * 2.0 ** (e - 7)
    return vals


def fp8_codes_argmin(y: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3FN code to each y: magnitudes at or above 448 saturate to 448,
    exact ties go to the code with an even mantissa, and the sign of y is kept (a negative
    y nearest to zero gives 0x80)."""
    table = fp8_value_table()
    mags = table[:0x7F]  # codes 0x00..0x7E, non-negative
    a = np.abs(y.astype(np.float64))
    a = np.minimum(a, 448.0)
    dist = np.abs(a[:, None] - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    tie = dist == best
    even = ((np.arange(0x7F) & 1) == 0)[None, :]
    pick = np.where(tie & even, 1, 0) * 2 + np.where(tie, 1, 0)
    code = pick.argmax(axis=1).astype(np.int64)
    sign = np.signbit(y).astype(np.int64)
    return code | (sign << 7)


def attention_loops(q, K, V, lens, scale, sink=None, softcap=0.0, window=0):
    """Pure-Python softmax attention.  q [B, Tq, Hq, D] floats, K, V [B, Hkv, L, D].
    softcap > 0: each scaled logit z becomes softcap * tanh(z / softcap).
    window > 0: the query at position pos attends tokens pos - window + 1 .. pos."""
    B, Tq, Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Tq, Hq, D))
    for b in range(B):
        for j in range(Tq):
            for h in range(Hq):
                hk = h // G
                pos = int(lens[b]) - Tq + j
                seen = [t for t in range(int(lens[b]))
                        if t <= pos and (window == 0 or t > pos - window)]
                if not seen:
                    continue
                zs = []
                for t in seen:
                    z = 0.0
                    for d in range(D):
                        z += float(q[b, j, h, d]) * float(K[b, hk, t, d])
                    z *= scale
                    if softcap > 0:
                        z = softcap * math.tanh(z / softcap)
                    zs.append(z)
                m = max(zs)
                ws = [math.exp(z - m) for z in zs]
                l = sum(ws)
                for d in range(D):
                    acc = 0.0
                    for i, t in enumerate(seen):
                        acc += ws[i] * float(V[b, hk, t, d])
                    out[b, j, h, d] = acc / l
                if sink is not None:
                    lse = m + math.log(l)
                    out[b, j, h, :] *= 1.0 / (1.0 + math.exp(float(sink[h]) - lse))
    return out
