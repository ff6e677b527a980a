"""Exact rational evaluation of weighted MQA logits, for tiny inputs.

Test infrastructure (see the package header).  Everything is a
fractions.Fraction: codes are decoded from their bit fields here (not through
the codec tables), the fp32 scales and weights are converted exactly, and the
ReLU and head sum are taken without rounding.  The float64 reference must agree
with this to a few ulp; the dots themselves must agree exactly.
"""

from fractions import Fraction

import numpy as np


def _e4m3(code):
    code = int(code) & 0xFF
    sign = -1 if code >> 7 else 1
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        raise ValueError("NaN code in brute-force input")
    if exp == 0:
        return sign * Fraction(man, 2 ** 9)
    return sign * Fraction(8 + man, 8) * Fraction(2) ** (exp - 7)


def _e2m1(nibble):
    nibble = int(nibble) & 0xF
    sign = -1 if nibble >> 3 else 1
    exp = (nibble >> 1) & 0x3
    man = nibble & 0x1
    if exp == 0:
        return sign * Fraction(man, 2)
    return sign * Fraction(2 + man, 2) * Fraction(2) ** (exp - 1)


def _e8m0(code):
    code = int(code)
    if code == 0xFF:
        raise ValueError("NaN scale in brute-force input")
    return Fraction(2) ** (code - 127)


def decode_row(fmt, codes, scales):
    """Exact values of one row of D elements."""
    if fmt == "mxfp4":
        elems = []
        for byte in codes:
            elems.append(_e2m1(int(byte) & 0xF))
            elems.append(_e2m1(int(byte) >> 4))
    else:
        elems = [_e4m3(c) for c in codes]
    if fmt == "fp8":
        return elems
    return [v * _e8m0(scales[d // 32]) for d, v in enumerate(elems)]


def dot(fmt, q_row, q_sf_row, kv_row, kv_sf_row):
    a = decode_row(fmt, q_row, q_sf_row)
    b = decode_row(fmt, kv_row, kv_sf_row)
    return sum((x * y for x, y in zip(a, b)), Fraction(0))


def logit(fmt, q, q_sf, kv, kv_sf, kv_scale, weights, i, j):
    """Exact logits[i, j] (no range check): sum_h w * max(0, s * <q, kv>)."""
    s = Fraction(1) if kv_scale is None else Fraction(float(np.float32(kv_scale[j])))
    total = Fraction(0)
    for h in range(q.shape[1]):
        d = dot(fmt, q[i, h], None if q_sf is None else q_sf[i, h],
                kv[j], None if kv_sf is None else kv_sf[j])
        x = s * d
        total += Fraction(float(np.float32(weights[i, h]))) * (x if x > 0 else Fraction(0))
    return total


def dense_logits(fmt, q, q_sf, kv, kv_sf, kv_scale, weights, k_start, k_end):
    """Exact dense clean logits as a nested list; None marks -inf."""
    sq, skv = q.shape[0], kv.shape[0]
    out = []
    for i in range(sq):
        s = min(max(int(k_start[i]), 0), skv)
        e = min(max(int(k_end[i]), s), skv)
        out.append([logit(fmt, q, q_sf, kv, kv_sf, kv_scale, weights, i, j)
                    if s <= j < e else None for j in range(skv)])
    return out
