"""Exact decoders for the element and scale formats of the MQA-logits inputs.

Test infrastructure (see the package header).  Each table is built from the
bit-field definition of its format, never from a library conversion; the
tests pin the tables against library dtypes and against the OCP MX value list.

Formats, as the pages name them:
  * FP8 e4m3 for Q and KV ([P1] "Implementing Standard MQA Logits
    Computation": q and kv are float8_e4m3fn tensors; [P4] reproducer builds
    them as torch.float8_e4m3fn).  This is the OCP "fn" variant: bias 7, no
    infinities, codes 0x7F/0xFF are NaN, largest finite 448.
  * MXFP8 / MXFP4 ([P4] Description and Performance table): e4m3 or e2m1
    elements with one e8m0 power-of-two scale per 32 consecutive elements.
    The reproducer packs four e8m0 scale bytes into one int32 for D = 128 and
    stores two e2m1 elements per byte for FP4.
"""

import numpy as np


def e4m3fn_value(code: int) -> float:
    """Value of one OCP e4m3fn byte: 1 sign, 4 exponent (bias 7), 3 mantissa bits."""
    code &= 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        # subnormal: 0.mmm * 2^(1 - 7)
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e2m1_value(code: int) -> float:
    """Value of one OCP e2m1 nibble: 1 sign, 2 exponent (bias 1), 1 mantissa bit."""
    code &= 0xF
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        # subnormal: 0.m * 2^(1 - 1)
        return sign * man * 0.5
    return sign * (1.0 + man / 2.0) * 2.0 ** (exp - 1)


def e8m0_value(code: int) -> float:
    """Value of one e8m0 scale byte: 2^(code - 127); 0xFF is NaN."""
    code &= 0xFF
    if code == 0xFF:
        return float("nan")
    return 2.0 ** (code - 127)


E4M3_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)

MX_BLOCK = 32


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """float64 values of an array of e4m3fn codes (uint8), same shape."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    """Unpack [..., n] bytes into [..., 2n] e2m1 nibbles.

    Element 2k sits in the low nibble of byte k and element 2k+1 in the high
    nibble (the OCP MX packing order for FP4).
    """
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & 0x0F
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)


def decode_e2m1_packed(packed: np.ndarray) -> np.ndarray:
    """float64 values of packed e2m1 bytes [..., n] -> [..., 2n]."""
    return E2M1_TABLE[unpack_e2m1(packed)]


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    return E8M0_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode(fmt: str, codes: np.ndarray, scales: np.ndarray = None) -> np.ndarray:
    """Decode Q or KV codes to exact float64 values along the last axis (D).

    fmt "fp8":   codes [..., D] e4m3fn, no block scale.
    fmt "mxfp8": codes [..., D] e4m3fn, scales [..., D/32] e8m0.
    fmt "mxfp4": codes [..., D/2] packed e2m1, scales [..., D/32] e8m0.
    The block scale of element d is scales[..., d // 32].
    """
    if fmt == "fp8":
        return decode_e4m3(codes)
    if fmt == "mxfp8":
        vals = decode_e4m3(codes)
    elif fmt == "mxfp4":
        vals = decode_e2m1_packed(codes)
    else:
        raise ValueError(f"unknown format {fmt!r}")
    d = vals.shape[-1]
    scales = np.asarray(scales, dtype=np.uint8)
    if scales.shape[-1] * MX_BLOCK != d:
        raise ValueError(f"{scales.shape[-1]} scales cannot cover D={d} in blocks of {MX_BLOCK}")
    return vals * np.repeat(decode_e8m0(scales), MX_BLOCK, axis=-1)
