"""Pins for the oracle's decode tables (CPU only).

The e4m3fn and e8m0 tables are compared with torch's own dtypes over every
code; the e2m1 table with the value list of the OCP Microscaling Formats v1.0
specification (torch has no e2m1 conversion).  The block-scale indexing of the
MX decode is pinned by scaling one block at a time.
"""

import math

import numpy as np
import pytest
import torch

from oracle import codecs
from synth import encode_e2m1, encode_e4m3, pack_e2m1


def test_e4m3fn_table_matches_torch_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = codecs.E4M3_TABLE
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # sign of zero too
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x44, 3.0), (0x7E, 448.0),
    (0xB8, -1.0), (0xFE, -448.0),
])
def test_e4m3fn_spec_values(code, value):
    assert codecs.e4m3fn_value(code) == value


def test_e4m3fn_nan_codes_only():
    nan_codes = [c for c in range(256) if math.isnan(codecs.e4m3fn_value(c))]
    assert nan_codes == [0x7F, 0xFF]


def test_e8m0_table_matches_torch_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    ours = codecs.E8M0_TABLE
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert codecs.e8m0_value(127) == 1.0 and codecs.e8m0_value(0) == 2.0 ** -127


def test_e2m1_table_matches_ocp_value_list():
    # OCP MX v1.0, FP4 E2M1: magnitudes by code 0..7; bit 3 is the sign.
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(codecs.E2M1_TABLE[:8]) == mags
    assert list(codecs.E2M1_TABLE[8:]) == [-m for m in mags]
    assert np.signbit(codecs.E2M1_TABLE[8])


def test_e2m1_unpack_order_low_nibble_first():
    packed = np.array([[0x97, 0x03]], dtype=np.uint8)
    assert codecs.unpack_e2m1(packed).tolist() == [[7, 9, 3, 0]]
    assert codecs.decode_e2m1_packed(packed).tolist() == [[6.0, -0.5, 1.5, 0.0]]


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_block_scale_applies_to_its_32_elements(fmt):
    d = 128
    rng = np.random.default_rng(5)
    if fmt == "mxfp8":
        codes = encode_e4m3(rng.standard_normal((3, d)))
    else:
        codes = pack_e2m1(encode_e2m1(rng.standard_normal((3, d)) * 2))
    base = codecs.decode(fmt, codes, np.full((3, d // 32), 127, np.uint8))
    for blk in range(d // 32):
        sf = np.full((3, d // 32), 127, np.uint8)
        sf[:, blk] = 127 + 3                         # x 8 for block blk only
        got = codecs.decode(fmt, codes, sf)
        expect = base.copy()
        expect[:, blk * 32:(blk + 1) * 32] *= 8.0
        assert np.array_equal(got, expect)


def test_mx_decode_rejects_mismatched_scale_count():
    with pytest.raises(ValueError):
        codecs.decode("mxfp8", np.zeros((2, 64), np.uint8), np.zeros((2, 3), np.uint8))


# ---- input encoders (generator side; they feed both oracle and GPU) --------

def test_encode_e2m1_rounds_to_nearest_even_and_saturates():
    x = np.array([0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.3, -6.0])
    got = codecs.E2M1_TABLE[encode_e2m1(x)]
    assert got.tolist() == [0.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, -0.5, -6.0]


def test_encode_e4m3_clips_and_round_trips():
    x = np.array([1.0, -448.0, 1000.0, -1e6, 2.0 ** -9, 2.0 ** -10, 1.0625, 1.1875])
    got = codecs.decode_e4m3(encode_e4m3(x))
    # 1.0625 is a tie between 1.0 and 1.125 -> even mantissa 1.0;
    # 1.1875 is a tie between 1.125 and 1.25 -> even mantissa 1.25.
    assert got.tolist() == [1.0, -448.0, 448.0, -448.0, 2.0 ** -9, 0.0, 1.0, 1.25]
