"""The bf16 weight encoder of the input generators (host only).

bf16 weights are an input format: both sides take the values of the encoded
bits.  The encoder must be nearest-even rounding of fp32 -- checked against
torch's own fp32 -> bfloat16 conversion and on hand-made ties."""

import numpy as np
import torch

import synth


def test_encode_bf16_matches_torch_rounding():
    x = (np.random.default_rng(3).standard_normal(200000) * 7).astype(np.float32)
    x[:4] = [0.0, -0.0, 1e-40, -3.0e38]
    got = synth.encode_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_encode_bf16_ties_to_even_and_exact_decode():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: ties go to the even 1.0;
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6: goes up.
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1.5, -2.0 ** -130], np.float32)
    dec = synth.decode_bf16(synth.encode_bf16(x))
    assert dec.tolist() == [1.0, 1 + 2.0 ** -6, 1.5, -2.0 ** -130]
