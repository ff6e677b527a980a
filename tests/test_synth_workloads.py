"""The workload generators' variants (host only): the prefill shape in the MX
formats and the all-zero inputs the source pages time their kernels on."""

import numpy as np
import pytest

import synth


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_prefill_shape_in_mx_formats(fmt):
    case = synth.workload_case(1, fmt)
    assert (case.sq, case.skv, case.h, case.d, case.fmt) == (2048, 32768, 64, 128, fmt)
    assert case.name.endswith("_" + fmt)
    assert case.kv_scale is None and case.q_sf is not None and case.kv_sf is not None
    assert case.q.shape[-1] == (128 if fmt == "mxfp8" else 64)
    # the rows are the prefill workload's: [0, Skv - Sq + i)
    assert np.array_equal(case.k_end, 32768 - 2048 + np.arange(2048))


def test_default_workloads_keep_their_names():
    assert synth.workload_case(1).name == synth.WORKLOAD_NAMES[1]
    assert synth.workload_case(0).name == synth.WORKLOAD_NAMES[0]


@pytest.mark.parametrize("idx,fmt", [(0, None), (1, None), (1, "mxfp4"), (2, None)])
def test_all_zero_variant(idx, fmt):
    case = synth.workload_case(idx, fmt, zero=True)
    assert not case.q.any() and not case.kv.any() and not case.weights.any()
    if case.q_sf is not None:
        assert (case.q_sf == 127).all() and (case.kv_sf == 127).all()   # unit e8m0 scales
    ref = synth.workload_case(idx, fmt)
    assert np.array_equal(case.k_start, ref.k_start) and np.array_equal(case.k_end, ref.k_end)


def test_paged_has_no_all_zero_variant():
    with pytest.raises(ValueError):
        synth.workload_case(3, zero=True)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_paged_decode_shape_in_mx_formats(fmt):
    case = synth.workload_case(3, fmt)
    ref = synth.workload_case(3)
    assert case.fmt == fmt and case.name.endswith("_" + fmt)
    assert case.kv_scale_pool is None and case.kv_sf_pool is not None
    # the same sequences and block table as the paged decode workload
    assert np.array_equal(case.context_lens, ref.context_lens)
    assert np.array_equal(case.block_table, ref.block_table)


@pytest.mark.parametrize("fmt,d", [("fp8", 128), ("mxfp8", 64)])
def test_cancelling_case_properties(fmt, d):
    """The cancelling inputs hold what their description promises: the pair
    products cancel exactly in every group of 8, and every product is a
    multiple of 2^-9 with sum |products| < 2^14 (partial sums exact in fp32)."""
    from oracle.codecs import decode
    import synth
    case = synth.cancelling_dense_case(6, 50, 32, d, fmt, seed=5)
    Q = decode(fmt, case.q, case.q_sf)                 # [6, 32, d]
    K = decode(fmt, case.kv, case.kv_sf)               # [50, d]
    P = Q[:, :, None, :] * K[None, None, :, :]
    assert np.all(np.mod(P * 512.0, 1.0) == 0)
    assert np.abs(P).sum(-1).max() < 2.0 ** 14
    pairs = synth.cancel_pairs(5, d)
    g = np.arange(d // 8) * 8
    assert np.all(P[..., g + pairs[:, 0]] + P[..., g + pairs[:, 1]] == 0)
    assert np.all(np.abs(Q[..., g + pairs[:, 0]]) >= 64)
