"""Pins for the float64 reference (CPU only).

Each test fixes the oracle to something other than itself: a hand-worked
example, the pages' zero-problem check, exact rational brute force, or a
closed-form property of the definition
    logits[i, j] = sum_h w[i,h] * ReLU(kv_scale[j] * <q[i,h,:], kv[j,:]>).
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from synth import dense_case, paged_case, encode_e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# hand-worked examples
# ---------------------------------------------------------------------------

def _hand_fp8_case():
    # e4m3fn codes: 1.0=0x38 2.0=0x40 0.5=0x30 3.0=0x44 -1.0=0xB8 0=0x00
    q = np.array([[[0x38, 0x40, 0x00, 0xB8],     # q[0,0] = [ 1, 2, 0, -1]
                   [0x30, 0x00, 0x44, 0x38]],    # q[0,1] = [.5, 0, 3,  1]
                  [[0xB8, 0xB8, 0x38, 0x00],     # q[1,0] = [-1,-1, 1,  0]
                   [0x40, 0x40, 0x40, 0x40]]],   # q[1,1] = [ 2, 2, 2,  2]
                 dtype=np.uint8)
    kv = np.array([[0x38, 0x38, 0x38, 0x38],     # kv[0] = [1, 1, 1,  1]
                   [0x40, 0x00, 0x30, 0xB8],     # kv[1] = [2, 0,.5, -1]
                   [0x00, 0xB8, 0x44, 0x30]],    # kv[2] = [0,-1, 3, .5]
                  dtype=np.uint8)
    kv_scale = np.array([1.0, 0.5, -2.0], np.float32)
    w = np.array([[1.0, -0.5], [0.25, 2.0]], np.float32)
    return q, kv, kv_scale, w, np.array([0, 1], np.int32), np.array([3, 3], np.int32)


def test_hand_worked_fp8_example():
    # dots <q[i,h], kv[j]>:
    #   row 0: h0 -> [2, 3, -2.5]   h1 -> [4.5, 1.5, 9.5]
    #   row 1: h0 -> [-1, -1.5, 4]  h1 -> [8, 3, 5]
    # row 0, w = [1, -.5]:
    #   j0 (s=1):   1*2   - .5*4.5          = -0.25
    #   j1 (s=.5):  1*1.5 - .5*.75          =  1.125
    #   j2 (s=-2):  1*ReLU(5) - .5*ReLU(-19) = 5      (s*ReLU(x) would give 9.5)
    # row 1, w = [.25, 2], range [1, 3):
    #   j0 -> -inf;  j1: .25*ReLU(-.75) + 2*ReLU(1.5) = 3;  j2: both negative -> 0
    q, kv, s, w, ks, ke = _hand_fp8_case()
    ref, bound = oracle.dense_logits("fp8", q, None, kv, None, s, w, ks, ke)
    assert ref.tolist() == [[-0.25, 1.125, 5.0], [-np.inf, 3.0, 0.0]]
    # bound = 1e-4 * sum_h |w*s*dot| + 1e-6 ; row 0 j2: |1*-2*-2.5| + |-.5*-2*9.5| = 14.5
    assert bound[0, 2] == pytest.approx(1e-4 * 14.5 + 1e-6, rel=1e-12)
    assert bound[1, 0] == 0.0


def test_hand_worked_mxfp4_example():
    # one 32-element block, H = 1.  e2m1 nibbles: 6=7 -.5=9 1.5=3 1=2 2=4 4=6 .5=1 -3=13
    q = np.zeros((1, 1, 16), np.uint8)
    q[0, 0, :2] = [0x97, 0x03]                 # q  = [6, -.5, 1.5, 0, ...]
    kv = np.zeros((2, 16), np.uint8)
    kv[0, :2] = [0x42, 0x06]                   # kv0 = [1, 2, 4, 0, ...]
    kv[1, :2] = [0x11, 0x0D]                   # kv1 = [.5, .5, -3, 0, ...]
    q_sf = np.array([[[128]]], np.uint8)       # x2
    kv_sf = np.array([[126], [129]], np.uint8)  # x.5 and x4
    w = np.array([[0.75]], np.float32)
    # dot0 = 2*.5*(6 - 1 + 6) = 11 ; dot1 = 2*4*(3 - .25 - 4.5) = -14
    ref, _ = oracle.dense_logits("mxfp4", q, q_sf, kv, kv_sf, None, w,
                                 np.array([0]), np.array([2]))
    assert ref.tolist() == [[0.75 * 11, 0.0]]


def test_pages_zero_problem_check():
    spec = json.load(open(os.path.join(GOLDEN, "zero_problem_clean_mask.json")))
    for c in spec["cases"]:
        sq, skv = c["sq"], c["skv"]
        ends = skv - sq + np.arange(sq)
        case = dense_case(sq, skv, c["h"], c["d"], c["fmt"], seed=3, k_end=ends, zero=True)
        ref, _ = oracle.dense_logits(*case.args())
        valid = np.arange(skv)[None, :] < ends[:, None]
        assert np.array_equal(np.isneginf(ref), ~valid)
        assert np.all(ref[valid] == 0.0)


# ---------------------------------------------------------------------------
# brute force (exact rationals) on tiny inputs
# ---------------------------------------------------------------------------

def _ranges(rng, sq, skv):
    ks = rng.integers(-3, skv + 2, sq)
    ke = rng.integers(-2, skv + 4, sq)
    ks[0], ke[0] = 0, skv          # one full row
    if sq > 2:
        ks[1], ke[1] = 5, 2        # one empty row
    return ks.astype(np.int32), ke.astype(np.int32)


@pytest.mark.parametrize("fmt,d", [("fp8", 32), ("fp8", 64), ("mxfp8", 64), ("mxfp4", 64)])
def test_oracle_matches_brute_force(fmt, d):
    rng = np.random.default_rng(11)
    sq, skv, h = 5, 23, 3
    ks, ke = _ranges(rng, sq, skv)
    case = dense_case(sq, skv, h, d, fmt, seed=17, k_start=ks, k_end=ke)
    if fmt == "fp8":
        case.kv_scale[::4] *= -1.0          # negative scales take the literal order
    ref, bound = oracle.dense_logits(*case.args())
    exact = brute.dense_logits(*case.args())
    eps = np.finfo(np.float64).eps
    for i in range(sq):
        for j in range(skv):
            if exact[i][j] is None:
                assert np.isneginf(ref[i, j]) and bound[i, j] == 0.0
                continue
            # scale of the rounding: the exact sum of |w * s * dot| over heads
            s = 1.0 if case.kv_scale is None else float(case.kv_scale[j])
            mag = sum(abs(float(case.weights[i, hh]) * s * float(brute.dot(
                fmt, case.q[i, hh], None if case.q_sf is None else case.q_sf[i, hh],
                case.kv[j], None if case.kv_sf is None else case.kv_sf[j])))
                for hh in range(h))
            assert abs(ref[i, j] - float(exact[i][j])) <= 8 * eps * mag
            assert bound[i, j] == pytest.approx(1e-4 * mag + 1e-6, rel=1e-12)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4"])
def test_dots_are_exact(fmt):
    case = dense_case(3, 7, 2, 64, fmt, seed=23)
    from oracle.codecs import decode
    Q = decode(fmt, case.q, case.q_sf)
    K = decode(fmt, case.kv, case.kv_sf)
    S = Q @ K.T
    for i in range(3):
        for h in range(2):
            for j in range(7):
                exact = brute.dot(fmt, case.q[i, h], None if case.q_sf is None else case.q_sf[i, h],
                                  case.kv[j], None if case.kv_sf is None else case.kv_sf[j])
                assert S[i, h, j] == float(exact) and exact == S[i, h, j]


def test_dense_entries_matches_dense_rows():
    case = dense_case(9, 40, 4, 64, "fp8", seed=5,
                      k_start=np.arange(9), k_end=np.arange(9) + 30)
    ref, bound = oracle.dense_logits(*case.args())
    rng = np.random.default_rng(1)
    rows = rng.integers(0, 9, 50)
    cols = rng.integers(0, 40, 50)
    v, b = oracle.dense_entries(*case.args(), rows, cols)
    assert np.array_equal(v, ref[rows, cols])
    assert np.allclose(b, bound[rows, cols], rtol=1e-14, atol=0)


# ---------------------------------------------------------------------------
# closed forms and invariants of the definition
# ---------------------------------------------------------------------------

def test_single_head_single_dim_closed_form():
    rng = np.random.default_rng(2)
    qv = rng.standard_normal(6)
    kvv = rng.standard_normal(9)
    q = encode_e4m3(qv).reshape(6, 1, 1)
    kv = encode_e4m3(kvv).reshape(9, 1)
    s = rng.uniform(-2, 2, 9).astype(np.float32)
    w = rng.standard_normal((6, 1)).astype(np.float32)
    ref, _ = oracle.dense_logits("fp8", q, None, kv, None, s, w,
                                 np.zeros(6, np.int32), np.full(6, 9, np.int32))
    from oracle.codecs import decode_e4m3
    a = decode_e4m3(q[:, 0, 0])[:, None]
    b = decode_e4m3(kv[:, 0])[None, :]
    expect = w.astype(np.float64) * np.maximum(0.0, s.astype(np.float64)[None, :] * a * b)
    assert np.array_equal(ref, expect)


def test_zero_weights_give_zero():
    case = dense_case(4, 33, 8, 64, "fp8", seed=9)
    case.weights[...] = 0
    ref, _ = oracle.dense_logits(*case.args())
    assert np.all(ref == 0.0)


def test_all_negative_dots_give_zero():
    case = dense_case(4, 33, 8, 64, "fp8", seed=9)
    case.q[...] = case.q | 0x80            # every q element <= 0
    case.kv[...] = case.kv & 0x7F          # every kv element >= 0
    ref, _ = oracle.dense_logits(*case.args())
    assert np.all(ref == 0.0)


def test_kv_scale_power_of_two_scales_output_exactly():
    case = dense_case(4, 33, 8, 64, "fp8", seed=13)
    ref, _ = oracle.dense_logits(*case.args())
    case.kv_scale[...] *= 2.0
    ref2, _ = oracle.dense_logits(*case.args())
    assert np.array_equal(ref2, 2.0 * ref)


def test_negative_kv_scale_takes_relu_after_scaling():
    # ReLU(-s * x) == ReLU(s * (-x)): a negated scale equals negated q codes,
    # exactly.  Scaling after the ReLU instead would give -1 times the output.
    case = dense_case(4, 33, 8, 64, "fp8", seed=13)
    ref, _ = oracle.dense_logits(*case.args())
    case.kv_scale[...] *= -1.0
    neg_scale, _ = oracle.dense_logits(*case.args())
    case.kv_scale[...] *= -1.0
    case.q[...] ^= 0x80
    neg_q, _ = oracle.dense_logits(*case.args())
    assert np.array_equal(neg_scale, neg_q)
    assert not np.allclose(neg_scale, -ref)


def test_head_permutation_with_weights_is_invariant():
    case = dense_case(4, 33, 8, 64, "fp8", seed=21)
    ref, _ = oracle.dense_logits(*case.args())
    perm = np.random.default_rng(3).permutation(8)
    case.q = case.q[:, perm]
    case.weights = case.weights[:, perm]
    ref2, _ = oracle.dense_logits(*case.args())
    assert np.allclose(ref2, ref, rtol=1e-13, atol=1e-13)


def test_linear_in_weights():
    case = dense_case(4, 33, 8, 64, "fp8", seed=21)
    w1 = case.weights.copy()
    r1, _ = oracle.dense_logits(*case.args())
    case.weights = np.random.default_rng(4).standard_normal(w1.shape).astype(np.float32)
    r2, _ = oracle.dense_logits(*case.args())
    case.weights = w1 + case.weights
    # (w1 + w2) is rounded to fp32 before use; compare with a rounding allowance
    r12, _ = oracle.dense_logits(*case.args())
    assert np.allclose(r12, r1 + r2, rtol=1e-6, atol=1e-6)
    case.weights = w1 * 4.0
    r4, _ = oracle.dense_logits(*case.args())
    assert np.array_equal(r4, 4.0 * r1)


def test_out_of_range_entries_are_exactly_neg_inf_and_ranges_clamp():
    skv = 20
    ks = np.array([-5, 0, 7, 19, 25, 3], np.int32)
    ke = np.array([4, 20, 7, 40, 30, 1], np.int32)
    case = dense_case(6, skv, 2, 32, "fp8", seed=1, k_start=ks, k_end=ke)
    ref, bound = oracle.dense_logits(*case.args())
    s, e = oracle.row_ranges(ks, ke, skv)
    assert s.tolist() == [0, 0, 7, 19, 20, 3]
    assert e.tolist() == [4, 20, 7, 20, 20, 3]
    for i in range(6):
        cols = np.arange(skv)
        inside = (cols >= s[i]) & (cols < e[i])
        assert np.all(np.isneginf(ref[i, ~inside]))
        assert np.all(np.isfinite(ref[i, inside]))
        assert np.all(bound[i, inside] >= 1e-6)


# ---------------------------------------------------------------------------
# compressed and paged layouts
# ---------------------------------------------------------------------------

def test_compressed_rows_are_dense_slices():
    sq, skv = 12, 50
    ks = np.array([0, 3, 10, 49, 50, 7, 2, 0, 30, 20, 5, 44], np.int32)
    ke = np.array([50, 40, 10, 50, 50, 3, 9, 1, 45, 50, 6, 48], np.int32)
    case = dense_case(sq, skv, 4, 64, "fp8", seed=8, k_start=ks, k_end=ke)
    packed, pbound, off = oracle.compressed_logits(*case.args())
    ref, bound = oracle.dense_logits(*case.args())
    s, e = oracle.row_ranges(ks, ke, skv)
    assert np.array_equal(np.diff(off), e - s)
    assert off[0] == 0 and off[-1] == packed.size
    for i in range(sq):
        assert np.array_equal(packed[off[i]:off[i + 1]], ref[i, s[i]:e[i]])
        assert np.array_equal(pbound[off[i]:off[i + 1]], bound[i, s[i]:e[i]])
    assert np.all(np.isfinite(packed))


@pytest.mark.parametrize("next_n", [1, 2, 4])
def test_paged_equals_dense_on_gathered_kv(next_n):
    case = paged_case(batch=3, next_n=next_n, h=4, d=64, block_size=16, num_blocks=40,
                      ctx_lo=1, ctx_hi=60, max_context_len=64, seed=31,
                      context_lens=[37, 2, 64])
    ref, bound = oracle.paged_logits(*case.args())
    assert ref.shape == (3 * next_n, 64)
    for b in range(3):
        ctx = int(case.context_lens[b])
        kv, kvs = oracle.gather_paged_kv(case.kv_pool, case.kv_scale_pool,
                                         case.block_table, b, ctx, 16)
        assert np.all(kv != 0x7F)                       # never a poisoned block
        rows = slice(b * next_n, (b + 1) * next_n)
        ends = ctx - next_n + np.arange(next_n) + 1
        d_ref, _ = oracle.dense_logits("fp8", case.q[rows], None, kv, None, kvs,
                                       case.weights[rows], np.zeros(next_n), ends)
        assert np.array_equal(ref[rows, :ctx], d_ref)
        assert np.all(np.isneginf(ref[rows, ctx:]))
        for t in range(next_n):
            e = max(0, ctx - next_n + t + 1)
            assert np.all(np.isfinite(ref[b * next_n + t, :e]))
            assert np.all(np.isneginf(ref[b * next_n + t, e:]))


def test_paged_mx_equals_dense_on_gathered_kv():
    case = paged_case(batch=2, next_n=2, h=2, d=64, block_size=32, num_blocks=9,
                      ctx_lo=1, ctx_hi=60, max_context_len=96, fmt="mxfp4", seed=3,
                      context_lens=[70, 33])
    ref, _ = oracle.paged_logits(*case.args())
    for b in range(2):
        ctx = int(case.context_lens[b])
        kv, _ = oracle.gather_paged_kv(case.kv_pool, None, case.block_table, b, ctx, 32)
        sf, _ = oracle.gather_paged_kv(case.kv_sf_pool, None, case.block_table, b, ctx, 32)
        rows = slice(b * 2, b * 2 + 2)
        d_ref, _ = oracle.dense_logits("mxfp4", case.q[rows], case.q_sf[rows], kv, sf, None,
                                       case.weights[rows], np.zeros(2), ctx - 2 + np.arange(2) + 1)
        assert np.array_equal(ref[rows, :ctx], d_ref)


def test_hand_worked_paged_example():
    """Two sequences through a permuted block table, block_size 4, next_n 2,
    H = 2, D = 2; sequence 1's context (9) exceeds max_context_len (7), so its
    rows see only the first 7 tokens.  Every expected value below was worked
    out by hand from the definition (query token t of sequence b is row
    b*next_n + t and covers keys [0, ctx_b - next_n + t + 1) clamped to
    min(ctx_b, max_context_len); logical token j is slot j % 4 of physical
    block block_table[b, j // 4]).  Physical block 2 is never read and holds
    NaN codes and a NaN scale."""
    nan8 = 0x7F
    kv_vals = {0: [[1, 0], [0, 1], [1, 1], [2, 0]],
               1: [[0, 2], [1, -1], [-1, 1], [2, 2]],
               3: [[1, 2], [2, 1], [-1, 0], [0, -1]],
               4: [[3, 0], [0, 3], [1, -2], [-2, 1]]}
    kv_pool = np.full((5, 4, 2), nan8, np.uint8)
    for blk, v in kv_vals.items():
        kv_pool[blk] = encode_e4m3(np.array(v, np.float32))
    kvs_pool = np.array([[1, 1, 2, 0.5], [1, 2, 1, 1], [np.nan] * 4, [1, 0.5, 1, 2],
                         [2, 1, 1, 0.5]], np.float32)
    block_table = np.array([[3, 0], [4, 1]], np.int32)
    q = encode_e4m3(np.array([[[1, 0], [0, 1]],        # row 0 = (b 0, t 0)
                              [[1, 1], [-1, 1]],       # row 1 = (b 0, t 1)
                              [[1, -1], [2, 0]],       # row 2 = (b 1, t 0)
                              [[0, 1], [1, 1]]],       # row 3 = (b 1, t 1)
                             np.float32))
    w = np.array([[1, 2], [0.5, 1], [1, -1], [2, 0.5]], np.float32)
    ctx = np.array([6, 9], np.int32)

    # the gather alone: sequence 1's 7 visible tokens, in logical order
    kv1, s1 = oracle.gather_paged_kv(kv_pool, kvs_pool, block_table, 1, 7, 4)
    assert np.array_equal(kv1, encode_e4m3(np.array(
        [[3, 0], [0, 3], [1, -2], [-2, 1], [0, 2], [1, -1], [-1, 1]], np.float32)))
    assert np.array_equal(s1, np.array([2, 1, 1, 0.5, 1, 2, 1], np.float32))
    # the row ranges, with the clamp at max_context_len
    _, e = oracle.paged_row_ranges(ctx, 2, 7)
    assert e.tolist() == [5, 6, 7, 7]

    ninf = -np.inf
    expected = np.array([[5, 2, 0, 0, 1, ninf, ninf],
                         [2.5, 0.75, 1, 0, 0.5, 1.5, ninf],
                         [-6, 0, 1, 0, 0, 0, 0],
                         [3, 7.5, 0, 1, 5, 0, 2]])
    ref, bound = oracle.paged_logits("fp8", q, None, kv_pool, None, kvs_pool, w, ctx,
                                     block_table, 2, 4, 7)
    assert np.array_equal(ref, expected)
    assert np.all(bound[np.isneginf(expected)] == 0)
