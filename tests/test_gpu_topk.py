"""GPU parity of the top-k selection over logits rows (mqa_logits_topk).

On synthetic logits (ties, signed zeros, -inf holes, ranges that are full,
empty, short or past the end) the device indices must equal the oracle's bit
for bit.  After the logits kernel, the selection is checked for validity
against the oracle's float64 logits within their error bound (the device
logits are not an oracle input)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import dense_on_device, dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mqa_logits_amd  # noqa: F401


@pytest.mark.parametrize("sq,skv,topk,ranges,seed", [
    (40, 1000, 64, True, 1),
    (24, 32773, 2048, True, 2),
    (16, 5000, 1, True, 3),
    (33, 3000, 4096, False, 4),             # more than most rows hold
    (8, 65536, 2048, False, 5),
    (3, 1, 7, True, 6),
    (20, 10000, 700, True, 7),              # the register kernel at each row capacity
    (20, 20000, 2048, True, 8),
    (6, 70001, 2048, True, 9),              # longer rows: the streaming kernel
    (10, 20000, 5000, True, 10),            # topk past the LDS stage: the streaming kernel
    (520, 20000, 2048, True, 12),           # more rows than two per compute unit
    (5, 40000, 1001, True, 13),             # an odd topk
    (7, 24577, 4096, True, 14),             # a large topk over long rows
])
def test_topk_matches_oracle(sq, skv, topk, ranges, seed):
    import mqa_logits_amd as mq
    x, ks, ke = synth.topk_logits(sq, skv, seed, ranges=ranges)
    log(f"[topk] fp32 Sq={sq} Skv={skv} topk={topk} ranges={ranges}")
    got = mq.mqa_logits_topk(dev(x), topk, dev(ks), dev(ke))
    torch.cuda.synchronize()
    want = oracle.topk_indices(x, topk, ks, ke)
    assert np.array_equal(got.cpu().numpy(), want)


def test_topk_bf16_logits_and_guard_columns():
    import mqa_logits_amd as mq
    sq, skv, topk = 20, 7001, 300
    x, ks, ke = synth.topk_logits(sq, skv, 11, ties=False)
    bits = synth.encode_bf16(x)
    xb = synth.decode_bf16(bits).reshape(x.shape)
    buf = torch.full((sq, topk + 5), 12345, dtype=torch.int32, device="cuda")
    log("[topk] bf16 logits, wide indices rows")
    mq.mqa_logits_topk(dev(bits.view(np.int16)).view(torch.bfloat16), topk, dev(ks), dev(ke),
                       out=buf[:, :topk])
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:, topk:] == 12345)
    assert np.array_equal(b[:, :topk], oracle.topk_indices(xb, topk, ks, ke))


def test_topk_all_equal_and_all_neg_inf_rows():
    import mqa_logits_amd as mq
    x = np.zeros((3, 40000), np.float32)
    x[1] = 1.5
    x[2] = -np.inf
    log("[topk] all-equal rows")
    got = mq.mqa_logits_topk(dev(x), 2048).cpu().numpy()
    assert np.array_equal(got, oracle.topk_indices(x, 2048))
    assert got[0].tolist() == list(range(2048)) and np.all(got[2] == -1)


@pytest.mark.parametrize("skv", [1000, 10000, 30000, 60000, 70000])
@pytest.mark.parametrize("bf16", [False, True])
def test_topk_many_keys_equal_to_the_cut(skv, bf16):
    # values on a coarse grid: many keys equal the k-th largest, and equal keys
    # keep appearing in columns after the ones taken (every kernel size)
    import mqa_logits_amd as mq
    rng = np.random.default_rng(skv + bf16)
    x = (np.round(rng.standard_normal((4, skv)) * 2) / 2).astype(np.float32)
    t = dev(x)
    if bf16:
        t = dev(synth.encode_bf16(x).view(np.int16)).view(torch.bfloat16)   # exact: few bits
    log(f"[topk] ties at the cut skv={skv} bf16={bf16}")
    got = mq.mqa_logits_topk(t, 1500).cpu().numpy()
    assert np.array_equal(got, oracle.topk_indices(x, 1500))


def test_topk_streaming_kernel_edge_rows():
    # rows longer than the register kernel holds: an all-equal row (its top bin
    # is too large for the LDS lists, so every level is a pass over the row),
    # a row with fewer candidates than topk, and a random row
    import mqa_logits_amd as mq
    skv = 70000
    x = np.full((3, skv), -np.inf, np.float32)
    x[0] = 0.75
    x[1, ::50] = np.arange(skv // 50, dtype=np.float32)
    x[2] = np.random.default_rng(5).standard_normal(skv).astype(np.float32)
    log("[topk] streaming kernel edge rows")
    got = mq.mqa_logits_topk(dev(x), 3000).cpu().numpy()
    assert np.array_equal(got, oracle.topk_indices(x, 3000))


def test_topk_after_dense_logits_is_a_valid_selection():
    import mqa_logits_amd as mq
    sq, skv, topk = 48, 4096, 512
    ks = np.zeros(sq, np.int64)
    ke = skv - sq + np.arange(sq) + 1 - 3000 * (np.arange(sq) % 5 == 0)   # some short rows
    case = synth.dense_case(sq, skv, 64, 128, "fp8", seed=77, k_start=ks, k_end=ke)
    d = dense_on_device(case)
    log("[topk] after mqa_logits")
    logits = mq.mqa_logits(d["fmt"], d["q"], d["q_sf"], d["kv"], d["kv_sf"], d["kv_scale"],
                           d["weights"], d["k_start"], d["k_end"])
    idx = mq.mqa_logits_topk(logits, topk, d["k_start"], d["k_end"]).cpu().numpy()
    ref, bound = oracle.dense_logits(*case.args())
    s, e = oracle.row_ranges(case.k_start, case.k_end, skv)
    for i in range(sq):
        n = int(e[i] - s[i])
        row = idx[i]
        sel = row[row >= 0]
        assert sel.size == min(topk, n) and np.all(row[sel.size:] == -1)
        assert np.all(np.diff(sel) > 0) and (sel.size == 0 or (sel[0] >= s[i] and sel[-1] < e[i]))
        if n > topk:
            rest = np.setdiff1d(np.arange(s[i], e[i]), sel)
            # every selected true value is at least every unselected one, up to both bounds
            lo = (ref[i, sel] + bound[i, sel]).min()
            hi = (ref[i, rest] - bound[i, rest]).max()
            assert hi <= lo, f"row {i}: unselected {hi} above selected {lo}"


@pytest.mark.parametrize("skv", [7, 4095, 8191, 16383, 32767, 65535, 70001])
def test_topk_bf16_last_column_of_an_odd_row(skv):
    # bf16 rows of odd length whose last column holds the row's largest value:
    # the register kernels read four columns per 8-byte load, and the last
    # column shares its 4-byte half with the first column past the row
    import mqa_logits_amd as mq
    rng = np.random.default_rng(skv)
    x = rng.standard_normal((3, skv)).astype(np.float32)
    x[:, -1] = 8.0
    x[1, -1] = -8.0                         # and once the smallest
    bits = synth.encode_bf16(x)
    xb = synth.decode_bf16(bits).reshape(x.shape)
    t = dev(bits.view(np.int16)).view(torch.bfloat16)
    log(f"[topk] bf16 odd row Skv={skv}")
    for k in (1, min(skv, 5)):
        got = mq.mqa_logits_topk(t, k).cpu().numpy()
        assert np.array_equal(got, oracle.topk_indices(xb, k)), f"k={k}"


def _prefilter_rows(skv, rng):
    """Rows that lead the register kernel's sampled-threshold prefilter into
    each of its outcomes: taken (plain noise), a wave's list segment
    overflowing (the largest keys all in the columns one wave holds), the
    whole list overflowing (the largest keys only in columns the sample does
    not read), too few keys at or above the threshold (mostly -inf rows), a
    threshold among negative values (topk near half the row), one huge
    outlier (the radix window spans every key bit), and every key equal."""
    cols = np.arange(skv)
    noise = rng.standard_normal((8, skv))
    x = noise.copy()
    x[1, (cols % 4096) < 256] += 50.0              # thread 0..63's columns: wave 0's
    x[2, (cols % 4) == 1] += 50.0                  # the sample reads columns 4t only
    x[3, rng.random(skv) < 0.9] = -np.inf
    x[4] = -np.abs(noise[4]) - 1.0                 # all negative
    x[5, skv // 3] = 3.0e38
    x[6] = 0.75
    x[7] = np.round(noise[7] * 4) / 4              # coarse grid: wide ties at the cut
    return x.astype(np.float32)


@pytest.mark.parametrize("skv", [6000, 12000, 32768, 65536, 100000, 131072])
@pytest.mark.parametrize("topk", [1, 2048, 2560, 2561, 4096])
def test_topk_prefilter_outcomes(skv, topk):
    # every outcome must give the oracle's selection bit for bit, whichever
    # path the kernel took (topk 2560 is the largest the 32-key kernels
    # prefilter, 3072 and 2048 those of rows in two and four parts)
    import mqa_logits_amd as mq
    rng = np.random.default_rng(skv + topk)
    x = _prefilter_rows(skv, rng)
    log(f"[topk] prefilter outcomes Skv={skv} topk={topk}")
    for bf16 in (False, True):
        xs = x
        t = dev(x)
        if bf16:
            bits = synth.encode_bf16(x)
            xs = synth.decode_bf16(bits).reshape(x.shape)
            t = dev(bits.view(np.int16)).view(torch.bfloat16)
        got = mq.mqa_logits_topk(t, topk).cpu().numpy()
        want = oracle.topk_indices(xs, topk, None, None)
        for r in range(x.shape[0]):
            assert np.array_equal(got[r], want[r]), f"row {r} bf16={bf16}"


@pytest.mark.parametrize("skv", [100, 3000, 70000])
def test_topk_takes_every_candidate_including_nan_bit_patterns(skv):
    # rows with at most topk candidates take all of them: every column that
    # is not -inf, NaN bit patterns included (the order is IEEE 754 total
    # order of the bit patterns, where a NaN is not -inf), ascending, then -1
    import mqa_logits_amd as mq
    rng = np.random.default_rng(skv)
    bits = rng.standard_normal((4, skv)).astype(np.float32).view(np.uint32)
    nan_patterns = np.array([0x7FC00000, 0xFFC00000, 0xFFFFFFFF, 0x7FFFFFFF, 0xFF800001],
                            np.uint32)
    for r in range(4):
        cols = rng.choice(skv, size=min(skv, 5), replace=False)
        bits[r, cols] = nan_patterns[:cols.size]
    bits[:, rng.random(skv) < 0.3] = np.float32(-np.inf).view(np.uint32)
    topk = skv                                      # every row takes all its candidates
    log(f"[topk] take-all with NaN bit patterns Skv={skv}")
    got = mq.mqa_logits_topk(dev(bits.view(np.float32)), topk).cpu().numpy()
    neg_inf = np.float32(-np.inf).view(np.uint32)
    for r in range(4):
        want = np.nonzero(bits[r] != neg_inf)[0]
        assert np.array_equal(got[r, :want.size], want), f"row {r}"
        assert np.all(got[r, want.size:] == -1), f"row {r} padding"


def _values(rng, kind, shape):
    """Ten value distributions for the top-k: normal, exponential, integers
    (heavy ties), lognormal (wide range), normal with +-1e30 outliers, a
    narrow all-negative band, a coarse grid, four distinct values with both
    zeros, tiny (subnormal-scale) values, and two far-apart clusters."""
    if kind == 0:
        return rng.standard_normal(shape)
    if kind == 1:
        return rng.exponential(1.0, shape)
    if kind == 2:
        return rng.integers(-5, 6, shape).astype(np.float64)
    if kind == 3:
        return rng.lognormal(0.0, 2.0, shape)
    if kind == 4:
        x = rng.standard_normal(shape)
        x[rng.random(shape) < 0.001] = 1e30
        x[rng.random(shape) < 0.001] = -1e30
        return x
    if kind == 5:
        return -np.abs(rng.standard_normal(shape)) * 1e-3 - 7.0
    if kind == 6:
        return np.round(rng.standard_normal(shape) * 2) / 2
    if kind == 7:
        return rng.choice([0.0, -0.0, 1.0, 2.0], size=shape)
    if kind == 8:
        return rng.standard_normal(shape) * 1e-30
    return np.where(rng.random(shape) < 0.5, rng.standard_normal(shape) + 100,
                    rng.standard_normal(shape) - 100)


@pytest.mark.parametrize("kind", range(10))
def test_topk_value_distributions(kind):
    # the selection's thresholds and radix windows depend on the values'
    # spread, ties and signs; each distribution runs six seeded cases with
    # drawn row lengths (every kernel size), topk (around the prefilter's
    # limits), -inf holes, ranges and logits types
    import mqa_logits_amd as mq
    for case in range(6):
        rng = np.random.default_rng([kind, case, 77])
        sq = int(rng.integers(1, 9))
        skv = int(rng.choice([int(rng.integers(1, 9000)), int(rng.integers(9000, 33000)),
                              int(rng.integers(33000, 65537)), int(rng.integers(65537, 80000))]))
        topk = int(rng.choice([1, int(rng.integers(1, 2600)), 2048, 2560, 2561, 4096]))
        x = _values(rng, kind, (sq, skv))
        x[rng.random((sq, skv)) < rng.choice([0.0, 0.05, 0.5, 0.95])] = -np.inf
        x = x.astype(np.float32)
        ks = ke = None
        if rng.random() < 0.5:
            ks = rng.integers(-10, skv, sq).astype(np.int32)
            ke = (ks + rng.integers(-5, skv + 10, sq)).astype(np.int32)
        t = dev(x)
        bf16 = bool(rng.random() < 0.3)
        if bf16:
            bits = synth.encode_bf16(x)
            x = synth.decode_bf16(bits).reshape(x.shape)
            t = dev(bits.view(np.int16)).view(torch.bfloat16)
        what = f"kind {kind} case {case} Sq={sq} Skv={skv} topk={topk} bf16={bf16}"
        log(f"[topk] {what}")
        got = mq.mqa_logits_topk(t, topk, dev(ks), dev(ke)).cpu().numpy()
        assert np.array_equal(got, oracle.topk_indices(x, topk, ks, ke)), what


@pytest.mark.parametrize("skv", [3000, 12000, 40000])
def test_topk_range_ends_bound_the_reads(skv):
    # the row's buffer ends with its range: a huge value just past the end is
    # never a candidate, and the last column in range (odd or even end, bf16
    # and fp32) is read and taken
    import mqa_logits_amd as mq
    rng = np.random.default_rng(skv + 1)
    sq = 12
    x = rng.standard_normal((sq, skv)).astype(np.float32)
    ks = rng.integers(0, skv // 3, sq).astype(np.int32)
    ke = (ks + rng.integers(skv // 4, skv - skv // 3, sq)).astype(np.int32)
    ke[::2] |= 1                                   # odd ends on even rows
    ke[1::2] &= ~1                                 # even ends on odd rows
    ke = np.minimum(ke, skv - 1).astype(np.int32)
    for r in range(sq):
        x[r, ke[r]] = 1.0e30                       # just past the range
        x[r, ke[r] - 1] = 5.0e29                   # the range's last column
    log(f"[topk] range ends bound the reads Skv={skv}")
    for bf16 in (False, True):
        xs, t = x, dev(x)
        if bf16:
            bits = synth.encode_bf16(x)
            xs = synth.decode_bf16(bits).reshape(x.shape)
            t = dev(bits.view(np.int16)).view(torch.bfloat16)
        got = mq.mqa_logits_topk(t, 2048, dev(ks), dev(ke)).cpu().numpy()
        want = oracle.topk_indices(xs, 2048, ks, ke)
        assert np.array_equal(got, want), f"bf16={bf16}"
        for r in range(sq):
            assert ke[r] - 1 in got[r] and ke[r] not in got[r], f"row {r} bf16={bf16}"


@pytest.mark.parametrize("skv", [5000, 40000, 100000, 140000])
def test_topk_indices_into_a_wider_buffer(skv):
    # the indices' row stride is passed apart: rows of topk inside a wider
    # int32 buffer, whose guard columns every kernel (register, two and four
    # parts, streaming) leaves alone
    import mqa_logits_amd as mq
    sq, topk, width = 6, 2048, 2048 + 37
    x, ks, ke = synth.topk_logits(sq, skv, skv + 3, ties=True, ranges=True)
    buf = torch.full((sq, width), -777, dtype=torch.int32, device="cuda")
    log(f"[topk] indices into a wider buffer Skv={skv}")
    mq.mqa_logits_topk(dev(x), topk, dev(ks), dev(ke), out=buf[:, :topk])
    got = buf.cpu().numpy()
    assert np.all(got[:, topk:] == -777), "guard columns written"
    assert np.array_equal(got[:, :topk], oracle.topk_indices(x, topk, ks, ke))
