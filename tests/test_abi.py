"""The C-ABI library on a host without a GPU (CPU only).

Checks that libmqa_logits.so loads, exports every function include/mqa_logits.h
declares, rejects bad arguments on the host before any HIP call, and reports
a missing device as MQA_ERR_HIP.  No test here reaches a kernel launch: every
call with fake pointers is built to fail validation first.
"""

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mqa_logits.h")

mq = pytest.importorskip("mqa_logits_amd")
lib = mq.lib

OK, INVALID, UNSUPPORTED, HIP = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x100000)          # aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x100004)      # 4- but not 16-byte aligned
FAKE_2 = ctypes.c_void_p(0x100002)        # 2- but not 4-byte aligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"defined", "if", "extern"})


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ["mqa_logits", "mqa_logits_compressed", "mqa_logits_compressed_offsets",
               "paged_mqa_logits", "paged_mqa_logits_metadata",
               "paged_mqa_logits_metadata_size", "mqa_num_cus", "mqa_last_error",
               "paged_mqa_logits_default_splits"]:
        assert fn in names


def test_every_declared_symbol_is_exported():
    raw = ctypes.CDLL(mq.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} is declared but not exported"
    assert set(mq.EXPORTED) <= set(declared_functions())


def dense_args(**kw):
    a = dict(dt=0, q=FAKE, q_sf=None, kv=FAKE, kv_sf=None, kv_scale=FAKE, w=FAKE,
             ks=FAKE, ke=FAKE, out=FAKE, stride=64, sq=16, skv=64, h=64, d=128, clean=1,
             w_type=0, out_type=0, sched=None, splits=0, precision=0, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("change,expect", [
    (dict(precision=2), INVALID),
    (dict(precision=-1), INVALID),
    (dict(h=48), UNSUPPORTED),
    (dict(h=128), UNSUPPORTED),
    (dict(d=96), UNSUPPORTED),
    (dict(dt=7), INVALID),
    (dict(q=None), INVALID),
    (dict(kv=None), INVALID),
    (dict(w=None), INVALID),
    (dict(out=None), INVALID),
    (dict(ks=None), INVALID),
    (dict(q=FAKE_ODD), INVALID),
    (dict(kv_scale=None), INVALID),                 # FP8 needs a token scale
    (dict(q_sf=FAKE), INVALID),                     # FP8 takes no block scales
    (dict(dt=1), INVALID),                          # MX needs block scales ...
    (dict(dt=1, q_sf=FAKE, kv_sf=FAKE), INVALID),   # ... and takes no kv_scale
    (dict(stride=63), INVALID),
    (dict(sq=-1), INVALID),
    (dict(skv=-5), INVALID),
    (dict(stride=1 << 28), UNSUPPORTED),
    (dict(w_type=2), INVALID),
    (dict(out_type=-1), INVALID),
    (dict(out_type=1, stride=65), INVALID),         # bf16 logits need an even stride
    (dict(sched=FAKE, splits=0), INVALID),
    (dict(sched=FAKE, splits=70000), INVALID),
    (dict(sched=FAKE_2, splits=8), INVALID),
    (dict(sched=FAKE, splits=8, sq=40000, ks=FAKE, ke=FAKE), UNSUPPORTED),   # > 32768 rows
])
def test_dense_validation_fails_before_any_launch(change, expect):
    assert lib.mqa_logits(*dense_args(**change)) == expect
    assert lib.mqa_last_error()


def test_empty_problems_are_noops():
    assert lib.mqa_logits(*dense_args(sq=0)) == OK
    assert lib.mqa_logits(*dense_args(skv=0, stride=0)) == OK
    assert lib.mqa_logits_compressed(0, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, 0, 64, 64, 128, 0, 0, None, 0, 0, None) == OK
    # the precision is checked even for an empty problem
    assert lib.mqa_logits(*dense_args(sq=0, precision=3)) == INVALID


def test_compressed_validation():
    base = [0, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 64, 64, 128, 0, 0,
            None, 0, 0, None]
    bad = list(base)
    bad[9] = None                                   # row_offsets
    assert lib.mqa_logits_compressed(*bad) == INVALID
    bad = list(base)
    bad[13] = 40                                    # H
    assert lib.mqa_logits_compressed(*bad) == UNSUPPORTED
    bad = list(base)
    bad[16] = 5                                     # logits type
    assert lib.mqa_logits_compressed(*bad) == INVALID
    bad = list(base)
    bad[19] = 9                                     # precision
    assert lib.mqa_logits_compressed(*bad) == INVALID
    assert lib.mqa_logits_compressed_offsets(FAKE, FAKE, -1, 10, FAKE, None) == INVALID
    assert lib.mqa_logits_compressed_offsets(FAKE, FAKE, 4, 10, None, None) == INVALID


@pytest.mark.parametrize("args,expect", [
    ((FAKE, FAKE, 16, 64, 0, FAKE, None), INVALID),          # num_splits
    ((FAKE, FAKE, 16, 64, 8, None, None), INVALID),          # schedule
    ((None, FAKE, 16, 64, 8, FAKE, None), INVALID),          # k_start
    ((FAKE, FAKE, -1, 64, 8, FAKE, None), INVALID),
    ((FAKE, FAKE, 40000, 64, 8, FAKE, None), UNSUPPORTED),
    ((FAKE, FAKE, 16, 64, 8, FAKE_2, None), INVALID),
])
def test_dense_metadata_validation(args, expect):
    assert lib.mqa_logits_metadata(*args) == expect
    assert lib.mqa_logits_metadata_size(256) == 2 * 257
    assert lib.mqa_logits_metadata_size(0) == -1


def paged_meta_args(**kw):
    a = dict(ctx=FAKE, batch=64, next_n=4, bs=64, max_ctx=32768, splits=256, sched=FAKE,
             stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("change,expect", [
    (dict(batch=0), UNSUPPORTED),
    (dict(batch=9000), UNSUPPORTED),
    (dict(next_n=17), UNSUPPORTED),
    (dict(next_n=0), UNSUPPORTED),
    (dict(bs=128), UNSUPPORTED),
    (dict(bs=48), UNSUPPORTED),
    (dict(splits=0), INVALID),
    (dict(max_ctx=-1), INVALID),
    (dict(ctx=None), INVALID),
    (dict(sched=None), INVALID),
])
def test_paged_metadata_validation(change, expect):
    assert lib.paged_mqa_logits_metadata(*paged_meta_args(**change)) == expect


def paged_args(**kw):
    a = dict(dt=0, q=FAKE, q_sf=None, kv=FAKE, kv_sf=None, kvs=FAKE, w=FAKE, ctx=FAKE,
             bt=FAKE, bt_stride=512, sched=FAKE, out=FAKE, stride=32768, batch=64, next_n=4,
             h=64, d=128, bs=64, num_blocks=36000, max_ctx=32768, splits=1024, clean=1,
             w_type=0, out_type=0, precision=0, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("change,expect", [
    (dict(bt_stride=511), INVALID),
    (dict(stride=32767), INVALID),
    (dict(num_blocks=0), INVALID),
    (dict(bt=None), INVALID),
    (dict(sched=None), INVALID),
    (dict(h=24), UNSUPPORTED),
    (dict(next_n=20), UNSUPPORTED),
    (dict(kvs=None), INVALID),
    (dict(w_type=3), INVALID),
    (dict(out_type=1, stride=32769), INVALID),      # bf16 logits need an even stride
    (dict(precision=5), INVALID),
])
def test_paged_validation(change, expect):
    assert lib.paged_mqa_logits(*paged_args(**change)) == expect


def test_metadata_size():
    assert lib.paged_mqa_logits_metadata_size(256) == 2 * 257
    assert lib.paged_mqa_logits_metadata_size(0) == -1


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="needs a host without a GPU")
def test_missing_device_is_reported_as_hip_error():
    assert lib.mqa_num_cus(0) < 0
    assert "device" in lib.mqa_last_error().decode().lower()
    with pytest.raises(mq.MqaError):
        mq.mqa_num_cus(0)


def test_binding_passes_row_strided_tables_and_rejects_others():
    # the block table and the logits rows may sit inside wider buffers (their
    # row stride goes to the library); a table whose rows are not contiguous
    # is refused before any call
    import mqa_logits_amd as mq
    wide = torch.zeros(3, 10, dtype=torch.int32)
    assert mq._rows_ptr(wide[:, :7], "block_table").value == wide.data_ptr()
    with pytest.raises(ValueError, match="rows must be contiguous"):
        mq._rows_ptr(wide.t(), "block_table")
    with pytest.raises(ValueError, match="rows must be contiguous"):
        mq._rows_ptr(wide[:, ::2], "block_table")


def _dense_inputs(fmt="fp8", sq=5, skv=40, h=16, d=64):
    dq = d // 2 if fmt == "mxfp4" else d
    t = dict(q=torch.zeros(sq, h, dq, dtype=torch.uint8), kv=torch.zeros(skv, dq, dtype=torch.uint8),
             q_sf=None, kv_sf=None, kv_scale=torch.ones(skv), weights=torch.zeros(sq, h),
             k_start=torch.zeros(sq, dtype=torch.int32), k_end=torch.full((sq,), skv, dtype=torch.int32))
    if fmt != "fp8":
        t.update(q_sf=torch.zeros(sq, h, d // 32, dtype=torch.uint8),
                 kv_sf=torch.zeros(skv, d // 32, dtype=torch.uint8), kv_scale=None)
    return t


def _call_dense(t, fmt="fp8"):
    import mqa_logits_amd as mq
    return mq.mqa_logits(fmt, t["q"], t["q_sf"], t["kv"], t["kv_sf"], t["kv_scale"], t["weights"],
                         t["k_start"], t["k_end"])


@pytest.mark.parametrize("change,message", [
    (dict(k_start=torch.zeros(5, dtype=torch.int64)), "k_start must be torch.int32"),
    (dict(k_end=torch.zeros(4, dtype=torch.int32)), "k_end must have shape"),
    (dict(kv=torch.zeros(40, 32, dtype=torch.uint8)), "kv must have shape"),
    (dict(kv=torch.zeros(40, 64, dtype=torch.float32)), "kv must have 1-byte elements"),
    (dict(kv_scale=torch.ones(41)), "kv_scale must have shape"),
    (dict(kv_scale=torch.ones(40, dtype=torch.float64)), "kv_scale must be torch.float32"),
    (dict(weights=torch.zeros(5, 16, dtype=torch.float64)), "weights must be"),
    (dict(q=torch.zeros(5, 16, 128, dtype=torch.uint8)[:, :, ::2]), "q must be contiguous"),
    (dict(q_sf=torch.zeros(5, 16, 2, dtype=torch.uint8)), "fp8 takes no block scales"),
    (dict(), "q must be a GPU tensor"),
])
def test_binding_checks_dense_arguments_before_calling(change, message):
    t = _dense_inputs()
    t.update(change)
    with pytest.raises(ValueError, match=message):
        _call_dense(t)


def test_binding_checks_mx_scales_and_paged_tables():
    import mqa_logits_amd as mq
    t = _dense_inputs("mxfp4")
    t["kv_sf"] = torch.zeros(40, 3, dtype=torch.uint8)
    with pytest.raises(ValueError, match="kv_sf must have shape"):
        _call_dense(t, "mxfp4")
    t = _dense_inputs("mxfp8")
    t["kv_scale"] = torch.ones(40)
    with pytest.raises(ValueError, match="takes no kv_scale"):
        _call_dense(t, "mxfp8")
    # paged: rows of the weights must be batch * next_n, the block table int32
    q = torch.zeros(6, 16, 64, dtype=torch.uint8)
    pool = torch.zeros(10, 16, 64, dtype=torch.uint8)
    scales = torch.ones(10, 16)
    ctx = torch.tensor([5, 9], dtype=torch.int32)
    sched = torch.zeros(5, 2, dtype=torch.int32)
    with pytest.raises(ValueError, match="batch \\* next_n"):
        mq.paged_mqa_logits("fp8", q, None, pool, None, scales, torch.zeros(5, 16), ctx,
                            torch.zeros(2, 4, dtype=torch.int32), sched, 3, 64)
    with pytest.raises(ValueError, match="block_table must be torch.int32"):
        mq.paged_mqa_logits("fp8", q, None, pool, None, scales, torch.zeros(6, 16), ctx,
                            torch.zeros(2, 4, dtype=torch.int64), sched, 3, 64)
    with pytest.raises(ValueError, match="k_start and k_end go together"):
        mq.mqa_logits_topk(torch.zeros(3, 10), 2, torch.zeros(3, dtype=torch.int32))


def test_binding_requires_block_tables_wide_enough_for_max_context_len():
    # the library reads row b of the table up to ceil(min(ctx_b, max_ctx) / bs)
    # entries; the binding cannot see ctx_b without a device read, so it asks
    # for rows of ceil(max_ctx / bs)
    import mqa_logits_amd as mq
    batch, next_n, h, d, bs, nblk, max_ctx = 2, 2, 8, 64, 16, 12, 40
    rows = batch * next_n
    q = torch.zeros(rows, h, d, dtype=torch.uint8)
    kv = torch.zeros(nblk, bs, d, dtype=torch.uint8)
    kvs = torch.ones(nblk, bs)
    w = torch.ones(rows, h)
    ctx = torch.full((batch,), max_ctx, dtype=torch.int32)
    sched = torch.zeros(3, 2, dtype=torch.int32)
    narrow = torch.zeros(batch, 2, dtype=torch.int32)           # needs 3
    with pytest.raises(ValueError, match="block_table rows must hold .* = 3 blocks, got 2"):
        mq.paged_mqa_logits("fp8", q, None, kv, None, kvs, w, ctx, narrow, sched, next_n, max_ctx)
    # the width check passes at 3; the next refusal is the CPU tensor
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        mq.paged_mqa_logits("fp8", q, None, kv, None, kvs, w, ctx,
                            torch.zeros(batch, 3, dtype=torch.int32), sched, next_n, max_ctx)
