"""Python binding of libmqa_logits (weighted MQA logits on MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/mqa_logits.h.  PyTorch supplies
device memory and the current stream; nothing here computes logits, and there
is no CPU fallback -- if the shared library is missing, importing the package
raises.

Entry points (same names as the C ABI):
  mqa_logits                      dense clean (or keep) logits
  mqa_logits_metadata             work schedule for the dense / compressed calls
  mqa_logits_topk                 top-k column indices of logits rows
  mqa_logits_compressed_offsets   row offsets of the packed layout
  mqa_logits_compressed           packed logits
  paged_mqa_logits_metadata       paged work split
  paged_mqa_logits                paged decode logits
  mqa_num_cus, paged_mqa_logits_default_splits
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmqa_logits.so")

FORMATS = {"fp8": 0, "mxfp8": 1, "mxfp4": 2}
# mqa_precision of the C ABI: the matrix core's grouped summation, or every
# product exact (eight KV operand copies for fp8 elements)
PRECISIONS = {"default": 0, "exact": 1}
# mqa_float of the C ABI: element type of the weights and of the logits
FLOAT_TYPES = {torch.float32: 0, torch.bfloat16: 1}


class MqaError(RuntimeError):
    """A non-OK status from the C ABI, with mqa_last_error()'s message."""

    def __init__(self, status, message):
        super().__init__(f"status {status}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python mqa_logits_amd/build.py` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sigs = {
        "mqa_logits": [I32, P, P, P, P, P, P, P, P, P, I64, I32, I32, I32, I32, I32, I32, I32,
                       P, I32, I32, P],
        "mqa_logits_metadata": [P, P, I32, I32, I32, P, P],
        "mqa_logits_topk": [P, I32, I64, P, P, I32, I32, I32, P, I64, P],
        "mqa_logits_compressed_offsets": [P, P, I32, I32, P, P],
        "mqa_logits_compressed": [I32, P, P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                  P, I32, I32, P],
        "paged_mqa_logits_metadata": [P, I32, I32, I32, I32, I32, P, P],
        "paged_mqa_logits": [I32, P, P, P, P, P, P, P, P, I64, P, P, I64,
                             I32, I32, I32, I32, I32, I32, I32, I32, I32, I32, I32, I32, P],
    }
    for name, argtypes in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_int
    for name in ("paged_mqa_logits_metadata_size", "mqa_logits_metadata_size"):
        getattr(lib, name).argtypes = [I32]
        getattr(lib, name).restype = I64
    lib.mqa_num_cus.argtypes = [I32]
    lib.mqa_num_cus.restype = I32
    lib.paged_mqa_logits_default_splits.argtypes = [I32]
    lib.paged_mqa_logits_default_splits.restype = I32
    lib.mqa_last_error.argtypes = []
    lib.mqa_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()

EXPORTED = ("mqa_logits", "mqa_logits_metadata_size", "mqa_logits_metadata", "mqa_logits_topk",
            "mqa_logits_compressed_offsets", "mqa_logits_compressed",
            "paged_mqa_logits_metadata_size", "paged_mqa_logits_metadata",
            "paged_mqa_logits", "mqa_num_cus", "paged_mqa_logits_default_splits",
            "mqa_last_error")


def _check(status):
    if status != 0:
        raise MqaError(status, lib.mqa_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmqa_logits must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


I32_T, I64_T = (torch.int32,), (torch.int64,)


class _Args:
    """The tensor arguments of one call, checked against what the C ABI will
    read or write through their pointers: shape (None entries are free),
    element type or size, layout (contiguous, or rows contiguous when
    `rows`), then one GPU for all of them.  The library sees only pointers
    and sizes, so a mismatch would read or write outside a tensor."""

    def __init__(self):
        self.seen = []

    def want(self, t, name, shape, dtypes=None, itemsize=None, rows=False):
        if t is None:
            raise ValueError(f"{name} is required")
        got = t.shape                           # a tuple: compared whole when no entry is free
        if (got != shape) if None not in shape else (
                len(got) != len(shape) or not all(w is None or g == w for g, w in zip(got, shape))):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(got)}")
        dt = t.dtype
        if dtypes is not None and dt not in dtypes:
            raise ValueError(f"{name} must be {' or '.join(map(str, dtypes))}, got {dt}")
        if itemsize is not None and dt.itemsize != itemsize:
            raise ValueError(f"{name} must have {itemsize}-byte elements, got {dt}")
        if rows:
            if len(got) and t.stride(-1) != 1 and got[-1] > 1:
                raise ValueError(f"{name} rows must be contiguous")
        elif not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        self.seen.append((name, t))

    def on_gpu(self):
        # device indices compared as integers (-1 for a CPU tensor)
        first = self.seen[0][1].get_device()
        for name, t in self.seen:
            dev = t.get_device()
            if dev < 0:
                raise ValueError(f"{name} must be a GPU tensor (the library reads device memory)")
            if dev != first:
                raise ValueError(f"{name} must be on cuda:{first}, got {t.device}")


def _codes(a, fmt, q, kv, q_sf, kv_sf, kv_scale, rows_shape, kv_shape):
    """The Q and KV operands of a call: byte codes (two e2m1 per byte for
    mxfp4), e8m0 block scales for the MX formats, fp32 token scales for fp8.
    rows_shape: Q's leading dims; kv_shape: KV's leading dims.  Returns D."""
    _fmt(fmt)
    d = _head_dim(fmt, q)
    a.want(q, "q", (*rows_shape, q.shape[-1] if q.dim() else None), itemsize=1)
    a.want(kv, "kv", (*kv_shape, q.shape[-1]), itemsize=1)
    if fmt == "fp8":
        if q_sf is not None or kv_sf is not None:
            raise ValueError("fp8 takes no block scales (q_sf, kv_sf)")
        a.want(kv_scale, "kv_scale", tuple(kv_shape), (torch.float32,))
    else:
        if kv_scale is not None:
            raise ValueError(f"{fmt} takes no kv_scale")
        a.want(q_sf, "q_sf", (*rows_shape, d // 32), itemsize=1)
        a.want(kv_sf, "kv_sf", (*kv_shape, d // 32), itemsize=1)
    return d


def _rows_ptr(t, what):
    """A 2-D tensor whose rows are contiguous (its row stride is passed apart)."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{what} rows must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _fmt(fmt):
    if fmt not in FORMATS:
        raise ValueError(f"format must be one of {sorted(FORMATS)}, got {fmt!r}")
    return FORMATS[fmt]


def _precision(precision):
    if precision not in PRECISIONS:
        raise ValueError(f"precision must be one of {sorted(PRECISIONS)}, got {precision!r}")
    return PRECISIONS[precision]


def _head_dim(fmt, q):
    return q.shape[-1] * (2 if fmt == "mxfp4" else 1)


def _float_type(dtype, what):
    if dtype not in FLOAT_TYPES:
        raise ValueError(f"{what} must be float32 or bfloat16, got {dtype}")
    return FLOAT_TYPES[dtype]


def _logits_rows(rows, cols, dtype, device):
    """[rows, cols] logits; bf16 rows get an even stride (the C ABI needs one)."""
    width = cols + (cols & 1) if dtype == torch.bfloat16 else cols
    out = torch.empty(rows, width, dtype=dtype, device=device)
    return out[:, :cols] if width != cols else out


def mqa_num_cus(device=0):
    n = lib.mqa_num_cus(int(device))
    if n < 0:
        raise MqaError(3, lib.mqa_last_error().decode())
    return n


def paged_mqa_logits_default_splits(device=0):
    n = lib.paged_mqa_logits_default_splits(int(device))
    if n < 0:
        raise MqaError(3, lib.mqa_last_error().decode())
    return n


def _schedule(schedule):
    if schedule is None:
        return None, 0
    return _ptr(schedule), schedule.shape[0] - 1


def _dense_args(a, fmt, q, q_sf, kv, kv_sf, kv_scale, weights, k_start, k_end, schedule):
    sq, h = weights.shape
    _codes(a, fmt, q, kv, q_sf, kv_sf, kv_scale, (sq, h), (kv.shape[0],))
    a.want(weights, "weights", (sq, h), tuple(FLOAT_TYPES))
    a.want(k_start, "k_start", (sq,), I32_T)
    a.want(k_end, "k_end", (sq,), I32_T)
    if schedule is not None:
        a.want(schedule, "schedule", (None, 2), I32_T)


def mqa_logits_metadata(k_start, k_end, skv, num_splits=None, out=None):
    """int32 [num_splits + 1, 2] work schedule for mqa_logits /
    mqa_logits_compressed with these ranges."""
    a = _Args()
    if num_splits is None:
        num_splits = paged_mqa_logits_default_splits(k_start.device.index or 0)
    sq = k_start.shape[0]
    a.want(k_start, "k_start", (sq,), I32_T)
    a.want(k_end, "k_end", (sq,), I32_T)
    if out is None:
        out = torch.empty(num_splits + 1, 2, dtype=torch.int32, device=k_start.device)
    a.want(out, "out", (num_splits + 1, 2), I32_T)
    a.on_gpu()
    _check(lib.mqa_logits_metadata(_ptr(k_start), _ptr(k_end), k_start.shape[0], skv,
                                   num_splits, _ptr(out), _stream(k_start)))
    return out


def mqa_logits(fmt, q, q_sf, kv, kv_sf, kv_scale, weights, k_start, k_end,
               clean_logits=True, out=None, logits_dtype=torch.float32, schedule=None,
               precision="default"):
    """Dense logits [Sq, Skv] of logits_dtype (out may be a wider-strided row
    view; its dtype then decides).  weights: float32 or bfloat16.  schedule:
    None or mqa_logits_metadata's result for the same ranges.  precision:
    "default" or "exact" (mqa_precision)."""
    sq, h = weights.shape
    skv = kv.shape[0]
    a = _Args()
    _dense_args(a, fmt, q, q_sf, kv, kv_sf, kv_scale, weights, k_start, k_end, schedule)
    if out is None:
        out = _logits_rows(sq, skv, logits_dtype, q.device)
    a.want(out, "out", (sq, skv), tuple(FLOAT_TYPES), rows=True)
    a.on_gpu()
    _check(lib.mqa_logits(
        _fmt(fmt), _ptr(q), _ptr(q_sf), _ptr(kv), _ptr(kv_sf), _ptr(kv_scale),
        _ptr(weights), _ptr(k_start), _ptr(k_end), ctypes.c_void_p(out.data_ptr()),
        out.stride(0) if sq > 0 else skv, sq, skv, h, _head_dim(fmt, q),
        1 if clean_logits else 0, _float_type(weights.dtype, "weights"),
        _float_type(out.dtype, "logits"), *_schedule(schedule), _precision(precision),
        _stream(q)))
    return out


def mqa_logits_topk(logits, topk, k_start=None, k_end=None, out=None):
    """int32 [Sq, topk] columns of each row's topk largest non--inf logits in
    [k_start, k_end) (the whole row without ranges), ascending, -1 padded."""
    a = _Args()
    sq, skv = logits.shape
    a.want(logits, "logits", (sq, skv), tuple(FLOAT_TYPES), rows=True)
    if (k_start is None) != (k_end is None):
        raise ValueError("k_start and k_end go together")
    if k_start is not None:
        a.want(k_start, "k_start", (sq,), I32_T)
        a.want(k_end, "k_end", (sq,), I32_T)
    if out is None:
        out = torch.empty(sq, topk, dtype=torch.int32, device=logits.device)
    a.want(out, "out", (sq, topk), I32_T, rows=True)
    a.on_gpu()
    _check(lib.mqa_logits_topk(
        ctypes.c_void_p(logits.data_ptr()), _float_type(logits.dtype, "logits"),
        logits.stride(0) if sq > 0 else skv, _ptr(k_start), _ptr(k_end), sq, skv, topk,
        ctypes.c_void_p(out.data_ptr()), out.stride(0) if sq > 0 else topk,
        _stream(logits)))
    return out


def mqa_logits_compressed_offsets(k_start, k_end, skv, out=None):
    """int64 [Sq + 1] exclusive prefix sum of the clamped row lengths."""
    a = _Args()
    sq = k_start.shape[0]
    a.want(k_start, "k_start", (sq,), I32_T)
    a.want(k_end, "k_end", (sq,), I32_T)
    if out is None:
        out = torch.empty(sq + 1, dtype=torch.int64, device=k_start.device)
    a.want(out, "out", (sq + 1,), I64_T)
    a.on_gpu()
    _check(lib.mqa_logits_compressed_offsets(_ptr(k_start), _ptr(k_end), sq, skv,
                                             _ptr(out), _stream(k_start)))
    return out


def mqa_logits_compressed(fmt, q, q_sf, kv, kv_sf, kv_scale, weights, k_start, k_end,
                          row_offsets=None, out=None, logits_dtype=torch.float32,
                          schedule=None, precision="default"):
    """Packed logits; returns (packed [total] of logits_dtype, row_offsets int64
    [Sq+1]).

    Without `out`, the total length is read back from the device (a sync)."""
    sq, h = weights.shape
    skv = kv.shape[0]
    a = _Args()
    _dense_args(a, fmt, q, q_sf, kv, kv_sf, kv_scale, weights, k_start, k_end, schedule)
    if row_offsets is None:
        row_offsets = mqa_logits_compressed_offsets(k_start, k_end, skv)
    a.want(row_offsets, "row_offsets", (sq + 1,), I64_T)
    if out is None:
        out = torch.empty(int(row_offsets[-1].item()), dtype=logits_dtype, device=q.device)
    # out must hold row_offsets[-1] values (not checked here: that would read
    # the offsets back from the device)
    a.want(out, "out", (None,), tuple(FLOAT_TYPES))
    a.on_gpu()
    _check(lib.mqa_logits_compressed(
        _fmt(fmt), _ptr(q), _ptr(q_sf), _ptr(kv), _ptr(kv_sf), _ptr(kv_scale),
        _ptr(weights), _ptr(k_start), _ptr(k_end), _ptr(row_offsets), _ptr(out),
        sq, skv, h, _head_dim(fmt, q), _float_type(weights.dtype, "weights"),
        _float_type(out.dtype, "logits"), *_schedule(schedule), _precision(precision),
        _stream(q)))
    return out, row_offsets


def paged_mqa_logits_metadata(context_lens, next_n, block_size, max_context_len,
                              num_splits=None, out=None):
    """int32 [num_splits + 1, 2] schedule for paged_mqa_logits."""
    a = _Args()
    if num_splits is None:
        num_splits = paged_mqa_logits_default_splits(context_lens.device.index or 0)
    a.want(context_lens, "context_lens", (context_lens.shape[0],), I32_T)
    if out is None:
        out = torch.empty(num_splits + 1, 2, dtype=torch.int32, device=context_lens.device)
    a.want(out, "out", (num_splits + 1, 2), I32_T)
    a.on_gpu()
    _check(lib.paged_mqa_logits_metadata(_ptr(context_lens), context_lens.shape[0], next_n,
                                         block_size, max_context_len, num_splits, _ptr(out),
                                         _stream(context_lens)))
    return out


def paged_mqa_logits(fmt, q, q_sf, kv_pool, kv_sf_pool, kv_scale_pool, weights,
                     context_lens, block_table, schedule, next_n, max_context_len,
                     clean_logits=True, out=None, logits_dtype=torch.float32,
                     precision="default"):
    """Paged decode logits [batch * next_n, max_context_len] of logits_dtype."""
    a = _Args()
    batch = context_lens.shape[0]
    rows, h = weights.shape
    num_blocks, block_size = kv_pool.shape[0], kv_pool.shape[1]
    num_splits = schedule.shape[0] - 1
    if rows != batch * next_n:
        raise ValueError(f"weights must have batch * next_n = {batch * next_n} rows, got {rows}")
    _codes(a, fmt, q, kv_pool, q_sf, kv_sf_pool, kv_scale_pool, (rows, h), (num_blocks, block_size))
    a.want(weights, "weights", (rows, h), tuple(FLOAT_TYPES))
    a.want(context_lens, "context_lens", (batch,), I32_T)
    a.want(block_table, "block_table", (batch, None), I32_T, rows=True)
    need = -(-max_context_len // block_size) if block_size > 0 else 0
    if block_table.shape[1] < need:
        raise ValueError(f"block_table rows must hold ceil(max_context_len / block_size) = {need} "
                         f"blocks, got {block_table.shape[1]}")
    a.want(schedule, "schedule", (num_splits + 1, 2), I32_T)
    if out is None:
        out = _logits_rows(rows, max_context_len, logits_dtype, q.device)
    a.want(out, "out", (rows, max_context_len), tuple(FLOAT_TYPES), rows=True)
    a.on_gpu()
    _check(lib.paged_mqa_logits(
        _fmt(fmt), _ptr(q), _ptr(q_sf), _ptr(kv_pool), _ptr(kv_sf_pool), _ptr(kv_scale_pool),
        _ptr(weights), _ptr(context_lens), _rows_ptr(block_table, "block_table"),
        block_table.stride(0),
        _ptr(schedule), ctypes.c_void_p(out.data_ptr()), out.stride(0), batch, next_n, h,
        _head_dim(fmt, q), block_size, num_blocks, max_context_len, num_splits,
        1 if clean_logits else 0, _float_type(weights.dtype, "weights"),
        _float_type(out.dtype, "logits"), _precision(precision), _stream(q)))
    return out
