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


def mqa_logits_metadata(k_start, k_end, skv, num_splits=None, out=None):
    """int32 [num_splits + 1, 2] work schedule for mqa_logits /
    mqa_logits_compressed with these ranges."""
    if num_splits is None:
        num_splits = paged_mqa_logits_default_splits(k_start.device.index or 0)
    if out is None:
        out = torch.empty(num_splits + 1, 2, dtype=torch.int32, device=k_start.device)
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
    if out is None:
        out = _logits_rows(sq, skv, logits_dtype, q.device)
    if out.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
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
    sq, skv = logits.shape
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    if out is None:
        out = torch.empty(sq, topk, dtype=torch.int32, device=logits.device)
    _check(lib.mqa_logits_topk(
        ctypes.c_void_p(logits.data_ptr()), _float_type(logits.dtype, "logits"),
        logits.stride(0) if sq > 0 else skv, _ptr(k_start), _ptr(k_end), sq, skv, topk,
        ctypes.c_void_p(out.data_ptr()), out.stride(0) if sq > 0 else topk,
        _stream(logits)))
    return out


def mqa_logits_compressed_offsets(k_start, k_end, skv, out=None):
    """int64 [Sq + 1] exclusive prefix sum of the clamped row lengths."""
    sq = k_start.shape[0]
    if out is None:
        out = torch.empty(sq + 1, dtype=torch.int64, device=k_start.device)
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
    if row_offsets is None:
        row_offsets = mqa_logits_compressed_offsets(k_start, k_end, skv)
    if out is None:
        out = torch.empty(int(row_offsets[-1].item()), dtype=logits_dtype, device=q.device)
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
    if num_splits is None:
        num_splits = paged_mqa_logits_default_splits(context_lens.device.index or 0)
    if out is None:
        out = torch.empty(num_splits + 1, 2, dtype=torch.int32, device=context_lens.device)
    _check(lib.paged_mqa_logits_metadata(_ptr(context_lens), context_lens.shape[0], next_n,
                                         block_size, max_context_len, num_splits, _ptr(out),
                                         _stream(context_lens)))
    return out


def paged_mqa_logits(fmt, q, q_sf, kv_pool, kv_sf_pool, kv_scale_pool, weights,
                     context_lens, block_table, schedule, next_n, max_context_len,
                     clean_logits=True, out=None, logits_dtype=torch.float32,
                     precision="default"):
    """Paged decode logits [batch * next_n, max_context_len] of logits_dtype."""
    batch = context_lens.shape[0]
    rows, h = weights.shape
    num_blocks, block_size = kv_pool.shape[0], kv_pool.shape[1]
    num_splits = schedule.shape[0] - 1
    if out is None:
        out = _logits_rows(rows, max_context_len, logits_dtype, q.device)
    if out.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    _check(lib.paged_mqa_logits(
        _fmt(fmt), _ptr(q), _ptr(q_sf), _ptr(kv_pool), _ptr(kv_sf_pool), _ptr(kv_scale_pool),
        _ptr(weights), _ptr(context_lens), _rows_ptr(block_table, "block_table"),
        block_table.stride(0),
        _ptr(schedule), ctypes.c_void_p(out.data_ptr()), out.stride(0), batch, next_n, h,
        _head_dim(fmt, q), block_size, num_blocks, max_context_len, num_splits,
        1 if clean_logits else 0, _float_type(weights.dtype, "weights"),
        _float_type(out.dtype, "logits"), _precision(precision), _stream(q)))
    return out
