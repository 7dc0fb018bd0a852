"""Python binding of libkvq (KV-cache quantise-on-write and dequant-fused paged
decode attention for MI355X / gfx950).

Argument marshalling only: every step runs in the HIP kernels of libkvq.so,
called through its C ABI (include/kvq.h) with the same entry-point names.
PyTorch supplies device memory and the current HIP stream.  The library must
have been built (``python -m quantized_decode_attention_amd._build`` or
``__graft_entry__.build()``); importing without it fails loudly.
"""
from __future__ import annotations

import ctypes
import os

# torch first: it carries its own HIP runtime (soname libamdhip64.so.7), and
# libkvq.so must bind to that same runtime rather than load a second copy.
import torch  # noqa: F401

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvq.so")

KVQ_FP8_PER_TENSOR = 1
KVQ_INT8_PTH = 2
KVQ_FP8_PTH = 3
KVQ_NVFP4 = 4
KVQ_KVARN_K4V2_G128 = 5
KVQ_INT4_PTH = 6
KVQ_MXFP4 = 7
KVQ_FLAG_NVFP4_4OVER6 = 1

FORMAT_NAMES = {1: "fp8_per_tensor", 2: "int8_per_token_head", 3: "fp8_per_token_head", 4: "nvfp4",
                5: "kvarn_k4v2_g128", 6: "int4_per_token_head", 7: "mxfp4"}

STATUS = {0: "KVQ_OK", 1: "KVQ_ERR_INVALID_ARG", 2: "KVQ_ERR_UNSUPPORTED", 3: "KVQ_ERR_WORKSPACE_TOO_SMALL",
          4: "KVQ_ERR_DEVICE", 5: "KVQ_ERR_HIP", 6: "KVQ_ERR_SCRATCH_TOO_SMALL"}
KVQ_DECODE_SCRATCH_BYTES = 16 << 20


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({kvq_status_string(status)})")


class KvqLayout(ctypes.Structure):
    """kvq_layout of include/kvq.h."""
    _fields_ = [
        ("format", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
    ]


def layout(fmt, num_kv_heads, head_dim, page_size, num_pages, k_scale=1.0, v_scale=1.0, flags=0) -> KvqLayout:
    return KvqLayout(fmt, flags, num_kv_heads, head_dim, page_size, num_pages, k_scale, v_scale)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m quantized_decode_attention_amd._build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    LP = ctypes.POINTER(KvqLayout)
    sigs = {
        "kvq_page_bytes": (I64, [LP]),
        "kvq_check_device": (ctypes.c_int, [ctypes.c_int]),
        "kvq_take_device_errors": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), P]),
        "kvq_quantize_write": (ctypes.c_int, [LP, P, P, P, I64, P, P]),
        "kvq_decode_workspace_bytes": (I64, [LP, I32, I32, I32, I32]),
        "kvq_decode_num_splits": (I32, [LP, I32, I32, I32, I32]),
        "kvq_decode_attention": (ctypes.c_int, [LP, P, P, I32, P, I32, P, I32, F32, P, P, P, I64, I32, P]),
        "kvq_decode_attention_append": (ctypes.c_int, [LP, P, P, P, P, P, I32, P, I32, P, I32, F32, P, P, I64, I32,
                                                        P]),
        "kvq_decode_attention_noalloc": (ctypes.c_int, [LP, P, P, I32, P, I32, P, I32, F32, P, P, I32, P]),
        "kvq_dequantize": (ctypes.c_int, [LP, P, P, I64, P, P, P]),
        "kvq_kvarn_append": (ctypes.c_int, [LP, P, P, P, P, I64, P, I32, P, I32, P, P]),
        "kvq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


_lib = _load()
lib = _lib


def kvq_status_string(status: int) -> str:
    return _lib.kvq_status_string(status).decode()


def _check(st: int, where: str):
    if st != 0:
        raise KvqError(st, where)


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() and t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    return ctypes.c_void_p(t.data_ptr())


# ---- entry points (same names as the C ABI) ---------------------------------

def kvq_page_bytes(lay: KvqLayout) -> int:
    return int(_lib.kvq_page_bytes(ctypes.byref(lay)))


def kvq_check_device(device: int = 0) -> int:
    return int(_lib.kvq_check_device(device))


KVQ_DEVERR_KVARN_TILE_SLOTS = 1 << 0
KVQ_DEVERR_KVARN_APPEND_SPAN = 1 << 1


def kvq_take_device_errors(stream=None) -> int:
    """Waits for the stream, returns the KVQ_DEVERR_* bits raised on the current device since the previous
    call and clears them."""
    flags = ctypes.c_uint32(0)
    _check(_lib.kvq_take_device_errors(ctypes.byref(flags), _stream(stream)), "kvq_take_device_errors")
    return int(flags.value)


def kvq_quantize_write(lay: KvqLayout, k, v, slot_mapping, cache, stream=None):
    """k, v: float16 [n_tok, H, D]; slot_mapping: int64 [n_tok]; cache: uint8."""
    import torch
    n = slot_mapping.shape[0]
    if k.shape != v.shape or k.shape[0] != n:
        raise ValueError("k, v must be [n_tok, H, D] and match slot_mapping")
    _check(_lib.kvq_quantize_write(ctypes.byref(lay), _ptr(k, torch.float16, "k"), _ptr(v, torch.float16, "v"),
                                   _ptr(slot_mapping, torch.int64, "slot_mapping"), n,
                                   _ptr(cache, torch.uint8, "cache"), _stream(stream)), "kvq_quantize_write")


def kvq_decode_workspace_bytes(lay: KvqLayout, batch: int, num_q_heads: int, max_pages_per_seq: int,
                               num_splits: int = 0) -> int:
    return int(_lib.kvq_decode_workspace_bytes(ctypes.byref(lay), batch, num_q_heads, max_pages_per_seq, num_splits))


def kvq_decode_num_splits(lay: KvqLayout, batch: int, num_q_heads: int, max_pages_per_seq: int,
                          num_splits: int = 0) -> int:
    return int(_lib.kvq_decode_num_splits(ctypes.byref(lay), batch, num_q_heads, max_pages_per_seq, num_splits))


def _decode_args(lay, cache, q, block_tables, context_lens, sm_scale, out, workspace, kvarn_tail, num_splits,
                 stream):
    import torch
    B, Hq, _ = q.shape
    return (ctypes.byref(lay), _ptr(cache, torch.uint8, "cache"), _ptr(q, torch.float16, "q"), Hq,
            _ptr(block_tables, torch.int32, "block_tables"), block_tables.shape[1],
            _ptr(context_lens, torch.int32, "context_lens"), B, float(sm_scale),
            _ptr(kvarn_tail, torch.float16, "kvarn_tail"), _ptr(out, torch.float16, "out"),
            _ptr(workspace, torch.uint8, "workspace") if workspace is not None and workspace.numel() else None,
            0 if workspace is None else workspace.numel(), num_splits, _stream(stream))


def kvq_decode_attention(lay: KvqLayout, cache, q, block_tables, context_lens, sm_scale, out, workspace,
                         kvarn_tail=None, num_splits: int = 0, stream=None):
    """q, out: float16 [B, Hq, D]; block_tables: int32 [B, max_pages]; context_lens: int32 [B];
    workspace: uint8 of at least kvq_decode_workspace_bytes(...) bytes (or None when that is 0)."""
    _check(_lib.kvq_decode_attention(*_decode_args(lay, cache, q, block_tables, context_lens, sm_scale, out,
                                                   workspace, kvarn_tail, num_splits, stream)),
           "kvq_decode_attention")


def kvq_decode_attention_noalloc(lay: KvqLayout, cache, q, block_tables, context_lens, sm_scale, out,
                                 kvarn_tail=None, num_splits: int = 0, stream=None):
    """kvq_decode_attention with the library's fixed device workspace instead of a caller's buffer (no
    allocation in the call; calls that overlap in time on one GPU race)."""
    import torch
    B, Hq, _ = q.shape
    _check(_lib.kvq_decode_attention_noalloc(
        ctypes.byref(lay), _ptr(cache, torch.uint8, "cache"), _ptr(q, torch.float16, "q"), Hq,
        _ptr(block_tables, torch.int32, "block_tables"), block_tables.shape[1],
        _ptr(context_lens, torch.int32, "context_lens"), B, float(sm_scale),
        _ptr(kvarn_tail, torch.float16, "kvarn_tail"), _ptr(out, torch.float16, "out"), num_splits,
        _stream(stream)), "kvq_decode_attention_noalloc")


def _append_args(lay, cache, k_new, v_new, slot_mapping, q, block_tables, context_lens, sm_scale, out, workspace,
                 num_splits, stream):
    import torch
    B, Hq, _ = q.shape
    return (ctypes.byref(lay), _ptr(cache, torch.uint8, "cache"), _ptr(k_new, torch.float16, "k_new"),
            _ptr(v_new, torch.float16, "v_new"), _ptr(slot_mapping, torch.int64, "slot_mapping"),
            _ptr(q, torch.float16, "q"), Hq, _ptr(block_tables, torch.int32, "block_tables"), block_tables.shape[1],
            _ptr(context_lens, torch.int32, "context_lens"), B, float(sm_scale), _ptr(out, torch.float16, "out"),
            _ptr(workspace, torch.uint8, "workspace") if workspace is not None and workspace.numel() else None,
            0 if workspace is None else workspace.numel(), num_splits, _stream(stream))


def kvq_decode_attention_append(lay: KvqLayout, cache, k_new, v_new, slot_mapping, q, block_tables, context_lens,
                                sm_scale, out, workspace, num_splits: int = 0, stream=None):
    """One decode step: k_new, v_new: float16 [B, H, D] (one new token per sequence); slot_mapping: int64 [B];
    q, out: float16 [B, Hq, D]; block_tables: int32 [B, max_pages]; context_lens: int32 [B] (new token
    included); workspace as for kvq_decode_attention."""
    _check(_lib.kvq_decode_attention_append(*_append_args(lay, cache, k_new, v_new, slot_mapping, q, block_tables,
                                                          context_lens, sm_scale, out, workspace, num_splits,
                                                          stream)),
           "kvq_decode_attention_append")


def _kvarn_append_args(lay, k, v, seq, pos, tail, block_tables, cache, stream):
    import torch
    return (ctypes.byref(lay), _ptr(k, torch.float16, "k"), _ptr(v, torch.float16, "v"),
            _ptr(seq, torch.int32, "seq"), _ptr(pos, torch.int32, "pos"), seq.shape[0],
            _ptr(tail, torch.float16, "tail"), tail.shape[0], _ptr(block_tables, torch.int32, "block_tables"),
            block_tables.shape[1], _ptr(cache, torch.uint8, "cache"), _stream(stream))


def kvq_kvarn_append(lay: KvqLayout, k, v, seq, pos, tail, block_tables, cache, stream=None):
    """k, v: float16 [n, H, 128]; seq, pos: int32 [n]; tail: float16 [B, 2, H, 128, 128];
    block_tables: int32 [B, max_pages]; cache: uint8."""
    _check(_lib.kvq_kvarn_append(*_kvarn_append_args(lay, k, v, seq, pos, tail, block_tables, cache, stream)),
           "kvq_kvarn_append")


def kvq_dequantize(lay: KvqLayout, cache, slot_mapping, k_out, v_out, stream=None):
    """k_out, v_out: float32 [n_tok, H, D]."""
    import torch
    _check(_lib.kvq_dequantize(ctypes.byref(lay), _ptr(cache, torch.uint8, "cache"),
                               _ptr(slot_mapping, torch.int64, "slot_mapping"), slot_mapping.shape[0],
                               _ptr(k_out, torch.float32, "k_out"), _ptr(v_out, torch.float32, "v_out"),
                               _stream(stream)), "kvq_dequantize")


# ---- prepared calls -----------------------------------------------------------
# A serving loop that repeats a call with the same buffers can marshal its
# arguments once: prepare_<entry point>(same arguments) returns a callable
# that makes only the C call (and raises KvqError on a nonzero status).  The
# stream is fixed when the call is prepared (the current stream by default);
# the callable holds references to the tensors it was given, so they stay
# allocated while it exists.

def _prepared(fn, args, where, keep):
    def call():
        st = fn(*args)
        if st != 0:
            raise KvqError(st, where)
    call.tensors = keep
    return call


def prepare_decode_attention(lay: KvqLayout, cache, q, block_tables, context_lens, sm_scale, out, workspace,
                             kvarn_tail=None, num_splits: int = 0, stream=None):
    return _prepared(_lib.kvq_decode_attention, _decode_args(lay, cache, q, block_tables, context_lens, sm_scale,
                                                             out, workspace, kvarn_tail, num_splits, stream),
                     "kvq_decode_attention", (lay, cache, q, block_tables, context_lens, out, workspace, kvarn_tail))


def prepare_decode_attention_append(lay: KvqLayout, cache, k_new, v_new, slot_mapping, q, block_tables,
                                    context_lens, sm_scale, out, workspace, num_splits: int = 0, stream=None):
    return _prepared(_lib.kvq_decode_attention_append,
                     _append_args(lay, cache, k_new, v_new, slot_mapping, q, block_tables, context_lens, sm_scale,
                                  out, workspace, num_splits, stream), "kvq_decode_attention_append",
                     (lay, cache, k_new, v_new, slot_mapping, q, block_tables, context_lens, out, workspace))


def prepare_kvarn_append(lay: KvqLayout, k, v, seq, pos, tail, block_tables, cache, stream=None):
    return _prepared(_lib.kvq_kvarn_append, _kvarn_append_args(lay, k, v, seq, pos, tail, block_tables, cache,
                                                               stream), "kvq_kvarn_append",
                     (lay, k, v, seq, pos, tail, block_tables, cache))


# ---- small conveniences over the entry points --------------------------------

class DecodeWorkspace:
    """A decode workspace sized for a problem."""

    def __init__(self, lay: KvqLayout, batch: int, num_q_heads: int, max_pages_per_seq: int, num_splits: int = 0,
                 device="cuda", stream=None):
        import torch
        nbytes = kvq_decode_workspace_bytes(lay, batch, num_q_heads, max_pages_per_seq, num_splits)
        if nbytes < 0:
            raise KvqError(1, "kvq_decode_workspace_bytes")
        self.num_splits = kvq_decode_num_splits(lay, batch, num_q_heads, max_pages_per_seq, num_splits)
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
