"""ctypes binding of the CPU oracle (kvq_oracle.c).

TEST INFRASTRUCTURE: only tests/, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The product library
(quantized_decode_attention_amd) never imports it and shares no code with it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkvq_oracle.so")

FP8_PER_TENSOR, INT8_PTH, FP8_PTH, NVFP4, KVARN_K4V2_G128, INT4_PTH, MXFP4 = 1, 2, 3, 4, 5, 6, 7
FLAG_NVFP4_4OVER6 = 1


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH, defines=()) -> str:
    """Compile the oracle with gcc (binary32 semantics: no contraction, no
    fast-math, SSE arithmetic)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Wno-unused-function",
             *[f"-D{d}" for d in defines], "-o", tmp, src, "-lm"],
            check=True,
        )
        os.replace(tmp, out)
    return out


class Layout(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
    ]


def layout(fmt, num_kv_heads, head_dim, page_size, num_pages, k_scale=1.0, v_scale=1.0, flags=0):
    return Layout(fmt, flags, num_kv_heads, head_dim, page_size, num_pages, k_scale, v_scale)



_SIGS = None


def _sigs():
    P, I32, I64, F32, F64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
    U8, U16, INT = ctypes.c_uint8, ctypes.c_uint16, ctypes.c_int
    return {
        "kvqo_half_to_float": (F32, [U16]),
        "kvqo_e4m3_decode": (F64, [U8]),
        "kvqo_e4m3_encode": (U8, [F32]),
        "kvqo_e2m1_decode": (F64, [U8]),
        "kvqo_e2m1_encode": (U8, [F32]),
        "kvqo_quantize_row": (INT, [INT, INT, F32, P, INT, P, P]),
        "kvqo_kvarn_rotate_f32": (None, [P]),
        "kvqo_kvarn_tile": (None, [P, I64, INT, P, P, P, P, P, P, P, P]),
        "kvqo_chunk_bytes": (I64, [P]),
        "kvqo_page_bytes": (I64, [P]),
        "kvqo_quantize_write": (INT, [P, P, P, P, I64, P]),
        "kvqo_dequantize": (INT, [P, P, P, I64, P, P]),
        "kvqo_attention_dense": (None, [P, P, P, I64, INT, F64, P]),
        "kvqo_decode_attention": (INT, [P, P, P, I32, P, I32, P, I32, F32, P, P, I32, P]),
    }


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16
    return a


class Oracle:
    """One loaded build of the oracle (the default build, or a test mutant)."""

    def __init__(self, path: str | None = None):
        self.path = path or build()
        self.L = ctypes.CDLL(self.path)
        for name, (res, args) in _sigs().items():
            fn = getattr(self.L, name)
            fn.restype = res
            fn.argtypes = args

    # ---- scalar encoders ----------------------------------------------------
    def half_to_float(self, bits):
        return self.L.kvqo_half_to_float(bits)

    def e4m3_encode(self, y):
        return self.L.kvqo_e4m3_encode(y)

    def e4m3_decode(self, c):
        return self.L.kvqo_e4m3_decode(c)

    def e2m1_encode(self, y):
        return self.L.kvqo_e2m1_encode(y)

    def e2m1_decode(self, c):
        return self.L.kvqo_e2m1_decode(c)

    # ---- rows, tiles, pages -------------------------------------------------
    def quantize_row(self, fmt, x16, scale=1.0, flags=0):
        """(codes uint8[D] unpacked, scale bytes) for one token-head row."""
        x = _u16(x16)
        D = x.shape[0]
        codes = np.zeros(D, np.uint8)
        scales = np.zeros(max(4, D // 16), np.uint8)
        rc = self.L.kvqo_quantize_row(fmt, flags, scale, _ptr(x), D, _ptr(codes), _ptr(scales))
        if rc:
            raise ValueError(f"kvqo_quantize_row rc={rc}")
        return codes, scales

    def kvarn_rotate(self, row):
        y = np.array(row, dtype=np.float32)
        assert y.shape == (128,)
        self.L.kvqo_kvarn_rotate_f32(_ptr(y))
        return y

    def kvarn_tile(self, x16, side):
        """KVarN pipeline on one [128 tokens][128 channels] binary16 tile."""
        x = _u16(x16).reshape(128, 128)
        out = {k: np.zeros((128, 128), np.float32) for k in ("y_rot", "y_norm")}
        for k in ("r", "c", "qs", "qm"):
            out[k] = np.zeros(128, np.float32)
        out["codes"] = np.zeros((128, 128), np.uint8)
        out["meta"] = np.zeros((3, 128), np.float32)
        self.L.kvqo_kvarn_tile(_ptr(x), 128, side, _ptr(out["y_rot"]), _ptr(out["y_norm"]), _ptr(out["r"]),
                               _ptr(out["c"]), _ptr(out["codes"]), _ptr(out["qs"]), _ptr(out["qm"]),
                               _ptr(out["meta"]))
        return out

    def chunk_bytes(self, lay):
        return self.L.kvqo_chunk_bytes(ctypes.byref(lay))

    def page_bytes(self, lay):
        return self.L.kvqo_page_bytes(ctypes.byref(lay))

    def quantize_write(self, lay, k16, v16, slots, cache=None):
        """k16, v16 [n_tok, H, D] binary16; slots int64 [n_tok]; returns the
        uint8 cache (num_pages * page_bytes)."""
        k, v = _u16(k16), _u16(v16)
        s = np.ascontiguousarray(slots, dtype=np.int64)
        if cache is None:
            cache = np.zeros(lay.num_pages * self.page_bytes(lay), np.uint8)
        rc = self.L.kvqo_quantize_write(ctypes.byref(lay), _ptr(k), _ptr(v), _ptr(s), s.shape[0], _ptr(cache))
        if rc:
            raise ValueError(f"kvqo_quantize_write rc={rc}")
        return cache

    def dequantize(self, lay, cache, slots):
        s = np.ascontiguousarray(slots, dtype=np.int64)
        n = s.shape[0]
        k = np.zeros((n, lay.num_kv_heads, lay.head_dim), np.float64)
        v = np.zeros_like(k)
        rc = self.L.kvqo_dequantize(ctypes.byref(lay), _ptr(cache), _ptr(s), n, _ptr(k), _ptr(v))
        if rc:
            raise ValueError(f"kvqo_dequantize rc={rc}")
        return k, v

    def attention_dense(self, q, k, v, scale):
        q = np.ascontiguousarray(q, np.float64)
        k = np.ascontiguousarray(k, np.float64)
        v = np.ascontiguousarray(v, np.float64)
        D = q.shape[-1]
        out = np.zeros(D, np.float64)
        self.L.kvqo_attention_dense(_ptr(q), _ptr(k), _ptr(v), k.shape[0], D, scale, _ptr(out))
        return out

    def decode_attention(self, lay, cache, q16, block_tables, ctx_lens, sm_scale, tail16=None, pairs=None):
        """binary64 outputs [n_pairs, D]; all (b, h) pairs -> [B, Hq, D]."""
        q = _u16(q16)
        B, Hq, D = q.shape
        bt = np.ascontiguousarray(block_tables, np.int32)
        cl = np.ascontiguousarray(ctx_lens, np.int32)
        full = pairs is None
        if full:
            pairs = np.array([(b, h) for b in range(B) for h in range(Hq)], np.int32)
        pairs = np.ascontiguousarray(pairs, np.int32).reshape(-1, 2)
        tail = None if tail16 is None else _u16(tail16)
        out = np.zeros((pairs.shape[0], D), np.float64)
        rc = self.L.kvqo_decode_attention(ctypes.byref(lay), _ptr(cache), _ptr(q), Hq, _ptr(bt), bt.shape[1],
                                          _ptr(cl), B, sm_scale, _ptr(tail), _ptr(pairs), pairs.shape[0], _ptr(out))
        if rc:
            raise ValueError(f"kvqo_decode_attention rc={rc}")
        return out.reshape(B, Hq, D) if full else out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
