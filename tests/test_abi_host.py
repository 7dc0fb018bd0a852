"""C-ABI checks that need no GPU: the library loads, exports every symbol the
public header declares, sizes pages exactly as the oracle does, and rejects
invalid requests before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(K):
    syms = declared_symbols()
    assert len(syms) >= 8
    lib = ctypes.CDLL(K.LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), f"{s} declared in include/kvq.h but not exported"


def _layouts():
    for fmt in (1, 2, 3, 4, 6, 7):
        for D in (32, 64, 128):
            for P in (16, 32, 64, 128, 256):
                yield fmt, 0, 3, D, P
    yield 4, 1, 8, 128, 16
    yield 5, 0, 8, 128, 128
    yield 5, 0, 8, 128, 256


@pytest.mark.parametrize("fmt,flags,H,D,P", list(_layouts()))
def test_page_bytes_match_oracle(K, fmt, flags, H, D, P):
    lay = K.layout(fmt, H, D, P, 10, 0.5, 0.25, flags)
    olay = oracle.layout(fmt, H, D, P, 10, 0.5, 0.25, flags)
    assert K.kvq_page_bytes(lay) == oracle.default().page_bytes(olay) > 0


@pytest.mark.parametrize("bad", [
    dict(fmt=0), dict(fmt=8), dict(fmt=7, flags=1), dict(D=96), dict(D=256), dict(P=8), dict(P=24), dict(P=48), dict(P=512), dict(H=0),
    dict(pages=0), dict(fmt=5, P=16), dict(fmt=5, P=64), dict(fmt=5, D=64), dict(flags=1), dict(flags=2, fmt=4),
    dict(fmt=1, ks=0.0), dict(fmt=1, ks=float("inf")), dict(fmt=4, vs=-1.0), dict(fmt=4, vs=1e-30),
])
def test_invalid_layouts_rejected(K, bad):
    a = dict(fmt=2, H=4, D=128, P=16, pages=4, ks=1.0, vs=1.0, flags=0)
    a.update(bad)
    lay = K.layout(a["fmt"], a["H"], a["D"], a["P"], a["pages"], a["ks"], a["vs"], a["flags"])
    assert K.kvq_page_bytes(lay) == -1
    assert K.kvq_decode_workspace_bytes(lay, 2, 4, 4) == -1
    st = K.lib.kvq_quantize_write(ctypes.byref(lay), None, None, None, 0, None, None)
    assert st in (1, 2)


def test_argument_errors_before_launch(K):
    lay = K.layout(2, 4, 128, 16, 4)
    L = K.lib
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    assert L.kvq_quantize_write(None, p, p, p, 1, p, None) == 1
    assert L.kvq_quantize_write(ctypes.byref(lay), p, p, p, -1, p, None) == 1
    assert L.kvq_quantize_write(ctypes.byref(lay), None, p, p, 1, p, None) == 1
    klay = K.layout(5, 4, 128, 128, 4)
    assert L.kvq_quantize_write(ctypes.byref(klay), p, p, p, 100, p, None) == 1  # not whole tiles
    # decode: GQA group must divide and be <= 8
    ws = K.kvq_decode_workspace_bytes(lay, 2, 8, 4)
    assert L.kvq_decode_attention(ctypes.byref(lay), p, p, 6, p, 4, p, 2, 0.1, None, p, p, ws, 0, None) == 1
    assert L.kvq_decode_attention(ctypes.byref(lay), p, p, 64, p, 4, p, 2, 0.1, None, p, p, 1 << 30, 0, None) == 2
    assert L.kvq_decode_attention(ctypes.byref(lay), p, p, 8, p, 4, p, 2, 0.1, p, p, p, ws, 0, None) == 1  # tail
    assert L.kvq_decode_attention(ctypes.byref(lay), p, p, 8, p, 4, p, 2, 0.1, None, p, p, ws - 1, 0, None) == 3
    assert L.kvq_decode_attention(ctypes.byref(lay), p, p, 8, p, 4, p, 2, float("nan"), None, p, p, ws, 0, None) == 1
    # one-call decode step: not for KVarN, the new rows are required, then the decode's own checks
    big = 1 << 30
    assert L.kvq_decode_attention_append(ctypes.byref(klay), p, p, p, p, p, 8, p, 4, p, 2, 0.1, p, p, big, 0,
                                         None) == 1
    assert L.kvq_decode_attention_append(ctypes.byref(lay), p, None, p, p, p, 8, p, 4, p, 2, 0.1, p, p, ws, 0,
                                         None) == 1
    assert L.kvq_decode_attention_append(ctypes.byref(lay), p, p, p, None, p, 8, p, 4, p, 2, 0.1, p, p, ws, 0,
                                         None) == 1
    assert L.kvq_decode_attention_append(ctypes.byref(lay), p, p, p, p, p, 64, p, 4, p, 2, 0.1, p, p, big, 0,
                                         None) == 2
    assert L.kvq_decode_attention_append(ctypes.byref(lay), p, p, p, p, p, 8, p, 4, p, 2, 0.1, p, p, ws - 1, 0,
                                         None) == 3
    assert L.kvq_dequantize(ctypes.byref(lay), None, p, 1, p, p, None) == 1
    # allocation-free decode: the decode's checks, then the fixed workspace's size
    assert L.kvq_decode_attention_noalloc(ctypes.byref(lay), p, p, 6, p, 4, p, 2, 0.1, None, p, 0, None) == 1
    assert L.kvq_decode_attention_noalloc(ctypes.byref(lay), p, p, 64, p, 4, p, 2, 0.1, None, p, 0, None) == 2
    assert L.kvq_decode_attention_noalloc(ctypes.byref(lay), p, p, 8, p, 4, p, 2, 0.1, p, p, 0, None) == 1
    assert L.kvq_decode_attention_noalloc(ctypes.byref(lay), None, p, 8, p, 4, p, 2, 0.1, None, p, 0, None) == 1
    rec = (2 * 8 + 8 * 128) * 4
    fits = K.KVQ_DECODE_SCRATCH_BYTES // rec  # records the fixed workspace holds
    assert fits == 4032
    # KVarN always keeps one record per (sequence, kv head): batch * 4 records at one split
    big_b = fits // 4 + 1
    assert L.kvq_decode_attention_noalloc(ctypes.byref(klay), p, p, 32, p, 4, p, big_b, 0.1, None, p, 1,
                                          None) == 6
    assert K.kvq_decode_workspace_bytes(klay, big_b, 32, 4, 1) > K.KVQ_DECODE_SCRATCH_BYTES
    assert K.kvq_decode_workspace_bytes(klay, big_b - 1, 32, 4, 1) <= K.KVQ_DECODE_SCRATCH_BYTES
    assert L.kvq_decode_attention_noalloc(ctypes.byref(lay), p, p, 8, p, 4000, p, 16, 0.1, None, p, 256,
                                          None) == 6


def test_misaligned_pointers_rejected(K):
    """Every entry point rejects a data pointer off its 16-byte alignment (or
    an index array off its own size) with KVQ_ERR_INVALID_ARG before it
    looks for a device."""
    L = K.lib
    lay = K.layout(2, 8, 128, 16, 64)
    klay = K.layout(5, 8, 128, 128, 8)
    a = 1 << 20              # aligned stand-in address (never dereferenced)
    P = lambda x: ctypes.c_void_p(x)
    for off in (2, 8):
        m = a + off          # binary16 data off 16 bytes
        assert L.kvq_quantize_write(ctypes.byref(lay), P(m), P(a), P(a), 16, P(a), None) == 1
        assert L.kvq_quantize_write(ctypes.byref(lay), P(a), P(a), P(a), 16, P(m), None) == 1
        assert L.kvq_decode_attention(ctypes.byref(lay), P(a), P(m), 64, P(a), 4, P(a), 2, 0.1, None, P(a),
                                      None, 0, 1, None) == 1
        assert L.kvq_decode_attention(ctypes.byref(lay), P(a), P(a), 64, P(a), 4, P(a), 2, 0.1, None, P(m),
                                      None, 0, 1, None) == 1
        assert L.kvq_decode_attention_noalloc(ctypes.byref(lay), P(m), P(a), 64, P(a), 4, P(a), 2, 0.1, None,
                                              P(a), 1, None) == 1
        assert L.kvq_decode_attention_append(ctypes.byref(lay), P(a), P(m), P(a), P(a), P(a), 64, P(a), 4, P(a),
                                             2, 0.1, P(a), None, 0, 1, None) == 1
        assert L.kvq_kvarn_append(ctypes.byref(klay), P(a), P(a), P(a), P(a), 2, P(m), 2, P(a), 4, P(a), None) == 1
        assert L.kvq_dequantize(ctypes.byref(lay), P(m), P(a), 16, P(a), P(a), None) == 1
    # index arrays off their own size, a workspace off 16 bytes, a misaligned KVarN tail
    assert L.kvq_quantize_write(ctypes.byref(lay), P(a), P(a), P(a + 4), 16, P(a), None) == 1
    assert L.kvq_decode_attention(ctypes.byref(lay), P(a), P(a), 64, P(a + 2), 4, P(a), 2, 0.1, None, P(a),
                                  None, 0, 1, None) == 1
    assert L.kvq_decode_attention(ctypes.byref(lay), P(a), P(a), 64, P(a), 4, P(a), 2, 0.1, None, P(a),
                                  P(a + 4), 1 << 20, 4, None) == 1
    assert L.kvq_decode_attention(ctypes.byref(klay), P(a), P(a), 64, P(a), 4, P(a), 2, 0.1, P(a + 8), P(a),
                                  P(a), 1 << 20, 1, None) == 1
    assert L.kvq_dequantize(ctypes.byref(lay), P(a), P(a), 16, P(a + 2), P(a), None) == 1
    # the same calls with aligned pointers get past these checks (no device here: KVQ_ERR_DEVICE)
    import torch
    if not torch.cuda.is_available():
        assert L.kvq_quantize_write(ctypes.byref(lay), P(a), P(a), P(a), 16, P(a), None) == 4
        assert L.kvq_dequantize(ctypes.byref(lay), P(a), P(a), 16, P(a), P(a), None) == 4


def test_split_plan_and_workspace(K):
    import torch
    if torch.cuda.is_available():
        pytest.skip("the automatic plan follows the device; covered by the GPU tests")
    lay = K.layout(2, 8, 128, 16, 16384)
    # no device: 256 compute units x 2 workgroups, one resident round of 512
    assert K.kvq_decode_num_splits(lay, 8, 64, 2048) == 8
    assert K.kvq_decode_num_splits(lay, 16, 64, 256) == 4
    # a (sequence, kv head) per compute unit: one split of eight-wave workgroups
    assert K.kvq_decode_num_splits(lay, 32, 64, 256) == 1
    assert K.kvq_decode_workspace_bytes(lay, 32, 64, 256) == 0
    assert K.kvq_decode_num_splits(lay, 32, 64, 256, 2) == 2  # an explicit count is kept
    assert K.kvq_decode_num_splits(lay, 2, 64, 1) == 1
    assert K.kvq_decode_num_splits(lay, 2, 64, 10, 3) == 3
    assert K.kvq_decode_num_splits(lay, 2, 64, 9, 4) == 3  # empty trailing split dropped
    assert K.kvq_decode_num_splits(lay, 2, 60, 9, 4) == -1  # q heads not a multiple of kv heads
    assert K.kvq_decode_workspace_bytes(lay, 2, 60, 9, 4) == -1
    assert K.kvq_decode_workspace_bytes(lay, 8, 64, 2048, 1) == 0
    for splits in (3, 16):
        b = K.kvq_decode_workspace_bytes(lay, 8, 64, 2048, splits)
        rec = (2 * 8 + 8 * 128) * 4
        assert b == 8 * 8 * splits * rec
    # KVarN always merges (binary16 tail, rotation back): a record even for one split
    klay = K.layout(5, 8, 128, 128, 2048)
    assert K.kvq_decode_workspace_bytes(klay, 16, 64, 128, 1) == 16 * 8 * 1 * (2 * 8 + 8 * 128) * 4
    assert K.kvq_decode_num_splits(klay, 16, 64, 128) == 4


def test_status_strings(K):
    for st in range(7):
        assert K.kvq_status_string(st)
    assert "KVQ_DECODE_SCRATCH_BYTES" in K.kvq_status_string(6)
    assert "gfx950" in K.kvq_status_string(4)


def test_device_check_without_gpu(K):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    assert K.kvq_check_device(0) == 4
    # the device-error query checks its pointer first, then the device
    assert K.lib.kvq_take_device_errors(None, None) == 1
    flags = ctypes.c_uint32(7)
    assert K.lib.kvq_take_device_errors(ctypes.byref(flags), None) == 4
    assert flags.value == 7  # untouched


def test_single_hip_runtime_in_process(K):
    """The binding loads libkvq.so against the HIP runtime torch already
    carries: exactly one libamdhip64 is mapped."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(line.split()[-1])
    assert len(paths) == 1, paths
