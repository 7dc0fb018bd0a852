"""kvq_decode_attention_noalloc (the decode with the library's fixed device
workspace) against kvq_decode_attention with a caller's workspace, through the
C ABI: the same outputs bit for bit, on two calls in a row, the second with a
smaller problem (the array keeps the first call's records, which must not
matter), for a split format, a single-split plan, KVarN with a tail and a
plan that fills most of the array; and both against the oracle."""
import ctypes
import math

import numpy as np
import pytest

import workloads
from gpu_util import assert_attn_close, dev, gpu_decode, log, olayout, paged_problem
from test_gpu_kvarn import kvarn_problem
from test_gpu_parity import layout_for

pytestmark = pytest.mark.gpu


def noalloc(K, lay, cache_dev, q16, bt, ctx, sm, tail16=None, num_splits=0):
    import torch
    B, Hq, D = q16.shape
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float16, device="cuda")
    K.kvq_decode_attention_noalloc(lay, cache_dev, dev(q16), dev(np.asarray(bt, np.int32)),
                                   dev(np.asarray(ctx, np.int32)), sm, out,
                                   None if tail16 is None else dev(tail16), num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def problem(K, O, rng, fmt, B, ctx, G=8, H=2, D=128, P=16):
    ctx = np.asarray(ctx, np.int32)
    bt, num_pages, slots = paged_problem(rng, B, H, G, D, P, ctx)
    k16 = workloads.random_halves(rng, (slots.size, H, D))
    v16 = workloads.random_halves(rng, (slots.size, H, D))
    lay = layout_for(K, fmt, 0, H, D, P, num_pages, k16, v16)
    cache = O.quantize_write(olayout(lay), k16, v16, slots)
    q16 = workloads.random_halves(rng, (B, H * G, D))
    return lay, cache, q16, bt, ctx


@pytest.mark.parametrize("fmt,splits", [(2, 0), (4, 5), (1, 1), (6, 0)])
def test_noalloc_matches_workspace_decode(K, O, fmt, splits):
    rng = np.random.default_rng(7100 + 10 * fmt + splits)
    sm = 1.0 / math.sqrt(128)
    # a larger call, then a smaller one on the same (now dirty) array
    for B, ctx in ((4, [3000, 17, 1200, 640]), (2, [33, 500])):
        lay, cache, q16, bt, ctx = problem(K, O, rng, fmt, B, ctx)
        cdev = dev(cache)
        log(f"noalloc fmt={fmt} B={B} splits={splits}")
        ref_ws, ws = gpu_decode(K, lay, cdev, q16, bt, ctx, sm, num_splits=splits)
        got = noalloc(K, lay, cdev, q16, bt, ctx, sm, num_splits=splits)
        assert np.array_equal(got, ref_ws), f"B={B}: max diff {np.abs(got - ref_ws).max():.3e}"
        assert_attn_close(got, O.decode_attention(olayout(lay), cache, q16, bt, ctx, sm), f"B={B}")
        log(f"  {ws.num_splits} splits, {ws.buffer.numel()} workspace bytes: equal")


def test_noalloc_kvarn_with_tail(K, O):
    rng = np.random.default_rng(7200)
    sm = 1.0 / math.sqrt(128)
    for B, ctx in ((3, [128 * 9 + 5, 128 * 4, 300]), (1, [128 * 2 + 127])):
        bt, num_pages, slots, kfull, vfull, tail = kvarn_problem(rng, B, 2, ctx)
        lay = K.layout(5, 2, 128, 128, num_pages)
        cache = O.quantize_write(olayout(lay), kfull, vfull, slots)
        q16 = workloads.random_halves(rng, (B, 16, 128))
        cdev = dev(cache)
        log(f"noalloc kvarn B={B}")
        ref_ws, _ = gpu_decode(K, lay, cdev, q16, bt, ctx, sm, tail16=tail)
        got = noalloc(K, lay, cdev, q16, bt, ctx, sm, tail16=tail)
        assert np.array_equal(got, ref_ws)
        assert_attn_close(got, O.decode_attention(olayout(lay), cache, q16, bt, ctx, sm, tail16=tail))


def test_noalloc_near_the_limit_and_beyond(K, O):
    """A plan whose records fill most of the fixed array (4032 records of
    4160 bytes at head size 128), then one that needs more: refused before
    any launch, and the next call still correct."""
    import torch
    rng = np.random.default_rng(7300)
    sm = 1.0 / math.sqrt(128)
    rec = (2 * 8 + 8 * 128) * 4
    B, H, splits = 16, 2, 120  # 3840 records, 15.97 MB
    ctx = np.full(B, 16 * 240, np.int32)
    lay, cache, q16, bt, ctx = problem(K, O, rng, 2, B, ctx, H=H)
    assert K.kvq_decode_workspace_bytes(lay, B, H * 8, bt.shape[1], splits) == B * H * splits * rec
    assert B * H * splits * rec <= K.KVQ_DECODE_SCRATCH_BYTES
    cdev = dev(cache)
    log("noalloc near the limit")
    ref_ws, ws = gpu_decode(K, lay, cdev, q16, bt, ctx, sm, num_splits=splits)
    assert ws.num_splits == splits
    got = noalloc(K, lay, cdev, q16, bt, ctx, sm, num_splits=splits)
    assert np.array_equal(got, ref_ws)
    # 16 * 2 * 240 records do not fit: refused with its own status, nothing launched
    assert K.kvq_decode_workspace_bytes(lay, B, H * 8, bt.shape[1], 240) > K.KVQ_DECODE_SCRATCH_BYTES
    out = torch.zeros((B, H * 8, 128), dtype=torch.float16, device="cuda")
    qd, btd, ctxd = dev(q16), dev(bt), dev(ctx)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = K.lib.kvq_decode_attention_noalloc(ctypes.byref(lay), ptr(cdev), ptr(qd), H * 8, ptr(btd), bt.shape[1],
                                            ptr(ctxd), B, sm, None, ptr(out), 240, None)
    torch.cuda.synchronize()
    assert st == 6
    assert not torch.any(out)
    got = noalloc(K, lay, cdev, q16[:3], bt[:3], ctx[:3], sm, num_splits=7)
    ref_ws, _ = gpu_decode(K, lay, cdev, q16[:3], bt[:3], ctx[:3], sm, num_splits=7)
    assert np.array_equal(got, ref_ws)
