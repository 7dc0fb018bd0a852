"""Helpers shared by the GPU tests: move seeded host arrays to the device, run
the library through its binding, and compare with the oracle."""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def olayout(lay):
    return oracle.layout(lay.format, lay.num_kv_heads, lay.head_dim, lay.page_size, lay.num_pages, lay.k_scale,
                         lay.v_scale, lay.flags)


def gpu_write(K, lay, k16, v16, slots, cache=None):
    import torch
    if cache is None:
        cache = torch.zeros(lay.num_pages * K.kvq_page_bytes(lay), dtype=torch.uint8, device="cuda")
    K.kvq_quantize_write(lay, dev(k16), dev(v16), dev(np.asarray(slots, np.int64)), cache)
    torch.cuda.synchronize()
    return cache


def gpu_decode(K, lay, cache_dev, q16, bt, ctx, sm_scale, tail16=None, num_splits=0):
    import torch
    B, Hq, D = q16.shape
    ws = K.DecodeWorkspace(lay, B, Hq, bt.shape[1], num_splits)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
    K.kvq_decode_attention(lay, cache_dev, dev(q16), dev(np.asarray(bt, np.int32)), dev(np.asarray(ctx, np.int32)),
                           sm_scale, out, ws.buffer, None if tail16 is None else dev(tail16), num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), ws


def attn_tolerance(ref):
    """2e-3 absolute, widened by 2^-10 |o| where binary16 output rounding alone
    exceeds it (|o| > 8)."""
    return 2e-3 + 2.0 ** -10 * np.abs(ref)


def assert_attn_close(got, ref, what=""):
    tol = attn_tolerance(ref)
    err = np.abs(got - ref)
    bad = err > tol
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if np.any(bad):
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} outputs beyond tolerance; first at {tuple(i)}: "
                             f"got {got[tuple(i)]}, ref {ref[tuple(i)]}, max err {err.max():.3e}")
    return float(err.max())


def assert_flat_where_representable(got, ref, what="", bound=2e-3):
    """A flat 2e-3 on every output whose binary16 rounding alone stays well
    inside it (|o_ref| <= 4, half an ulp <= 2^-10): there the contract's flat
    bound holds without the 2^-10 |o| widening."""
    small = np.abs(ref) <= 4.0
    err = np.abs(got - ref)[small]
    assert not np.any(err > bound), f"{what}: max err {err.max():.3e} beyond a flat {bound} at |o| <= 4"
    return float(err.max()) if err.size else 0.0


def first_mismatch(a, b):
    d = np.nonzero(a != b)[0]
    return None if d.size == 0 else (int(d[0]), int(a[d[0]]), int(b[d[0]]), int(d.size))


def paged_problem(rng, B, H, G, D, P, ctx, extra_pages=2):
    """Random block tables (a shuffled pool) and the slot of every cached token,
    sequence-major."""
    ctx = np.asarray(ctx, np.int32)
    max_pages = max(1, int(math.ceil(int(ctx.max()) / P)))
    num_pages = B * max_pages + extra_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = perm[:B * max_pages].reshape(B, max_pages)
    slots = []
    for b in range(B):
        t = np.arange(int(ctx[b]))
        slots.append(bt[b, t // P].astype(np.int64) * P + t % P)
    slots = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    return bt, num_pages, slots
