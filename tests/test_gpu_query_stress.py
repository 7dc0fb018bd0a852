"""Decode parity with queries that stress the key path.  [P1] §1.1 notes that
a key's quantisation error reaches the score multiplied by the query's norm,
so besides zero-mean queries the kernels must hold the tolerance for
non-centred queries (mean 4, 16, 64), queries with a few channels x100 and
wide ones (N(0, 8)), over keys with x10 outlier channels as in the 32K
workload.  Every format, against the binary64 oracle: the contract's bound,
the 0.5 ulp + 1e-4 bound of the other parity tests, and a flat 2e-3 wherever
the binary16 output can hold it (|o| <= 4)."""
import math

import numpy as np
import pytest

import workloads
from gpu_util import (assert_attn_close, assert_flat_where_representable, dev, gpu_decode, log, olayout,
                      paged_problem)
from test_gpu_kvarn import kvarn_problem
from test_gpu_parity import FMT_IDS, FORMATS, layout_for

pytestmark = pytest.mark.gpu

QUERY_KINDS = ["mean4", "mean16", "mean64", "spikes100", "wide8"]


def stress_queries(rng, shape, kind):
    q = rng.standard_normal(shape)
    if kind.startswith("mean"):
        q += float(kind[4:])
    elif kind == "spikes100":
        D = shape[-1]
        for idx in np.ndindex(shape[:-1]):
            q[idx + (rng.choice(D, 3, replace=False),)] *= 100.0
    elif kind == "wide8":
        q *= 8.0
    return q.astype(np.float16)


def outlier_rows(rng, n, H, D, scale=10.0):
    """N(0, 1) rows with 10 of the H*D channels scaled (the 32K workload's
    recipe), drawn separately for each call."""
    x = workloads.random_halves(rng, (n, H, D))
    cols = rng.choice(H * D, 10, replace=False)
    for c in cols:
        x[:, c // D, c % D] *= np.float16(scale)
    return x


def tight_bound(got, ref, what):
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    bad = np.abs(got - ref) > 0.5 * ulp + 1e-4 + 1e-4 * np.abs(ref)
    assert not np.any(bad), f"{what}: {bad.sum()} outputs beyond 0.5 ulp + 1e-4; max err {np.abs(got - ref).max():.3e}"


@pytest.mark.parametrize("kind", QUERY_KINDS)
@pytest.mark.parametrize("fmt,flags", FORMATS, ids=FMT_IDS)
def test_decode_stress_queries(K, O, fmt, flags, kind):
    rng = np.random.default_rng(9000 + 37 * fmt + flags + 101 * QUERY_KINDS.index(kind))
    B, H, G, D, P = 3, 2, 8, 128, 16
    ctx = np.array([300, 1000, 77], np.int32)
    bt, num_pages, slots = paged_problem(rng, B, H, G, D, P, ctx)
    n = slots.shape[0]
    k16 = outlier_rows(rng, n, H, D)
    v16 = outlier_rows(rng, n, H, D)
    lay = layout_for(K, fmt, flags, H, D, P, num_pages, k16, v16)
    cache = O.quantize_write(olayout(lay), k16, v16, slots)
    q16 = stress_queries(rng, (B, H * G, D), kind)
    sm = 1.0 / math.sqrt(D)
    ref = O.decode_attention(olayout(lay), cache, q16, bt, ctx, sm)
    cache_dev = dev(cache)
    for splits in (0, 1, 3):
        what = f"fmt={fmt} flags={flags} q={kind} splits={splits}"
        log(f"stress decode {what}")
        got, _ = gpu_decode(K, lay, cache_dev, q16, bt, ctx, sm, num_splits=splits)
        assert_attn_close(got, ref, what)
        tight_bound(got, ref, what)
        assert_flat_where_representable(got, ref, what)


@pytest.mark.parametrize("kind", QUERY_KINDS)
def test_kvarn_decode_stress_queries(K, O, kind):
    rng = np.random.default_rng(9500 + QUERY_KINDS.index(kind))
    B, H, G, D = 2, 2, 8, 128
    ctx = np.array([128 * 5 + 37, 128 * 3], np.int32)
    bt, num_pages, slots, kfull, vfull, tail = kvarn_problem(rng, B, H, ctx)
    lay = K.layout(5, H, D, 128, num_pages)
    cache = O.quantize_write(olayout(lay), kfull, vfull, slots)
    q16 = stress_queries(rng, (B, H * G, D), kind)
    sm = 1.0 / math.sqrt(D)
    ref = O.decode_attention(olayout(lay), cache, q16, bt, ctx, sm, tail16=tail)
    for splits in (0, 1, 2):
        what = f"kvarn q={kind} splits={splits}"
        log(f"stress decode {what}")
        got, _ = gpu_decode(K, lay, dev(cache), q16, bt, ctx, sm, tail16=tail, num_splits=splits)
        assert_attn_close(got, ref, what)
        tight_bound(got, ref, what)
        assert_flat_where_representable(got, ref, what)
