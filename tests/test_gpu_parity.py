"""GPU path vs the oracle through the C ABI: bit-exact cache bytes (codes and
scales), bit-exact dequantisation, and decode attention within
|o - o_ref| <= 2e-3 + 2^-10 |o_ref| of the binary64 oracle on the same cache."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (assert_attn_close, dev, first_mismatch, gpu_decode, gpu_write, log, olayout,
                      paged_problem)

pytestmark = pytest.mark.gpu

FORMATS = [(1, 0), (2, 0), (3, 0), (4, 0), (4, 1), (6, 0), (7, 0)]
FMT_IDS = ["fp8pt", "int8pth", "fp8pth", "nvfp4", "nvfp4_4over6", "int4pth", "mxfp4"]


def edge_rows(rng, n, H, D):
    """Token rows with the cases the formats must handle: plain normal data,
    an attention-sink token (x20), zero rows, single outliers, tiny and huge
    magnitudes, binary16 subnormals, exact E4M3 / E2M1 boundary values."""
    x = workloads.random_halves(rng, (n, H, D))
    x[0] *= np.float16(20)
    if n > 3:
        x[1] = 0
        x[2, :, 5] = np.float16(3000.0)
        x[3] = (rng.standard_normal((H, D)) * 1e-5).astype(np.float16)
    if n > 6:
        x[4] = np.float16(-0.0)
        x[5] = (np.arange(H * D).reshape(H, D) % 7 - 3).astype(np.float16) * np.float16(2.0 ** -24)
        x[6] = rng.uniform(-60000, 60000, (H, D)).astype(np.float16)
    if n > 8:
        grid = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 448, 464], np.float16)
        x[7] = rng.choice(grid, (H, D)) * rng.choice(np.float16([-1, 1]), (H, D))
        x[8] = np.float16(-2.5)
    return x


def layout_for(K, fmt, flags, H, D, P, num_pages, k16=None, v16=None, saturate=False):
    ks = vs = 1.0
    if fmt in (1, 4) and k16 is not None:
        top = 448.0 if fmt == 1 else 2688.0
        if saturate:
            top *= 1.5  # push some values beyond the representable range
        ks = float(np.float32(np.abs(k16).max()) / np.float32(top)) or 1.0
        vs = float(np.float32(np.abs(v16).max()) / np.float32(top)) or 1.0
    return K.layout(fmt, H, D, P, num_pages, ks, vs, flags)


@pytest.mark.parametrize("fmt,flags", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("D,P", [(128, 16), (64, 32), (32, 16), (128, 64)])
def test_write_bytes_match_oracle(K, O, fmt, flags, D, P):
    rng = np.random.default_rng(1000 * fmt + 10 * D + P + flags)
    H, num_pages, n = 3, 7, 70
    pool = num_pages * P
    slots = rng.choice(pool, n, replace=False).astype(np.int64)
    slots[10] = -1
    slots[11] = pool + 5  # past the pool: skipped
    k16 = edge_rows(rng, n, H, D)
    v16 = edge_rows(rng, n, H, D)
    for saturate in (False, True) if fmt in (1, 4) else (False,):
        lay = layout_for(K, fmt, flags, H, D, P, num_pages, k16, v16, saturate)
        log(f"write fmt={fmt} flags={flags} D={D} P={P} sat={saturate}")
        ref = O.quantize_write(olayout(lay), k16, v16, slots)
        got = gpu_write(K, lay, k16, v16, slots).cpu().numpy()
        mm = first_mismatch(got, ref)
        assert mm is None, f"cache byte {mm[0]}: gpu {mm[1]:#x} oracle {mm[2]:#x} ({mm[3]} bytes differ)"


def run_slots(rng, P, num_pages, n_runs):
    """Slot mappings as a prefill writes them: runs of consecutive slots that
    fill pages in order (aligned 16-token groups), plus runs that start
    mid-group, a group with two tokens swapped, a skipped slot and ragged
    run ends.  Every slot is written at most once."""
    pages = rng.permutation(num_pages)
    slots = []
    for r in range(n_runs):
        pg = int(pages[r])
        start = 0 if r % 3 else 5  # every third run starts off a 16-token group
        n = P - start if r % 4 else P // 2 + 3
        slots.append(pg * P + start + np.arange(n))
    s = np.concatenate(slots).astype(np.int64)
    s[[36, 37]] = s[[37, 36]]  # two tokens swapped: a group out of order
    s[40] = -1                  # skipped
    return s


@pytest.mark.parametrize("fmt,flags", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("D,P", [(128, 16), (64, 32), (32, 64), (128, 128)])
def test_write_runs_match_oracle(K, O, fmt, flags, D, P):
    """Prefill-style slot runs (the coalesced group path) and the breaks in
    them (the per-row path) give the oracle's bytes."""
    rng = np.random.default_rng(3000 + 100 * fmt + D + P + flags)
    H, num_pages = 3, 9
    slots = run_slots(rng, P, num_pages, 7)
    n = slots.size
    k16 = edge_rows(rng, n, H, D)
    v16 = edge_rows(rng, n, H, D)
    lay = layout_for(K, fmt, flags, H, D, P, num_pages, k16, v16)
    log(f"write runs fmt={fmt} flags={flags} D={D} P={P} n={n}")
    ref = O.quantize_write(olayout(lay), k16, v16, slots)
    got = gpu_write(K, lay, k16, v16, slots).cpu().numpy()
    mm = first_mismatch(got, ref)
    assert mm is None, f"cache byte {mm[0]}: gpu {mm[1]:#x} oracle {mm[2]:#x} ({mm[3]} bytes differ)"


@pytest.mark.parametrize("fmt,flags", FORMATS, ids=FMT_IDS)
def test_dequantize_matches_oracle(K, O, fmt, flags):
    import torch
    rng = np.random.default_rng(77 + fmt + flags)
    H, D, P, num_pages, n = 2, 128, 16, 6, 90
    slots = rng.choice(num_pages * P, n, replace=False).astype(np.int64)
    k16 = edge_rows(rng, n, H, D)
    v16 = edge_rows(rng, n, H, D)
    lay = layout_for(K, fmt, flags, H, D, P, num_pages, k16, v16)
    cache_ref = O.quantize_write(olayout(lay), k16, v16, slots)
    kr, vr = O.dequantize(olayout(lay), cache_ref, slots)
    kout = torch.full((n, H, D), 7.0, dtype=torch.float32, device="cuda")
    vout = torch.full((n, H, D), 7.0, dtype=torch.float32, device="cuda")
    K.kvq_dequantize(lay, dev(cache_ref), dev(slots), kout, vout)
    torch.cuda.synchronize()
    # one binary32 rounding of the exact binary64 value
    assert np.array_equal(kout.cpu().numpy(), kr.astype(np.float32))
    assert np.array_equal(vout.cpu().numpy(), vr.astype(np.float32))


DECODE_CASES = []
for fmt, flags in FORMATS:
    for G in (1, 2, 4, 8):
        for D, P in ((128, 16), (64, 32), (32, 16)):
            DECODE_CASES.append((fmt, flags, G, D, P))


@pytest.mark.parametrize("fmt,flags,G,D,P", DECODE_CASES)
def test_decode_matches_oracle(K, O, fmt, flags, G, D, P):
    rng = np.random.default_rng(fmt * 131 + flags * 7 + G * 17 + D + P)
    B, H = 5, 2
    ctx = np.array([0, 1, 17, 2 * P - 1, 9 * P + 3], np.int32)
    bt, num_pages, slots = paged_problem(rng, B, H, G, D, P, ctx)
    n = slots.shape[0]
    k16 = workloads.random_halves(rng, (n, H, D))
    v16 = workloads.random_halves(rng, (n, H, D))
    k16[int(ctx[:4].sum())] *= np.float16(20)  # a sink in the last sequence
    v16[int(ctx[:4].sum())] *= np.float16(20)
    lay = layout_for(K, fmt, flags, H, D, P, num_pages, k16, v16)
    cache = O.quantize_write(olayout(lay), k16, v16, slots)
    q16 = workloads.random_halves(rng, (B, H * G, D))
    sm = 1.0 / math.sqrt(D)
    ref = O.decode_attention(olayout(lay), cache, q16, bt, ctx, sm)
    cache_dev = dev(cache)
    for splits in (0, 1, 3, 7):
        log(f"decode fmt={fmt} flags={flags} G={G} D={D} P={P} splits={splits}")
        got, _ = gpu_decode(K, lay, cache_dev, q16, bt, ctx, sm, num_splits=splits)
        assert_attn_close(got, ref, f"splits={splits}")
        # beyond the contract: apart from the final binary16 rounding the
        # result tracks the binary64 oracle to ~1e-4
        ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(got - ref) <= 0.5 * ulp + 1e-4 + 1e-4 * np.abs(ref))
    assert not np.any(got[0]), "empty context must give a zero row"


@pytest.mark.parametrize("fmt,flags", FORMATS, ids=FMT_IDS)
def test_decode_closed_forms(K, O, fmt, flags):
    """ctx = 1 gives the token's value; identical keys give the mean value."""
    import torch
    rng = np.random.default_rng(5 + fmt + flags)
    H, G, D, P = 1, 4, 128, 16
    T = 48
    bt = np.array([[2, 0, 1]], np.int32)
    slots = bt[0, np.arange(T) // P].astype(np.int64) * P + np.arange(T) % P
    k16 = np.repeat(workloads.random_halves(rng, (1, H, D)), T, axis=0)
    v16 = workloads.random_halves(rng, (T, H, D))
    lay = layout_for(K, fmt, flags, H, D, P, 3, k16, v16)
    cache = O.quantize_write(olayout(lay), k16, v16, slots)
    _, vh = O.dequantize(olayout(lay), cache, slots)
    q16 = workloads.random_halves(rng, (1, G, D))
    got, _ = gpu_decode(K, lay, dev(cache), q16, bt, [T], 0.3)
    for h in range(G):
        assert_attn_close(got[0, h], vh[:, 0].mean(axis=0), "identical keys")
    got, _ = gpu_decode(K, lay, dev(cache), q16, bt, [1], 0.3)
    for h in range(G):
        assert_attn_close(got[0, h], vh[0, 0], "one token")


def test_decode_invalid_pages(K, O):
    """Block-table entries outside the pool are skipped without faulting."""
    rng = np.random.default_rng(9)
    B, H, G, D, P = 2, 2, 4, 128, 16
    ctx = np.array([64, 64], np.int32)
    bt, num_pages, slots = paged_problem(rng, B, H, G, D, P, ctx)
    k16 = workloads.random_halves(rng, (slots.size, H, D))
    v16 = workloads.random_halves(rng, (slots.size, H, D))
    lay = K.layout(2, H, D, P, num_pages)
    cache = O.quantize_write(olayout(lay), k16, v16, slots)
    bad = bt.copy()
    bad[0, 1] = -5
    bad[1, 2] = num_pages + 100
    got, _ = gpu_decode(K, lay, dev(cache), workloads.random_halves(rng, (B, H * G, D)), bad, ctx, 0.1,
                        num_splits=2)
    assert np.all(np.isfinite(got))


def test_workspace_reuse_many_calls(K, O):
    """Repeated calls on one workspace, with different batch sizes and split
    counts, stay correct (the workspace carries nothing between calls)."""
    import torch
    rng = np.random.default_rng(21)
    H, G, D, P = 2, 8, 128, 16
    ctx = np.array([200, 31, 500, 64], np.int32)
    bt, num_pages, slots = paged_problem(rng, 4, H, G, D, P, ctx)
    k16 = workloads.random_halves(rng, (slots.size, H, D))
    v16 = workloads.random_halves(rng, (slots.size, H, D))
    lay = K.layout(3, H, D, P, num_pages)
    cache = O.quantize_write(olayout(lay), k16, v16, slots)
    q16 = workloads.random_halves(rng, (4, H * G, D))
    ref = O.decode_attention(olayout(lay), cache, q16, bt, ctx, 0.09)
    ws = K.DecodeWorkspace(lay, 4, H * G, bt.shape[1], 9)
    cdev = dev(cache)
    for it, (nb, splits) in enumerate([(4, 9), (4, 9), (2, 5), (4, 3), (3, 9), (4, 9)]):
        out = torch.empty((nb, H * G, D), dtype=torch.float16, device="cuda")
        K.kvq_decode_attention(lay, cdev, dev(q16[:nb]), dev(bt[:nb]), dev(ctx[:nb]), 0.09, out, ws.buffer, None,
                               splits)
        torch.cuda.synchronize()
        assert_attn_close(out.cpu().numpy().astype(np.float64), ref[:nb], f"call {it}")


@pytest.mark.parametrize("splits", [16, 64])
def test_split_records_are_fresh_each_call(K, O, splits):
    """Back-to-back calls in one stream on one workspace, alternating two
    query sets: the merge must read the records of its own call, written on
    other XCDs a moment before, never those the previous call left in the
    same place."""
    import torch
    rng = np.random.default_rng(2200 + splits)
    B, H, G, D, P = 8, 4, 8, 128, 16
    ctx = rng.integers(1500, 2049, B).astype(np.int32)
    ctx[0] = 2048  # 128 pages: 16 or 64 splits of whole pages
    bt, num_pages, slots = paged_problem(rng, B, H, G, D, P, ctx)
    k16 = workloads.random_halves(rng, (slots.size, H, D))
    v16 = workloads.random_halves(rng, (slots.size, H, D))
    lay = K.layout(2, H, D, P, num_pages)
    cache = O.quantize_write(olayout(lay), k16, v16, slots)
    qs = [workloads.random_halves(rng, (B, H * G, D)) * 2.0 for _ in range(2)]
    refs = [O.decode_attention(olayout(lay), cache, q, bt, ctx, 0.09) for q in qs]
    ws = K.DecodeWorkspace(lay, B, H * G, bt.shape[1], splits)
    assert ws.num_splits == splits
    cdev, btd, ctxd = dev(cache), dev(bt), dev(ctx)
    qd = [dev(q) for q in qs]
    outs = [torch.empty((B, H * G, D), dtype=torch.float16, device="cuda") for _ in range(8)]
    for i, out in enumerate(outs):
        K.kvq_decode_attention(lay, cdev, qd[i % 2], btd, ctxd, 0.09, out, ws.buffer, None, splits)
    torch.cuda.synchronize()
    for i, out in enumerate(outs):
        assert_attn_close(out.cpu().numpy().astype(np.float64), refs[i % 2], f"call {i}")
    assert not np.array_equal(outs[0].cpu().numpy(), outs[1].cpu().numpy())


@pytest.mark.parametrize("fmt,flags", [(2, 0), (4, 1), (6, 0), (7, 0)], ids=["int8pth", "nvfp4_4over6", "int4pth", "mxfp4"])
def test_decode_long_splits_and_limits(K, O, fmt, flags):
    """One split walking more than 256 pages (several block-table chunks in
    LDS), the largest page size, the maximum split count, and a batch whose
    sequences mix empty, one-page and long contexts."""
    rng = np.random.default_rng(4000 + fmt + flags)
    H, G, D = 2, 8, 128
    for P, ctx in ((16, [16 * 600 + 7, 0, 16, 5000]), (256, [256 * 3 + 1, 255, 256 * 9])):
        ctx = np.array(ctx, np.int32)
        B = ctx.size
        bt, num_pages, slots = paged_problem(rng, B, H, G, D, P, ctx)
        n = slots.shape[0]
        k16 = workloads.random_halves(rng, (n, H, D))
        v16 = workloads.random_halves(rng, (n, H, D))
        lay = layout_for(K, fmt, flags, H, D, P, num_pages, k16, v16)
        cache = O.quantize_write(olayout(lay), k16, v16, slots)
        q16 = workloads.random_halves(rng, (B, H * G, D))
        sm = 1.0 / math.sqrt(D)
        pairs = np.array([(b, h) for b in range(B) for h in (0, 5, H * G - 1)], np.int32)
        ref = O.decode_attention(olayout(lay), cache, q16, bt, ctx, sm, pairs=pairs)
        cdev = dev(cache)
        for splits in (1, 256):
            log(f"long decode fmt={fmt} P={P} splits={splits} max_pages={bt.shape[1]}")
            got, ws = gpu_decode(K, lay, cdev, q16, bt, ctx, sm, num_splits=splits)
            mp = bt.shape[1]
            pps = -(-mp // min(splits, mp))  # pages per split; empty trailing splits are dropped
            assert ws.num_splits == -(-mp // pps)
            for (b, h), r in zip(pairs, ref):
                assert_attn_close(got[b, h], r, f"P={P} splits={splits} b={b} h={h}")


def test_mxfp4_decode_small_and_large_blocks(K, O):
    """MXFP4 blocks across the whole binary16 range: block exponents from -26
    (subnormal inputs, whose binary16 operands round) to 13 (values near
    65504), mixed within one token row and across tokens."""
    rng = np.random.default_rng(4242)
    B, H, G, D, P = 3, 2, 8, 128, 16
    ctx = np.array([40, 130, 77], np.int32)
    bt, num_pages, slots = paged_problem(rng, B, H, G, D, P, ctx)
    n = slots.shape[0]
    mags = 2.0 ** rng.integers(-24, 15, (n, H, D // 32))  # per-block magnitude
    k16 = (rng.uniform(-1, 1, (n, H, D)) * np.repeat(mags, 32, axis=-1)).astype(np.float16)
    mags = 2.0 ** rng.integers(-24, 15, (n, H, D // 32))
    v16 = (rng.uniform(-1, 1, (n, H, D)) * np.repeat(mags, 32, axis=-1)).astype(np.float16)
    lay = K.layout(7, H, D, P, num_pages)
    cache = O.quantize_write(olayout(lay), k16, v16, slots)
    got_cache = gpu_write(K, lay, k16, v16, slots).cpu().numpy()
    mm = first_mismatch(got_cache, cache)
    assert mm is None, f"cache byte {mm[0]}: gpu {mm[1]:#x} oracle {mm[2]:#x}"
    # queries small enough that the huge keys give finite, spread-out logits
    q16 = (workloads.random_halves(rng, (B, H * G, D)) * np.float16(2.0 ** -14)).astype(np.float16)
    sm = 1.0 / math.sqrt(D)
    ref = O.decode_attention(olayout(lay), cache, q16, bt, ctx, sm)
    for splits in (1, 4):
        log(f"mxfp4 wide-range decode splits={splits}")
        got, _ = gpu_decode(K, lay, dev(cache), q16, bt, ctx, sm, num_splits=splits)
        assert_attn_close(got, ref, f"splits={splits}")


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 5, 6, 7])
def test_auto_split_plan_fills_the_device(K, O, fmt):
    """The automatic plan gives one resident round of the split kernel (2 to
    4 workgroups per compute unit on MI355X's 256), and a workspace of exactly
    the queried size is accepted while one byte less is refused."""
    import ctypes
    import torch
    B, H, G, D = 16, 8, 8, 128
    P = 128 if fmt == 5 else 16
    mp = 16384 // P
    lay = K.layout(fmt, H, D, P, B * mp, 0.05, 0.05)
    s = K.kvq_decode_num_splits(lay, B, H * G, mp)
    log(f"auto plan fmt={fmt}: {s} splits, {s * B * H} workgroups")
    assert 2 * 256 <= s * B * H <= 4 * 256 or s == -(-mp // 8)
    need = K.kvq_decode_workspace_bytes(lay, B, H * G, mp)
    assert need == B * H * s * (2 * 8 + 8 * D) * 4
    # the call validates the workspace size before touching any buffer
    cache = torch.zeros(16, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(cache.data_ptr())
    st = K.lib.kvq_decode_attention(ctypes.byref(lay), p, p, H * G, p, mp, p, B, 0.1, None, p, p, need - 1, 0, None)
    assert st == 3
    if fmt in (1, 2, 3):
        # a (sequence, kv head) per compute unit or more: one split of
        # eight-wave workgroups, no workspace
        assert K.kvq_decode_num_splits(lay, 32, H * 4, mp) == 1
        assert K.kvq_decode_workspace_bytes(lay, 32, H * 4, mp) == 0


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_decode_single_split_eight_waves(K, O, fmt):
    """Enough (sequence, kv head) pairs to give every compute unit one: the
    automatic plan runs one eight-wave workgroup per pair (no split
    partials); every output matches the oracle, empty and ragged contexts
    included."""
    rng = np.random.default_rng(8100 + fmt)
    B, H, G, D, P = 64, 4, 4, 128, 16
    ctx = rng.integers(0, 300, B).astype(np.int32)
    ctx[0], ctx[1], ctx[2] = 0, 1, 16 * 18
    bt, num_pages, slots = paged_problem(rng, B, H, G, D, P, ctx)
    n = slots.shape[0]
    k16 = workloads.random_halves(rng, (n, H, D))
    v16 = workloads.random_halves(rng, (n, H, D))
    lay = layout_for(K, fmt, 0, H, D, P, num_pages, k16, v16)
    assert K.kvq_decode_num_splits(lay, B, H * G, bt.shape[1]) == 1
    cache = O.quantize_write(olayout(lay), k16, v16, slots)
    q16 = workloads.random_halves(rng, (B, H * G, D))
    sm = 1.0 / math.sqrt(D)
    ref = O.decode_attention(olayout(lay), cache, q16, bt, ctx, sm)
    log(f"decode eight-wave single split fmt={fmt}")
    got, ws = gpu_decode(K, lay, dev(cache), q16, bt, ctx, sm)
    assert ws.num_splits == 1 and ws.buffer.numel() == 0
    assert_attn_close(got, ref)
    assert not np.any(got[0])


@pytest.mark.parametrize("fmt,flags", FORMATS, ids=FMT_IDS)
def test_decode_edge_context_lengths(K, O, fmt, flags):
    """Context lengths around the 16-token sub-page and page boundaries, a
    long one, and block tables that repeat pages: a page listed twice in one
    sequence and a sequence that shares another's pages (the reads see the
    same bytes twice; nothing in the decode assumes distinct pages)."""
    rng = np.random.default_rng(700 + fmt * 3 + flags)
    H, G, D, P = 2, 4, 128, 16
    ctx = np.array([1, 15, 16, 17, 127, 128, 129, 4095], np.int32)
    B = ctx.size
    bt, num_pages, slots = paged_problem(rng, B, H, G, D, P, ctx)
    n = slots.shape[0]
    k16 = workloads.random_halves(rng, (n, H, D))
    v16 = workloads.random_halves(rng, (n, H, D))
    lay = layout_for(K, fmt, flags, H, D, P, num_pages, k16, v16)
    cache = O.quantize_write(olayout(lay), k16, v16, slots)
    # repeated pages (after the write: the cache holds each page once)
    bt = bt.copy()
    bt[5, 4:8] = bt[5, 0]        # ctx 128 = pages 0..7: page 0 read five times
    bt[6, :9] = bt[7, :9]        # ctx 129: the first 9 pages of the 4095-token sequence
    q16 = workloads.random_halves(rng, (B, H * G, D))
    sm = 1.0 / math.sqrt(D)
    ref = O.decode_attention(olayout(lay), cache, q16, bt, ctx, sm)
    cache_dev = dev(cache)
    for splits in (0, 1, 5):
        log(f"edge contexts fmt={fmt} flags={flags} splits={splits}")
        got, _ = gpu_decode(K, lay, cache_dev, q16, bt, ctx, sm, num_splits=splits)
        assert_attn_close(got, ref, f"splits={splits}")
        ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(got - ref) <= 0.5 * ulp + 1e-4 + 1e-4 * np.abs(ref))
