"""KVarN k4v2 g128 through the C ABI against the oracle: bit-exact tile
quantisation (codes and binary32 metadata), bit-exact binary64 dequantisation,
and decode attention (complete tiles from the cache plus a binary16 tail)
within |o - o_ref| <= 2e-3 + 2^-10 |o_ref|."""
import math

import numpy as np
import pytest

import workloads
from gpu_util import assert_attn_close, dev, first_mismatch, gpu_decode, gpu_write, log, olayout

pytestmark = pytest.mark.gpu

D = P = 128


def kvarn_problem(rng, B, H, ctx, extra_pages=2, outliers=True, skip_page0=False):
    """Shuffled block tables; K/V rows of every token (sequence-major); the
    slots and source rows of the complete tiles; the binary16 tail buffer
    [B][2][H][128][D] holding each sequence's last ctx % 128 tokens."""
    ctx = np.asarray(ctx, np.int32)
    max_pages = max(1, int(math.ceil(int(ctx.max()) / P)))
    num_pages = B * max_pages + extra_pages
    pool = rng.permutation(num_pages).astype(np.int32)
    if skip_page0:
        pool = pool[pool != 0]
    bt = pool[:B * max_pages].reshape(B, max_pages)
    T = int(ctx.sum())
    k16 = workloads.random_halves(rng, (T, H, D))
    v16 = workloads.random_halves(rng, (T, H, D))
    if outliers:  # a few channels scaled x8, as in the long-context workload
        for x in (k16, v16):
            for h in range(H):
                x[:, h, rng.choice(D, 2, replace=False)] *= np.float16(8)
    slots, rows = [], []
    tail = np.zeros((B, 2, H, P, D), np.float16)
    off = 0
    for b in range(B):
        nfull = int(ctx[b]) // P
        for t in range(nfull):
            slots.append(bt[b, t].astype(np.int64) * P + np.arange(P))
            rows.append(off + t * P + np.arange(P))
        nt = int(ctx[b]) - nfull * P
        tail[b, 0, :, :nt] = k16[off + nfull * P: off + int(ctx[b])].transpose(1, 0, 2)
        tail[b, 1, :, :nt] = v16[off + nfull * P: off + int(ctx[b])].transpose(1, 0, 2)
        off += int(ctx[b])
    slots = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    rows = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    return bt, num_pages, slots, k16[rows], v16[rows], tail


def edge_tiles(rng, n_tiles, H):
    """Tiles with the cases the pipeline must handle: plain normal data, a
    sink token, outlier channels, an all-zero tile, constant rows and
    constant columns (zero deviations, zero quantiser steps), negative zeros,
    binary16 subnormals and the largest binary16 magnitudes."""
    x = workloads.random_halves(rng, (n_tiles * P, H, D))
    x[0] *= np.float16(20)
    x[:P, :, 7] *= np.float16(8)
    if n_tiles > 1:
        x[P:2 * P] = 0
    if n_tiles > 2:
        x[2 * P:3 * P] = np.float16(-0.0)
        x[2 * P:3 * P, :, 3] = np.float16(1.5)
    if n_tiles > 3:
        x[3 * P:4 * P] = rng.standard_normal((1, H, D)).astype(np.float16)  # identical rows
    if n_tiles > 4:
        x[4 * P:5 * P] = rng.standard_normal((P, H, 1)).astype(np.float16)  # constant rows
    if n_tiles > 5:
        x[5 * P:6 * P] = (rng.integers(-3, 4, (P, H, D)) * 2.0 ** -24).astype(np.float16)
    if n_tiles > 6:
        x[6 * P:7 * P] = rng.uniform(-65504, 65504, (P, H, D)).astype(np.float16)
    return x


def test_kvarn_write_bytes_match_oracle(K, O):
    rng = np.random.default_rng(501)
    H, n_tiles, num_pages = 3, 9, 12
    pages = rng.permutation(num_pages)[:n_tiles]
    slots = (pages[:, None].astype(np.int64) * P + np.arange(P)).reshape(-1)
    slots[7 * P] = -1                # a tile whose first slot is negative: skipped
    slots[8 * P] = num_pages * P     # ... or past the pool: skipped
    k16 = edge_tiles(rng, n_tiles, H)
    v16 = edge_tiles(rng, n_tiles, H)
    lay = K.layout(5, H, D, P, num_pages)
    log(f"kvarn write H={H} tiles={n_tiles}")
    ref = O.quantize_write(olayout(lay), k16, v16, slots)
    got = gpu_write(K, lay, k16, v16, slots).cpu().numpy()
    mm = first_mismatch(got, ref)
    assert mm is None, f"cache byte {mm[0]}: gpu {mm[1]:#x} oracle {mm[2]:#x} ({mm[3]} bytes differ)"


def test_kvarn_write_many_tiles(K, O):
    """A larger write (64 tiles x 8 kv heads, several workgroup rounds)."""
    rng = np.random.default_rng(502)
    H, n_tiles = 8, 64
    num_pages = n_tiles + 3
    pages = rng.permutation(num_pages)[:n_tiles]
    slots = (pages[:, None].astype(np.int64) * P + np.arange(P)).reshape(-1)
    k16 = workloads.random_halves(rng, (n_tiles * P, H, D))
    v16 = workloads.random_halves(rng, (n_tiles * P, H, D), 2.0)
    lay = K.layout(5, H, D, P, num_pages)
    log(f"kvarn write H={H} tiles={n_tiles}")
    ref = O.quantize_write(olayout(lay), k16, v16, slots)
    got = gpu_write(K, lay, k16, v16, slots).cpu().numpy()
    mm = first_mismatch(got, ref)
    assert mm is None, f"cache byte {mm[0]}: gpu {mm[1]:#x} oracle {mm[2]:#x} ({mm[3]} bytes differ)"


def test_kvarn_dequantize_matches_oracle(K, O):
    import torch
    rng = np.random.default_rng(503)
    H, n_tiles, num_pages = 2, 7, 9
    pages = rng.permutation(num_pages)[:n_tiles]
    slots = (pages[:, None].astype(np.int64) * P + np.arange(P)).reshape(-1)
    k16 = edge_tiles(rng, n_tiles, H)
    v16 = edge_tiles(rng, n_tiles, H)
    lay = K.layout(5, H, D, P, num_pages)
    cache = O.quantize_write(olayout(lay), k16, v16, slots)
    sel = rng.permutation(slots.size)[:300]
    sel_slots = slots[sel].copy()
    sel_slots[5] = -1  # skipped: row left untouched
    kr, vr = O.dequantize(olayout(lay), cache, sel_slots)
    kout = torch.full((sel.size, H, D), 7.0, dtype=torch.float32, device="cuda")
    vout = torch.full((sel.size, H, D), 7.0, dtype=torch.float32, device="cuda")
    log("kvarn dequantize")
    K.kvq_dequantize(lay, dev(cache), dev(sel_slots), kout, vout)
    torch.cuda.synchronize()
    kg, vg = kout.cpu().numpy(), vout.cpu().numpy()
    assert np.all(kg[5] == 7.0) and np.all(vg[5] == 7.0)
    keep = np.arange(sel.size) != 5
    # binary64 rebuild and rotation, one rounding to binary32
    assert np.array_equal(kg[keep], kr[keep].astype(np.float32))
    assert np.array_equal(vg[keep], vr[keep].astype(np.float32))


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_kvarn_decode_matches_oracle(K, O, G):
    rng = np.random.default_rng(510 + G)
    B, H = 5, 2
    ctx = np.array([0, 1, 128, 300, 9 * 128 + 127], np.int32)
    bt, num_pages, slots, kq, vq, tail = kvarn_problem(rng, B, H, ctx)
    lay = K.layout(5, H, D, P, num_pages)
    cache = O.quantize_write(olayout(lay), kq, vq, slots)
    q16 = workloads.random_halves(rng, (B, H * G, D))
    sm = 1.0 / math.sqrt(D)
    ref = O.decode_attention(olayout(lay), cache, q16, bt, ctx, sm, tail16=tail)
    cache_dev = dev(cache)
    # 10 splits of one tile each: more than one group of 8 partial records
    for splits in (0, 1, 3, 7, 10):
        log(f"kvarn decode G={G} splits={splits}")
        got, ws = gpu_decode(K, lay, cache_dev, q16, bt, ctx, sm, tail16=tail, num_splits=splits)
        if splits == 10:
            assert ws.num_splits == 10
        assert_attn_close(got, ref, f"splits={splits}")
        ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(got - ref) <= 0.5 * ulp + 1e-4 + 1e-4 * np.abs(ref))
    assert not np.any(got[0]), "empty context must give a zero row"


def test_kvarn_decode_whole_tiles_no_tail(K, O):
    """Contexts that are whole tiles need no tail buffer (NULL)."""
    rng = np.random.default_rng(520)
    B, H, G = 3, 2, 8
    ctx = np.array([128, 512, 256], np.int32)
    bt, num_pages, slots, kq, vq, _ = kvarn_problem(rng, B, H, ctx)
    lay = K.layout(5, H, D, P, num_pages)
    cache = O.quantize_write(olayout(lay), kq, vq, slots)
    q16 = workloads.random_halves(rng, (B, H * G, D))
    ref = O.decode_attention(olayout(lay), cache, q16, bt, ctx, 0.088)
    log("kvarn decode no tail")
    got, _ = gpu_decode(K, lay, dev(cache), q16, bt, ctx, 0.088)
    assert_attn_close(got, ref)


def test_kvarn_decode_closed_forms(K, O):
    """Identical keys in a tile give the mean of the dequantised values; a
    context of one token (tail only) gives that token's value."""
    rng = np.random.default_rng(530)
    H, G = 1, 4
    bt = np.array([[1, 0]], np.int32)
    slots = (np.int64(1) * P + np.arange(P))
    k16 = np.repeat(workloads.random_halves(rng, (1, H, D)), P, axis=0)
    v16 = workloads.random_halves(rng, (P, H, D))
    lay = K.layout(5, H, D, P, 2)
    cache = O.quantize_write(olayout(lay), k16, v16, slots)
    _, vh = O.dequantize(olayout(lay), cache, slots)
    q16 = workloads.random_halves(rng, (1, G, D))
    log("kvarn closed forms")
    got, _ = gpu_decode(K, lay, dev(cache), q16, bt, [P], 0.3)
    for h in range(G):
        assert_attn_close(got[0, h], vh[:, 0].mean(axis=0), "identical keys")
    tail = np.zeros((1, 2, H, P, D), np.float16)
    tail[0, :, 0, 0] = workloads.random_halves(rng, (2, D))
    got, _ = gpu_decode(K, lay, dev(cache), q16, bt, [1], 0.3, tail16=tail)
    for h in range(G):
        assert np.array_equal(got[0, h], tail[0, 1, 0, 0].astype(np.float64)), "one tail token"


def test_kvarn_decode_invalid_pages(K, O):
    """Pages outside the pool are skipped without faulting, even when the
    pool's first page holds garbage metadata."""
    rng = np.random.default_rng(540)
    B, H, G = 2, 2, 4
    ctx = np.array([384, 300], np.int32)
    bt, num_pages, slots, kq, vq, tail = kvarn_problem(rng, B, H, ctx, skip_page0=True)
    lay = K.layout(5, H, D, P, num_pages)
    cache = O.quantize_write(olayout(lay), kq, vq, slots)
    cache[:K.kvq_page_bytes(lay)] = 0xFF  # NaN metadata in page 0, which no entry uses
    bad = bt.copy()
    bad[0, 1] = -3
    bad[1, 0] = num_pages + 7
    q16 = workloads.random_halves(rng, (B, H * G, D))
    log("kvarn decode invalid pages")
    got, _ = gpu_decode(K, lay, dev(cache), q16, bad, ctx, 0.1, tail16=tail, num_splits=2)
    assert np.all(np.isfinite(got))


def test_kvarn_incremental_append_matches_oracle(K, O):
    """Tokens appended step by step (a 50-token chunk, then one token per
    sequence per call) give the same pages as one whole-tile write, the tail
    holds the raw tokens of the incomplete tile, and decode over pages + tail
    matches the oracle."""
    import torch
    rng = np.random.default_rng(560)
    B, H, G = 3, 2, 4
    ctx = np.array([128 + 5, 256, 3 * 128 - 1], np.int32)
    bt, num_pages, slots, kq, vq, tail_ref = kvarn_problem(rng, B, H, ctx)
    # every token of every sequence, sequence-major, as kvarn_problem drew them
    T = int(ctx.sum())
    rng2 = np.random.default_rng(561)
    k_all = workloads.random_halves(rng2, (T, H, D))
    v_all = workloads.random_halves(rng2, (T, H, D))
    starts = np.concatenate([[0], np.cumsum(ctx)[:-1]])
    full_slots, full_rows = [], []
    tail_ref = np.zeros((B, 2, H, P, D), np.float16)
    for b in range(B):
        n_full = int(ctx[b]) // P
        for t in range(n_full):
            full_slots.append(bt[b, t].astype(np.int64) * P + np.arange(P))
            full_rows.append(starts[b] + t * P + np.arange(P))
        nt = int(ctx[b]) - n_full * P
        tail_ref[b, 0, :, :nt] = k_all[starts[b] + n_full * P: starts[b] + ctx[b]].transpose(1, 0, 2)
        tail_ref[b, 1, :, :nt] = v_all[starts[b] + n_full * P: starts[b] + ctx[b]].transpose(1, 0, 2)
    full_slots = np.concatenate(full_slots)
    full_rows = np.concatenate(full_rows)
    lay = K.layout(5, H, D, P, num_pages)
    ref_cache = O.quantize_write(olayout(lay), k_all[full_rows], v_all[full_rows], full_slots)

    cache = torch.zeros(num_pages * K.kvq_page_bytes(lay), dtype=torch.uint8, device="cuda")
    tail = torch.zeros((B, 2, H, P, D), dtype=torch.float16, device="cuda")
    kd, vd, btd = dev(k_all), dev(v_all), dev(bt)

    def append(pairs):
        rows = np.array([starts[b] + p for b, p in pairs], np.int64)
        K.kvq_kvarn_append(lay, kd[dev(rows)], vd[dev(rows)], dev(np.array([b for b, _ in pairs], np.int32)),
                           dev(np.array([p for _, p in pairs], np.int32)), tail, btd, cache)

    log("kvarn incremental append")
    append([(b, p) for b in range(B) for p in range(50)])  # a chunk within the first tile
    for p in range(50, int(ctx.max())):
        append([(b, p) for b in range(B) if p < ctx[b]])
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    pb = K.kvq_page_bytes(lay)
    for b in range(B):
        for t in range(int(ctx[b]) // P):
            pg = int(bt[b, t])
            assert np.array_equal(got[pg * pb:(pg + 1) * pb], ref_cache[pg * pb:(pg + 1) * pb]), (b, t)
    gt = tail.cpu().numpy()
    for b in range(B):
        nt = int(ctx[b]) % P
        assert np.array_equal(gt[b, :, :, :nt].view(np.uint16), tail_ref[b, :, :, :nt].view(np.uint16)), b
    q16 = workloads.random_halves(rng, (B, H * G, D))
    ref = O.decode_attention(olayout(lay), ref_cache, q16, bt, ctx, 0.088, tail16=tail_ref)
    out = torch.empty((B, H * G, D), dtype=torch.float16, device="cuda")
    ws = K.DecodeWorkspace(lay, B, H * G, bt.shape[1])
    K.kvq_decode_attention(lay, cache, dev(q16), btd, dev(ctx), 0.088, out, ws.buffer, tail)
    torch.cuda.synchronize()
    assert_attn_close(out.cpu().numpy().astype(np.float64), ref)


def test_kvarn_decode_edge_contexts_and_repeated_tiles(K, O):
    """Contexts around the tile boundary (127, 128, 129, 255, 256, 257, 8191)
    and block tables that list a tile's page twice or share pages between
    sequences: the tail is per sequence, the tiles are read as listed."""
    rng = np.random.default_rng(733)
    B, H, G = 7, 2, 8
    ctx = np.array([127, 128, 129, 255, 256, 257, 8191], np.int32)
    bt, num_pages, slots, kq, vq, tail = kvarn_problem(rng, B, H, ctx)
    lay = K.layout(5, H, D, P, num_pages)
    cache = O.quantize_write(olayout(lay), kq, vq, slots)
    bt = bt.copy()
    bt[4, 1] = bt[4, 0]      # ctx 256: its first tile read twice
    bt[5, :2] = bt[6, :2]    # ctx 257: the first two tiles of the 8191-token sequence
    q16 = workloads.random_halves(rng, (B, H * G, D))
    sm = 1.0 / math.sqrt(D)
    ref = O.decode_attention(olayout(lay), cache, q16, bt, ctx, sm, tail16=tail)
    cache_dev = dev(cache)
    for splits in (0, 1, 9):
        log(f"kvarn edge contexts splits={splits}")
        got, _ = gpu_decode(K, lay, cache_dev, q16, bt, ctx, sm, tail16=tail, num_splits=splits)
        assert_attn_close(got, ref, f"splits={splits}")
        ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(got - ref) <= 0.5 * ulp + 1e-4 + 1e-4 * np.abs(ref))


def test_kvarn_contract_violations_are_reported(K, O):
    """The KVarN inputs the host cannot check (they live in device memory)
    are checked by the kernels: a whole-tile write run whose slots are not
    one tile of a page in order is skipped and raises
    KVQ_DEVERR_KVARN_TILE_SLOTS; an append whose tokens of one sequence span
    two tiles or repeat a position raises KVQ_DEVERR_KVARN_APPEND_SPAN.  Valid
    runs are written bit for bit as the oracle writes them, and every flag is
    cleared once read."""
    import torch
    rng = np.random.default_rng(560)
    H, n_tiles, num_pages = 2, 5, 8
    lay = K.layout(5, H, D, P, num_pages)
    K.kvq_take_device_errors()  # start clean
    pages = rng.permutation(num_pages)[:n_tiles]
    good = (pages[:, None].astype(np.int64) * P + np.arange(P)).reshape(-1)
    k16 = workloads.random_halves(rng, (n_tiles * P, H, D))
    v16 = workloads.random_halves(rng, (n_tiles * P, H, D))
    log("kvarn write: valid runs")
    got = gpu_write(K, lay, k16, v16, good).cpu().numpy()
    assert K.kvq_take_device_errors() == 0
    assert first_mismatch(got, O.quantize_write(olayout(lay), k16, v16, good)) is None

    bad = good.copy()
    bad[1 * P + 5], bad[1 * P + 6] = bad[1 * P + 6], bad[1 * P + 5]  # run 1: two slots swapped
    bad[3 * P: 4 * P] += 64  # run 3: starts half way into a tile
    bad[4 * P] = -1  # run 4: first slot negative, skipped without a report
    kept = good.copy()
    for r in (1, 3, 4):
        kept[r * P] = -1
    log("kvarn write: runs that break the tile rule")
    got = gpu_write(K, lay, k16, v16, bad).cpu().numpy()
    assert K.kvq_take_device_errors() == K.KVQ_DEVERR_KVARN_TILE_SLOTS
    assert K.kvq_take_device_errors() == 0
    assert first_mismatch(got, O.quantize_write(olayout(lay), k16, v16, kept)) is None

    # appends: one token per sequence is fine; a sequence's tokens at 127 and
    # 128 (two tiles), or twice at one position, are reported
    B = 2
    bt = dev(np.arange(B * 2, dtype=np.int32).reshape(B, 2))
    cache = torch.zeros(num_pages * K.kvq_page_bytes(lay), dtype=torch.uint8, device="cuda")
    tail = torch.zeros((B, 2, H, P, D), dtype=torch.float16, device="cuda")
    for seq, pos, want in (([0, 1], [5, 9], 0), ([0, 1, 0], [127, 3, 128], K.KVQ_DEVERR_KVARN_APPEND_SPAN),
                           ([1, 1], [7, 7], K.KVQ_DEVERR_KVARN_APPEND_SPAN), ([0, 1], [6, 10], 0)):
        n = len(seq)
        log(f"kvarn append seq={seq} pos={pos}")
        kd = dev(workloads.random_halves(rng, (n, H, D)))
        vd = dev(workloads.random_halves(rng, (n, H, D)))
        K.kvq_kvarn_append(lay, kd, vd, dev(np.array(seq, np.int32)), dev(np.array(pos, np.int32)), tail, bt, cache)
        assert K.kvq_take_device_errors() == want
