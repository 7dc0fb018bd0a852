"""kvq_decode_attention_append (one decode step in one call) against the
oracle: the cache bytes equal the oracle's write of the new tokens bit for
bit, and the output equals the oracle's binary64 decode over the updated
cache within the decode tolerance.  Also the library's own write-then-decode
gives the same result."""
import math

import numpy as np
import pytest

import workloads
from gpu_util import assert_attn_close, dev, first_mismatch, gpu_decode, log, olayout, paged_problem
from test_gpu_parity import FMT_IDS, FORMATS, edge_rows, layout_for

pytestmark = pytest.mark.gpu


def step_problem(rng, B, H, G, D, P, ctx, skip):
    """Block tables for contexts `ctx` (the new token included), the cached
    tokens before the step and the new token's slot per sequence.  A sequence
    in `skip` gets slot -1 (nothing stored, all ctx tokens cached); ctx = 0
    gets a slot on a page no sequence reads."""
    bt, num_pages, _ = paged_problem(rng, B, H, G, D, P, ctx, extra_pages=2)
    free_page = int(np.setdiff1d(np.arange(num_pages), bt.ravel())[0])
    old, new_slots = [], np.empty(B, np.int64)
    for b in range(B):
        c = int(ctx[b])
        n_old = c if (b in skip or c == 0) else c - 1
        old += [int(bt[b, t // P]) * P + t % P for t in range(n_old)]
        if b in skip:
            new_slots[b] = -1
        elif c == 0:
            new_slots[b] = free_page * P + 3
        else:
            new_slots[b] = int(bt[b, (c - 1) // P]) * P + (c - 1) % P
    return bt, num_pages, np.array(old, np.int64), new_slots


@pytest.mark.parametrize("fmt,flags", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("D,P,G", [(128, 16, 8), (64, 32, 2), (32, 16, 1)])
def test_append_decode_matches_oracle(K, O, fmt, flags, D, P, G):
    import torch
    rng = np.random.default_rng(900 + 10 * fmt + flags + D + G)
    H = 2
    ctx = np.array([1, 2, 16, 17, 300, 1000, 0, 129, 40], np.int32)
    B = ctx.size
    skip = {7}
    bt, num_pages, slots_old, slots_new = step_problem(rng, B, H, G, D, P, ctx, skip)
    k_old = workloads.random_halves(rng, (slots_old.size, H, D))
    v_old = workloads.random_halves(rng, (slots_old.size, H, D))
    k_new = edge_rows(rng, B, H, D)
    v_new = edge_rows(rng, B, H, D)[::-1].copy()
    lay = layout_for(K, fmt, flags, H, D, P, num_pages, np.concatenate([k_old, k_new]),
                     np.concatenate([v_old, v_new]))
    before = O.quantize_write(olayout(lay), k_old, v_old, slots_old)
    after = O.quantize_write(olayout(lay), k_new, v_new, slots_new, cache=before.copy())
    q16 = workloads.random_halves(rng, (B, H * G, D))
    sm = 1.0 / math.sqrt(D)
    ref = O.decode_attention(olayout(lay), after, q16, bt, ctx, sm)

    args = [dev(k_new), dev(v_new), dev(slots_new)]
    for splits in (0, 1, 3, 9):
        log(f"append+decode fmt={fmt} flags={flags} D={D} P={P} G={G} splits={splits}")
        ws = K.DecodeWorkspace(lay, B, H * G, bt.shape[1], splits)
        cache = dev(before)
        out = torch.empty((B, H * G, D), dtype=torch.float16, device="cuda")
        K.kvq_decode_attention_append(lay, cache, *args, dev(q16), dev(bt), dev(ctx), sm, out, ws.buffer, splits)
        torch.cuda.synchronize()
        got_cache = cache.cpu().numpy()
        assert first_mismatch(got_cache, after) is None, f"splits={splits}: cache {first_mismatch(got_cache, after)}"
        got = out.cpu().numpy().astype(np.float64)
        # the new tokens are edge rows (binary16 extremes, outliers): scores
        # of ~1e5 in binary32, so only the decode tolerance applies
        assert_attn_close(got, ref, f"splits={splits}")
        # the same step as two calls: write, then decode
        cache2 = dev(before)
        K.kvq_quantize_write(lay, *args, cache2)
        got2, _ = gpu_decode(K, lay, cache2, q16, bt, ctx, sm, num_splits=splits)
        assert_attn_close(got2, got, f"splits={splits}: write + decode vs one call")



@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("fmt,flags", [(2, 0), (3, 0), (4, 1), (6, 0)], ids=["int8pth", "fp8pth", "nvfp4_4over6",
                                                                          "int4pth"])
def test_append_slot_elsewhere(K, O, fmt, flags, splits):
    """A new token whose slot is not position ctx-1's (here: on a page no
    sequence reads) is stored at that slot and still attended as position
    ctx-1, with one split (the split kernel attends it) and with several (the
    merge does)."""
    import torch
    rng = np.random.default_rng(950 + 10 * fmt + flags + splits)
    B, H, G, D, P = 3, 2, 8, 128, 16
    ctx = np.array([100, 37, 64], np.int32)
    bt, num_pages, slots_old, slots_new = step_problem(rng, B, H, G, D, P, ctx, set())
    free = np.setdiff1d(np.arange(num_pages), bt.ravel())
    assert free.size >= 2
    at_ctx = slots_new.copy()           # position ctx-1's slots
    slots_new[1] = int(free[-1]) * P + 5  # sequence 1 writes elsewhere
    k_old = workloads.random_halves(rng, (slots_old.size, H, D))
    v_old = workloads.random_halves(rng, (slots_old.size, H, D))
    k_new = workloads.random_halves(rng, (B, H, D))
    v_new = workloads.random_halves(rng, (B, H, D))
    lay = layout_for(K, fmt, flags, H, D, P, num_pages, np.concatenate([k_old, k_new]),
                     np.concatenate([v_old, v_new]))
    before = O.quantize_write(olayout(lay), k_old, v_old, slots_old)
    after = O.quantize_write(olayout(lay), k_new, v_new, slots_new, cache=before.copy())
    attended = O.quantize_write(olayout(lay), k_new, v_new, at_ctx, cache=before.copy())
    q16 = workloads.random_halves(rng, (B, H * G, D))
    sm = 1.0 / math.sqrt(D)
    ref = O.decode_attention(olayout(lay), attended, q16, bt, ctx, sm)
    log(f"append, slot elsewhere: fmt={fmt} flags={flags} splits={splits}")
    ws = K.DecodeWorkspace(lay, B, H * G, bt.shape[1], splits)
    assert ws.num_splits == splits
    cache = dev(before)
    out = torch.empty((B, H * G, D), dtype=torch.float16, device="cuda")
    K.kvq_decode_attention_append(lay, cache, dev(k_new), dev(v_new), dev(slots_new), dev(q16), dev(bt), dev(ctx),
                                  sm, out, ws.buffer, splits)
    torch.cuda.synchronize()
    assert first_mismatch(cache.cpu().numpy(), after) is None
    assert_attn_close(out.cpu().numpy().astype(np.float64), ref, f"splits={splits}")


def test_prepared_calls_match_the_plain_binding(K, O):
    """The prepared calls (arguments marshalled once, then one C call per
    use) give bit for bit the plain binding's results: the append step, the
    decode and the KVarN append, each used twice."""
    import torch
    rng = np.random.default_rng(955)
    H, G, D, P = 2, 8, 128, 16
    ctx = np.array([300, 17, 1000, 1], np.int32)
    B = ctx.size
    bt, num_pages, slots_old, slots_new = step_problem(rng, B, H, G, D, P, ctx, set())
    k_old = workloads.random_halves(rng, (slots_old.size, H, D))
    v_old = workloads.random_halves(rng, (slots_old.size, H, D))
    k_new = workloads.random_halves(rng, (B, H, D))
    v_new = workloads.random_halves(rng, (B, H, D))
    lay = K.layout(2, H, D, P, num_pages)
    before = O.quantize_write(olayout(lay), k_old, v_old, slots_old)
    q16 = workloads.random_halves(rng, (B, H * G, D))
    q, btd, ctxd, kn, vn, sn = dev(q16), dev(bt), dev(ctx), dev(k_new), dev(v_new), dev(slots_new)
    ws = K.DecodeWorkspace(lay, B, H * G, bt.shape[1], 3)
    log("prepared append / decode")
    res = []
    for prepared in (False, True):
        cache = dev(before)
        out = torch.zeros((B, H * G, D), dtype=torch.float16, device="cuda")
        out2 = torch.zeros_like(out)
        if prepared:
            step = K.prepare_decode_attention_append(lay, cache, kn, vn, sn, q, btd, ctxd, 0.09, out, ws.buffer, 3)
            dec = K.prepare_decode_attention(lay, cache, q, btd, ctxd, 0.09, out2, ws.buffer, None, 3)
            step(), step(), dec(), dec()
        else:
            for _ in range(2):
                K.kvq_decode_attention_append(lay, cache, kn, vn, sn, q, btd, ctxd, 0.09, out, ws.buffer, 3)
            for _ in range(2):
                K.kvq_decode_attention(lay, cache, q, btd, ctxd, 0.09, out2, ws.buffer, None, 3)
        torch.cuda.synchronize()
        res.append((cache.cpu().numpy(), out.cpu().numpy(), out2.cpu().numpy()))
    for a, b in zip(*res):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))

    # KVarN: two appended tokens per sequence through prepared calls
    klay = K.layout(5, H, D, 128, 8)
    kbt = np.arange(8, dtype=np.int32).reshape(2, 4)
    seq = dev(np.arange(2, dtype=np.int32))
    kv = [dev(workloads.random_halves(rng, (2, H, D))) for _ in range(4)]
    log("prepared kvarn append")
    res = []
    for prepared in (False, True):
        cache = torch.zeros(8 * K.kvq_page_bytes(klay), dtype=torch.uint8, device="cuda")
        tail = torch.zeros((2, 2, H, 128, D), dtype=torch.float16, device="cuda")
        for j in range(2):
            pos = dev(np.full(2, j, np.int32))
            if prepared:
                K.prepare_kvarn_append(klay, kv[2 * j], kv[2 * j + 1], seq, pos, tail, dev(kbt), cache)()
            else:
                K.kvq_kvarn_append(klay, kv[2 * j], kv[2 * j + 1], seq, pos, tail, dev(kbt), cache)
        torch.cuda.synchronize()
        res.append((cache.cpu().numpy(), tail.cpu().numpy()))
    for a, b in zip(*res):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
