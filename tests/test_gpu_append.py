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

