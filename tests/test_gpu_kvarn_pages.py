"""KVarN with pages of 256 tokens (two 128-token tiles per page) through the
C ABI against the oracle: bit-exact whole-tile writes into either tile of a
page, bit-exact dequantisation, decode over tiles spread across pages plus
the binary16 tail, and the incremental append completing tiles in both
positions of a page."""
import math

import numpy as np
import pytest

import workloads
from gpu_util import assert_attn_close, dev, first_mismatch, gpu_decode, gpu_write, log, olayout

pytestmark = pytest.mark.gpu

D = T = 128  # head size, tile
PS = 256     # page size


def problem(rng, B, H, ctx, extra_pages=2):
    """Shuffled block tables of 256-token pages; slots and rows of every
    complete tile; the binary16 tail of each sequence's incomplete tile."""
    ctx = np.asarray(ctx, np.int32)
    max_pages = max(1, int(math.ceil(int(ctx.max()) / PS)))
    num_pages = B * max_pages + extra_pages
    bt = rng.permutation(num_pages).astype(np.int32)[:B * max_pages].reshape(B, max_pages)
    n = int(ctx.sum())
    k16 = workloads.random_halves(rng, (n, H, D))
    v16 = workloads.random_halves(rng, (n, H, D))
    slots, rows = [], []
    tail = np.zeros((B, 2, H, T, D), np.float16)
    off = 0
    for b in range(B):
        nfull = int(ctx[b]) // T
        for t in range(nfull):
            tok = t * T + np.arange(T)
            slots.append(bt[b, tok // PS].astype(np.int64) * PS + tok % PS)
            rows.append(off + tok)
        nt = int(ctx[b]) - nfull * T
        tail[b, 0, :, :nt] = k16[off + nfull * T: off + int(ctx[b])].transpose(1, 0, 2)
        tail[b, 1, :, :nt] = v16[off + nfull * T: off + int(ctx[b])].transpose(1, 0, 2)
        off += int(ctx[b])
    slots = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    rows = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    return bt, num_pages, slots, k16, v16, rows, tail


def test_kvarn256_write_and_dequantize_match_oracle(K, O):
    import torch
    rng = np.random.default_rng(7100)
    H, num_pages = 3, 5
    # tiles into both positions of several pages, in a scrambled order
    starts = np.array([1 * PS + 128, 3 * PS, 0, 4 * PS + 128, 2 * PS, 3 * PS + 128], np.int64)
    slots = np.concatenate([s + np.arange(T) for s in starts])
    k16 = workloads.random_halves(rng, (slots.size, H, D))
    v16 = workloads.random_halves(rng, (slots.size, H, D), 3.0)
    k16[5, :, 9] = np.float16(4000.0)
    v16[T:2 * T] = 0
    lay = K.layout(5, H, D, PS, num_pages)
    log("kvarn 256-token pages: write")
    ref = O.quantize_write(olayout(lay), k16, v16, slots)
    got = gpu_write(K, lay, k16, v16, slots).cpu().numpy()
    mm = first_mismatch(got, ref)
    assert mm is None, f"cache byte {mm[0]}: gpu {mm[1]:#x} oracle {mm[2]:#x} ({mm[3]} bytes differ)"
    kr, vr = O.dequantize(olayout(lay), ref, slots)
    kout = torch.full((slots.size, H, D), 7.0, dtype=torch.float32, device="cuda")
    vout = torch.full((slots.size, H, D), 7.0, dtype=torch.float32, device="cuda")
    K.kvq_dequantize(lay, dev(ref), dev(slots), kout, vout)
    torch.cuda.synchronize()
    # rebuilt in binary64 and rotated back, one final rounding to binary32
    assert np.array_equal(kout.cpu().numpy(), kr.astype(np.float32))
    assert np.array_equal(vout.cpu().numpy(), vr.astype(np.float32))


@pytest.mark.parametrize("G", [1, 8])
def test_kvarn256_decode_matches_oracle(K, O, G):
    rng = np.random.default_rng(7200 + G)
    B, H = 5, 2
    ctx = np.array([0, 100, 256, 300, 3 * PS + 128 + 37], np.int32)
    bt, num_pages, slots, k16, v16, rows, tail = problem(rng, B, H, ctx)
    lay = K.layout(5, H, D, PS, num_pages)
    cache = O.quantize_write(olayout(lay), k16[rows], v16[rows], slots)
    q16 = workloads.random_halves(rng, (B, H * G, D))
    sm = 1.0 / math.sqrt(D)
    ref = O.decode_attention(olayout(lay), cache, q16, bt, ctx, sm, tail16=tail)
    cdev = dev(cache)
    for splits in (0, 1, 3):
        log(f"kvarn 256-token pages: decode G={G} splits={splits}")
        got, _ = gpu_decode(K, lay, cdev, q16, bt, ctx, sm, tail16=tail, num_splits=splits)
        assert_attn_close(got, ref, f"splits={splits}")
    assert not np.any(got[0]), "empty context must give a zero row"


def test_kvarn256_incremental_append_matches_oracle(K, O):
    """One token per sequence per call from position 0: tiles complete in the
    first and in the second half of pages, with the same bytes as whole-tile
    writes, and decode over pages plus tail matches the oracle."""
    import torch
    rng = np.random.default_rng(7300)
    B, H, G = 2, 2, 4
    ctx = np.array([PS + 128 + 9, 2 * PS], np.int32)
    bt, num_pages, slots, k16, v16, rows, tail_ref = problem(rng, B, H, ctx)
    lay = K.layout(5, H, D, PS, num_pages)
    ref_cache = O.quantize_write(olayout(lay), k16[rows], v16[rows], slots)
    starts = np.concatenate([[0], np.cumsum(ctx)[:-1]])
    cache = torch.zeros(num_pages * K.kvq_page_bytes(lay), dtype=torch.uint8, device="cuda")
    tail = torch.zeros((B, 2, H, T, D), dtype=torch.float16, device="cuda")
    kd, vd, btd = dev(k16), dev(v16), dev(bt)
    log("kvarn 256-token pages: incremental append")
    for p in range(int(ctx.max())):
        pairs = [(b, p) for b in range(B) if p < ctx[b]]
        r = np.array([starts[b] + q for b, q in pairs], np.int64)
        K.kvq_kvarn_append(lay, kd[dev(r)], vd[dev(r)], dev(np.array([b for b, _ in pairs], np.int32)),
                           dev(np.array([q for _, q in pairs], np.int32)), tail, btd, cache)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    pb = K.kvq_page_bytes(lay)
    tb = pb // (2 * H)  # one tile of one head
    for b in range(B):
        for ti in range(int(ctx[b]) // T):
            for h in range(H):
                a = int(bt[b, ti // 2]) * pb + h * 2 * tb + (ti % 2) * tb
                assert np.array_equal(got[a:a + tb], ref_cache[a:a + tb]), (b, ti, h)
    gt = tail.cpu().numpy()
    for b in range(B):
        nt = int(ctx[b]) % T
        assert np.array_equal(gt[b, :, :, :nt].view(np.uint16), tail_ref[b, :, :, :nt].view(np.uint16)), b
    q16 = workloads.random_halves(rng, (B, H * G, D))
    ref = O.decode_attention(olayout(lay), ref_cache, q16, bt, ctx, 0.088, tail16=tail_ref)
    out = torch.empty((B, H * G, D), dtype=torch.float16, device="cuda")
    ws = K.DecodeWorkspace(lay, B, H * G, bt.shape[1])
    K.kvq_decode_attention(lay, cache, dev(q16), btd, dev(ctx), 0.088, out, ws.buffer, tail)
    torch.cuda.synchronize()
    assert_attn_close(out.cpu().numpy().astype(np.float64), ref)
