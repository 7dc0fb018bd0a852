"""Full-size workloads in the benchmark's launch configuration, checked on
samples the oracle can afford.

For each workload the GPU quantise-writes the whole context (every token of
every sequence, one call) and decodes every (sequence, q head) with the split
plan the benchmark uses.  As in the benchmark's steps, the formats other than
KVarN write all but the last token of each sequence first and then write and
decode the last one in a single kvq_decode_attention_append call.  The oracle quantise-writes two sampled sequences on
the CPU: every page of those sequences must match the GPU cache byte for byte,
and sampled (sequence, q head) outputs must match the binary64 oracle within
|o - o_ref| <= 2e-3 + 2^-10 |o_ref|."""
import concurrent.futures as cf
import math

import numpy as np
import pytest

import workloads
from gpu_util import assert_attn_close, assert_flat_where_representable, dev, log, olayout

pytestmark = pytest.mark.gpu

CASES = [("int8_32k", 2, 0), ("int8_32k", 6, 0), ("fp8_sink_4k", 1, 0), ("fp8_sink_4k", 3, 0),
         ("nvfp4_16k", 4, 0), ("nvfp4_16k", 4, 1), ("nvfp4_16k", 7, 0), ("kvarn_16k", 5, 0),
         ("nvfp4_16k_tp2", 4, 0), ("kvarn_16k_tp2", 5, 0)]
IDS = ["int8_32k", "int4pth_32k", "fp8pt_4k", "fp8pth_4k", "nvfp4_16k", "nvfp4_4over6_16k", "mxfp4_16k", "kvarn_16k",
       "nvfp4_16k_tp2", "kvarn_16k_tp2"]

_cache = {}


def workload(name):
    if name not in _cache:
        _cache.clear()  # one full workload in host memory at a time
        _cache[name] = workloads.make(name)
    return _cache[name]


@pytest.mark.parametrize("name,fmt,flags", CASES, ids=IDS)
def test_full_size_sampled(K, O, name, fmt, flags):
    import torch
    w = workload(name)
    sp = w.spec
    ks, vs = w.per_tensor_scales(fmt)
    lay = K.layout(fmt, sp.Hkv, sp.D, sp.P, w.num_pages, ks, vs, flags)
    olay = olayout(lay)
    pb = K.kvq_page_bytes(lay)
    log(f"full size {name} fmt={fmt} flags={flags}: B={w.B} T={w.T} pages={w.num_pages}")

    # GPU: the whole context in one write, then one decode with the
    # benchmark's automatic split plan
    cache = torch.zeros(w.num_pages * pb, dtype=torch.uint8, device="cuda")
    one_call = fmt != K.KVQ_KVARN_K4V2_G128
    last = np.arange(w.B) * w.T + (w.T - 1)
    keep = np.ones(w.B * w.T, bool)
    if one_call:
        keep[last] = False
    kd, vd = dev(w.k16[keep]), dev(w.v16[keep])
    K.kvq_quantize_write(lay, kd, vd, dev(w.slots[keep]), cache)
    del kd, vd
    ws = K.DecodeWorkspace(lay, w.B, sp.Hq, w.block_tables.shape[1])
    out = torch.empty((w.B, sp.Hq, sp.D), dtype=torch.float16, device="cuda")
    sm = 1.0 / math.sqrt(sp.D)
    if one_call:
        K.kvq_decode_attention_append(lay, cache, dev(w.k16[last]), dev(w.v16[last]), dev(w.slots[last]),
                                      dev(w.q16), dev(w.block_tables), dev(w.ctx_lens), sm, out, ws.buffer)
    else:
        K.kvq_decode_attention(lay, cache, dev(w.q16), dev(w.block_tables), dev(w.ctx_lens), sm, out, ws.buffer)
    torch.cuda.synchronize()
    got_cache = cache.cpu().numpy()
    got = out.cpu().numpy().astype(np.float64)
    del cache
    assert np.all(np.isfinite(got))

    # oracle: the first and last sequences
    seqs = [0, w.B - 1]
    ref_cache = np.zeros(w.num_pages * pb, np.uint8)
    T = w.T

    def write_seq(b):
        sl = slice(b * T, (b + 1) * T)
        O.quantize_write(olay, w.k16[sl], w.v16[sl], w.slots[sl], ref_cache)

    with cf.ThreadPoolExecutor(len(seqs)) as ex:
        list(ex.map(write_seq, seqs))
    for b in seqs:
        for pg in w.block_tables[b]:
            lo, hi = int(pg) * pb, (int(pg) + 1) * pb
            if not np.array_equal(got_cache[lo:hi], ref_cache[lo:hi]):
                d = int(np.nonzero(got_cache[lo:hi] != ref_cache[lo:hi])[0][0])
                raise AssertionError(f"sequence {b} page {int(pg)} byte {d}: gpu {got_cache[lo + d]:#x} "
                                     f"oracle {ref_cache[lo + d]:#x}")

    # sampled outputs: first and last q head of each sampled sequence, and one
    # whole GQA group
    G = sp.Hq // sp.Hkv
    heads = sorted({0, sp.Hq - 1, *range(G, 2 * G)})
    pairs = np.array([(b, h) for b in seqs for h in heads], np.int32)

    def dec(pr):
        return O.decode_attention(olay, ref_cache, w.q16, w.block_tables, w.ctx_lens, sm, pairs=pr[None])

    with cf.ThreadPoolExecutor(8) as ex:
        ref = np.concatenate(list(ex.map(dec, pairs)))
    for (b, h), r in zip(pairs, ref):
        assert_attn_close(got[b, h], r, f"{name} sequence {b} head {h}")
    # and a flat 2e-3 wherever the binary16 output's rounding stays well inside it
    sampled = np.stack([got[b, h] for b, h in pairs])
    flat = assert_flat_where_representable(sampled, ref, name)
    log(f"  {name}: max error {np.abs(sampled - ref).max():.2e}, {flat:.2e} at |o| <= 4")
