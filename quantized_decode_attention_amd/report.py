"""Tensor-level quantisation error report: the format gate of [P5] "NVFP4 KV
Cache：Blackwell 上的 4-bit 缓存量化", §量化误差该怎样测 (tensor level: MSE and
normalised MSE, max absolute error, cosine similarity, zero ratio, clipping /
saturation ratio, scale distribution, error by layer / head / position, K and V
counted separately), plus the attention-output error of the quantised decode
against unquantised attention.

Every quantised value comes from the GPU library (kvq_quantize_write, then
kvq_dequantize and kvq_decode_attention); this module only measures.

    python -m quantized_decode_attention_amd.report --workload fp8_sink_4k --seqs 2
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys

import numpy as np

# Largest code value of each format's scaled grid (used to express the row's
# largest reconstructed magnitude as an effective scale).
TOP_CODE = {1: 448.0, 2: 127.0, 3: 448.0, 4: 6.0, 6: 7.0, 7: 6.0}
# Relative margin above the row's largest reconstruction beyond which an input
# counts as clipped (above every format's half-step rounding error).
CLIP_MARGIN = 0.25


# --------------------------------------------------------------------------- #
# Metrics (pure numpy; x, xh: [n_tok, H, D] inputs and reconstructions)
# --------------------------------------------------------------------------- #

def tensor_metrics(x, xh):
    """Whole-tensor metrics of one side (K or V)."""
    x = np.asarray(x, np.float64)
    xh = np.asarray(xh, np.float64)
    e = xh - x
    mse = float(np.mean(e * e))
    power = float(np.mean(x * x))
    xf, hf = x.ravel(), xh.ravel()
    nx, nh = np.linalg.norm(xf), np.linalg.norm(hf)
    cos = float(xf @ hf / (nx * nh)) if nx > 0 and nh > 0 else float("nan")
    row_max = np.abs(xh).max(axis=-1, keepdims=True)
    clipped = np.abs(x) > row_max * (1.0 + CLIP_MARGIN) + 1e-30
    return {
        "mse": mse,
        "nmse": mse / power if power > 0 else float("nan"),
        "max_abs_error": float(np.abs(e).max()) if e.size else 0.0,
        "cosine": cos,
        "zero_ratio": float(np.mean(xh == 0.0)),
        "zero_ratio_input": float(np.mean(x == 0.0)),
        "clip_ratio": float(np.mean(clipped)),
    }


def scale_distribution(xh, top_code):
    """Distribution of the effective per-token-head scale max|x_hat| / top code
    (the stored scale for the per-token-head formats, whose row maximum lands
    on the top code)."""
    rs = np.abs(np.asarray(xh, np.float64)).max(axis=-1).ravel() / top_code
    rs = rs[rs > 0]
    if rs.size == 0:
        return {}
    p = np.percentile(rs, [1, 50, 99])
    return {"p01": float(p[0]), "p50": float(p[1]), "p99": float(p[2]), "min": float(rs.min()),
            "max": float(rs.max()), "log2_span": float(np.log2(rs.max() / rs.min()))}


def by_head(x, xh):
    """NMSE of each kv head (the worst head is the one to watch)."""
    x = np.asarray(x, np.float64)
    xh = np.asarray(xh, np.float64)
    out = []
    for h in range(x.shape[1]):
        p = np.mean(x[:, h] ** 2)
        out.append(float(np.mean((xh[:, h] - x[:, h]) ** 2) / p) if p > 0 else float("nan"))
    return out


def by_position(x, xh, T, buckets=8):
    """NMSE of the first token of every sequence (where attention sinks sit)
    and of equal position buckets over the context; tokens are sequence-major
    with T per sequence."""
    x = np.asarray(x, np.float64).reshape(-1, T, *x.shape[1:])
    xh = np.asarray(xh, np.float64).reshape(-1, T, *xh.shape[1:])

    def nmse(a, b):
        p = np.mean(a * a)
        return float(np.mean((b - a) ** 2) / p) if p > 0 else float("nan")

    edges = np.linspace(0, T, buckets + 1).astype(int)
    return {"first_token": nmse(x[:, 0], xh[:, 0]), "rest": nmse(x[:, 1:], xh[:, 1:]),
            "buckets": [nmse(x[:, a:b], xh[:, a:b]) for a, b in zip(edges[:-1], edges[1:]) if b > a]}


def attention_metrics(o, o_ref):
    """Quantised decode output vs unquantised attention, per (sequence, head)
    row: relative L2 error, max abs error, cosine."""
    o = np.asarray(o, np.float64).reshape(-1, o.shape[-1])
    r = np.asarray(o_ref, np.float64).reshape(-1, o_ref.shape[-1])
    rel = np.linalg.norm(o - r, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-30)
    cos = np.sum(o * r, axis=1) / np.maximum(np.linalg.norm(o, axis=1) * np.linalg.norm(r, axis=1), 1e-30)
    return {"rel_l2_mean": float(rel.mean()), "rel_l2_max": float(rel.max()),
            "max_abs_error": float(np.abs(o - r).max()), "cosine_min": float(cos.min())}


# --------------------------------------------------------------------------- #
# Driver (GPU)
# --------------------------------------------------------------------------- #

def _reference_attention(q16, k16, v16, B, T, G, sm_scale):
    """Unquantised attention in binary32 on the GPU (plain torch ops, per
    sequence and kv head, no batched products on transposed views)."""
    import torch
    q = torch.from_numpy(np.ascontiguousarray(q16)).cuda().float()          # [B, Hq, D]
    Hkv, D = k16.shape[1], k16.shape[2]
    out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device="cuda")
    for b in range(B):
        k = torch.from_numpy(np.ascontiguousarray(k16[b * T:(b + 1) * T])).cuda().float()  # [T, Hkv, D]
        v = torch.from_numpy(np.ascontiguousarray(v16[b * T:(b + 1) * T])).cuda().float()
        for h in range(Hkv):
            qh = q[b, h * G:(h + 1) * G]                      # [G, D]
            s = (qh @ k[:, h].T.contiguous()) * sm_scale       # [G, T]
            p = torch.softmax(s, dim=-1)
            out[b, h * G:(h + 1) * G] = p @ v[:, h].contiguous()
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def report_format(K, w, fmt, flags=0):
    """Quantise w's tensors with one format on the GPU and measure."""
    import torch
    sp = w.spec
    ks, vs = w.per_tensor_scales(fmt)
    lay = K.layout(fmt, sp.Hkv, sp.D, sp.P, w.num_pages, ks, vs, flags)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cache = torch.zeros(w.num_pages * K.kvq_page_bytes(lay), dtype=torch.uint8, device="cuda")
    slots = d(w.slots)
    K.kvq_quantize_write(lay, d(w.k16), d(w.v16), slots, cache)
    kh = torch.empty(w.k16.shape, dtype=torch.float32, device="cuda")
    vh = torch.empty(w.v16.shape, dtype=torch.float32, device="cuda")
    K.kvq_dequantize(lay, cache, slots, kh, vh)
    ws = K.DecodeWorkspace(lay, w.B, sp.Hq, w.block_tables.shape[1])
    out = torch.empty((w.B, sp.Hq, sp.D), dtype=torch.float16, device="cuda")
    sm = 1.0 / math.sqrt(sp.D)
    K.kvq_decode_attention(lay, cache, d(w.q16), d(w.block_tables), d(w.ctx_lens), sm, out, ws.buffer)
    torch.cuda.synchronize()
    kh, vh, o = kh.cpu().numpy(), vh.cpu().numpy(), out.cpu().numpy()
    res = {"format": K.FORMAT_NAMES[fmt] + ("_4over6" if flags else "")}
    for side, x, xh in (("k", w.k16, kh), ("v", w.v16, vh)):
        r = tensor_metrics(x, xh)
        if fmt in TOP_CODE:
            r["scale_distribution"] = scale_distribution(xh, TOP_CODE[fmt])
        hh = by_head(x, xh)
        r["nmse_by_head"] = {"max": max(hh), "min": min(hh), "values": hh}
        r["nmse_by_position"] = by_position(x, xh, w.T)
        res[side] = r
    o_ref = _reference_attention(w.q16, w.k16, w.v16, w.B, w.T, sp.Hq // sp.Hkv, sm)
    res["attention_output"] = attention_metrics(o, o_ref)
    return res


FORMATS_OF = {
    "glossary_int8": [(2, 0), (3, 0), (1, 0), (6, 0), (4, 0), (4, 1), (7, 0)],
    "fp8_sink_4k": [(1, 0), (3, 0), (2, 0), (6, 0), (4, 0), (4, 1), (7, 0)],
    "int8_32k": [(2, 0), (3, 0), (6, 0), (4, 0), (7, 0)],
    "nvfp4_16k": [(4, 0), (4, 1), (7, 0), (3, 0), (2, 0), (6, 0)],
    "kvarn_16k": [(5, 0), (2, 0), (4, 0), (7, 0), (6, 0)],
}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="fp8_sink_4k", choices=sorted(FORMATS_OF))
    ap.add_argument("--seqs", type=int, default=2, help="sequences of the workload to draw (full context each)")
    ap.add_argument("--out", default=None, help="also write the JSON report to this file")
    args = ap.parse_args(argv)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import quantized_decode_attention_amd as K
    import workloads
    w = workloads.make(args.workload, B=min(args.seqs, workloads.SPECS[args.workload].B))
    rep = {"workload": args.workload, "sequences": w.B, "context": w.T,
           "formats": [report_format(K, w, f, fl) for f, fl in FORMATS_OF[args.workload]
                       if f != 5 or (w.spec.D == 128 and w.spec.P == 128)]}
    text = json.dumps(rep, indent=1)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")
    print(text)
    return rep


if __name__ == "__main__":
    main()
