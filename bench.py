#!/usr/bin/env python3
"""Benchmark of the KV-cache quantisation hot path on one MI355X.

A step is one decode step of the workload: quantise-write the new token of
every sequence and run dequant-fused paged decode attention over the whole
context, new token included, in one call (kvq_decode_attention_append: the
split kernel, whose split-0 workgroups also quantise, store and attend the new
tokens, then the merge kernel when the context is split; KVarN steps append
through kvq_kvarn_append and then call kvq_decode_attention).  The headline
workload is INT8 per-token-head at 32K context (B=8, 64 q / 8 kv heads,
D=128, page 16): `value` is quantised-KV bytes read per second over the timed
steps.  Inputs are resident in HBM before timing starts; the cache is rotated
across copies so the 256 MB last-level cache does not hold the next step's
pages.

Also reported on the same line:
  write_mtok_s   whole-context quantise-on-write throughput (tokens/s / 1e6)
  roofline       the step's decode call (split kernel, which also writes and
                 attends the new tokens, plus the merge): algorithmic KV bytes
                 per call / mean call duration against 8 TB/s.  The duration
                 is the timed region's (one HIP event pair on the launch
                 stream around all the steps) per step, one call per step;
                 `event_timed_call_us` adds the distribution of an
                 instrumented pass right after, with an event pair around
                 each call (an event recorded between two launches holds the
                 next one back, so those read ~2 us long).  A KVarN step also
                 appends, so KVarN's decode calls are timed in a region of
                 their own: the instrumented steps' calls repeated back to
                 back
  copy           a 1 GiB device-to-device copy (read + write bytes / time):
                 the achievable bandwidth beside the specification
  roofline.access_pattern_floor, formats.*.read_floor_gbs
                 the decode's own pages read whole with no arithmetic
                 (libkvq_probe.so, a measurement helper outside libkvq): the
                 access pattern's ceiling
  cpu_baseline   the CPU oracle on a bounded sample of the same workload
  formats        the other formats' workloads (decode GB/s, write Mtok/s), and
                 one GPU's share of the 16K workloads under two-way tensor
                 parallelism (32 q / 4 kv heads); each times at least 200
                 steps (a shorter window makes the 40 us calls noisy)

Warm-up: W untimed steps (default 3000, about 0.3 s) before the timed ones,
and at least 200 ms of back-to-back writes before the write is timed.  The
chip's clocks take that long to settle under sustained load: at 10 warm-up
steps the headline's timed steps ran ~4% slower, and the ALU-bound KVarN
write ~15% slower right after the host-side set-up.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn quantised-KV GB/s (% of HBM peak) + quantize-write Mtok/s, 1 GPU"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Problem:
    """One workload on the device: inputs, rotated cache copies, workspace."""

    def __init__(self, K, name, fmt, flags=0, copies=0, min_rotation_bytes=1.0e9):
        import numpy as np
        import torch

        import workloads
        t0 = time.time()
        w = workloads.make(name)
        sp = w.spec
        self.w, self.sp, self.fmt, self.flags = w, sp, fmt, flags
        ks, vs = w.per_tensor_scales(fmt)
        self.lay = K.layout(fmt, sp.Hkv, sp.D, sp.P, w.num_pages, ks, vs, flags)
        self.page_bytes = K.kvq_page_bytes(self.lay)
        self.cache_bytes = self.page_bytes * w.num_pages
        self.kv_bytes = w.B * (w.T // sp.P) * self.page_bytes  # read by one decode
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.k, self.v = d(w.k16), d(w.v16)
        self.slots = d(w.slots)
        self.q, self.bt, self.ctx = d(w.q16), d(w.block_tables), d(w.ctx_lens)
        # the step's new token: the last position of every sequence
        last = np.arange(w.B) * w.T + (w.T - 1)
        self.k_new, self.v_new = d(w.k16[last]), d(w.v16[last])
        self.slots_new = d(w.slots[last])
        n = copies or max(2, math.ceil(min_rotation_bytes / self.cache_bytes))
        self.caches = [torch.zeros(self.cache_bytes, dtype=torch.uint8, device="cuda") for _ in range(n)]
        self.ws = K.DecodeWorkspace(self.lay, w.B, sp.Hq, w.block_tables.shape[1])
        self.out = torch.empty((w.B, sp.Hq, sp.D), dtype=torch.float16, device="cuda")
        self.sm = 1.0 / math.sqrt(sp.D)
        self.K = K
        self.kvarn = fmt == K.KVQ_KVARN_K4V2_G128
        torch.cuda.synchronize()
        log(f"[bench] {name} fmt={fmt} flags={flags}: inputs ready in {time.time() - t0:.1f}s, "
            f"cache {self.cache_bytes / 1e6:.1f} MB x {n} copies, {self.ws.num_splits} splits")

    def write_all(self, i):
        self.K.kvq_quantize_write(self.lay, self.k, self.v, self.slots, self.caches[i % len(self.caches)])

    def prepare_incremental(self, n_steps):
        """KVarN decode steps: contexts start n_steps tokens short of the full
        length; step i appends one token per sequence through the binary16
        tail (kvq_kvarn_append, completing a tile when it fills) and decodes
        over the complete tiles plus the tail.  Every cache copy has its own
        tail, prefilled with the tile that holds the first position, so each
        copy stays consistent whichever steps it serves."""
        import numpy as np
        import torch
        w, sp, P = self.w, self.sp, self.sp.P
        n_steps = max(1, min(n_steps, w.T - 1))
        c0 = w.T - n_steps
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        t0 = c0 // P * P  # first position of the tile holding c0
        tail = np.zeros((w.B, 2, sp.Hkv, P, sp.D), np.float16)
        for b in range(w.B):
            rows = b * w.T + t0 + np.arange(P)
            tail[b, 0] = w.k16[rows].transpose(1, 0, 2)
            tail[b, 1] = w.v16[rows].transpose(1, 0, 2)
        self.tails = [d(tail) for _ in self.caches]
        pos = c0 + np.arange(n_steps)
        rows = (np.arange(w.B)[None, :] * w.T + pos[:, None]).reshape(-1)
        self.k_steps = d(w.k16[rows].reshape(n_steps, w.B, sp.Hkv, sp.D))
        self.v_steps = d(w.v16[rows].reshape(n_steps, w.B, sp.Hkv, sp.D))
        self.pos_steps = d(np.repeat(pos[:, None], w.B, axis=1).astype(np.int32))
        self.ctx_steps = d(np.repeat(pos[:, None] + 1, w.B, axis=1).astype(np.int32))
        self.seq = d(np.arange(w.B, dtype=np.int32))
        ctx = pos + 1
        tile_bytes = (ctx // P) * self.page_bytes
        tail_bytes = (ctx % P) * sp.Hkv * 2 * sp.D * 2
        self.step_kv_bytes = w.B * (tile_bytes + tail_bytes)  # per step: pages + binary16 tail
        self.n_inc = n_steps

    def prepare_calls(self, n):
        """The library calls of steps 0 .. n-1 with their arguments marshalled
        now, so a timed step costs one C call per entry point on the host.
        Step i uses cache copy i % copies (and, for KVarN, the i-th appended
        token and context length)."""
        K, nc = self.K, len(self.caches)
        if self.kvarn:
            self.append_calls = [K.prepare_kvarn_append(self.lay, self.k_steps[i], self.v_steps[i], self.seq,
                                                        self.pos_steps[i], self.tails[i % nc], self.bt,
                                                        self.caches[i % nc]) for i in range(n)]
            self.decode_calls = [K.prepare_decode_attention(self.lay, self.caches[i % nc], self.q, self.bt,
                                                            self.ctx_steps[i], self.sm, self.out, self.ws.buffer,
                                                            self.tails[i % nc]) for i in range(n)]
        else:
            calls = [K.prepare_decode_attention_append(self.lay, c, self.k_new, self.v_new, self.slots_new, self.q,
                                                       self.bt, self.ctx, self.sm, self.out, self.ws.buffer)
                     for c in self.caches]
            self.step_calls = [calls[i % nc] for i in range(n)]

    def step(self, i):
        """One decode step: KVarN appends through its binary16 tail and then
        decodes (two calls); the other formats quantise-write the new tokens
        and decode in one call (kvq_decode_attention_append)."""
        if self.kvarn:
            self.append_calls[i]()
            self.decode_calls[i]()
        else:
            self.step_calls[i]()

    def time_write(self, reps=10, warm_ms=200.0):
        """Median of `reps` whole-context writes, each timed by an event pair,
        after at least `warm_ms` of back-to-back writes: the chip's clocks
        need that long under sustained load to settle (ALU-bound writes run up
        to ~15% slower right after the host-side set-up)."""
        import torch
        t0, i = time.perf_counter(), 0
        while i < len(self.caches) or (time.perf_counter() - t0) * 1e3 < warm_ms:
            self.write_all(i)
            i += 1
            if i % 8 == 0:
                torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(ev):
            a.record()
            self.write_all(i)
            b.record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
        n_tok = self.w.B * self.w.T
        return n_tok / (ms * 1e-3) / 1e6, ms

    def time_steps(self, steps, warmup):
        """Timed decode steps; returns (ms per step, mean decode call ms).
        The timed region is `steps` steps bracketed by one event pair: an
        event recorded between two launches holds the next launch back by a
        few microseconds, so per-call events stay out of it.  The per-call
        durations come from an instrumented pass of `steps` more steps right
        after it (an event pair around every decode call).  The step index
        keeps counting across warm-up, timed and instrumented steps."""
        import torch
        if self.kvarn:
            if warmup + 2 * steps > self.w.T - 1:
                raise SystemExit(f"bench: a KVarN workload appends one token per step, so warm-up + 2 x steps "
                                 f"({warmup + 2 * steps}) must stay below its context ({self.w.T})")
            self.prepare_incremental(warmup + 2 * steps)
        self.prepare_calls(warmup + 2 * steps)
        torch.cuda.synchronize()
        for i in range(warmup):
            self.step(i)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            self.step(warmup + i)
        end.record()
        torch.cuda.synchronize()
        total = start.elapsed_time(end)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            j = warmup + steps + i
            if self.kvarn:
                self.append_calls[j]()
                ev[i][0].record()
                self.decode_calls[j]()
            else:
                ev[i][0].record()
                self.step(j)
            ev[i][1].record()
        torch.cuda.synchronize()
        self.dec_region_ms = None
        if self.kvarn:
            # the instrumented steps' decode calls once more, back to back in
            # one event pair: the same work per call (same tiles and tail
            # rows) without an event between launches
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(steps):
                self.decode_calls[warmup + steps + i]()
            b.record()
            torch.cuda.synchronize()
            self.dec_region_ms = a.elapsed_time(b) / steps
        if self.kvarn:  # mean KV bytes (tiles + binary16 tail) of the timed and of the instrumented steps
            self.kv_bytes = int(self.step_kv_bytes[warmup:warmup + steps].mean())
            self.call_kv_bytes = int(self.step_kv_bytes[warmup + steps:warmup + 2 * steps].mean())
        else:
            self.call_kv_bytes = self.kv_bytes
        self.dec_ms = sorted(a.elapsed_time(b) for a, b in ev)
        return total / steps, sum(self.dec_ms) / len(self.dec_ms)

    def time_read_floor(self, reps=20):
        """The decode's access pattern with no arithmetic (libkvq_probe.so):
        every (page, kv head) chunk of the cache read whole, split as the
        decode splits it, over the same rotated cache copies.  Returns GB/s of
        cache bytes read per launch (the decode's algorithmic bytes)."""
        import ctypes

        import torch
        L = read_probe_lib()
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        chunk = self.page_bytes // self.sp.Hkv
        if self.kvarn:
            chunk = chunk // (self.sp.P // 128)  # one 128-token tile per unit of the walk
        splits = max(1, self.ws.num_splits)
        # the decode's eight-wave single-split plan (see decode_kernel_name)
        waves = 8 if splits == 1 and self.fmt in (1, 2, 3) and self.w.B * self.sp.Hkv >= 256 else 4

        def go(i):
            rc = L.kvq_probe_read_pattern(ctypes.c_void_p(self.caches[i % len(self.caches)].data_ptr()),
                                          ctypes.c_void_p(self.bt.data_ptr()), self.w.B, self.sp.Hkv,
                                          self.w.block_tables.shape[1], chunk, self.w.num_pages, splits, waves,
                                          ctypes.c_void_p(sink.data_ptr()), stream)
            assert rc == 0, rc
        for i in range(3):
            go(i)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(ev):
            a.record()
            go(i)
            b.record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
        nbytes = self.w.B * (self.w.T // self.sp.P) * self.page_bytes
        return nbytes / (ms * 1e-3) / 1e9, ms * 1e3

    def dec_percentiles_us(self):
        d = self.dec_ms
        pick = lambda f: round(d[min(len(d) - 1, int(f * len(d)))] * 1e3, 2)
        return {"p10_us": pick(0.1), "p50_us": pick(0.5), "p90_us": pick(0.9)}

    def call_ms(self, ms_step, ms_dec):
        """Mean duration of the decode call, from one event pair around
        back-to-back calls.  Every format but KVarN runs one call per step, so
        it is the timed region's time per step.  A KVarN step also appends
        through the tail, so its decode calls are timed in a region of their
        own: the instrumented steps' calls run once more back to back (an
        event pair around each call holds the next launch back and reads
        ~2 us long)."""
        return self.dec_region_ms if self.kvarn else ms_step

    def call_timing(self):
        return ("HIP event pair around the instrumented steps' decode calls, repeated back to back" if self.kvarn
                else "HIP event pair around the timed steps, one decode call per step")


_READ_PROBE = None


def read_probe_lib():
    """libkvq_probe.so: the benchmark's access-pattern read helper (built with
    the library; not part of libkvq)."""
    global _READ_PROBE
    if _READ_PROBE is None:
        import ctypes
        path = os.path.join(ROOT, "quantized_decode_attention_amd", "libkvq_probe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python quantized_decode_attention_amd/_build.py`")
        L = ctypes.CDLL(path)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.kvq_probe_read_pattern.restype = I
        L.kvq_probe_read_pattern.argtypes = [P, P, I, I, I, I, I, I, I, P, P]
        _READ_PROBE = L
    return _READ_PROBE


def copy_bandwidth(nbytes=1 << 30, reps=10):
    """Device-to-device copy of a known size (read + write counted): the
    achievable HBM reference beside the 8 TB/s specification, and the
    calibration kernel for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "gbs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
            "us": round(ms * 1e3, 2)}


# HBM traffic of every workload's decode call and whole-context write,
# measured with rocprofv3 counters and kept in a profile summary together with
# a digest of the kernels' sources: a figure is reported only while those
# sources are unchanged (comments and blank lines aside).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_all_formats.md")
# every source a decode call or a write launch compiles from, and the build flags
KERNEL_SOURCES = ("decode_attn.hip", "quant_write.hip", "kvarn_decode.hip", "kvarn_write.hip", "decode_common.h",
                  "row_encode.h", "kvq_device.h", "kvq_internal.h")


def _code_only(text):
    """Source text without // and /* */ comments, blank lines or trailing
    blanks (string literals in these sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_sources_digest():
    import hashlib

    from quantized_decode_attention_amd import _build
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(_build.CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    for src in ("decode_attn.hip", "quant_write.hip", "kvarn_decode.hip", "kvarn_write.hip"):
        h.update(" ".join(_build.SOURCES[src]).encode())
    h.update(" ".join(_build.COMMON[:4]).encode())
    return h.hexdigest()


def _traffic_table():
    """{(key, what): bytes} from the summary's machine-readable lines
    `traffic <key> <decode|write> = <bytes>`, or {} when the digest no longer
    matches the sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    vals, digest = {}, None
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.strip().strip("`").split(" = ")
            if len(parts) != 2:
                continue
            lhs, rhs = parts[0].split(), parts[1].strip()
            if lhs == ["kernel_sources_sha256"]:
                digest = rhs
            elif len(lhs) == 3 and lhs[0] == "traffic":
                try:
                    vals[(lhs[1], lhs[2])] = int(rhs)
                except ValueError:
                    pass
    return vals if digest == kernel_sources_digest() else {}


def measured_traffic(key, what="decode"):
    """HBM bytes per decode call (or per whole-context write) of a workload
    entry (`workload/format`), from the committed counter summary; None when
    there is none or the kernels changed since the counters were taken."""
    return _traffic_table().get((key, what))


def cpu_formats(K):
    """The other formats' workloads for --cpu-formats (the headline's is added first)."""
    return [("fp8_sink_4k", K.KVQ_FP8_PER_TENSOR, 0), ("fp8_sink_4k", K.KVQ_FP8_PTH, 0),
            ("nvfp4_16k", K.KVQ_NVFP4, 0), ("nvfp4_16k", K.KVQ_NVFP4, K.KVQ_FLAG_NVFP4_4OVER6),
            ("nvfp4_16k", K.KVQ_MXFP4, 0), ("kvarn_16k", K.KVQ_KVARN_K4V2_G128, 0),
            ("int8_32k", K.KVQ_INT4_PTH, 0)]


def cpu_baseline(name, fmt, flags, n_seq, threads):
    """The oracle on a bounded sample of the workload: quantise-write every
    token of n_seq sequences, then decode every q head of those sequences.
    Parallel over (sequence, kv head) units with one thread each (ctypes
    releases the GIL)."""
    import numpy as np

    import oracle
    import workloads
    O = oracle.default()
    w = workloads.make(name, B=n_seq)
    sp = w.spec
    ks, vs = w.per_tensor_scales(fmt)
    lay = oracle.layout(fmt, sp.Hkv, sp.D, sp.P, w.num_pages, ks, vs, flags)
    cache = np.zeros(w.num_pages * O.page_bytes(lay), np.uint8)
    per_seq = w.T
    t0 = time.time()
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda b: O.quantize_write(lay, w.k16[b * per_seq:(b + 1) * per_seq],
                                               w.v16[b * per_seq:(b + 1) * per_seq],
                                               w.slots[b * per_seq:(b + 1) * per_seq], cache), range(n_seq)))
    t_write = time.time() - t0
    G = sp.Hq // sp.Hkv
    units = [(b, h) for b in range(n_seq) for h in range(sp.Hkv)]

    def dec(u):
        b, h = u
        pairs = np.array([(b, h * G + g) for g in range(G)], np.int32)
        return O.decode_attention(lay, cache, w.q16, w.block_tables, w.ctx_lens, 1.0 / math.sqrt(sp.D), pairs=pairs)

    t0 = time.time()
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(dec, units))
    t_dec = time.time() - t0
    kv_bytes = n_seq * (w.T // sp.P) * O.page_bytes(lay)
    return {
        "value": round(kv_bytes / t_dec / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{name}: {n_seq} of {sp.B} sequences, all {sp.Hq} q heads (decode, binary64), "
                   f"after quantise-writing their {n_seq * w.T} tokens (binary32)"),
        "seconds": round(t_dec, 2),
        "write_mtok_s": round(n_seq * w.T / t_write / 1e6, 4),
        "write_seconds": round(t_write, 2),
    }


# format name -> (kvq_format, flags)
FORMAT_CHOICES = {"fp8_per_tensor": (1, 0), "int8_per_token_head": (2, 0), "fp8_per_token_head": (3, 0),
                  "nvfp4": (4, 0), "nvfp4_4over6": (4, 1), "kvarn_k4v2_g128": (5, 0), "int4_per_token_head": (6, 0),
                  "mxfp4": (7, 0)}


WORKLOAD_FORMAT = {"int8_32k": "int8_per_token_head", "fp8_sink_4k": "fp8_per_token_head", "nvfp4_16k": "nvfp4",
                   "kvarn_16k": "kvarn_k4v2_g128", "nvfp4_16k_tp2": "nvfp4", "kvarn_16k_tp2": "kvarn_k4v2_g128"}


def main_format(workload, fmt_name=""):
    """(kvq_format, flags) of the main workload: its own format, or the one
    named; None for an unknown name or a KVarN / paged-format mismatch."""
    if workload not in WORKLOAD_FORMAT:
        return None
    f = FORMAT_CHOICES.get(fmt_name or WORKLOAD_FORMAT[workload])
    if f is None or (f[0] == 5) != workload.startswith("kvarn"):
        return None
    return f


def entry_key(K, name, fmt, flags):
    """`workload/format` key of a bench entry (and of its traffic figures)."""
    return f"{name}/{K.FORMAT_NAMES[fmt]}" + ("_4over6" if flags else "")


def decode_kernel_name(p):
    """The kernels of one decode call of a bench entry."""
    G = p.sp.Hq // p.sp.Hkv
    if p.kvarn:
        return f"kvarn_decode_kernel<{G}> + kvarn_merge_kernel<{G}>"
    # eight-wave workgroups when the plan runs a single split over at least
    # one (sequence, kv head) per compute unit (kvq.h)
    waves = 8 if p.ws.num_splits == 1 and p.fmt in (1, 2, 3) and p.w.B * p.sp.Hkv >= 256 else 4
    return (f"decode_kernel<{p.fmt}, {p.sp.D}, {G}, {waves}>"
            + (" + decode_merge_kernel" if p.ws.num_splits > 1 else ""))


def write_bytes(p):
    """Bytes a whole-context write moves: the binary16 K and V read, the cache written."""
    w, sp = p.w, p.sp
    return 2 * w.B * w.T * sp.Hkv * sp.D * 2 + w.B * (w.T // sp.P) * p.page_bytes


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3000,
                    help="untimed steps first (the default, ~0.3 s of steps, lets the clocks settle under load)")
    ap.add_argument("--workload", default="int8_32k", choices=sorted(WORKLOAD_FORMAT))
    ap.add_argument("--format", default="", help="format of the main workload (default: the workload's own; "
                    "one of " + ", ".join(FORMAT_CHOICES) + ")")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-formats", action="store_true", help="skip the other formats' workloads")
    ap.add_argument("--cpu-seqs", type=int, default=0, help="sequences of the CPU baseline (0 = the whole batch)")
    ap.add_argument("--cpu-formats", action="store_true",
                    help="also time the oracle on every format's workload (whole batch on the host threads, "
                         "and one sequence on one thread); adds about a minute")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py measures one GPU: the hot path shards by (sequence, kv head) with no exchange, and this "
            "build runs and reports a single MI355X only.  Use --gpus 1.")
        sys.exit(2)

    main_fmt = main_format(args.workload, args.format)
    if main_fmt is None:
        log(f"no format {args.format!r} for workload {args.workload!r}: KVarN runs only on the kvarn workloads "
            f"(page 128) and they only with KVarN; formats: {', '.join(FORMAT_CHOICES)}")
        sys.exit(2)

    import torch

    import quantized_decode_attention_amd as K
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    st = K.kvq_check_device(0)
    if st != 0:
        log(f"device check failed: {K.kvq_status_string(st)}")
        sys.exit(1)


    pb = Problem(K, args.workload, *main_fmt)
    write_mtok, write_ms = pb.time_write()
    log(f"[bench] whole-context write: {write_mtok:.1f} Mtok/s ({write_ms:.3f} ms)")
    ms_step, ms_dec = pb.time_steps(args.steps, args.warmup)
    floor_gbs, floor_us = pb.time_read_floor()
    log(f"[bench] access-pattern read floor: {floor_us:.1f} us ({floor_gbs:.0f} GB/s)")
    value = pb.kv_bytes / (ms_step * 1e-3) / 1e9
    ms_call = pb.call_ms(ms_step, ms_dec)
    achieved = pb.call_kv_bytes / (ms_call * 1e-3) / 1e9
    log(f"[bench] step {ms_step * 1e3:.1f} us ({value:.0f} GB/s), decode call {ms_call * 1e3:.1f} us "
        f"({achieved:.0f} GB/s, {achieved / HBM_PEAK_GBS:.1%} of peak); per-call events {ms_dec * 1e3:.1f} us")
    sp, w = pb.sp, pb.w
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma/f32-acc",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "format": K.FORMAT_NAMES[pb.fmt], "batch": w.B, "context": w.T,
            "q_heads": sp.Hq, "kv_heads": sp.Hkv, "head_dim": sp.D, "page_size": sp.P,
            "splits": pb.ws.num_splits, "cache_copies": len(pb.caches),
            "step": "quantize-write 1 new token per sequence + paged decode attention over the context "
                    "(one kvq_decode_attention_append call)",
        },
        "kv_bytes_per_step": pb.kv_bytes,
        "write_mtok_s": round(write_mtok, 2),
        "write_gbs": round(write_bytes(pb) / (write_ms * 1e-3) / 1e9, 2),
        "write_frac_of_peak": round(write_bytes(pb) / (write_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "write_traffic": measured_traffic(entry_key(K, args.workload, *main_fmt), "write"),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(entry_key(K, args.workload, *main_fmt)),
            # eight-wave workgroups when the plan runs a single split over
            # at least one (sequence, kv head) per compute unit (kvq.h)
            "kernel": decode_kernel_name(pb),
            "algorithmic_bytes": pb.call_kv_bytes, "traffic_unit": "HBM bytes per decode call (rocprofv3 "
            "FETCH_SIZE and WRITE_SIZE, each scaled by its reading for a 1 GiB device copy)",
            "mean_launch_us": round(ms_call * 1e3, 2), "timing": pb.call_timing(),
            # the instrumented pass right after the timed steps: an event pair
            # around each call (upper bounds: an event between two launches
            # holds the next one back)
            "event_timed_call_us": {"mean": round(ms_dec * 1e3, 2), **pb.dec_percentiles_us()},
            # the same pages read whole with no arithmetic (libkvq_probe.so):
            # the access pattern's own ceiling beside the 8 TB/s specification
            "access_pattern_floor": {"gbs": round(floor_gbs, 1), "us": round(floor_us, 2),
                                     "frac_of_peak": round(floor_gbs / HBM_PEAK_GBS, 4)},
        },
    }
    del pb
    torch.cuda.empty_cache()
    result["copy"] = copy_bandwidth()
    log(f"[bench] device copy: {result['copy']}")

    if not args.no_formats:
        fmts = {}
        others = [("fp8_sink_4k", K.KVQ_FP8_PER_TENSOR, 0), ("fp8_sink_4k", K.KVQ_FP8_PTH, 0),
                  ("nvfp4_16k", K.KVQ_NVFP4, 0), ("nvfp4_16k", K.KVQ_NVFP4, K.KVQ_FLAG_NVFP4_4OVER6),
                  ("nvfp4_16k", K.KVQ_MXFP4, 0), ("kvarn_16k", K.KVQ_KVARN_K4V2_G128, 0),
                  ("int8_32k", K.KVQ_INT4_PTH, 0),
                  ("nvfp4_16k_tp2", K.KVQ_NVFP4, 0), ("kvarn_16k_tp2", K.KVQ_KVARN_K4V2_G128, 0)]
        for name, fmt, flags in others:
            if name == args.workload and fmt == main_fmt[0] and flags == main_fmt[1]:
                continue
            p = Problem(K, name, fmt, flags)
            wm, wms = p.time_write()
            ms_s, ms_d = p.time_steps(max(200, args.steps), args.warmup)
            fl_gbs, _ = p.time_read_floor()
            key = K.FORMAT_NAMES[fmt] + ("_4over6" if flags else "") + ("_tp2_share" if name.endswith("_tp2") else "")
            ms_c = p.call_ms(ms_s, ms_d)
            fmts[key] = {"workload": name, "decode_gbs": round(p.call_kv_bytes / (ms_c * 1e-3) / 1e9, 1),
                         "decode_frac_of_peak": round(p.call_kv_bytes / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "decode_us": round(ms_c * 1e3, 2), "decode_timing": p.call_timing(),
                         "event_timed_call_us": {"mean": round(ms_d * 1e3, 2), **p.dec_percentiles_us()},
                         "step_us": round(ms_s * 1e3, 2),
                         "write_mtok_s": round(wm, 1),
                         "write_frac_of_peak": round(write_bytes(p) / (wms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(entry_key(K, name, fmt, flags)),
                         "write_traffic": measured_traffic(entry_key(K, name, fmt, flags), "write"),
                         "algorithmic_bytes": p.call_kv_bytes, "splits": p.ws.num_splits,
                         "read_floor_gbs": round(fl_gbs, 1),
                         "step": ("append to the binary16 tail (tile quantised when complete) + decode over "
                                  "tiles and tail" if fmt == K.KVQ_KVARN_K4V2_G128
                                  else "write + decode in one kvq_decode_attention_append call")}
            log(f"[bench] {key}: {fmts[key]}")
            del p
            torch.cuda.empty_cache()
        result["formats"] = fmts

    if not args.no_cpu_baseline:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        log(f"[bench] CPU oracle baseline on {threads} threads ...")
        import workloads
        n_seq = args.cpu_seqs or workloads.SPECS[args.workload].B
        result["cpu_baseline"] = cpu_baseline(args.workload, *main_fmt, n_seq, threads)
    if args.cpu_formats:
        import workloads
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        cpu = {}
        for name, fmt, flags in [(args.workload, *main_fmt)] + cpu_formats(K):
            key = f"{name}/{K.FORMAT_NAMES[fmt]}" + ("_4over6" if flags else "")
            log(f"[bench] oracle timing {key} ...")
            cpu[key] = {"all_threads": cpu_baseline(name, fmt, flags, workloads.SPECS[name].B, threads),
                        "one_thread": cpu_baseline(name, fmt, flags, 1, 1)}
        result["cpu_formats"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
