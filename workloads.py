"""Seeded synthetic inputs for the KV-cache quantisation hot path.

This module holds no part of the method's arithmetic: it only draws random
K/V/Q tensors, block tables and slot mappings with the shapes and value
distributions of the five workloads below, and picks the per-layer scale
arguments the way a calibration checkpoint would (host-side max|x| divided by
the format's top value).  Both the CPU oracle and the GPU library consume the
exact same binary16 arrays.

Workloads (drawn with numpy's PCG64: K and V in fixed chunks of 2^22 values, each
from its own child of the stated seed's SeedSequence; cast to binary16 with
round-to-nearest-even):

  glossary_int8   B=2, H_q=H_kv=4, T=16, D=32, page 16, seed 137.  q, k, v are
                  drawn with torch.manual_seed(137) / torch.randn in the order
                  q, k, v as the glossary's fake-quant script does, then rounded
                  to binary16.
  fp8_sink_4k     B=32, 32q/8kv, T=4096, D=128, page 16, seed 2002; K, V ~ N(0,1)
                  with token 0 of every sequence scaled x20 (attention sink).
  int8_32k        B=8, 64q/8kv, T=32768, D=128, page 16, seed 3003; K, V ~ N(0,1)
                  with 10 of the 1024 (kv head, channel) columns scaled x10,
                  drawn separately for K and V.
  nvfp4_16k       B=16, 64q/8kv, T=16384, D=128, page 16, seed 4004; K, V ~
                  Student-t with 4 degrees of freedom (drawn as Z / sqrt(chi2_4 / 4)).
  kvarn_16k       B=16, 64q/8kv, T=16384, D=128, page 128, seed 5005; K, V ~ N(0,1)
                  with 10 of the 1024 columns scaled x8.
  nvfp4_16k_tp2,  one GPU's share of the two 16K workloads under tensor
  kvarn_16k_tp2   parallelism over two GPUs: 32q/4kv, otherwise as above.

Q ~ N(0,1) for all.  The block tables are a random permutation of all pool pages
(exactly B*T/P pages), so every sequence's pages are scattered.
"""
from __future__ import annotations

import dataclasses

import numpy as np

FP8_PER_TENSOR, INT8_PTH, FP8_PTH, NVFP4, KVARN_K4V2_G128 = 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    formats: tuple
    B: int
    Hq: int
    Hkv: int
    T: int
    D: int
    P: int
    seed: int
    dist: str


SPECS = {
    "glossary_int8": Spec("glossary_int8", (INT8_PTH,), 2, 4, 4, 16, 32, 16, 137, "glossary"),
    "fp8_sink_4k": Spec("fp8_sink_4k", (FP8_PER_TENSOR, FP8_PTH), 32, 32, 8, 4096, 128, 16, 2002, "sink20"),
    "int8_32k": Spec("int8_32k", (INT8_PTH,), 8, 64, 8, 32768, 128, 16, 3003, "chan10"),
    "nvfp4_16k": Spec("nvfp4_16k", (NVFP4,), 16, 64, 8, 16384, 128, 16, 4004, "student_t4"),
    "kvarn_16k": Spec("kvarn_16k", (KVARN_K4V2_G128,), 16, 64, 8, 16384, 128, 128, 5005, "chan8"),
    # one GPU's share of the 16K workloads under tensor parallelism over two
    # GPUs (half the kv heads, each with all of its query heads)
    "nvfp4_16k_tp2": Spec("nvfp4_16k_tp2", (NVFP4,), 16, 32, 4, 16384, 128, 16, 4004, "student_t4"),
    "kvarn_16k_tp2": Spec("kvarn_16k_tp2", (KVARN_K4V2_G128,), 16, 32, 4, 16384, 128, 128, 5005, "chan8"),
}


@dataclasses.dataclass
class Workload:
    spec: Spec
    B: int
    T: int
    k16: np.ndarray        # [B*T, Hkv, D] float16, sequence-major token order
    v16: np.ndarray
    q16: np.ndarray        # [B, Hq, D] float16
    block_tables: np.ndarray  # [B, T/P] int32
    ctx_lens: np.ndarray   # [B] int32
    slots: np.ndarray      # [B*T] int64
    num_pages: int
    k_amax: float          # host max|K| over the tensor (binary32)
    v_amax: float

    def per_tensor_scales(self, fmt):
        """Per-layer scale arguments standing in for checkpoint scales:
        max|x| / 448 for FP8 per-tensor, max|x| / (448 * 6) for the NVFP4
        global scale (block scales then fit E4M3), 1.0 otherwise."""
        if fmt == FP8_PER_TENSOR:
            return float(np.float32(self.k_amax) / np.float32(448.0)), float(np.float32(self.v_amax) / np.float32(448.0))
        if fmt == NVFP4:
            return float(np.float32(self.k_amax) / np.float32(2688.0)), float(np.float32(self.v_amax) / np.float32(2688.0))
        return 1.0, 1.0


_CHUNK = 1 << 22  # elements per independently seeded chunk


def _fill(ss, n, dist, out):
    """Draw n binary32 values into out from seed sequence ss, in fixed chunks
    (chunk i uses ss.spawn(...)[i]), so the values do not depend on how many
    threads draw them."""
    import concurrent.futures as cf
    import os
    kids = ss.spawn((n + _CHUNK - 1) // _CHUNK)

    def one(i):
        rng = np.random.default_rng(kids[i])
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        seg = out[lo:hi]
        if dist == "student_t4":
            # Student-t with 4 degrees of freedom as Z / sqrt(chi2_4 / 4) with
            # chi2_4 = 2 * Gamma(2, 1): the textbook construction, in binary32
            rng.standard_normal(out=seg, dtype=np.float32)
            g = rng.standard_gamma(2.0, size=hi - lo, dtype=np.float32)
            np.multiply(g, np.float32(0.5), out=g)
            np.sqrt(g, out=g)
            np.divide(seg, g, out=seg)
        else:
            rng.standard_normal(out=seg, dtype=np.float32)

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, range(len(kids))))


def _to_half(x):
    """binary32 -> binary16, round-to-nearest-even (torch's multi-threaded cast)."""
    import torch
    return torch.from_numpy(x).to(torch.float16).numpy()


def _absmax(x16):
    import torch
    return float(torch.from_numpy(x16).abs().max().float())


def make(name: str, B: int | None = None, T: int | None = None, seed: int | None = None) -> Workload:
    """Draw a workload.  B and T may be reduced for tests (same distribution);
    seed overrides the spec's seed."""
    sp = SPECS[name]
    B = sp.B if B is None else B
    T = sp.T if T is None else T
    seed = sp.seed if seed is None else seed
    assert T % sp.P == 0, "contexts are whole pages"
    H, D = sp.Hkv, sp.D
    ss = np.random.SeedSequence(seed)
    ss_k, ss_v, ss_rest = ss.spawn(3)
    rng = np.random.default_rng(ss_rest)
    if sp.dist == "glossary":
        import torch
        g = torch.Generator().manual_seed(seed)
        q = torch.randn(B, sp.Hq, 1, D, generator=g, dtype=torch.float32)
        k = torch.randn(B, H, T, D, generator=g, dtype=torch.float32)
        v = torch.randn(B, H, T, D, generator=g, dtype=torch.float32)
        q16 = q[:, :, 0, :].numpy().astype(np.float16)
        k16 = k.permute(0, 2, 1, 3).reshape(B * T, H, D).numpy().astype(np.float16)
        v16 = v.permute(0, 2, 1, 3).reshape(B * T, H, D).numpy().astype(np.float16)
    else:
        n = B * T * H * D
        k = np.empty(n, np.float32)
        _fill(ss_k, n, sp.dist, k)
        v = np.empty(n, np.float32)
        _fill(ss_v, n, sp.dist, v)
        k = k.reshape(B, T, H, D)
        v = v.reshape(B, T, H, D)
        q16 = rng.standard_normal((B, sp.Hq, D), dtype=np.float32).astype(np.float16)
        if sp.dist == "sink20":
            k[:, 0] *= np.float32(20.0)
            v[:, 0] *= np.float32(20.0)
        elif sp.dist in ("chan10", "chan8"):
            f = np.float32(10.0 if sp.dist == "chan10" else 8.0)
            for x in (k, v):
                cols = rng.choice(H * D, size=10, replace=False)
                mult = np.ones(H * D, np.float32)
                mult[cols] = f
                xv = x.reshape(B * T, H * D)
                np.multiply(xv, mult, out=xv)
        k16 = _to_half(k.reshape(B * T, H, D))
        del k
        v16 = _to_half(v.reshape(B * T, H, D))
        del v
    pages_per_seq = T // sp.P
    num_pages = B * pages_per_seq
    perm = rng.permutation(num_pages).astype(np.int32)
    block_tables = perm.reshape(B, pages_per_seq)
    t = np.arange(T, dtype=np.int64)
    slots = (block_tables[:, t // sp.P].astype(np.int64) * sp.P + (t % sp.P)[None, :]).reshape(-1)
    return Workload(sp, B, T, k16, v16, q16, block_tables, np.full(B, T, np.int32), slots,
                    num_pages, _absmax(k16), _absmax(v16))


def random_halves(rng, shape, scale=1.0, dist="normal"):
    """Generic binary16 test data (edge-case generators for tests)."""
    if dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    elif dist == "uniform":
        x = rng.uniform(-scale, scale, size=shape).astype(np.float32)
    else:
        raise ValueError(dist)
    return x.astype(np.float16)
