"""Pins of the CPU oracle against what the pages and mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError on
a violation, so the same checks run against the real oracle
(test_oracle_pins.py) and against deliberately broken builds of it
(test_oracle_mutants.py).  None of them re-types the oracle's formula: they use
library routines (numpy / torch / scipy), brute force, closed forms, exact
invariants or the pages' printed numbers.
"""
from __future__ import annotations

import math
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32 = np.float32


def golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            vals.setdefault(parts[0], []).append(parts[1:])
    return vals


def _torch_e4m3(y):
    """Library E4M3 encoding (torch, round-to-nearest-even; NaN above 464)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_decode(codes):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


def _e2m1_brute(y):
    """Nearest of the 15 signed E2M1 values by exhaustive search; sign kept on
    zero; ties to the even code."""
    grid = [float(g) for g in golden("e2m1_grid.txt")["0"][0]]
    grid = [0.0] + grid  # the line starts with 0; first token consumed as key
    out = []
    for v in np.asarray(y, np.float64).ravel():
        neg = math.copysign(1.0, v) < 0
        best, bestd = None, None
        for code in range(8):
            d = abs(abs(v) - grid[code])
            if best is None or d < bestd or (d == bestd and code % 2 == 0 and best % 2 == 1):
                best, bestd = code, d
        out.append(best | (8 if neg else 0))
    return np.array(out, np.uint8)


def _rows(rng, D, n=40):
    """Rows covering the edge cases of per-token-head scaling."""
    rows = [workloads.random_halves(rng, (D,)) for _ in range(n)]
    rows.append(np.zeros(D, np.float16))
    one = np.zeros(D, np.float16)
    one[D // 3] = 3.0
    rows.append(one)
    out = workloads.random_halves(rng, (D,), 0.01)
    out[5] = 1000.0
    rows.append(out)
    rows.append(workloads.random_halves(rng, (D,), 1e-6))
    big = workloads.random_halves(rng, (D,), 6e4, "uniform")
    big[0] = 65504.0
    rows.append(big)
    rows.append(np.full(D, -2.0, np.float16))
    rows.append(np.arange(1, D + 1).astype(np.float16) * np.float16(2.0 ** -24))  # subnormal halves
    rows.append(workloads.random_halves(rng, (D,), 3.0, "uniform"))
    return rows


# --------------------------------------------------------------------------- #
# number formats
# --------------------------------------------------------------------------- #

def pin_half_widening(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([O.half_to_float(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def pin_e4m3_decode(O):
    codes = np.arange(256, dtype=np.uint8)
    ref = _torch_e4m3_decode(codes)
    got = np.array([O.e4m3_decode(int(c)) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def _e4m3_probe_values(rng):
    finite = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    finite = finite[np.isfinite(finite)]
    grid = _torch_e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    mids = mids.astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))])
    rnd = rng.uniform(-470, 470, 20000).astype(np.float32)
    small = (rng.standard_normal(5000) * 0.01).astype(np.float32)
    return np.concatenate([finite, near, -near, rnd, small, np.float32([0.0, -0.0, 448.0, 464.0, -500.0])])


def pin_e4m3_encode(O, rng=None):
    rng = rng or np.random.default_rng(1)
    y = _e4m3_probe_values(rng)
    got = np.array([O.e4m3_encode(float(v)) for v in y], np.uint8)
    sat = np.abs(y) >= 464
    ref = _torch_e4m3(y)
    assert np.array_equal(got[~sat], ref[~sat]), "E4M3 encode differs from torch below 464"
    exp_sat = np.where(np.signbit(y[sat]), 0xFE, 0x7E).astype(np.uint8)
    assert np.array_equal(got[sat], exp_sat), "E4M3 encode must saturate at 448"
    # every finite code round-trips
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert O.e4m3_encode(float(O.e4m3_decode(c))) == c


def pin_e2m1_encode(O, rng=None):
    rng = rng or np.random.default_rng(2)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(9)), np.nextafter(mids, np.float32(-9))])
    sweep = np.arange(-8 * 64, 8 * 64 + 1, dtype=np.float32) / 64
    y = np.concatenate([near, -near, sweep, rng.uniform(-10, 10, 3000).astype(np.float32),
                        np.float32([-0.0, 0.0, -1e-30, 6.0, 6.5, 100.0, -7.0])])
    got = np.array([O.e2m1_encode(float(v)) for v in y], np.uint8)
    ref = _e2m1_brute(y)
    assert np.array_equal(got, ref), f"E2M1 mismatch at {y[got != ref][:5]}"
    # decode reproduces the page's grid
    for c in range(16):
        v = O.e2m1_decode(c)
        assert v == (-1 if c & 8 else 1) * float(grid[c & 7]) or (v == 0 and grid[c & 7] == 0)


# --------------------------------------------------------------------------- #
# row quantisers
# --------------------------------------------------------------------------- #

def pin_int8_pth(O, rng=None):
    rng = rng or np.random.default_rng(3)
    for D in (32, 128):
        for x16 in _rows(rng, D):
            codes, sb = O.quantize_row(oracle.INT8_PTH, x16)
            q = codes.view(np.int8).astype(np.int64)
            s = sb[:4].view(np.float32)[0]
            x = x16.astype(np.float64)
            assert np.isfinite(s) and s > 0
            assert np.all(np.abs(q) <= 127)
            if not np.any(x):
                assert not np.any(q)
                continue
            # brute force: nearest integer in [-127, 127] to fl32(x / s), ties to even
            y = (x16.astype(np.float32) / F32(s)).astype(np.float64)
            cand = np.arange(-127, 128)
            dist = np.abs(y[:, None] - cand[None, :])
            best = dist.min(axis=1, keepdims=True)
            tie_ok = (dist == best) & (cand[None, :] % 2 == 0)
            single = (dist == best).sum(axis=1) == 1
            brute = np.where(single, cand[np.argmin(dist, axis=1)], cand[np.argmax(tie_ok, axis=1)])
            assert np.array_equal(q, brute)
            # rounding moves a value by at most half a step (page: +-0.5 level)
            assert np.all(np.abs(x - float(s) * q) <= float(s) * (0.5 + 2.0 ** -17))
            # the largest magnitude lands on the top code
            i = np.argmax(np.abs(x))
            assert abs(q[i]) == 127


def pin_int4_pth(O, rng=None):
    """INT4 per-token-head (reading: the INT8 rule at 4 bits): brute-force
    nearest code in [-7, 7] with ties to even, the half-step bound, the top
    code, and the cache round trip through the signed nibbles."""
    rng = rng or np.random.default_rng(12)
    for D in (32, 128):
        for x16 in _rows(rng, D):
            codes, sb = O.quantize_row(oracle.INT4_PTH, x16)
            assert np.all(codes < 16)
            q = ((codes.astype(np.int64) ^ 8) - 8)  # two's-complement nibble
            s = sb[:4].view(np.float32)[0]
            x = x16.astype(np.float64)
            assert np.isfinite(s) and s > 0
            assert s == F32(max(F32(np.abs(x16.astype(np.float32)).max()), F32(1e-8))) / F32(7)
            assert np.all(np.abs(q) <= 7)
            if not np.any(x):
                assert not np.any(q)
                continue
            y = (x16.astype(np.float32) / F32(s)).astype(np.float64)
            cand = np.arange(-7, 8)
            dist = np.abs(y[:, None] - cand[None, :])
            best = dist.min(axis=1, keepdims=True)
            tie_ok = (dist == best) & (cand[None, :] % 2 == 0)
            single = (dist == best).sum(axis=1) == 1
            brute = np.where(single, cand[np.argmin(dist, axis=1)], cand[np.argmax(tie_ok, axis=1)])
            assert np.array_equal(q, brute)
            assert np.all(np.abs(x - float(s) * q) <= float(s) * (0.5 + 2.0 ** -17))
            assert abs(q[np.argmax(np.abs(x))]) == 7
    # round trip through the paged cache: x_hat = q * s with the signed codes
    D, P, H = 64, 16, 2
    k = workloads.random_halves(rng, (20, H, D))
    v = workloads.random_halves(rng, (20, H, D), 3.0)
    slots = rng.choice(3 * P, 20, replace=False).astype(np.int64)
    lay = oracle.layout(oracle.INT4_PTH, H, D, P, 3)
    cache = O.quantize_write(lay, k, v, slots)
    kh, vh = O.dequantize(lay, cache, slots)
    for src, got in ((k, kh), (v, vh)):
        for i in range(20):
            for h in range(H):
                codes, sb = O.quantize_row(oracle.INT4_PTH, src[i, h])
                q = ((codes.astype(np.int64) ^ 8) - 8)
                assert np.array_equal(got[i, h], q * float(sb[:4].view(np.float32)[0]))


def _torch_int_pth(x16, qmax):
    """The glossary's per-token-head rule as its script states it, run by torch
    in binary32 on the CPU: |x| maximum floored at 1e-8, then / qmax; codes
    torch.round(x / scale) (half to even), clamped to +-qmax."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x16, dtype=np.float16)).to(torch.float32)
    scale = t.abs().amax(dim=-1, keepdim=True).clamp_min(1e-8) / qmax
    q = torch.round(t / scale).clamp(-qmax, qmax)
    return q.to(torch.int64).numpy(), scale.numpy()[..., 0]


def _finite_halves_upto(M):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    h = h[np.isfinite(h)]
    return h[np.abs(h.astype(np.float64)) <= M]


def _sweep_rows(M, D=128):
    """Every finite binary16 value of magnitude <= M, in rows of D whose first
    entry is M (so M is every row's maximum)."""
    vals = _finite_halves_upto(M)
    n = D - 1
    pad = (-len(vals)) % n
    vals = np.concatenate([vals, np.zeros(pad, np.float16)]).reshape(-1, n)
    return np.concatenate([np.full((len(vals), 1), M, np.float16), vals], axis=1)


# row maxima of the sweep: the exact-tie maxima 127 * 7 * 2^-9, 127 * 13 * 2^-9,
# 127 * 15 * 2^-9 (scale 7, 13, 15 * 2^-9), 7 * 7 (INT4 scale 7), plus plain ones
_SWEEP_MAXIMA = (1.736328125, 3.224609375, 3.720703125, 49.0, 3.0, 0.1, 65504.0, 2.0 ** -24)


def pin_int_rule_order(O):
    """[P3] §可运行 fake-quant 实验 fixes the integer rule's order of operations:
    the maximum is floored at 1e-8 before the division by 127, and values are
    divided by the scale (not multiplied by a reciprocal), rounding half to even.
    Pinned two ways: hand-worked rows whose expected codes and scale bits follow
    from exact rational arithmetic (tests/golden/int_rule_order.txt: all-zero
    rows, a subnormal maximum, exact .5 ties), and torch running the script's
    rule on every finite binary16 value under several row maxima (INT8 and, by
    reading R39, INT4 with 7 for 127), codes and scale bits equal."""
    fmt_of = {127: oracle.INT8_PTH, 7: oracle.INT4_PTH}
    n_lines = 0
    with open(os.path.join(GOLDEN, "int_rule_order.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("->")
            name, qmax, sbits, *vals = lhs.split()
            want = [int(c) for c in rhs.split()]
            x16 = np.zeros(128, np.float16)
            x16[:len(vals)] = [float(v) for v in vals]
            assert np.array_equal(x16[:len(vals)].astype(np.float64), [float(v) for v in vals]), name
            codes, sb = O.quantize_row(fmt_of[int(qmax)], x16)
            q = codes.view(np.int8).astype(np.int64) if int(qmax) == 127 else (codes.astype(np.int64) ^ 8) - 8
            got_bits = int(sb[:4].view(np.uint32)[0])
            assert got_bits == int(sbits, 16), f"{name}/{qmax}: scale bits {got_bits:#010x} != {sbits}"
            assert list(q[:len(want)]) == want, f"{name}/{qmax}: codes {list(q[:len(want)])} != {want}"
            assert not np.any(q[len(vals):]), name
            n_lines += 1
    assert n_lines == 6
    for qmax, fmt in ((127, oracle.INT8_PTH), (7, oracle.INT4_PTH)):
        for M in _SWEEP_MAXIMA:
            rows = _sweep_rows(M)
            rows = np.concatenate([rows, np.zeros((1, 128), np.float16)])
            tq, ts = _torch_int_pth(rows, qmax)
            for i, x16 in enumerate(rows):
                codes, sb = O.quantize_row(fmt, x16)
                q = codes.view(np.int8).astype(np.int64) if qmax == 127 else (codes.astype(np.int64) ^ 8) - 8
                assert sb[:4].view(np.float32)[0].view(np.uint32) == np.float32(ts[i]).view(np.uint32), \
                    (qmax, M, i)
                bad = np.nonzero(q != tq[i])[0]
                assert not len(bad), f"qmax {qmax}, max {M}: x={x16[bad[:3]]} oracle {q[bad[:3]]} torch {tq[i][bad[:3]]}"


def pin_fp8_pth(O, rng=None):
    rng = rng or np.random.default_rng(4)
    for D in (32, 128):
        for x16 in _rows(rng, D):
            codes, sb = O.quantize_row(oracle.FP8_PTH, x16)
            s = sb[:4].view(np.float32)[0]
            x = x16.astype(np.float64)
            assert np.isfinite(s) and s > 0
            y = x16.astype(np.float32) / F32(s)
            assert np.all(np.abs(y) < 464)
            assert np.array_equal(codes, _torch_e4m3(y))
            if not np.any(x):
                continue
            xh = float(s) * _torch_e4m3_decode(codes)
            # half-step bound of E4M3 at the value's binade (2^-10 below 2^-6)
            ay = np.abs(y.astype(np.float64))
            e = np.floor(np.log2(np.maximum(ay, 2.0 ** -6)))
            assert np.all(np.abs(x - xh) <= float(s) * (2.0 ** (e - 4)) * (1 + 2.0 ** -10))
            i = np.argmax(np.abs(x))
            assert codes[i] & 0x7F == 0x7E  # max |x| maps to 448 = FP8_MAX
    # hand-worked exact ties (tests/golden/fp8_pth_ties.txt)
    with open(os.path.join(GOLDEN, "fp8_pth_ties.txt")) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(lines) == 1
    for line in lines:
        lhs, rhs = line.split("->")
        _, sbits, *vals = lhs.split()
        x16 = np.zeros(128, np.float16)
        x16[:len(vals)] = [float(v) for v in vals]
        codes, sb = O.quantize_row(oracle.FP8_PTH, x16)
        assert int(sb[:4].view(np.uint32)[0]) == int(sbits, 16)
        assert [int(c) for c in codes[:len(vals)]] == [int(c, 16) for c in rhs.split()], codes[:len(vals)]
    # every finite binary16 value under row maxima with exact ties (448 * 7, 448 * 13,
    # 448 * 15 * 2^-10) and plain ones: the scale is the page's max / 448 and the
    # codes torch's E4M3 of the true quotient
    for M in (3136.0, 5824.0, 6.5625, 448.0, 1.0):
        for x16 in _sweep_rows(M):
            codes, sb = O.quantize_row(oracle.FP8_PTH, x16)
            s = F32(M) / F32(448)
            assert sb[:4].view(np.float32)[0] == s
            assert np.array_equal(codes, _torch_e4m3(x16.astype(np.float32) / s)), M


def pin_fp8_pt(O, rng=None):
    rng = rng or np.random.default_rng(5)
    for scale in (1.0, 0.01, 0.37, 3.0):
        for x16 in _rows(rng, 128, 10):
            codes, _ = O.quantize_row(oracle.FP8_PER_TENSOR, x16, scale)
            y = x16.astype(np.float32) / F32(scale)
            sat = np.abs(y) >= 464
            assert np.array_equal(codes[~sat], _torch_e4m3(y[~sat]))
            assert np.all(codes[sat] & 0x7F == 0x7E)


def _nvfp4_check(O, x16, st, flags):
    D = x16.shape[0]
    codes, bsc = O.quantize_row(oracle.NVFP4, x16, st, flags)
    x = x16.astype(np.float32)
    for b in range(D // 16):
        xb = x[16 * b:16 * (b + 1)]
        sbv = _torch_e4m3_decode(bsc[b:b + 1])[0]
        a = float(np.abs(xb).max())
        cb = codes[16 * b:16 * (b + 1)]
        if sbv == 0:
            assert not np.any(cb & 7)
            continue
        d = F32(st) * F32(sbv)
        # brute-force E2M1 of fl32(x / d)
        assert np.array_equal(cb, _e2m1_brute(xb / d))
        if not flags:
            # block max lands near the top of the grid: 6 * s_t * s_b ~ max|x| within E4M3 rounding
            if a / 6 / st >= 2.0 ** -6 and a / 6 / st < 440:
                assert abs(6 * st * sbv - a) <= a * 2.0 ** -4 * 1.0001
        else:
            # 4over6: the kept scale has the smaller squared error (ties keep max/6)
            def sse(sv):
                if sv == 0:
                    return float(np.sum(xb.astype(np.float64) ** 2))
                dd = F32(st) * F32(sv)
                q = _e2m1_brute(xb / dd)
                vals = np.array([O.e2m1_decode(int(c)) for c in q], np.float32)
                return float(np.sum((xb.astype(np.float64) - (dd * vals).astype(np.float64)) ** 2))
            s6 = _torch_e4m3_decode(_torch_e4m3(np.float32([F32(a) / F32(6) / F32(st)])))[0]
            s4 = _torch_e4m3_decode(_torch_e4m3(np.float32([min(F32(a) / F32(4) / F32(st), 448.0)])))[0]
            e6, e4 = sse(s6), sse(s4)
            assert sbv in (s6, s4)
            if abs(e4 - e6) > 1e-6 * max(e4, e6):
                assert sbv == (s4 if e4 < e6 else s6), (e4, e6, sbv, s4, s6)


def pin_nvfp4(O, rng=None):
    rng = rng or np.random.default_rng(6)
    for flags in (0, oracle.FLAG_NVFP4_4OVER6):
        for st in (1.0, 0.05, 2.0 ** -3):
            for x16 in _rows(rng, 128, 12):
                _nvfp4_check(O, x16, st, flags)
            t4 = rng.standard_t(4, 128).astype(np.float16)
            _nvfp4_check(O, t4, st, flags)
    # round trip: inputs already on s_t * s_b * grid reproduce exactly
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    st = 0.125
    for sbv in (1.0, 1.125, 1.75, 0.5, 2.5, 12.0):
        v = rng.choice(grid, 128) * rng.choice([-1, 1], 128)
        v[::16] = 6.0
        x = (st * sbv * v).astype(np.float16)
        assert np.array_equal(x.astype(np.float64), st * sbv * v)
        codes, bsc = O.quantize_row(oracle.NVFP4, x, st)
        vals = np.array([O.e2m1_decode(int(c)) for c in codes])
        rec = st * np.repeat(_torch_e4m3_decode(bsc[:8]), 16) * vals
        assert np.array_equal(rec, x.astype(np.float64))


def pin_nvfp4_scale_order(O):
    """Hand-worked blocks (tests/golden/nvfp4_scale_order.txt) whose E4M3 block
    scale depends on the association of the reading's (max / 6) / s_t: its
    quotient lands on one side of an E4M3 midpoint while max / (6 s_t) lands
    on the other, or exactly on it.  The expected codes follow from exact
    rational arithmetic, written out in the fixture."""
    n = 0
    with open(os.path.join(GOLDEN, "nvfp4_scale_order.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("->")
            name, st_bits, amax = lhs.split()
            st = float(np.uint32(int(st_bits, 16)).view(np.float32))
            x16 = np.zeros(128, np.float16)
            for b in range(8):
                x16[16 * b] = float(amax)
            assert float(x16[0]) == float(amax)
            for flags in (0, oracle.FLAG_NVFP4_4OVER6):
                codes, bsc = O.quantize_row(oracle.NVFP4, x16, st, flags)
                if flags == 0:
                    assert list(bsc[:8]) == [int(rhs)] * 8, f"{name}: block scale {bsc[:8]} != {rhs}"
            n += 1
    assert n == 2


def _pow2_exponent_brute(a):
    """The integer k with 4 * 2^k <= a < 8 * 2^k, by search (a > 0)."""
    hits = [k for k in range(-160, 140) if 4.0 * 2.0 ** k <= a < 8.0 * 2.0 ** k]
    assert len(hits) == 1
    return hits[0]


def pin_mxfp4(O, rng=None):
    """MXFP4 (reading: the OCP MX block conversion): per 32-value block the
    power of two 2^k with 4 * 2^k <= max|x| < 8 * 2^k, found by search, the
    biased E8M0 byte k + 127, brute-force E2M1 of x / 2^k with saturation at
    6; hand-worked blocks; exact round trip of values already on the grid;
    the cache round trip."""
    rng = rng or np.random.default_rng(13)
    rows = []
    for D in (32, 128):
        rows += _rows(rng, D)
        rows.append(rng.standard_t(4, D).astype(np.float16))
    for x16 in rows:
        D = x16.shape[0]
        codes, sb = O.quantize_row(oracle.MXFP4, x16)
        x = x16.astype(np.float64)
        for b in range(D // 32):
            xb, cb = x[32 * b:32 * (b + 1)], codes[32 * b:32 * (b + 1)]
            a = float(np.abs(xb).max())
            if a == 0.0:
                assert sb[b] == 0 and not np.any(cb & 7)
                continue
            k = _pow2_exponent_brute(a)
            assert int(sb[b]) == k + 127
            assert np.array_equal(cb, _e2m1_brute(xb / 2.0 ** k))
            # only the top binade [6, 8) * 2^k can clip; the max never rounds to zero
            assert cb[np.argmax(np.abs(xb))] & 7 >= 6
    # hand-worked blocks (32 values: the listed ones, then zeros)
    cases = [
        ([6.0, 5.0, 0.25, -0.75], 127, [7, 6, 0, 8 | 2]),       # max 6: 2^0; ties go to the even code
        ([7.0, -7.0, 1.25], 127, [7, 8 | 7, 2]),                # max 7: 2^0, 7 saturates to 6
        ([8.0, 7.0, 3.0], 128, [6, 6, 3]),                      # max 8: 2^1; 7/2 = 3.5 ties 3|4 -> 4
        ([0.75, 0.09375, -0.0], 124, [7, 2, 8]),                # max 0.75: 2^-3; 0.09375 * 8 = 0.75 ties 0.5|1
        ([65504.0, 1.0], 140, [7, 0]),                          # max 65504: 2^13; 1 / 8192 -> 0
        ([2.0 ** -24], 101, [6]),                               # smallest subnormal half: 2^-26, value 4
    ]
    for vals, byte, want in cases:
        x16 = np.zeros(32, np.float16)
        x16[:len(vals)] = vals
        codes, sb = O.quantize_row(oracle.MXFP4, x16)
        assert int(sb[0]) == byte, (vals, int(sb[0]))
        assert list(codes[:len(vals)]) == want, (vals, list(codes[:len(vals)]))
        assert not np.any(codes[len(vals):])
    # values already on 2^k * grid with a block max of 4 or 6 (times 2^k) reproduce exactly
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    D, P, H = 128, 16, 2
    k16 = np.zeros((P, H, D), np.float16)
    v16 = np.zeros((P, H, D), np.float16)
    for t in range(P):
        for h in range(H):
            for dst in (k16, v16):
                e = rng.integers(-20, 12, D // 32)
                vals = rng.choice(grid, D) * rng.choice([-1, 1], D)
                vals[::32] = rng.choice([4.0, 6.0], D // 32)
                dst[t, h] = (vals * np.repeat(2.0 ** e, 32)).astype(np.float16)
                assert np.array_equal(dst[t, h].astype(np.float64), vals * np.repeat(2.0 ** e, 32))
    lay = oracle.layout(oracle.MXFP4, H, D, P, 2)
    slots = (P + rng.permutation(P)).astype(np.int64)
    cache = O.quantize_write(lay, k16, v16, slots)
    kh, vh = O.dequantize(lay, cache, slots)
    assert np.array_equal(kh, k16.astype(np.float64)) and np.array_equal(vh, v16.astype(np.float64))
    # cache round trip of random rows: x_hat = 2^(byte - 127) * e2m1(code)
    k = workloads.random_halves(rng, (20, H, D))
    v = workloads.random_halves(rng, (20, H, D), 3.0)
    slots = rng.choice(2 * P, 20, replace=False).astype(np.int64)
    cache = O.quantize_write(lay, k, v, slots)
    kh, vh = O.dequantize(lay, cache, slots)
    for src, got in ((k, kh), (v, vh)):
        for i in range(20):
            for h in range(H):
                codes, sb = O.quantize_row(oracle.MXFP4, src[i, h])
                vals = np.array([O.e2m1_decode(int(c)) for c in codes])
                assert np.array_equal(got[i, h], vals * np.repeat(2.0 ** (sb[:D // 32].astype(np.int64) - 127), 32))


# --------------------------------------------------------------------------- #
# page layout
# --------------------------------------------------------------------------- #

def pin_page_bytes(O):
    g = golden("page_content.txt")
    sb = int(g["pth_scale_bytes_per_side"][0][0])
    for D in (32, 64, 128):
        P = 16
        # per token and kv head: (hs_k + hs_v) * 1 byte + 2 fp32 scales
        lay = oracle.layout(oracle.INT8_PTH, 8, D, P, 4)
        assert O.chunk_bytes(lay) == P * ((D + D) * 1 + 2 * sb)
        assert O.page_bytes(lay) == 8 * P * (2 * D + 2 * sb)
        lay = oracle.layout(oracle.FP8_PTH, 8, D, P, 4)
        assert O.chunk_bytes(lay) == P * ((D + D) * 1 + 2 * sb)
        lay = oracle.layout(oracle.FP8_PER_TENSOR, 8, D, P, 4)
        assert O.chunk_bytes(lay) == P * 2 * D
        lay = oracle.layout(oracle.NVFP4, 8, D, P, 4)
        assert O.chunk_bytes(lay) == P * 2 * (D // 2 + D // 16)
        div = int(g["int4_head_size_divisor"][0][0])
        lay = oracle.layout(oracle.INT4_PTH, 8, D, P, 4)
        assert O.chunk_bytes(lay) == P * ((D // div + D // div) * 1 + 2 * sb)
        # MXFP4: the NVFP4 code bytes with one E8M0 byte per 32 values
        mx = golden("mxfp4_block.txt")
        blk = int(mx["block_values"][0][0])
        lay = oracle.layout(oracle.MXFP4, 8, D, P, 4)
        assert O.chunk_bytes(lay) == P * 2 * (D // 2 + (D // blk) * int(mx["block_scale_bits"][0][0]) // 8)
    # MXFP4 metadata is sparser than NVFP4's: 4.25 against 4.5 bits per value
    lay = oracle.layout(oracle.MXFP4, 1, 128, 16, 1)
    mx_bits = O.chunk_bytes(lay) * 8 / (2 * 16 * 128)
    assert mx_bits == (int(mx["block_code_bits"][0][0]) + int(mx["block_scale_bits"][0][0])) / blk
    # NVFP4: 4.5 bits per value from the 16-value micro-block
    nb = golden("nvfp4_bits.txt")
    lay = oracle.layout(oracle.NVFP4, 1, 128, 16, 1)
    bits = O.chunk_bytes(lay) * 8 / (2 * 16 * 128)
    assert bits == float(nb["bits_per_value"][0][0])
    assert mx_bits < bits
    assert round(16 / bits, 2) == float(nb["ratio_vs_bf16"][0][0])
    assert round(8 / bits, 2) == float(nb["ratio_vs_fp8"][0][0])
    # 4-bit per-token KV bytes are about 0.28 of FP16 at head size 128
    frac = O.chunk_bytes(lay) / 16 / (2 * 2 * 128)
    assert round(frac, 2) == float(g["four_bit_fraction_of_fp16"][0][0])
    # KVarN: 128-token tile, capacity within the page's 3-5x
    kc = golden("kvarn_capacity.txt")
    lay = oracle.layout(oracle.KVARN_K4V2_G128, 1, 128, 128, 1)
    ratio = (2 * 128 * 128 * 2) / O.chunk_bytes(lay)
    assert float(kc["capacity_vs_fp16_low"][0][0]) <= ratio <= float(kc["capacity_vs_fp16_high"][0][0])
    # per-token-head scale count (K and V together) from the overhead table
    for toks, _, heads, _, n in golden("scale_count.txt")["tokens"]:
        P = 16
        lay = oracle.layout(oracle.INT8_PTH, int(heads), 128, P, int(toks) // P)
        data = int(toks) * int(heads) * 2 * 128
        scale_bytes = O.page_bytes(lay) * lay.num_pages - data
        assert scale_bytes // sb == int(n)


def pin_glossary_bytes(O):
    """The glossary's byte accounting, reproduced by our paged layout."""
    g = golden("glossary_int8_bytes.txt")
    w = workloads.make("glossary_int8")
    lay = oracle.layout(oracle.INT8_PTH, 4, 32, 16, w.num_pages)
    cache = O.quantize_write(lay, w.k16, w.v16, w.slots)
    fp16 = 2 * w.k16.size * 2
    assert fp16 == int(g["fp16_payload_bytes"][0][0])
    total = cache.size
    payload = 2 * w.k16.size
    assert payload == int(g["int8_payload_bytes"][0][0])
    assert total - payload == int(g["scale_metadata_bytes"][0][0])
    assert round(fp16 / total, 3) == float(g["effective_compression_ratio"][0][0])
    kh, vh = O.dequantize(lay, cache, w.slots)
    atol = float(g["assert_close_atol"][0][0])
    assert np.abs(kh - w.k16.astype(np.float64)).max() <= atol
    assert np.abs(vh - w.v16.astype(np.float64)).max() <= atol


def _written_nibbles(O, lay, k16, v16, slots):
    n = lay.num_pages * O.page_bytes(lay)
    a = O.quantize_write(lay, k16, v16, slots, np.zeros(n, np.uint8))
    b = O.quantize_write(lay, k16, v16, slots, np.full(n, 0xFF, np.uint8))
    lo_eq = (a & 15) == (b & 15)
    hi_eq = (a >> 4) == (b >> 4)
    return np.stack([lo_eq, hi_eq], axis=1).ravel()


def pin_layout_bijective(O, rng=None):
    """Every token-head row owns its own nibbles; a full page covers the chunk
    exactly once."""
    rng = rng or np.random.default_rng(7)
    for fmt in (oracle.INT8_PTH, oracle.FP8_PTH, oracle.FP8_PER_TENSOR, oracle.NVFP4, oracle.INT4_PTH, oracle.MXFP4):
        D, P, H = 64, 16, 2
        lay = oracle.layout(fmt, H, D, P, 2, 0.05, 0.05)
        k = workloads.random_halves(rng, (P, H, D))
        v = workloads.random_halves(rng, (P, H, D))
        owner = np.full(2 * lay.num_pages * O.page_bytes(lay), -1)
        for t in range(P):
            slots = np.full(P, -1, np.int64)
            slots[t] = P + t  # page 1
            w = _written_nibbles(O, lay, k, v, slots)
            assert np.all(owner[w] == -1), f"format {fmt}: token {t} overlaps another token"
            owner[w] = t
        half = owner.size // 2
        assert np.all(owner[:half] == -1), "page 0 must be untouched"
        assert np.all(owner[half:] >= 0), f"format {fmt}: chunk bytes never written"
    lay = oracle.layout(oracle.KVARN_K4V2_G128, 2, 128, 128, 2)
    k = workloads.random_halves(rng, (128, 2, 128))
    v = workloads.random_halves(rng, (128, 2, 128))
    w = _written_nibbles(O, lay, k, v, 128 + np.arange(128))
    half = w.size // 2
    assert not np.any(w[:half]) and np.all(w[half:])
    # two tiles per page: each owns its own bytes, together they cover page 1
    lay = oracle.layout(oracle.KVARN_K4V2_G128, 2, 128, 256, 2)
    w0 = _written_nibbles(O, lay, k, v, 256 + np.arange(128))
    w1 = _written_nibbles(O, lay, k, v, 384 + np.arange(128))
    half = w0.size // 2
    assert not np.any(w0 & w1)
    assert not np.any(w0[:half] | w1[:half]) and np.all((w0 | w1)[half:])


# --------------------------------------------------------------------------- #
# KVarN
# --------------------------------------------------------------------------- #

def pin_kvarn_rotation(O, rng=None):
    from scipy.linalg import hadamard
    rng = rng or np.random.default_rng(8)
    H = hadamard(128).astype(np.float32)
    c = F32(1.0) / F32(math.sqrt(128.0))  # RN(1/sqrt(128))
    for i in range(128):
        e = np.zeros(128, np.float32)
        e[i] = 1
        assert np.array_equal(O.kvarn_rotate(e), H[:, i] * c), f"column {i} is not Sylvester H / sqrt(128)"
    assert np.array_equal(H.astype(np.int64) @ H.T.astype(np.int64), 128 * np.eye(128, dtype=np.int64))
    for _ in range(20):
        q = rng.standard_normal(128).astype(np.float32)
        k = rng.standard_normal(128).astype(np.float32)
        rq, rk = O.kvarn_rotate(q), O.kvarn_rotate(k)
        # orthogonal: scores unchanged; involutory: applying twice restores the row
        assert abs(float(rq.astype(np.float64) @ rk) - float(q.astype(np.float64) @ k)) <= 1e-5 * 128
        assert np.allclose(O.kvarn_rotate(rq), q, rtol=0, atol=1e-5)


def pin_kvarn_tile(O, rng=None):
    rng = rng or np.random.default_rng(9)
    x = rng.standard_normal((128, 128)).astype(np.float32)
    x[:, 7] *= 8
    x[:, 90] *= 8
    x16 = x.astype(np.float16)
    for side, levels in ((0, 15), (1, 3)):
        o = O.kvarn_tile(x16, side)
        yr, yn, r, c = o["y_rot"], o["y_norm"], o["r"], o["c"]
        # stage 2: each token row rotated
        for t in range(0, 128, 17):
            assert np.array_equal(yr[t], O.kvarn_rotate(x16[t].astype(np.float32)))
        # stage 3 ends with a channel pass: every channel has unit population deviation
        assert np.allclose(yn.astype(np.float64).std(axis=0), 1.0, atol=2e-5)
        # the alternation converges: token deviations are near 1 as well
        assert np.allclose(yn.astype(np.float64).std(axis=1), 1.0, atol=0.05)
        # factors account for the whole transform: y_rot = r_t c_j y_norm
        rec = r[:, None].astype(np.float64) * c[None, :] * yn
        assert np.allclose(rec, yr, rtol=1e-5, atol=1e-6)
        # stage 4: asymmetric RTN within half a step, group min -> 0, group max -> top code
        codes, qs, qm = o["codes"].astype(np.float64), o["qs"].astype(np.float64), o["qm"].astype(np.float64)
        if side == 0:
            yh = qs[None, :] * codes + qm[None, :]
            assert np.all(np.abs(yn - yh) <= qs[None, :] * (0.5 + 1e-5))
            assert np.all(codes.min(axis=0) == 0) and np.all(codes.max(axis=0) == levels)
            assert np.array_equal(codes[np.argmin(yn, axis=0), np.arange(128)], np.zeros(128))
        else:
            yh = qs[:, None] * codes + qm[:, None]
            assert np.all(np.abs(yn - yh) <= qs[:, None] * (0.5 + 1e-5))
            assert np.all(codes.min(axis=1) == 0) and np.all(codes.max(axis=1) == levels)
        # stored metadata rebuilds the rotated tile up to the quantisation error
        m = o["meta"].astype(np.float64)
        if side == 0:
            kh = m[2][:, None] * (m[0][None, :] * codes + m[1][None, :])
        else:
            kh = m[2][None, :] * (m[0][:, None] * codes + m[1][:, None])
        step = (qs[None, :] if side == 0 else qs[:, None]) * r[:, None] * c[None, :]
        assert np.all(np.abs(kh - yr) <= 0.5 * step * (1 + 1e-4) + 1e-6)
    # degenerate tiles
    o = O.kvarn_tile(np.zeros((128, 128), np.float16), 0)
    assert np.all(o["codes"] == 0) and np.all(o["meta"][:2] == 0)
    o = O.kvarn_tile(np.full((128, 128), 1.5, np.float16), 1)
    assert np.all(np.isfinite(o["meta"]))


def _kvarn_factors_log_domain(x16, sweeps):
    """[P2] §技术原理's normalisation in its own terms, in binary64: rotate
    every token row by the normalised Walsh-Hadamard matrix (scipy), then per
    sweep add log sigma of every token row to the row's log factor, and then
    log sigma of every channel column to the column's log factor, sigma being
    the population deviation of the rotated tile divided by the current
    factors.  Returns the factors exp(log r), exp(log c)."""
    from scipy.linalg import hadamard
    Hm = hadamard(128).astype(np.float64) / math.sqrt(128.0)
    X = x16.astype(np.float64) @ Hm
    lr, lc = np.zeros(128), np.zeros(128)
    for _ in range(sweeps):
        sd = (X * np.exp(-lr[:, None] - lc[None, :])).std(axis=1)
        lr += np.log(np.where(sd > 0, sd, 1.0))
        sd = (X * np.exp(-lr[:, None] - lc[None, :])).std(axis=0)
        lc += np.log(np.where(sd > 0, sd, 1.0))
    return np.exp(lr), np.exp(lc)


def pin_kvarn_sweeps(O, rng=None):
    """The KVarN preset runs 4 sweeps (token pass, then channel pass): the
    oracle's binary32 token and channel factors, and the metadata that stores
    them (K rho = r, V gamma = c), match the binary64 log-domain formulation
    at 4 sweeps to 1e-5 relative; 3 or 5 sweeps differ by ~1e-3, so a wrong
    count fails."""
    rng = rng or np.random.default_rng(15)
    x = rng.standard_normal((128, 128)).astype(np.float32)
    x[:, 7] *= 8
    x[:, 90] *= 8
    y = (rng.standard_normal((128, 128)) * np.exp(rng.standard_normal((128, 1)))
         * np.exp(rng.standard_normal((1, 128))))
    for tile in (x.astype(np.float16), y.astype(np.float16)):
        for side in (0, 1):
            o = O.kvarn_tile(tile, side)
            r, c = _kvarn_factors_log_domain(tile, 4)
            assert np.max(np.abs(o["r"] / r - 1)) <= 1e-5, np.max(np.abs(o["r"] / r - 1))
            assert np.max(np.abs(o["c"] / c - 1)) <= 1e-5, np.max(np.abs(o["c"] / c - 1))
            stored = o["meta"][2]
            assert np.array_equal(stored, o["r"] if side == 0 else o["c"])
            for other in (3, 5):
                r2, c2 = _kvarn_factors_log_domain(tile, other)
                assert np.max(np.abs(r2 / r - 1)) > 1e-4 and np.max(np.abs(c2 / c - 1)) > 1e-4


# --------------------------------------------------------------------------- #
# attention
# --------------------------------------------------------------------------- #

def _dense_ref(q, K, V, scale):
    lg = (K @ q) * scale
    p = np.exp(lg - lg.max())
    return (p / p.sum()) @ V


def pin_attention(O, rng=None):
    rng = rng or np.random.default_rng(10)
    B, H, Hq, D, P = 3, 2, 8, 64, 16
    G = Hq // H
    for fmt, flags in ((oracle.INT8_PTH, 0), (oracle.FP8_PER_TENSOR, 0), (oracle.FP8_PTH, 0),
                       (oracle.NVFP4, 0), (oracle.NVFP4, 1)):
        maxp = 5
        num_pages = B * maxp
        lay = oracle.layout(fmt, H, D, P, num_pages, 0.02, 0.03, flags)
        ctx = np.array([37, 80, 1], np.int32)
        bt = rng.permutation(num_pages).astype(np.int32).reshape(B, maxp)
        toks, slots = [], []
        for b in range(B):
            for t in range(ctx[b]):
                toks.append((b, t))
                slots.append(bt[b, t // P] * P + t % P)
        n = len(toks)
        k16 = workloads.random_halves(rng, (n, H, D))
        v16 = workloads.random_halves(rng, (n, H, D))
        slots = np.array(slots, np.int64)
        cache = O.quantize_write(lay, k16, v16, slots)
        kh, vh = O.dequantize(lay, cache, slots)
        q16 = workloads.random_halves(rng, (B, Hq, D))
        sm = 1.0 / math.sqrt(D)
        out = O.decode_attention(lay, cache, q16, bt, ctx, sm)
        i0 = 0
        for b in range(B):
            rows = slice(i0, i0 + ctx[b])
            for h in range(Hq):
                ref = _dense_ref(q16[b, h].astype(np.float64), kh[rows, h // G], vh[rows, h // G], F32(sm))
                assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-12)
            i0 += ctx[b]
        # one cached token: the output is that token's dequantised value
        for h in range(Hq):
            assert np.allclose(out[2, h], vh[i0 - 1, h // G], rtol=1e-14, atol=1e-14)
    # identical keys: uniform weights, the output is the mean value
    lay = oracle.layout(oracle.INT8_PTH, 1, 32, 16, 2)
    k16 = np.repeat(workloads.random_halves(rng, (1, 1, 32)), 32, axis=0)
    v16 = workloads.random_halves(rng, (32, 1, 32))
    slots = np.arange(32)
    cache = O.quantize_write(lay, k16, v16, slots)
    _, vh = O.dequantize(lay, cache, slots)
    out = O.decode_attention(lay, cache, workloads.random_halves(rng, (1, 1, 32)), np.array([[0, 1]]),
                             np.array([32]), 0.3)
    assert np.allclose(out[0, 0], vh[:, 0].mean(axis=0), rtol=1e-13, atol=1e-14)
    # empty context gives zeros
    out = O.decode_attention(lay, cache, workloads.random_halves(rng, (1, 1, 32)), np.array([[0, 1]]),
                             np.array([0]), 0.3)
    assert not np.any(out)
    # GQA grouping: q head h reads kv head h // G
    H, Hq = 4, 8
    lay = oracle.layout(oracle.INT8_PTH, H, 32, 16, 1)
    k16 = np.zeros((16, H, 32), np.float16)
    v16 = np.zeros((16, H, 32), np.float16)
    for h in range(H):
        v16[:, h, :] = h + 1
    cache = O.quantize_write(lay, k16, v16, np.arange(16))
    out = O.decode_attention(lay, cache, workloads.random_halves(rng, (1, Hq, 32)), np.array([[0]]),
                             np.array([16]), 0.2)
    for h in range(Hq):
        assert np.allclose(out[0, h], h // (Hq // H) + 1, rtol=1e-6)


def pin_kvarn_pages(O, rng=None):
    """Pages of 256 tokens hold two independent 128-token tiles: their bytes
    are exactly the bytes of the same tokens written as two 128-token pages,
    placed back to back in each (page, head) chunk."""
    rng = rng or np.random.default_rng(14)
    H, D = 2, 128
    k = workloads.random_halves(rng, (256, H, D))
    v = workloads.random_halves(rng, (256, H, D), 2.0)
    l256 = oracle.layout(oracle.KVARN_K4V2_G128, H, D, 256, 2)
    l128 = oracle.layout(oracle.KVARN_K4V2_G128, H, D, 128, 2)
    tb = O.chunk_bytes(l128)
    assert O.chunk_bytes(l256) == 2 * tb
    c256 = O.quantize_write(l256, k, v, 256 + np.arange(256))  # page 1
    c128 = O.quantize_write(l128, k, v, np.arange(256))        # pages 0 and 1
    pb = O.page_bytes(l256)
    assert not np.any(c256[:pb])
    for h in range(H):
        for tile in range(2):
            got = c256[pb + h * 2 * tb + tile * tb:pb + h * 2 * tb + (tile + 1) * tb]
            want = c128[tile * H * tb + h * tb:tile * H * tb + (h + 1) * tb]
            assert np.array_equal(got, want), (h, tile)
    # and read back as the same values
    k2, v2 = O.dequantize(l256, c256, 256 + np.arange(256))
    k1, v1 = O.dequantize(l128, c128, np.arange(256))
    assert np.array_equal(k2, k1) and np.array_equal(v2, v1)
    # a tile must start on a multiple of 128 inside the page
    try:
        O.quantize_write(l256, k[:128], v[:128], 256 + 64 + np.arange(128))
    except ValueError:
        pass
    else:
        raise AssertionError("a tile starting mid-page must be refused")


def pin_attention_kvarn(O, rng=None):
    rng = rng or np.random.default_rng(11)
    for P in (128, 256):
        _attention_kvarn_case(O, rng, P)


def _attention_kvarn_case(O, rng, P):
    B, H, Hq, D = 2, 2, 4, 128
    ctx = np.array([256 + 37, 128], np.int32) if P == 128 else np.array([512 + 128 + 37, 384], np.int32)
    maxp = int(-(-ctx.max() // P))
    bt = rng.permutation(B * maxp).astype(np.int32).reshape(B, maxp)
    lay = oracle.layout(oracle.KVARN_K4V2_G128, H, D, P, B * maxp)
    cache = np.zeros(lay.num_pages * O.page_bytes(lay), np.uint8)
    K, V = {}, {}
    tail = np.zeros((B, 2, H, 128, D), np.float16)
    for b in range(B):
        full = ctx[b] // 128 * 128
        k16 = workloads.random_halves(rng, (ctx[b], H, D))
        v16 = workloads.random_halves(rng, (ctx[b], H, D))
        slots = (bt[b, np.arange(full) // P].astype(np.int64) * P + np.arange(full) % P)
        O.quantize_write(lay, k16[:full], v16[:full], slots, cache)
        kh, vh = O.dequantize(lay, cache, slots)
        nt = ctx[b] - full
        tail[b, 0, :, :nt] = k16[full:].transpose(1, 0, 2)
        tail[b, 1, :, :nt] = v16[full:].transpose(1, 0, 2)
        K[b] = np.concatenate([kh, k16[full:].astype(np.float64)])
        V[b] = np.concatenate([vh, v16[full:].astype(np.float64)])
        # 4-bit keys and 2-bit values stay close to the input (sanity of the whole pipeline)
        err_k = np.mean((kh - k16[:full]) ** 2) / np.mean(k16[:full].astype(np.float64) ** 2)
        err_v = np.mean((vh - v16[:full]) ** 2) / np.mean(v16[:full].astype(np.float64) ** 2)
        assert err_k < 0.03 and err_v < 0.25, (err_k, err_v)
    q16 = workloads.random_halves(rng, (B, Hq, D))
    out = O.decode_attention(lay, cache, q16, bt, ctx, 0.088, tail)
    for b in range(B):
        for h in range(Hq):
            ref = _dense_ref(q16[b, h].astype(np.float64), K[b][:, h // 2], V[b][:, h // 2], F32(0.088))
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-12)


ALL_PINS = [
    pin_half_widening, pin_e4m3_decode, pin_e4m3_encode, pin_e2m1_encode, pin_int8_pth, pin_int4_pth, pin_fp8_pth,
    pin_fp8_pt, pin_nvfp4, pin_mxfp4, pin_page_bytes, pin_glossary_bytes, pin_layout_bijective, pin_kvarn_rotation,
    pin_kvarn_tile, pin_kvarn_pages, pin_attention, pin_attention_kvarn, pin_int_rule_order, pin_nvfp4_scale_order,
    pin_kvarn_sweeps,
]
