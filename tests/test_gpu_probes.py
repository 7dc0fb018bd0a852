"""gfx950 conversion builtins against the oracle's encoders and decoders.

The library's encoders are integer code on the binary32 bit pattern; these
tests record whether the hardware conversions agree with the same rules
(round-to-nearest-even, saturation handled by the caller for E4M3, E2M1 ties
to the even code), so that a kernel may use them.  The probe kernels live in
tests/gpu_probes/ (test-only, not part of libkvq)."""
import ctypes
import os

import numpy as np
import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def PL():
    path = os.path.join(ROOT, "tests", "gpu_probes", "libkvq_probes.so")
    if not os.path.exists(path):
        from quantized_decode_attention_amd import _build
        _build.build_probes()
    import torch  # noqa: F401  (one HIP runtime: torch's)
    return ctypes.CDLL(path)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def e4m3_grid(O):
    return np.array([O.e4m3_decode(c) for c in range(127)], np.float64)


def test_cvt_f32_to_e4m3_matches_oracle(PL, O):
    import torch
    rng = np.random.default_rng(0)
    grid = e4m3_grid(O)
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)  # exact ties
    x = np.concatenate([mids, -mids, np.nextafter(mids, np.float32(1e9)), np.nextafter(mids, np.float32(-1e9)),
                        rng.uniform(-448, 448, 100000).astype(np.float32),
                        (rng.standard_normal(20000) * 1e-3).astype(np.float32),
                        np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -2.0 ** -10, 1e-30])]).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    out = torch.zeros(x.size, dtype=torch.uint8, device="cuda")
    log("probe cvt f32->e4m3")
    assert PL.probe_cvt_f32_fp8(_ptr(xd), ctypes.c_int64(x.size), _ptr(out)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = np.array([O.e4m3_encode(float(v)) for v in x], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(ref[i])) for i in bad[:8]]


def test_cvt_f32_to_e2m1_matches_oracle(PL, O):
    import torch
    rng = np.random.default_rng(1)
    g = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    x = np.concatenate([mids, -mids, np.nextafter(mids, np.float32(9)), np.nextafter(mids, np.float32(-9)),
                        rng.uniform(-7, 7, 20000).astype(np.float32),
                        np.float32([0.0, -0.0, 6.0, -6.0, 6.5, -1e9, 1e-30, 5.0, -5.0])]).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    out = torch.zeros(x.size, dtype=torch.uint8, device="cuda")
    log("probe cvt f32->e2m1")
    assert PL.probe_cvt_f32_fp4(_ptr(xd), ctypes.c_int64(x.size), _ptr(out)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = np.array([O.e2m1_encode(float(v)) for v in x], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(ref[i])) for i in bad[:8]]


def _all_byte_positions(rng):
    """Every byte value at every byte position of a word, the other bytes random."""
    words = rng.integers(0, 2 ** 32, 1024, dtype=np.uint64).astype(np.uint32)
    for pos in range(4):
        for b in range(256):
            w = int(words[pos * 256 + b]) & ~(0xFF << (8 * pos))
            words[pos * 256 + b] = w | (b << (8 * pos))
    return words


def test_cvt_e4m3_to_f16_exact(PL, O):
    """E4M3 -> binary16 (scale 1), as the decode issues it: exact value of
    every finite code, in code order, in both halves."""
    import torch
    words = _all_byte_positions(np.random.default_rng(2))
    src = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.zeros(words.size * 2, dtype=torch.int32, device="cuda")
    log("probe cvt e4m3->f16")
    assert PL.probe_cvt_fp8_f16_asm(_ptr(src), words.size, _ptr(out)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.float16).astype(np.float64).reshape(words.size, 4)
    dec = np.array([O.e4m3_decode(c) for c in range(256)])
    for i, w in enumerate(words):
        for k in range(4):
            c = (int(w) >> (8 * k)) & 0xFF
            if (c & 0x7F) == 0x7F:
                assert np.isnan(got[i, k])
            else:
                assert got[i, k] == dec[c] and np.signbit(got[i, k]) == np.signbit(dec[c]), (hex(int(w)), k)


def test_cvt_e2m1_to_f16_exact(PL, O):
    """E2M1 pairs -> binary16 (scale 1), as the decode issues them: every
    byte at every position gives (low nibble, high nibble) exactly."""
    import torch
    words = _all_byte_positions(np.random.default_rng(3))
    src = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.zeros(words.size * 4, dtype=torch.int32, device="cuda")
    log("probe cvt e2m1->f16")
    assert PL.probe_cvt_fp4_f16_asm(_ptr(src), words.size, ctypes.c_float(1.0), _ptr(out)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.float16).astype(np.float64).reshape(words.size, 4, 2)
    dec = np.array([O.e2m1_decode(c) for c in range(16)])
    for i, w in enumerate(words):
        for k in range(4):
            b = (int(w) >> (8 * k)) & 0xFF
            for e, c in enumerate((b & 15, b >> 4)):
                assert got[i, k, e] == dec[c] and np.signbit(got[i, k, e]) == np.signbit(dec[c]), (hex(int(w)), k, e)


def test_cvt_e2m1_to_f16_power_of_two_scales(PL, O):
    """E2M1 pairs -> binary16 with scale 2^k, as the MXFP4 decode issues them
    (the block's E8M0 byte placed in a binary32 exponent field): every code
    gives E2M1 value * 2^k exactly for every k whose products are binary16
    numbers, binary16 subnormals included (k in [-23, 13]); binary16 inputs
    give MXFP4 block exponents in [-26, 13], and below -23 the conversion
    stays within 2^-24 of the exact value.  Byte 0 (scale +0) turns the zero
    codes into zeros."""
    import torch
    words = _all_byte_positions(np.random.default_rng(4))
    src = torch.from_numpy(words.view(np.int32)).cuda()
    dec = np.array([O.e2m1_decode(c) for c in range(16)])
    codes = np.stack([(words[:, None] >> (8 * np.arange(4))) & 15, (words[:, None] >> (8 * np.arange(4) + 4)) & 15],
                     axis=-1).astype(np.int64)  # [word, byte, nibble]
    for k in list(range(-30, 14)):
        scale = np.float32(2.0 ** k)
        out = torch.zeros(words.size * 4, dtype=torch.int32, device="cuda")
        assert PL.probe_cvt_fp4_f16_asm(_ptr(src), words.size, ctypes.c_float(float(scale)), _ptr(out)) == 0
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.float16).astype(np.float64).reshape(words.size, 4, 2)
        exact = dec[codes] * 2.0 ** k
        if k >= -23:
            assert np.array_equal(got, exact), f"k={k}"
            assert np.array_equal(np.signbit(got), np.signbit(exact)), f"k={k}"
        else:
            assert np.all(np.abs(got - exact) <= 2.0 ** -24), f"k={k}"
    log("probe cvt e2m1->f16 with 2^k scales: exact for k >= -23")
    zero = torch.from_numpy(np.array([0x80808080 - 2 ** 32, 0], np.int64).astype(np.int32)).cuda()
    out = torch.ones(8, dtype=torch.int32, device="cuda")
    assert PL.probe_cvt_fp4_f16_asm(_ptr(zero), 2, ctypes.c_float(0.0), _ptr(out)) == 0
    torch.cuda.synchronize()
    assert not np.any(out.cpu().numpy().view(np.float16).astype(np.float64))


def test_mfma_f16_subnormal_operands(PL):
    """The QK product takes binary16 subnormal operands (MXFP4 keys of small
    blocks) without flushing: 16x16x32 products of m * 2^-24 values with small
    integers come out exactly."""
    import torch
    rng = np.random.default_rng(5)
    A = (rng.integers(-7, 8, (16, 32)) * 2.0 ** -24).astype(np.float16)  # subnormals
    A[3] = (rng.integers(-7, 8, 32) * 2.0 ** -14).astype(np.float16)     # normal row for contrast
    B = rng.integers(-4, 5, (32, 16)).astype(np.float16)
    assert np.array_equal(A.astype(np.float64), np.round(A.astype(np.float64) * 2.0 ** 24) * 2.0 ** -24)
    # lane l: A row l % 16 and B column l % 16, k = 8 * (l // 16) + 0..7
    la = np.stack([A[l % 16, 8 * (l // 16):8 * (l // 16) + 8] for l in range(64)])
    lb = np.stack([B[8 * (l // 16):8 * (l // 16) + 8, l % 16] for l in range(64)])
    out = torch.zeros((64, 4), dtype=torch.float32, device="cuda")
    assert PL.probe_mfma_f16(_ptr(torch.from_numpy(la).cuda()), _ptr(torch.from_numpy(lb).cuda()), _ptr(out)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = A.astype(np.float64) @ B.astype(np.float64)  # exact: small integers times 2^-24
    # lane l: column l % 16, rows 4 * (l // 16) + 0..3
    want = np.stack([ref[4 * (l // 16):4 * (l // 16) + 4, l % 16] for l in range(64)])
    assert np.array_equal(got, want), np.abs(got - want).max()


def _e4m3_inputs(O, rng):
    grid = e4m3_grid(O)
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    x = np.concatenate([mids, -mids, np.nextafter(mids, np.float32(1e9)), np.nextafter(mids, np.float32(-1e9)),
                        rng.uniform(-448, 448, 40000).astype(np.float32),
                        (rng.standard_normal(20000) * 1e-3).astype(np.float32),
                        np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -2.0 ** -10, 1e-30, -1e-30])])
    x = x[:x.size // 4 * 4]
    return rng.permutation(x).astype(np.float32)


def test_cvt_f32_to_e4m3_pairs_in_both_words(PL, O):
    """The packed binary32 -> E4M3 conversion used by the FP8 writes: both
    values of a pair and both words of a dword match the oracle's encoder
    for every |y| <= 448 (the writes clamp to +-448 first)."""
    import torch
    x = _e4m3_inputs(O, np.random.default_rng(6))
    out = torch.zeros(x.size // 4, dtype=torch.int32, device="cuda")
    log("probe cvt f32->e4m3 pairs")
    assert PL.probe_cvt_f32_fp8_pairs(_ptr(torch.from_numpy(x).cuda()), ctypes.c_int64(x.size // 4), _ptr(out)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint8)
    ref = np.array([O.e4m3_encode(float(v)) for v in x], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(ref[i])) for i in bad[:8]]


def test_cvt_f32_to_e2m1_x8_packing(PL, O):
    """The scaled binary32 -> E2M1 conversion used by the 4-bit writes, eight
    values into one dword (byte selects 0..3): every nibble matches the
    oracle's encoder, ties and saturation included."""
    import torch
    rng = np.random.default_rng(7)
    g = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    x = np.concatenate([mids, -mids, np.nextafter(mids, np.float32(9)), np.nextafter(mids, np.float32(-9)),
                        rng.uniform(-8, 8, 40000).astype(np.float32),
                        np.float32([0.0, -0.0, 6.0, -6.0, 6.5, -7.9, 1e-30, 5.0, -5.0, 0.25, -0.25, 7.0])])
    x = rng.permutation(x[:x.size // 8 * 8]).astype(np.float32)
    out = torch.zeros(x.size // 8, dtype=torch.int32, device="cuda")
    log("probe cvt f32->e2m1 x8")
    assert PL.probe_cvt_f32_fp4_x8(_ptr(torch.from_numpy(x).cuda()), ctypes.c_int64(x.size // 8), _ptr(out)) == 0
    torch.cuda.synchronize()
    b = out.cpu().numpy().view(np.uint8)
    got = np.stack([b & 15, b >> 4], axis=1).ravel()
    ref = np.array([O.e2m1_encode(float(v)) for v in x], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(ref[i])) for i in bad[:8]]


def test_cvt_e4m3_nibbles_to_f16_integers(PL):
    """KVarN key codes: a byte holding c in 0..15, read as E4M3 (c * 2^-9)
    and converted with scale 2^9, gives exactly the integer c, in both
    bytes of both words."""
    import torch
    rng = np.random.default_rng(8)
    words = rng.integers(0, 2 ** 32, 4096, dtype=np.uint64).astype(np.uint32) & np.uint32(0x0F0F0F0F)
    words[:16] = np.arange(16, dtype=np.uint32) * np.uint32(0x01010101)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.zeros(words.size * 2, dtype=torch.int32, device="cuda")
    log("probe cvt e4m3 nibbles -> integers")
    assert PL.probe_cvt_fp8_f16_scaled(_ptr(src), words.size, ctypes.c_float(512.0), _ptr(out)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.float16).astype(np.float64).reshape(words.size, 4)
    want = np.stack([(words >> (8 * k)) & 0xFF for k in range(4)], axis=1).astype(np.float64)
    assert np.array_equal(got, want)


def test_cvt_e2m1_to_f32_every_code_and_byte(PL, O):
    """The scaled E2M1 -> binary32 conversion at scale 1 (used for NVFP4's
    4over6 reconstruction error) returns the exact grid value of every code
    from every byte position of a word (the sign of a zero is not compared:
    it cannot change x - d * v or its square)."""
    import torch
    rng = np.random.default_rng(5)
    words = _all_byte_positions(rng)
    wd = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.zeros(words.size * 8, dtype=torch.float32, device="cuda")
    log("probe cvt e2m1 -> f32, byte selects")
    assert PL.probe_cvt_fp4_f32_bytes(_ptr(wd), words.size, _ptr(out)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, 8)
    for i, w in enumerate(words):
        for j in range(8):
            code = (int(w) >> (4 * j)) & 15
            ref = np.float32(O.e2m1_decode(code))
            assert got[i, j] == ref, (hex(int(w)), j, got[i, j], ref)
