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


def test_cvt_e4m3_to_f16_unit_scale_exact(PL, O):
    """E4M3 -> binary16 with scale 1 gives the exact value of every finite code."""
    import torch
    scales = torch.tensor([1.0], dtype=torch.float32, device="cuda")
    out = torch.zeros(512, dtype=torch.int16, device="cuda")
    log("probe cvt e4m3->f16")
    assert PL.probe_cvt_fp8_f16(_ptr(scales), 1, _ptr(out)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.float16).astype(np.float64).reshape(256, 2)
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue  # NaN codes
        v = O.e4m3_decode(c)
        assert got[c, 0] == v and got[c, 1] == v, (c, got[c], v)
