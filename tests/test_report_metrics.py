"""The error-report metrics on inputs with known answers (CPU)."""
import numpy as np
import pytest

from quantized_decode_attention_amd import report


def test_tensor_metrics_known_values():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((10, 2, 16))
    e = np.full_like(x, 0.01)
    m = report.tensor_metrics(x, x + e)
    assert m["mse"] == pytest.approx(1e-4)
    assert m["nmse"] == pytest.approx(1e-4 / np.mean(x * x))
    assert m["max_abs_error"] == pytest.approx(0.01)
    assert m["zero_ratio"] == 0.0 and m["clip_ratio"] == 0.0
    m = report.tensor_metrics(x, 2 * x)
    assert m["cosine"] == pytest.approx(1.0)
    m = report.tensor_metrics(x, -x)
    assert m["cosine"] == pytest.approx(-1.0)
    # zeros and clipping: a row reconstructed with max 1.0 while the input
    # holds 2.0 has that element clipped
    x = np.array([[[2.0, 0.5, 0.0, -0.25]]])
    xh = np.array([[[1.0, 0.5, 0.0, 0.0]]])
    m = report.tensor_metrics(x, xh)
    assert m["clip_ratio"] == pytest.approx(0.25)
    assert m["zero_ratio"] == pytest.approx(0.5)
    assert m["zero_ratio_input"] == pytest.approx(0.25)


def test_scale_distribution_recovers_row_scale():
    s = np.array([0.5, 1.0, 2.0, 4.0])
    xh = np.zeros((4, 1, 8))
    xh[:, 0, 3] = 127 * s
    d = report.scale_distribution(xh, 127.0)
    assert d["min"] == pytest.approx(0.5) and d["max"] == pytest.approx(4.0)
    assert d["log2_span"] == pytest.approx(3.0)


def test_by_position_and_head():
    rng = np.random.default_rng(1)
    T = 16
    x = rng.standard_normal((2 * T, 3, 8))
    xh = x.copy()
    xh[0::T, 1] += 0.5  # error on the first token of each sequence, head 1 only
    p = report.by_position(x, xh, T, buckets=4)
    assert p["first_token"] > 0 and p["rest"] == 0.0
    assert p["buckets"][0] > 0 and all(b == 0.0 for b in p["buckets"][1:])
    h = report.by_head(x, xh)
    assert h[0] == 0.0 and h[2] == 0.0 and h[1] > 0


def test_attention_metrics():
    rng = np.random.default_rng(2)
    o = rng.standard_normal((3, 4, 32))
    m = report.attention_metrics(o, o)
    assert m["rel_l2_max"] == 0.0 and m["max_abs_error"] == 0.0 and m["cosine_min"] == pytest.approx(1.0)
    m = report.attention_metrics(1.1 * o, o)
    assert m["rel_l2_mean"] == pytest.approx(0.1)
