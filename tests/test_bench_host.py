"""Host-side checks of the benchmark, no GPU: the one-GPU guard, the
per-step algorithmic KV bytes of every workload (from the library's page
size), and the source digest that decides whether the committed HBM
counter figures still describe the decode kernel."""
import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
    assert r.stdout == ""  # no JSON line


# Per-step KV bytes read by one decode (K+V codes and in-page scales) of the
# workloads at full size: bytes per token-head times B * T * H_kv.
STEP_BYTES = [
    ("fp8_sink_4k", 1, 256, 268_435_456),
    ("fp8_sink_4k", 3, 264, 276_824_064),
    ("int8_32k", 2, 264, 553_648_128),
    ("int8_32k", 6, 136, 285_212_672),
    ("nvfp4_16k", 4, 144, 301_989_888),
    ("nvfp4_16k", 7, 136, 285_212_672),
    ("kvarn_16k", 5, 120, 251_658_240),
    ("nvfp4_16k_tp2", 4, 144, 150_994_944),
    ("kvarn_16k_tp2", 5, 120, 125_829_120),
]


@pytest.mark.parametrize("name,fmt,per_token_head,total", STEP_BYTES)
def test_step_kv_bytes(K, name, fmt, per_token_head, total):
    sp = workloads.SPECS[name]
    lay = K.layout(fmt, sp.Hkv, sp.D, sp.P, 1, 1.0, 1.0, 0)
    page = K.kvq_page_bytes(lay)
    assert page == per_token_head * sp.P * sp.Hkv
    assert sp.B * (sp.T // sp.P) * page == total


def test_traffic_digest_ignores_comments_only():
    code = "int a = 1;  // one\n/* block\n comment */\nint b = 2;\n\n"
    assert bench._code_only(code) == "int a = 1;\nint b = 2;"
    assert bench._code_only(code) == bench._code_only(code.replace("one", "two"))
    assert bench._code_only(code) != bench._code_only(code.replace("= 2", "= 3"))


def test_traffic_table_follows_the_digest(monkeypatch, tmp_path):
    """Figures are read per `workload/format` entry, and only while the
    summary's digest matches the kernels' sources."""
    f = tmp_path / "traffic.md"
    body = ("    traffic int8_32k/int8_per_token_head decode = 565181228\n"
            "    traffic int8_32k/int8_per_token_head write = 1700000000\n"
            "    traffic nvfp4_16k/nvfp4_4over6 decode = 310000000\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(body + f"    kernel_sources_sha256 = {bench.kernel_sources_digest()}\n")
    assert bench.measured_traffic("int8_32k/int8_per_token_head") == 565181228
    assert bench.measured_traffic("int8_32k/int8_per_token_head", "write") == 1700000000
    assert bench.measured_traffic("nvfp4_16k/nvfp4_4over6") == 310000000
    assert bench.measured_traffic("nvfp4_16k/nvfp4") is None
    f.write_text(body + "    kernel_sources_sha256 = 0123\n")
    assert bench.measured_traffic("int8_32k/int8_per_token_head") is None


def test_committed_traffic_is_near_the_algorithmic_bytes():
    # null once the kernel sources changed since the counters were taken,
    # else within a few percent of the algorithmic 553.6 MB
    got = bench.measured_traffic("int8_32k/int8_per_token_head")
    assert got is None or 553_648_128 <= got <= 1.1 * 553_648_128


def test_format_choice():
    assert bench.main_format("int8_32k") == (2, 0)
    assert bench.main_format("nvfp4_16k", "nvfp4_4over6") == (4, 1)
    assert bench.main_format("nvfp4_16k", "mxfp4") == (7, 0)
    assert bench.main_format("kvarn_16k_tp2") == (5, 0)
    assert bench.main_format("int8_32k", "kvarn_k4v2_g128") is None
    assert bench.main_format("kvarn_16k", "nvfp4") is None
    assert bench.main_format("int8_32k", "int2") is None
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "kvarn_16k", "--format",
                        "int8_per_token_head"], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and r.stdout == ""


def test_call_time_source():
    """The decode call's time comes from back-to-back calls inside one event
    pair: the timed region's time per step where a step is one call, and the
    KVarN decode calls' own region where a step also appends; the per-call
    event timing (which reads long) is never the figure."""
    p = object.__new__(bench.Problem)
    p.dec_region_ms = 0.061
    p.kvarn = False
    assert p.call_ms(0.0905, 0.0927) == 0.0905
    assert "timed steps" in p.call_timing()
    p.kvarn = True
    assert p.call_ms(0.0660, 0.0629) == 0.061
    assert "back to back" in p.call_timing()

