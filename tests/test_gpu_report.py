"""The error report on the glossary's small INT8 case and every format
(GPU): the glossary's own tolerance holds for INT8, finer formats have
smaller errors, and 4-bit formats stay well correlated."""
import numpy as np
import pytest

import workloads
from gpu_util import log
from oracle_pins import golden
from quantized_decode_attention_amd import report

pytestmark = pytest.mark.gpu


def test_error_report_orders_formats(K):
    w = workloads.make("glossary_int8")
    log("error report glossary_int8")
    res = {r["format"]: r for r in (report.report_format(K, w, f, fl) for f, fl in report.FORMATS_OF["glossary_int8"])}
    atol = float(golden("glossary_int8_bytes.txt")["assert_close_atol"][0][0])
    for side in ("k", "v"):
        assert res["int8_per_token_head"][side]["max_abs_error"] <= atol
        n8 = res["int8_per_token_head"][side]["nmse"]
        assert n8 < res["fp8_per_token_head"][side]["nmse"] < res["nvfp4"][side]["nmse"]
        assert n8 < res["int4_per_token_head"][side]["nmse"]
        # NVFP4's finer E4M3 block scales beat MXFP4's 32-value power-of-two
        # scales, the comparison the NVFP4 page draws
        assert res["nvfp4"][side]["nmse"] < res["mxfp4"][side]["nmse"]
        for name in ("int4_per_token_head", "nvfp4", "nvfp4_4over6", "mxfp4"):
            assert res[name][side]["cosine"] > 0.98
        for r in res.values():
            # MXFP4 saturates the top binade [6, 8) * 2^k of each block by design
            assert r[side]["clip_ratio"] == 0.0 or r["format"] in ("fp8_per_tensor", "nvfp4", "nvfp4_4over6",
                                                                   "mxfp4")
    for r in res.values():
        eight_bit = r["format"] in ("int8_per_token_head", "fp8_per_token_head", "fp8_per_tensor")
        assert r["attention_output"]["cosine_min"] > (0.99 if eight_bit else 0.95), r["format"]
        assert np.isfinite(r["attention_output"]["rel_l2_max"])
