"""The benchmark's profile summaries file rocprofv3 kernel names under the
library's kernels: every template instance of a kernel must land under its
own name (a misfiled instance silently nulls or mixes the traffic figures)."""

import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def _full(short: str) -> str:
    return f"void sikv::(anonymous namespace)::{short}(int, int, float*)"


def test_attention_instances_by_value_format():
    for g in range(1, 9):
        for o32 in ("true", "false"):
            assert bench.library_kernel(_full(f"attn_kernel<{g}, false, {o32}>")) == "attn"
            assert bench.library_kernel(_full(f"attn_kernel<{g}, true, {o32}>")) == "attn_qv"


def test_other_library_kernels_and_foreign_names():
    assert bench.library_kernel(_full("score_kernel<8, false, false, 8>")) == "score"
    assert bench.library_kernel(_full("score_kernel<16, true, true, 8>")) == "score"
    assert bench.library_kernel(_full("select_kernel<4>")) == "select"
    assert bench.library_kernel(_full("combine_kernel")) == "combine"
    assert bench.library_kernel(_full("codes_kernel<true>")) == "codes"
    assert bench.library_kernel(_full("mu_partial_kernel")) == "mu_partial"
    assert bench.library_kernel("void at::native::vectorized_elementwise_kernel<4>(int)") is None
    assert bench.library_kernel("Cijk_Ailk_Bljk_BBS_BH_Bias_HA_S_SAV") is None
