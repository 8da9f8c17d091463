"""Host-side pieces of bench.py (no GPU): the attention kernel's own roof and
the stage each profiled kernel name is counted under."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from mla_inputs import CONFIGS  # noqa: E402


def _run(name, tokens, cache_bytes, attn_ms):
    return {"cfg": CONFIGS[name], "total_tokens": tokens, "cache_bytes": cache_bytes,
            "attn_ms": attn_ms}


def test_fp8_roof_is_the_matrix_cores():
    """32 x 16384 tokens, 128 heads, 644 B per token: HBM 337.6 MB / 8 TB/s =
    42.2 us; matrix cores 67.1M token-heads x (2*64 + 2*512) flops at 2.5
    PFLOP/s (30.9 us) plus x 2*2*512 at 5 PFLOP/s (27.5 us) = 58.4 us."""
    tokens = 32 * 16384
    r = bench.attention_roof(_run("dsv3_fp8_16k", tokens, tokens * 644, 0.1168))
    assert r["attn_hbm_us"] == pytest.approx(42.2, abs=0.05)
    assert r["attn_mfma_floor_us"] == pytest.approx(58.4, abs=0.05)
    assert r["attn_roof_bound"] == "mfma" and r["attn_roof_us"] == r["attn_mfma_floor_us"]
    assert r["attn_frac_of_roof"] == pytest.approx(0.5, abs=0.001)


def test_bf16_roof_is_hbm():
    """123444 tokens of 1152 B: 142.2 MB / 8 TB/s = 17.8 us, above the
    matrix-core time 15.8M x 2176 flops / 2.5 PFLOP/s = 13.75 us."""
    tokens = 123444
    r = bench.attention_roof(_run("dsv3_ragged_32k", tokens, tokens * 1152, 0.0356))
    assert r["attn_roof_bound"] == "hbm"
    assert r["attn_roof_us"] == pytest.approx(17.8, abs=0.05)
    assert r["attn_mfma_floor_us"] == pytest.approx(13.75, abs=0.06)   # 13.753, to 0.1 us
    assert r["attn_frac_of_roof"] == pytest.approx(0.5, abs=0.002)


@pytest.mark.parametrize("name,cls", [
    ("void mla::(anonymous namespace)::attend64_kernel<false, 1>(mla::AttnArgs)", "attention"),
    ("void mla::(anonymous namespace)::attend64_fp8_kernel<false>(mla::AttnArgs)", "attention"),
    ("void mla::(anonymous namespace)::up16_mfma_kernel<true, 0>(mla::AttnArgs, float const*)", "merge_up"),
    ("void mla::(anonymous namespace)::up16_mfma_kernel<false, 1>(mla::AttnArgs, float const*)", "up_project"),
    ("void mla::merge_kernel<1>(mla::AttnArgs, float*)", "combine"),
    ("void mla::combine_kernel(mla::AttnArgs, float*)", "combine"),
    ("void mla::(anonymous namespace)::absorb_mfma_kernel<1>(unsigned short const*)", "absorb"),
    ("mla::plan_kernel(mla::PlanInput)", "plan"),
    ("__amd_rocclr_copyBuffer", "copy"),
    ("void at::native::vectorized_elementwise_kernel<4>", None),
])
def test_kernel_classes(name, cls):
    assert bench.kernel_class(name) == cls
