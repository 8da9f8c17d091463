"""Named decode workloads.

Shapes follow the pages' workloads:
  * the TransMLA-converted LLaMA-2-7B layer (32 heads, 512 latent + 64 rope
    values cached per token) from "TransMLA: Multi-Head Latent Attention Is All
    You Need", Table 4 / Figure 5 (throughput at 1K-32K context);
  * the DeepSeek-V3 attention shape (128 heads, d_nope = 128, latent 512,
    rope 64, d_v = 128) from "TPLA: Tensor Parallel Latent Attention ...",
    section 3.4 ("MLA Matrix Absorption", W_UV of shape 512 x 16384) and the
    DeepSeek-V3 configuration chapter of "TransMLA & Sparse Latent Attention".
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class MLAConfig:
    name: str
    batch: int
    heads: int
    d_nope: int
    d_latent: int
    d_rope: int
    d_v: int
    page_size: int
    seq_len: Optional[int] = None                  # every sequence this long
    seq_len_range: Optional[Tuple[int, int]] = None  # inclusive uniform range
    cache_dtype: str = "bf16"    # "f32" | "bf16" | "e4m3"
    q_dtype: str = "bf16"        # "f32" | "bf16"
    rope_dtype: str = "bf16"
    weight_dtype: str = "bf16"
    out_dtype: str = "f32"       # the decode output; bf16 storage is also supported
    permuted: bool = True        # random physical block permutation
    seed: int = 1000
    spare_blocks: int = 3        # unused, NaN-poisoned pool blocks

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(self.d_nope + self.d_rope) ** 0.5

    @property
    def max_seq_len(self) -> int:
        return self.seq_len if self.seq_len is not None else self.seq_len_range[1]

    def replace(self, **kw) -> "MLAConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return MLAConfig(**d)


_DSV3 = dict(heads=128, d_nope=128, d_latent=512, d_rope=64, d_v=128, page_size=64)

CONFIGS = {
    # tiny fp32 step: one contiguous 64-token block per sequence
    "tiny_fp32": MLAConfig(
        name="tiny_fp32", batch=2, heads=4, d_nope=16, d_latent=32, d_rope=8, d_v=16,
        page_size=64, seq_len=64, cache_dtype="f32", q_dtype="f32", rope_dtype="f32",
        weight_dtype="f32", out_dtype="f32", permuted=False, seed=1000),
    # TransMLA-converted LLaMA-2-7B layer, 8K context
    "transmla_llama2_7b": MLAConfig(
        name="transmla_llama2_7b", batch=16, heads=32, d_nope=128, d_latent=512, d_rope=64,
        d_v=128, page_size=64, seq_len=8192, permuted=False, seed=1001),
    # DeepSeek-V3 shape, batch 64, 4K context, permuted pages
    "dsv3_b64_4k": MLAConfig(name="dsv3_b64_4k", batch=64, seq_len=4096, seed=1002, **_DSV3),
    # DeepSeek-V3 shape, ragged 1K..32K context, batch 8
    "dsv3_ragged_32k": MLAConfig(
        name="dsv3_ragged_32k", batch=8, seq_len_range=(1024, 32768), seed=1003, **_DSV3),
    # DeepSeek-V3 shape, fp8-e4m3 latent with per-token fp32 scale, batch 32, 16K context
    "dsv3_fp8_16k": MLAConfig(
        name="dsv3_fp8_16k", batch=32, seq_len=16384, cache_dtype="e4m3", seed=1004, **_DSV3),
    # DeepSeek-V3 shape, batch 8, every sequence at 32K context (supplemental)
    "dsv3_b8_32k": MLAConfig(name="dsv3_b8_32k", batch=8, seq_len=32768, seed=1005, **_DSV3),
}


def config_by_name(name: str) -> MLAConfig:
    return CONFIGS[name]
