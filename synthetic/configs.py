"""Workload shapes for Grouped Value Attention (GVA) decode.

Each entry names one synthetic decode workload by what it is: batch ``B`` of
independent sequences, ``H`` query heads sharing ``G`` value groups, value
head width ``d_h`` split into an unrotated content slice ``d_n`` and a shared
rotated position slice ``d_r`` (Grouped Value Attention, onedev.kr review,
section "How it differs": the decoupled-RoPE split of each head).

The shapes carry no arithmetic of the method; they are shared by the float64
oracle and by the HIP path through the input generator in
``synthetic.inputs``.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class GVAConfig:
    name: str
    B: int
    H: int
    G: int
    d_h: int
    d_n: int
    d_r: int
    # Fixed context length, or None when ``len_range`` gives a ragged draw.
    T: Optional[int]
    cache_dtype: str  # "float32" or "bfloat16"
    len_range: Optional[Tuple[int, int]] = None  # inclusive uniform range
    append: bool = False  # new token's V / k_rope written before attention
    shuffled_blocks: bool = False
    block_size: int = 64
    rope_base: float = 10000.0
    seed: int = 0
    with_gqa: bool = False  # a same-shape GQA decode is timed beside it
    notes: str = field(default="", compare=False)

    @property
    def heads_per_group(self) -> int:
        return self.H // self.G


CONFIGS = {
    "tiny_fp32": GVAConfig(
        name="tiny_fp32", B=1, H=4, G=2, d_h=32, d_n=24, d_r=8, T=128,
        cache_dtype="float32",
        notes="single fp32 decode step, seed 0, RoPE base 10000"),
    "decode_350m": GVAConfig(
        name="decode_350m", B=32, H=16, G=4, d_h=64, d_n=48, d_r=16, T=4096,
        cache_dtype="bfloat16",
        notes="350M-shaped decode, one query token per sequence"),
    "wide_rope_append": GVAConfig(
        name="wide_rope_append", B=64, H=16, G=4, d_h=64, d_n=40, d_r=24,
        T=8192, cache_dtype="bfloat16", append=True,
        notes="wider position slice; new token appended before attention"),
    "long_ragged": GVAConfig(
        name="long_ragged", B=8, H=16, G=4, d_h=64, d_n=48, d_r=16, T=None,
        len_range=(1024, 131072), cache_dtype="bfloat16",
        shuffled_blocks=True,
        notes="ragged lengths, 64-token blocks, shuffled block table"),
    "large_model": GVAConfig(
        name="large_model", B=128, H=32, G=8, d_h=128, d_n=96, d_r=32,
        T=16384, cache_dtype="bfloat16", with_gqa=True,
        notes="larger-model shape, timed beside a same-shape GQA decode"),
}

# The order in which the workloads are listed (smallest first).
CONFIG_ORDER = ["tiny_fp32", "decode_350m", "wide_rope_append",
                "long_ragged", "large_model"]


def get_config(name: str) -> GVAConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {CONFIG_ORDER}")
