"""Seeded synthetic workloads for GVA decode (shapes and random inputs only).

Shared by the float64 oracle (``oracle/``) and the HIP path
(``compressed_kv_cache_amd``); holds none of the method's arithmetic.
"""
from .configs import CONFIGS, CONFIG_ORDER, GVAConfig, get_config
from .inputs import (block_layout, draw_seq_lens, make_gqa_inputs, make_gqa_multi_inputs,
                     make_gva_inputs, make_gva_multi_inputs, with_overrides)

__all__ = ["CONFIGS", "CONFIG_ORDER", "GVAConfig", "get_config",
           "block_layout", "draw_seq_lens", "make_gqa_inputs", "make_gqa_multi_inputs",
           "make_gva_inputs", "make_gva_multi_inputs", "with_overrides"]
