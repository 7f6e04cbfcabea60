"""libgva: Grouped Value Attention absorbed decode on MI355X (gfx950).

Importing the package loads the in-tree ``libgva.so`` and fails loudly when it
is missing; every operation runs in its HIP kernels.
"""
from . import _lib
from ._lib import NOALLOC_SCRATCH_BYTES, PROBE_BLOCKS, GvaError, GvaShape, LIB_PATH
from .ops import (BLOCK_SIZE, absorb_query, absorb_query_multi, append_cache,
                  append_cache_multi, cache_scalars_per_token, decode_attention,
                  decode_attention_lens, decode_attention_multi, decode_rope_keys,
                  decode_step, decode_step_lens, decode_step_multi, decode_step_noalloc,
                  decode_step_workspace_bytes_lens, decode_workspace_bytes_lens,
                  decode_step_workspace_bytes, decode_workspace_bytes,
                  decode_workspace_bytes_multi, gqa_decode_attention,
                  gqa_decode_attention_multi, gqa_decode_workspace_bytes, make_shape,
                  stream_read_probe)

lib = _lib.load()

__all__ = ["BLOCK_SIZE", "GvaError", "GvaShape", "LIB_PATH", "absorb_query",
           "absorb_query_multi", "append_cache", "append_cache_multi",
           "cache_scalars_per_token", "decode_attention", "decode_attention_lens",
           "decode_attention_multi", "decode_step_lens", "decode_step_workspace_bytes_lens",
           "decode_workspace_bytes_lens",
           "decode_rope_keys",
           "decode_step", "decode_step_multi", "decode_step_noalloc",
           "decode_step_workspace_bytes", "NOALLOC_SCRATCH_BYTES",
           "decode_workspace_bytes", "decode_workspace_bytes_multi",
           "gqa_decode_attention", "gqa_decode_attention_multi", "gqa_decode_workspace_bytes",
           "lib", "make_shape", "PROBE_BLOCKS", "stream_read_probe"]
