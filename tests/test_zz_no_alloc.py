"""The step that allocates nothing (gva_decode_step_noalloc), through the C
ABI: two calls in a row, the second with a smaller batch and context, each
bit-identical to the step with a caller-provided workspace on the same
inputs (the two entry points share their kernels), and within the bf16 bar
of the float64 oracle.

Runs alone in a fresh process and after the other GPU tests: the second
call's sizes differ from the first, and the library clears the split
counters it uses in every call, so no earlier call's scratch contents can
leak into a later one.
"""
import numpy as np
import pytest
import torch

import oracle as o
import synthetic as syn
from parity_util import announce, assert_bf16_parity, cpu

pytestmark = pytest.mark.gpu


def _inputs(dev, B, T, seed):
    cfg = syn.with_overrides(syn.get_config("wide_rope_append"), B=B, T=T)
    return cfg, syn.make_gva_inputs(cfg, device=dev, seed=seed)


def _check(g, dev, B, T, seed):
    cfg, x = _inputs(dev, B, T, seed)
    announce("noalloc step", "B", B, "T", T, "seed", seed)
    h = {k: cpu(v) for k, v in x.items() if isinstance(v, torch.Tensor)}
    args = (x["q_nope"], x["q_rope"], x["M"], x["v_pool"], x["k_pool"], x["block_table"],
            x["seq_lens"], x["max_seq_len"])
    out_ref = torch.full((B, cfg.H, cfg.d_h), float("nan"), device=dev)
    lse_ref = torch.full((B, cfg.H), float("nan"), device=dev)
    g.decode_step(*args, v_new=x["v_new"], k_new=x["k_new"], rope_base=cfg.rope_base,
                  out=out_ref, lse=lse_ref)
    out = torch.full_like(out_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    g.decode_step_noalloc(*args, v_new=x["v_new"], k_new=x["k_new"],
                          rope_base=cfg.rope_base, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    assert torch.equal(lse, lse_ref)
    # and the oracle (after its own append)
    vp, kp = o.append_token(h["v_pool"], h["k_pool"], h["v_new"], h["k_new"], h["pos"],
                            h["block_table"], base=cfg.rope_base, cache_dtype="bfloat16")
    ref, ref_lse = o.gva_decode_materialized(h["q_nope"], h["q_rope"], h["M"], vp, kp,
                                             h["block_table"], h["seq_lens"],
                                             base=cfg.rope_base)
    assert_bf16_parity(cpu(out).double().numpy(), ref, what="noalloc out")
    np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, atol=1e-3)


def test_noalloc_step_two_calls_second_smaller(gpu):
    import compressed_kv_cache_amd as g
    _check(g, gpu, B=12, T=3000, seed=5)
    _check(g, gpu, B=3, T=700, seed=6)
