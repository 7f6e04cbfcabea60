"""The seeded synthetic input generator: determinism and the stated recipe."""
import math

import numpy as np
import torch

import synthetic as syn


def test_deterministic_by_seed():
    cfg = syn.get_config("tiny_fp32")
    a = syn.make_gva_inputs(cfg)
    b = syn.make_gva_inputs(cfg)
    c = syn.make_gva_inputs(cfg, seed=1)
    for k in ("q_nope", "q_rope", "M", "v_pool", "k_pool"):
        assert torch.equal(a[k].nan_to_num(7.0), b[k].nan_to_num(7.0))
    assert not torch.equal(a["q_nope"], c["q_nope"])


def test_scale_matched_maps_match_query_rms():
    """sigma_M = sigma_Q / (sigma_V sqrt(d_in)) makes the reconstructed content
    keys K_h = V M_h as large as the queries (agihunt.info summary,
    initialisation paragraph; onedev.kr review, "How it differs")."""
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=4, T=1024)
    x = syn.make_gva_inputs(cfg)
    V = x["v_pool"][:4].float().reshape(-1, cfg.G, cfg.d_h)
    K = torch.einsum("tgd,hdn->thn", V[:, :1], x["M"])  # group 0 for all heads
    rms_k = K.pow(2).mean().sqrt().item()
    rms_q = x["q_nope"].pow(2).mean().sqrt().item()
    assert abs(rms_k / rms_q - 1) < 0.1
    assert abs(x["sigma_M"] - 1 / math.sqrt(cfg.d_h)) < 1e-15


def test_ragged_layout_and_poison():
    cfg = syn.with_overrides(syn.get_config("long_ragged"),
                             len_range=(100, 700))
    x = syn.make_gva_inputs(cfg)
    lens = x["seq_lens_host"].tolist()
    assert all(100 <= n <= 700 for n in lens)
    bs = cfg.block_size
    nblk = [-(-n // bs) for n in lens]
    ids = torch.cat([x["block_table_host"][b, :nblk[b]] for b in range(cfg.B)])
    assert sorted(ids.tolist()) == list(range(x["num_blocks"]))  # permutation
    assert ids.tolist() != list(range(x["num_blocks"]))          # shuffled
    for b, n in enumerate(lens):
        blk = int(x["block_table_host"][b, (n - 1) // bs])
        s = (n - 1) % bs
        assert torch.isfinite(x["v_pool"][blk, s]).all()
        if s + 1 < bs:
            assert torch.isnan(x["v_pool"][blk, s + 1:].float()).all()
            assert torch.isnan(x["k_pool"][blk, s + 1:].float()).all()


def test_append_slot_is_poisoned():
    cfg = syn.with_overrides(syn.get_config("wide_rope_append"), B=3, T=100)
    x = syn.make_gva_inputs(cfg)
    for b in range(cfg.B):
        p = int(x["pos"][b])
        blk = int(x["block_table_host"][b, p // 64])
        assert torch.isnan(x["v_pool"][blk, p % 64].float()).all()
        assert torch.isnan(x["k_pool"][blk, p % 64].float()).all()
    assert x["v_new"].shape == (3, cfg.G, cfg.d_h)
    assert x["k_new"].shape == (3, cfg.d_r)


def test_bf16_cache_values_are_bf16():
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=2, T=64)
    x = syn.make_gva_inputs(cfg)
    assert x["v_pool"].dtype == torch.bfloat16
    assert x["k_pool"].dtype == torch.bfloat16


def test_configs_have_split_head_width():
    for name in syn.CONFIG_ORDER:
        c = syn.get_config(name)
        assert c.d_n + c.d_r == c.d_h
        assert c.H % c.G == 0 and c.d_r % 2 == 0
