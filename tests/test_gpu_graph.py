"""A decode step captured in a HIP graph replays to the eager result.

Every replay is checked bit for bit against the eager step, with eager work
and synchronisations between the replays.  The library records no memset
nodes: every buffer it writes is fully overwritten by its kernels.
"""
import pytest
import torch

import synthetic as syn

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager(gpu):
    import compressed_kv_cache_amd as g
    cfg = syn.with_overrides(syn.get_config("wide_rope_append"), B=8, T=3000)
    x = syn.make_gva_inputs(cfg, device=gpu)
    ws = torch.zeros(g.decode_workspace_bytes(cfg.B, cfg.H, x["v_pool"], x["k_pool"],
                                              x["block_table"], x["max_seq_len"]),
                     dtype=torch.uint8, device=gpu)
    qa = torch.empty((cfg.B, cfg.H, cfg.d_h + cfg.d_r), device=gpu)
    out = torch.empty((cfg.B, cfg.H, cfg.d_h), device=gpu)
    lse = torch.empty((cfg.B, cfg.H), device=gpu)

    def step():
        g.append_cache(x["v_new"], x["k_new"], x["pos"], x["block_table"],
                       x["v_pool"], x["k_pool"])
        g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"], out=qa)
        g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"],
                           x["seq_lens"], x["max_seq_len"], workspace=ws, out=out,
                           lse=lse)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step()
    for i in range(5):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        qa.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {i}"
        assert torch.equal(lse, ref_lse), f"replay {i}"
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)


def test_prefill_step_graph_replays_match_eager(gpu):
    """The many-token step (append L new tokens, absorb, blocked prefill
    kernel) captured in a graph: every replay equals the eager result."""
    import compressed_kv_cache_amd as g
    L = 96
    base = syn.get_config("long_ragged")
    cfg = syn.with_overrides(base, B=3, H=16, G=4, d_h=64, d_n=48, d_r=16,
                             cache_dtype="bfloat16", len_range=None, T=None, append=True)
    x = syn.make_gva_multi_inputs(cfg, L, device=gpu,
                                  seq_lens=torch.tensor([96, 200, 321], dtype=torch.int32),
                                  shuffled=True)
    ws = torch.zeros(1 << 24, dtype=torch.uint8, device=gpu)
    out = torch.empty((cfg.B, cfg.H, L, cfg.d_h), device=gpu)
    lse = torch.empty((cfg.B, cfg.H, L), device=gpu)

    def step():
        g.decode_step_multi(x["q_nope"], x["q_rope"], x["M"], x["v_pool"], x["k_pool"],
                            x["block_table"], x["seq_lens"], x["max_seq_len"],
                            v_new=x["v_new"], k_new=x["k_new"], workspace=ws, out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    ref_out, ref_lse = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step()
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {i}"
        assert torch.equal(lse, ref_lse), f"replay {i}"
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
