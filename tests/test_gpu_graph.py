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
