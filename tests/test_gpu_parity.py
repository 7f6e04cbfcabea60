"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Every workload is checked end to end -- append (where the workload has it),
absorb, decode -- against the oracle that materialises K_h = V_g(h) M_h.
Small workloads are compared in full; the large ones in full on the GPU and
on sampled (sequence, head) pairs for the oracle, in the same launch
configuration the benchmark times.
"""
import math

import numpy as np
import pytest
import torch

import oracle as o
import synthetic as syn
from parity_util import (announce, assert_bf16_parity, assert_bf16_split_precision,
                         assert_fp32_parity, cpu, seq_subpool)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g(gpu):
    import compressed_kv_cache_amd as pkg
    return pkg


def run_step(g, x, cfg):
    """append (if any) -> absorb -> decode on the GPU; returns (qa, out, lse)."""
    if cfg.append:
        g.append_cache(x["v_new"], x["k_new"], x["pos"], x["block_table"],
                       x["v_pool"], x["k_pool"], rope_base=cfg.rope_base)
    qa = g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"],
                        rope_base=cfg.rope_base)
    out, lse = g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                  x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    return qa, out, lse


def oracle_pools(x, cfg):
    """The caches the oracle attends over (after its own append)."""
    if not cfg.append:
        return x["v_pool"], x["k_pool"]
    return o.append_token(x["v_pool"], x["k_pool"], x["v_new"], x["k_new"],
                          x["pos_host"], x["block_table_host"], base=cfg.rope_base,
                          cache_dtype=cfg.cache_dtype)


def gen(cfg, dev, **kw):
    x = syn.make_gva_inputs(cfg, device=dev, **kw)
    x["pos_host"] = cpu(x["pos"])
    host = {k: cpu(v) for k, v in x.items() if isinstance(v, torch.Tensor)}
    return x, host


# ----------------------------------------------------------- tiny fp32 ----

def test_tiny_fp32_end_to_end(g, gpu):
    cfg = syn.get_config("tiny_fp32")
    announce("tiny_fp32 end to end")
    x, h = gen(cfg, gpu)
    qa, out, lse = run_step(g, x, cfg)
    ref_out, ref_lse = o.gva_decode_materialized(
        h["q_nope"], h["q_rope"], h["M"], h["v_pool"], h["k_pool"],
        h["block_table"], h["seq_lens"], base=cfg.rope_base)
    ref_qa = o.absorb_query(h["q_nope"], h["q_rope"], h["M"], h["pos"])
    assert_fp32_parity(cpu(qa), ref_qa, tol=1e-6, what="qa")
    assert_fp32_parity(cpu(out), ref_out, what="out")
    assert_fp32_parity(cpu(lse), ref_lse, what="lse")


# ------------------------------------------------------ bf16 workloads ----

def _check_all(g, gpu, cfg, seqs=None, heads=None, **kw):
    x, h = gen(cfg, gpu, **kw)
    announce(cfg.name, "B", cfg.B, "lens", x["seq_lens_host"][:8].tolist())
    qa, out, lse = run_step(g, x, cfg)
    vp, kp = oracle_pools(h, cfg)
    ref_out, ref_lse = o.gva_decode_materialized(
        h["q_nope"], h["q_rope"], h["M"], vp, kp, h["block_table"],
        h["seq_lens"], base=cfg.rope_base, seqs=seqs, heads=heads)
    sel = np.isfinite(ref_lse)
    got = cpu(out).double().numpy()
    assert_bf16_parity(got[sel], ref_out[sel], what=cfg.name + " out")
    assert_bf16_split_precision(got[sel], ref_out[sel], what=cfg.name + " out")
    np.testing.assert_allclose(cpu(lse).double().numpy()[sel], ref_lse[sel],
                               rtol=0, atol=1e-3)
    return x, h, out


def test_decode_350m_full(g, gpu):
    _check_all(g, gpu, syn.get_config("decode_350m"))


def test_wide_rope_append_full(g, gpu):
    cfg = syn.get_config("wide_rope_append")
    x, h, _ = _check_all(g, gpu, cfg)
    # appended slots, bit for bit against the oracle's own append
    vp, kp = o.append_token(h["v_pool"], h["k_pool"], h["v_new"], h["k_new"],
                            h["pos"], h["block_table"], base=cfg.rope_base,
                            cache_dtype="bfloat16")
    for b in range(cfg.B):
        p = int(h["pos"][b])
        blk = int(h["block_table"][b, p // 64])
        gv = cpu(x["v_pool"][blk, p % 64]).double().numpy()
        gk = cpu(x["k_pool"][blk, p % 64]).double().numpy()
        np.testing.assert_array_equal(gv, vp[blk, p % 64])
        np.testing.assert_array_equal(gk, kp[blk, p % 64])


def test_long_ragged_sampled_heads(g, gpu):
    cfg = syn.get_config("long_ragged")
    _check_all(g, gpu, cfg, heads=[0, 7, 15])


def test_large_model_sampled(g, gpu):
    cfg = syn.get_config("large_model")
    announce("large_model generate")
    x = syn.make_gva_inputs(cfg, device=gpu)
    announce("large_model run")
    qa, out, lse = run_step(g, x, cfg)
    qh, qrh, Mh = cpu(x["q_nope"]), cpu(x["q_rope"]), cpu(x["M"])
    pairs = [(0, 0), (37, 13), (127, 31), (64, 4)]
    for b, hh in pairs:
        sub = seq_subpool(x, b)
        ref, ref_lse = o.gva_decode_materialized(
            qh[b:b + 1], qrh[b:b + 1], Mh, sub["v_pool"], sub["k_pool"],
            sub["block_table"], sub["seq_lens"], base=cfg.rope_base, heads=[hh])
        assert_bf16_parity(cpu(out[b, hh]).double().numpy(), ref[0, hh],
                           what=f"large_model b={b} h={hh}")
        assert_bf16_split_precision(cpu(out[b, hh]).double().numpy(), ref[0, hh],
                                    what=f"large_model b={b} h={hh}")
        assert abs(float(lse[b, hh]) - ref_lse[0, hh]) < 1e-3


# ----------------------------------------------------------- edge cases ----

EDGE_LENS = [1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 127, 128, 129, 1000]


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
@pytest.mark.parametrize("shape", [
    # (H, G, d_h, d_n, d_r)
    (16, 4, 64, 48, 16),
    (8, 8, 32, 24, 8),
    (4, 1, 128, 96, 32),
    (32, 8, 128, 96, 32),
    (16, 4, 64, 40, 24),
    (16, 2, 64, 62, 2),
    (16, 4, 64, 32, 32),     # matrix cores: d_h 64, d_r 32
    (16, 4, 128, 112, 16),   # matrix cores: d_h 128, d_r 16
    (64, 16, 64, 48, 16),    # matrix cores: four head tiles per block
    (128, 32, 64, 48, 16),   # matrix cores: eight head tiles, 8 waves per block
])
def test_ragged_edges(g, gpu, shape, dtype):
    H, G, d_h, d_n, d_r = shape
    base = syn.get_config("long_ragged")
    cfg = syn.with_overrides(base, B=len(EDGE_LENS), H=H, G=G, d_h=d_h, d_n=d_n,
                             d_r=d_r, cache_dtype=dtype, len_range=None, T=None)
    lens = torch.tensor(EDGE_LENS, dtype=torch.int32)
    x, h = gen(cfg, gpu, seq_lens=lens, shuffled=True)
    announce("ragged edges", shape, dtype)
    if dtype == "float32" and H == 128:
        # fp32 caches run on the vector kernel, whose per-block head state
        # does not hold 128 heads: reported, not computed
        with pytest.raises(g.GvaError) as e:
            run_step(g, x, cfg)
        assert e.value.status == 3  # GVA_ERR_UNSUPPORTED
        return
    qa, out, lse = run_step(g, x, cfg)
    ref, ref_lse = o.gva_decode_materialized(
        h["q_nope"], h["q_rope"], h["M"], h["v_pool"], h["k_pool"],
        h["block_table"], h["seq_lens"], base=cfg.rope_base)
    if dtype == "float32":
        assert_fp32_parity(cpu(out), ref)
        assert_fp32_parity(cpu(lse), ref_lse)
    else:
        assert_bf16_parity(cpu(out).double().numpy(), ref)
        np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, atol=1e-3)


def test_zero_length_and_slack_max_seq_len(g, gpu):
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=4, T=None)
    lens = torch.tensor([0, 5, 0, 300], dtype=torch.int32)
    x, h = gen(cfg, gpu, seq_lens=lens)
    qa = g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    # max_seq_len larger than any length: the extra chunks are empty
    mx = 64 * x["block_table"].shape[1]
    out, lse = g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                  x["seq_lens"], mx)
    torch.cuda.synchronize()
    o_ = cpu(out).double().numpy()
    l_ = cpu(lse).double().numpy()
    assert np.all(o_[0] == 0) and np.all(o_[2] == 0)
    assert np.all(l_[0] == -np.inf) and np.all(l_[2] == -np.inf)
    ref, ref_lse = o.gva_decode_materialized(
        h["q_nope"], h["q_rope"], h["M"], h["v_pool"], h["k_pool"],
        h["block_table"], h["seq_lens"], seqs=[1, 3])
    assert_bf16_parity(o_[[1, 3]], ref[[1, 3]])


def test_out_of_range_device_values_give_nan(g, gpu):
    """A length beyond max_seq_len or a block id beyond the pool is reported as
    NaN output for that sequence; the others are unaffected."""
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=3, T=128)
    x, h = gen(cfg, gpu)
    qa = g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    bt = x["block_table"].clone()
    bt[1, 1] = x["num_blocks"] + 5       # block id past the pool
    sl = x["seq_lens"].clone()
    sl[2] = 10_000                       # longer than max_seq_len
    out, lse = g.decode_attention(qa, x["v_pool"], x["k_pool"], bt, sl, 128)
    torch.cuda.synchronize()
    o_ = cpu(out)
    assert torch.isnan(o_[1]).all() and torch.isnan(o_[2]).all()
    assert torch.isfinite(o_[0]).all()


# ------------------------------------------------------------ properties ----

def test_constant_values_give_constant_output(g, gpu):
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=2, T=777)
    x, _ = gen(cfg, gpu)
    nb = x["num_blocks"]
    x["v_pool"].fill_(1.0)
    qa = g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    out, _ = g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    np.testing.assert_allclose(cpu(out).numpy(), 1.0, rtol=0, atol=1e-6)


def test_zero_query_gives_mean_of_values(g, gpu):
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=2, T=500)
    x, h = gen(cfg, gpu)
    qa = torch.zeros((cfg.B, cfg.H, cfg.d_h + cfg.d_r), device=gpu)
    out, lse = g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                  x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    for b in range(cfg.B):
        sub = seq_subpool(x, b)
        V = o.gather_tokens(o.to_f64(sub["v_pool"]), sub["block_table"][0], 500, 64)
        for hh in range(cfg.H):
            ref = V[:, hh // 4].mean(0)
            np.testing.assert_allclose(cpu(out[b, hh]).numpy(), ref, atol=1e-5)
        np.testing.assert_allclose(cpu(lse[b]).numpy(), math.log(500), atol=1e-5)


def test_bitwise_deterministic(g, gpu):
    cfg = syn.with_overrides(syn.get_config("long_ragged"), len_range=(100, 5000))
    x, _ = gen(cfg, gpu)
    qa = g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    a, la = g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"],
                               x["seq_lens"], x["max_seq_len"])
    b, lb = g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"],
                               x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_paged_shuffled_equals_contiguous(g, gpu):
    """The same token rows reached through a shuffled table or through the
    identity table give bit-identical results."""
    cfg = syn.with_overrides(syn.get_config("long_ragged"), len_range=(300, 3000))
    x, h = gen(cfg, gpu)
    qa = g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    a, _ = g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"],
                              x["seq_lens"], x["max_seq_len"])
    # lay the same rows out contiguously: block i of seq b -> slot order
    lens = x["seq_lens_host"].tolist()
    nbs = [-(-n // 64) for n in lens]
    ids = torch.cat([x["block_table_host"][b, :nbs[b]] for b in range(cfg.B)]).long()
    vp = x["v_pool"][ids.to(gpu)].contiguous()
    kp = x["k_pool"][ids.to(gpu)].contiguous()
    table = torch.zeros_like(x["block_table_host"])
    off = 0
    for b, nb in enumerate(nbs):
        table[b, :nb] = torch.arange(off, off + nb)
        off += nb
    b_, _ = g.decode_attention(qa, vp, kp, table.to(gpu), x["seq_lens"],
                               x["max_seq_len"])
    torch.cuda.synchronize()
    assert torch.equal(a, b_)


# -------------------------------------------------------------------- GQA ----

@pytest.mark.parametrize("name,sample", [("decode_350m", None),
                                         ("large_model", [(0, 0), (99, 30)])])
def test_gqa_decode(g, gpu, name, sample):
    cfg = syn.get_config(name)
    announce("gqa", name)
    x = syn.make_gqa_inputs(cfg, device=gpu)
    out, lse = g.gqa_decode_attention(x["q"], x["k_pool"], x["v_pool"],
                                      x["block_table"], x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    if sample is None:
        h = {k: cpu(v) for k, v in x.items() if isinstance(v, torch.Tensor)}
        ref, ref_lse = o.gqa_decode(h["q"], h["k_pool"], h["v_pool"], h["block_table"],
                                    h["seq_lens"])
        assert_bf16_parity(cpu(out).double().numpy(), ref, what="gqa out")
        np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, atol=1e-3)
    else:
        qh = cpu(x["q"])
        for b, hh in sample:
            sub = seq_subpool(x, b)
            ref, _ = o.gqa_decode(qh[b:b + 1], sub["k_pool"], sub["v_pool"],
                                  sub["block_table"], sub["seq_lens"], heads=[hh])
            assert_bf16_parity(cpu(out[b, hh]).double().numpy(), ref[0, hh])


def test_gqa_small_fp32(g, gpu):
    cfg = syn.with_overrides(syn.get_config("tiny_fp32"), B=3, T=None,
                             len_range=(1, 300), shuffled_blocks=True)
    x = syn.make_gqa_inputs(cfg, device=gpu)
    out, lse = g.gqa_decode_attention(x["q"], x["k_pool"], x["v_pool"],
                                      x["block_table"], x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    h = {k: cpu(v) for k, v in x.items() if isinstance(v, torch.Tensor)}
    ref, ref_lse = o.gqa_decode(h["q"], h["k_pool"], h["v_pool"], h["block_table"],
                                h["seq_lens"])
    assert_fp32_parity(cpu(out), ref)


def test_reference_kernel_on_matrix_core_shapes(g, gpu, monkeypatch):
    """The plain VALU kernel, forced on a bf16 shape the matrix-core kernel
    normally takes, agrees with the oracle and (to rounding) with it."""
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=3, T=None,
                             len_range=(1, 2000), shuffled_blocks=True)
    x, h = gen(cfg, gpu)
    qa = g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    fast, _ = g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                 x["seq_lens"], x["max_seq_len"])
    monkeypatch.setenv("GVA_FORCE_REF", "1")
    ref_k, _ = g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                  x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    ref, _ = o.gva_decode_materialized(h["q_nope"], h["q_rope"], h["M"], h["v_pool"],
                                       h["k_pool"], h["block_table"], h["seq_lens"])
    assert_bf16_parity(cpu(ref_k).double().numpy(), ref, what="reference kernel")
    assert_bf16_parity(cpu(fast).double().numpy(), ref, what="matrix-core kernel")


def test_workspace_reused_across_calls(g, gpu):
    """One zero-filled workspace serves many calls with different lengths (the
    per-sequence counters reset themselves): every call matches a call with
    a fresh workspace bit for bit."""
    cfg = syn.with_overrides(syn.get_config("long_ragged"), len_range=(3000, 20000))
    x, _ = gen(cfg, gpu)
    qa = g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    mx = x["max_seq_len"]
    ws = torch.zeros(g.decode_workspace_bytes(cfg.B, cfg.H, x["v_pool"], x["k_pool"],
                                              x["block_table"], mx),
                     dtype=torch.uint8, device=gpu)
    full = x["seq_lens"]
    variants = [full, (full // 3).clamp_min(1), full.clamp_max(64), full,
                torch.zeros_like(full), full]
    for i, lens in enumerate(variants):
        a, la = g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"], lens, mx,
                                   workspace=ws)
        b, lb = g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"], lens, mx)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(la, lb), f"call {i}"


# ------------------------------------------------------------ fused step ----

@pytest.mark.parametrize("name,kw", [
    ("wide_rope_append", {"B": 8, "T": 3000}),
    ("decode_350m", {"B": 4, "T": 1000, "append": True}),
    ("tiny_fp32", {"append": True}),
    ("large_model", {"B": 4, "T": 700, "append": True}),
])
def test_decode_step_matches_oracle_and_separate_calls(g, gpu, name, kw):
    """gva_decode_step (append + absorb + decode in two launches) equals the
    oracle, and equals the three separate calls bit for bit."""
    cfg = syn.with_overrides(syn.get_config(name), **kw)
    announce("decode_step", name, kw)
    x, h = gen(cfg, gpu)
    vp0, kp0 = x["v_pool"].clone(), x["k_pool"].clone()
    out, lse = g.decode_step(x["q_nope"], x["q_rope"], x["M"], x["v_pool"], x["k_pool"],
                             x["block_table"], x["seq_lens"], x["max_seq_len"],
                             v_new=x["v_new"], k_new=x["k_new"], rope_base=cfg.rope_base)
    torch.cuda.synchronize()
    # the same through the separate entry points, on fresh copies of the caches
    x2 = dict(x)
    x2["v_pool"], x2["k_pool"] = vp0, kp0
    _, out2, lse2 = run_step(g, x2, cfg)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    assert torch.equal(x["v_pool"].nan_to_num(7), vp0.nan_to_num(7))
    assert torch.equal(x["k_pool"].nan_to_num(7), kp0.nan_to_num(7))
    vp, kp = oracle_pools(h, cfg)
    ref, ref_lse = o.gva_decode_materialized(
        h["q_nope"], h["q_rope"], h["M"], vp, kp, h["block_table"], h["seq_lens"],
        base=cfg.rope_base)
    if cfg.cache_dtype == "float32":
        assert_fp32_parity(cpu(out), ref)
    else:
        assert_bf16_parity(cpu(out).double().numpy(), ref)
        assert_bf16_split_precision(cpu(out).double().numpy(), ref)


def test_decode_step_at_the_benchmark_configuration(g, gpu):
    """The call the benchmark times, at its sizes: gva_decode_step with the
    append on the 350M-shaped workload (B = 32, T = 4096), its workspace
    zero-filled once and reused, against the oracle over every sequence and
    head, on two calls in a row (the second starts from the counters the
    first left)."""
    cfg = syn.with_overrides(syn.get_config("decode_350m"), append=True)
    announce("decode_step at the benchmark configuration", cfg.B, cfg.T)
    x, h = gen(cfg, gpu)
    ws = torch.zeros(g.decode_step_workspace_bytes(x["q_nope"], x["q_rope"], x["v_pool"],
                                                   x["k_pool"], x["block_table"],
                                                   x["max_seq_len"]),
                     dtype=torch.uint8, device=gpu)
    vp, kp = oracle_pools(h, cfg)
    ref, ref_lse = o.gva_decode_materialized(
        h["q_nope"], h["q_rope"], h["M"], vp, kp, h["block_table"], h["seq_lens"],
        base=cfg.rope_base)
    first = None
    for call in range(2):
        out = torch.full((cfg.B, cfg.H, cfg.d_h), float("nan"), device=gpu)
        lse = torch.full((cfg.B, cfg.H), float("nan"), device=gpu)
        g.decode_step(x["q_nope"], x["q_rope"], x["M"], x["v_pool"], x["k_pool"],
                      x["block_table"], x["seq_lens"], x["max_seq_len"], v_new=x["v_new"],
                      k_new=x["k_new"], rope_base=cfg.rope_base, workspace=ws, out=out,
                      lse=lse)
        torch.cuda.synchronize()
        got = cpu(out).double().numpy()
        assert_bf16_parity(got, ref, what=f"call {call}")
        assert_bf16_split_precision(got, ref, what=f"call {call}")
        np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, rtol=0, atol=1e-3)
        if first is None:
            first = out.clone()
        else:
            assert torch.equal(out, first)  # bitwise reproducible
    assert int(ws[:4].view(torch.int32).item()) == 0  # counters left at zero


def test_decode_step_without_append(g, gpu):
    cfg = syn.with_overrides(syn.get_config("long_ragged"), len_range=(100, 3000))
    x, h = gen(cfg, gpu)
    out, _ = g.decode_step(x["q_nope"], x["q_rope"], x["M"], x["v_pool"], x["k_pool"],
                           x["block_table"], x["seq_lens"], x["max_seq_len"])
    _, out2, _ = run_step(g, x, cfg)
    assert torch.equal(out, out2)


# ------------------------------------------------------- split extremes ----

def test_one_long_sequence_many_chunks(g, gpu):
    """One sequence split over ~256 chunks: the final merge runs many rounds."""
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=1, T=70000)
    x, h = gen(cfg, gpu)
    announce("one long sequence", cfg.T)
    qa, out, lse = run_step(g, x, cfg)
    ref, ref_lse = o.gva_decode_materialized(
        h["q_nope"], h["q_rope"], h["M"], h["v_pool"], h["k_pool"], h["block_table"],
        h["seq_lens"], base=cfg.rope_base)
    assert_bf16_parity(cpu(out).double().numpy(), ref)
    np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, atol=1e-3)


def test_more_sequences_than_split_target(g, gpu):
    """B = 300 short sequences (more than the ~256 chunks aimed for)."""
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=300, T=None,
                             len_range=(1, 200))
    x, h = gen(cfg, gpu)
    announce("B=300")
    qa, out, lse = run_step(g, x, cfg)
    ref, ref_lse = o.gva_decode_materialized(
        h["q_nope"], h["q_rope"], h["M"], h["v_pool"], h["k_pool"], h["block_table"],
        h["seq_lens"], base=cfg.rope_base)
    assert_bf16_parity(cpu(out).double().numpy(), ref)
    np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, atol=1e-3)


@pytest.mark.parametrize("H,G,d_h", [(16, 4, 64), (32, 8, 128)])
def test_gqa_ragged_edges(g, gpu, H, G, d_h):
    base = syn.get_config("long_ragged")
    cfg = syn.with_overrides(base, B=len(EDGE_LENS), H=H, G=G, d_h=d_h, d_n=d_h - 16,
                             d_r=16, len_range=None, T=None)
    lens = torch.tensor(EDGE_LENS, dtype=torch.int32)
    y = syn.make_gqa_inputs(cfg, device=gpu, seq_lens=lens)  # shuffled block table
    announce("gqa ragged edges", H, G, d_h)
    out, lse = g.gqa_decode_attention(y["q"], y["k_pool"], y["v_pool"], y["block_table"],
                                      y["seq_lens"], y["max_seq_len"])
    h = {k: cpu(v) for k, v in y.items() if isinstance(v, torch.Tensor)}
    ref, ref_lse = o.gqa_decode(h["q"], h["k_pool"], h["v_pool"], h["block_table"],
                                h["seq_lens"])
    assert_bf16_parity(cpu(out).double().numpy(), ref)
    np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, atol=1e-3)


# --------------------------------------------------------- width variants ----

@pytest.mark.parametrize("H,G,d_h,d_n,dtype", [
    (16, 4, 64, 48, "bfloat16"),     # matrix cores, d_h 64
    (32, 8, 128, 96, "bfloat16"),    # matrix cores, d_h 128
    (8, 8, 32, 24, "float32"),       # vector path
])
def test_no_positional_slice(g, gpu, H, G, d_h, d_n, dtype):
    """d_r = 0: scores use the absorbed content slice only; the fused step
    appends values only."""
    base = syn.get_config("long_ragged")
    cfg = syn.with_overrides(base, B=len(EDGE_LENS), H=H, G=G, d_h=d_h, d_n=d_n, d_r=0,
                             cache_dtype=dtype, len_range=None, T=None, append=True)
    lens = torch.tensor(EDGE_LENS, dtype=torch.int32)
    x, h = gen(cfg, gpu, seq_lens=lens, shuffled=True)
    announce("no positional slice", H, G, d_h, dtype)
    out, lse = g.decode_step(x["q_nope"], x["q_rope"], x["M"], x["v_pool"], x["k_pool"],
                             x["block_table"], x["seq_lens"], x["max_seq_len"],
                             v_new=x["v_new"], k_new=x["k_new"], rope_base=cfg.rope_base)
    vp, kp = oracle_pools(h, cfg)
    ref, ref_lse = o.gva_decode_materialized(
        h["q_nope"], h["q_rope"], h["M"], vp, kp, h["block_table"], h["seq_lens"],
        base=cfg.rope_base)
    if dtype == "float32":
        assert_fp32_parity(cpu(out), ref)
    else:
        assert_bf16_parity(cpu(out).double().numpy(), ref)
    np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, atol=1e-3)


def test_keys_equal_values_variant(g, gpu):
    """M_h = I, d_n = d_h, d_r = 0: the keys are the values themselves, so the
    decode equals textbook attention of q_nope over K = V (bisque.today
    explainer, Figure 3: the K = V variant, half the GQA cache)."""
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=4, T=1500, d_n=64, d_r=0)
    x, h = gen(cfg, gpu)
    eye = torch.eye(cfg.d_h, dtype=torch.float32)
    x["M"] = eye.expand(cfg.H, -1, -1).contiguous().to(gpu)
    announce("K = V variant")
    qa, out, lse = run_step(g, x, cfg)
    q = cpu(x["q_nope"]).double().numpy()
    scale = 1.0 / math.sqrt(cfg.d_h)
    for b in range(cfg.B):
        sub = seq_subpool(x, b)
        n = int(x["seq_lens_host"][b])
        V = sub["v_pool"].double().numpy().reshape(-1, cfg.G, cfg.d_h)[:n]
        for hh in range(cfg.H):
            Vg = V[:, o.head_group(hh, cfg.H, cfg.G), :]
            ref = o.softmax_attention(q[b, hh], Vg, Vg, scale)[0]
            assert_bf16_parity(cpu(out[b, hh]).double().numpy(), ref, what=f"b={b} h={hh}")


def test_additive_head_split(g, gpu):
    """d_n + d_r > d_h (content width not reduced by the position slice)."""
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=6, T=2000, d_n=64, d_r=16)
    x, h = gen(cfg, gpu)
    announce("additive split")
    qa, out, lse = run_step(g, x, cfg)
    ref, _ = o.gva_decode_materialized(
        h["q_nope"], h["q_rope"], h["M"], h["v_pool"], h["k_pool"], h["block_table"],
        h["seq_lens"], base=cfg.rope_base)
    assert_bf16_parity(cpu(out).double().numpy(), ref)


# ------------------------------------------ several query tokens (L > 1) ----

MULTI_LENS = [4, 5, 63, 64, 65, 66, 67, 128, 129, 1000]


def _multi_case(gpu, H, G, d_h, d_n, d_r, dtype, L, lens=MULTI_LENS, append=False):
    base = syn.get_config("long_ragged")
    cfg = syn.with_overrides(base, B=len(lens), H=H, G=G, d_h=d_h, d_n=d_n, d_r=d_r,
                             cache_dtype=dtype, len_range=None, T=None, append=append)
    x = syn.make_gva_multi_inputs(cfg, L, device=gpu,
                                  seq_lens=torch.tensor(lens, dtype=torch.int32),
                                  shuffled=True)
    h = {k: cpu(v) for k, v in x.items() if isinstance(v, torch.Tensor)}
    return cfg, x, h


@pytest.mark.parametrize("H,G,d_h,d_n,d_r,dtype,L", [
    (16, 4, 64, 48, 16, "bfloat16", 4),     # matrix cores, one group per head tile
    (16, 4, 64, 48, 16, "bfloat16", 2),     # matrix cores, two groups per head tile
    (16, 4, 64, 40, 24, "bfloat16", 4),
    (32, 8, 128, 96, 32, "bfloat16", 2),    # matrix cores, d_h 128
    (32, 8, 128, 96, 32, "bfloat16", 4),    # d_h 128, 8 head tiles of one group: 8 waves
    (32, 8, 128, 128, 0, "bfloat16", 4),
    (16, 4, 64, 64, 0, "bfloat16", 4),      # no positional slice
    (8, 8, 32, 24, 8, "float32", 3),        # vector path
    (16, 4, 64, 48, 16, "float32", 4),      # vector path, fp32 cache
])
def test_multi_query_decode(g, gpu, H, G, d_h, d_n, d_r, dtype, L):
    """L query tokens per sequence (positions len-L .. len-1), each attending
    causally; lengths put the causal tail across 64-token chunk edges."""
    cfg, x, h = _multi_case(gpu, H, G, d_h, d_n, d_r, dtype, L)
    announce("multi-query decode", H, G, d_h, d_r, dtype, "L", L)
    qa = g.absorb_query_multi(x["q_nope"], x["q_rope"], x["M"], x["pos"],
                              rope_base=cfg.rope_base)
    out, lse = g.decode_attention_multi(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                        x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    ref_qa = o.absorb_queries(h["q_nope"], h["q_rope"], h["M"], h["pos"],
                              base=cfg.rope_base)
    assert_fp32_parity(cpu(qa), ref_qa, tol=1e-6, what="qa")
    ref, ref_lse = o.gva_decode_materialized_queries(
        h["q_nope"], h["q_rope"], h["M"], h["v_pool"], h["k_pool"], h["block_table"],
        h["seq_lens"], base=cfg.rope_base)
    if dtype == "float32":
        assert_fp32_parity(cpu(out), ref)
        assert_fp32_parity(cpu(lse), ref_lse)
    else:
        assert_bf16_parity(cpu(out).double().numpy(), ref)
        assert_bf16_split_precision(cpu(out).double().numpy(), ref)
        np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, rtol=0, atol=1e-3)
        # these shapes run on the split matrix-core kernels (the blocked
        # prefill kernel, the fallback, needs no workspace)
        assert g.decode_workspace_bytes_multi(cfg.B, H, L, x["v_pool"], x["k_pool"],
                                              x["block_table"], x["max_seq_len"]) > 0


@pytest.mark.parametrize("L", [2, 4])
def test_multi_query_step_with_append(g, gpu, L):
    """gva_decode_step_multi: the L new tokens are appended (values bit for bit,
    rotated keys as the oracle rounds them), then the L queries attend."""
    cfg, x, h = _multi_case(gpu, 16, 4, 64, 48, 16, "bfloat16", L, append=True)
    announce("multi-query step", "L", L)
    out, lse = g.decode_step_multi(x["q_nope"], x["q_rope"], x["M"], x["v_pool"],
                                   x["k_pool"], x["block_table"], x["seq_lens"],
                                   x["max_seq_len"], v_new=x["v_new"], k_new=x["k_new"],
                                   rope_base=cfg.rope_base)
    torch.cuda.synchronize()
    vp, kp = o.append_tokens(h["v_pool"], h["k_pool"], h["v_new"], h["k_new"], h["pos"],
                             h["block_table"], base=cfg.rope_base, cache_dtype="bfloat16")
    for b, n in enumerate(MULTI_LENS):
        for p in range(n - L, n):
            blk, sl = int(h["block_table"][b, p // 64]), p % 64
            np.testing.assert_array_equal(cpu(x["v_pool"][blk, sl]).double().numpy(),
                                          vp[blk, sl])
            np.testing.assert_array_equal(cpu(x["k_pool"][blk, sl]).double().numpy(),
                                          kp[blk, sl])
    ref, ref_lse = o.gva_decode_materialized_queries(
        h["q_nope"], h["q_rope"], h["M"], vp, kp, h["block_table"], h["seq_lens"],
        base=cfg.rope_base)
    assert_bf16_parity(cpu(out).double().numpy(), ref)
    np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, rtol=0, atol=1e-3)


def test_multi_query_one_token_is_the_single_query_call(g, gpu):
    """q_len = 1 through the *_multi entry points gives the single-token
    call's results bit for bit."""
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=5, T=777)
    x, h = gen(cfg, gpu)
    announce("multi-query q_len 1")
    qa1 = g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    out1, lse1 = g.decode_attention(qa1, x["v_pool"], x["k_pool"], x["block_table"],
                                    x["seq_lens"], x["max_seq_len"])
    qam = g.absorb_query_multi(x["q_nope"][:, :, None].contiguous(),
                               x["q_rope"][:, :, None].contiguous(), x["M"], x["pos"])
    outm, lsem = g.decode_attention_multi(qam, x["v_pool"], x["k_pool"], x["block_table"],
                                          x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    assert torch.equal(qam[:, :, 0], qa1)
    assert torch.equal(outm[:, :, 0], out1)
    assert torch.equal(lsem[:, :, 0], lse1)


def test_multi_query_short_and_empty_sequences(g, gpu):
    """0 < len < L is invalid (NaN for that sequence only); len = 0 gives
    zeros and lse = -inf."""
    L = 4
    lens = [0, 3, 4, 70]
    cfg, x, h = _multi_case(gpu, 16, 4, 64, 48, 16, "bfloat16", L, lens=lens)
    announce("multi-query short sequences")
    qa = g.absorb_query_multi(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    out, lse = g.decode_attention_multi(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                        x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    out, lse = cpu(out), cpu(lse)
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(torch.isnan(out[1]))
    ref, _ = o.gva_decode_materialized_queries(
        h["q_nope"], h["q_rope"], h["M"], h["v_pool"], h["k_pool"], h["block_table"],
        h["seq_lens"], base=cfg.rope_base, seqs=[2, 3])
    assert_bf16_parity(out[2:].double().numpy(), ref[2:])


def test_multi_query_350m_shape_sampled(g, gpu):
    """Four query tokens per sequence at the 350M decode shape (the launch
    the benchmark times); the oracle checks three sequences in full."""
    cfg = syn.get_config("decode_350m")
    announce("multi-query 350M shape")
    x = syn.make_gva_multi_inputs(cfg, 4, device=gpu)
    qa = g.absorb_query_multi(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    out, lse = g.decode_attention_multi(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                        x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    for b in (0, 17, 31):
        sub = seq_subpool(x, b)
        ref, ref_lse = o.gva_decode_materialized_queries(
            cpu(x["q_nope"][b:b + 1]), cpu(x["q_rope"][b:b + 1]), cpu(x["M"]),
            sub["v_pool"], sub["k_pool"], sub["block_table"], sub["seq_lens"],
            base=cfg.rope_base)
        assert_bf16_parity(cpu(out[b:b + 1]).double().numpy(), ref, what=f"b={b}")
        np.testing.assert_allclose(cpu(lse[b:b + 1]).double().numpy(), ref_lse, atol=1e-3)


# ------------------------------ ordinary RoPE on the reconstructed key ----

@pytest.mark.parametrize("H,G,d_h,d_k", [
    (16, 4, 64, 64),
    (16, 4, 64, 48),
    (32, 8, 128, 64),
    (8, 1, 64, 32),       # eight heads per group
])
def test_rope_on_keys_decode(g, gpu, H, G, d_h, d_k):
    """Keys rebuilt and rotated per token, query rotated at len-1, against
    the float64 oracle that forms every rotated key; ragged lengths."""
    base = syn.get_config("long_ragged")
    cfg = syn.with_overrides(base, B=len(EDGE_LENS), H=H, G=G, d_h=d_h, d_n=d_k, d_r=0,
                             len_range=None, T=None)
    lens = torch.tensor(EDGE_LENS, dtype=torch.int32)
    x, h = gen(cfg, gpu, seq_lens=lens, shuffled=True)
    announce("rope on keys", H, G, d_h, d_k)
    out, lse = g.decode_rope_keys(x["q_nope"], x["M"], x["v_pool"], x["block_table"],
                                  x["seq_lens"], x["max_seq_len"], rope_base=cfg.rope_base)
    torch.cuda.synchronize()
    ref, ref_lse = o.gva_decode_rope_on_keys(h["q_nope"], h["M"], h["v_pool"],
                                             h["block_table"], h["seq_lens"],
                                             base=cfg.rope_base)
    assert_bf16_parity(cpu(out).double().numpy(), ref)
    np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, rtol=0, atol=1e-3)


def test_rope_on_keys_350m_shape_sampled(g, gpu):
    """The 350M decode shape without a positional slice (d_k = d_h = 64) at
    full size; the oracle checks three sequences in full."""
    cfg = syn.with_overrides(syn.get_config("decode_350m"), d_n=64, d_r=0)
    announce("rope on keys 350M shape")
    x = syn.make_gva_inputs(cfg, device=gpu)
    out, lse = g.decode_rope_keys(x["q_nope"], x["M"], x["v_pool"], x["block_table"],
                                  x["seq_lens"], x["max_seq_len"], rope_base=cfg.rope_base)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    for b in (0, 13, 31):
        sub = seq_subpool(x, b, keys=("v_pool",))
        ref, ref_lse = o.gva_decode_rope_on_keys(
            cpu(x["q_nope"][b:b + 1]), cpu(x["M"]), sub["v_pool"], sub["block_table"],
            sub["seq_lens"], base=cfg.rope_base)
        assert_bf16_parity(cpu(out[b:b + 1]).double().numpy(), ref, what=f"b={b}")
        np.testing.assert_allclose(cpu(lse[b:b + 1]).double().numpy(), ref_lse, atol=1e-3)


def test_rope_on_keys_invalid_lengths(g, gpu):
    """Zero length: zeros and -inf; a length past max_seq_len: NaN."""
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=3, T=None, d_n=64, d_r=0,
                             len_range=(1, 300))
    lens = torch.tensor([0, 200, 150], dtype=torch.int32)
    x, h = gen(cfg, gpu, seq_lens=lens)
    x["seq_lens"][2] = 10 ** 6
    announce("rope on keys invalid lengths")
    out, lse = g.decode_rope_keys(x["q_nope"], x["M"], x["v_pool"], x["block_table"],
                                  x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    out, lse = cpu(out), cpu(lse)
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(torch.isfinite(out[1]))
    assert torch.all(torch.isnan(out[2]))


# --------------------------------- many query tokens (prefill kernel) ----

@pytest.mark.parametrize("H,G,d_h,d_n,d_r,L,lens", [
    (16, 4, 64, 48, 16, 100, [100, 101, 163, 640]),   # prefill and prefix + chunk
    (16, 4, 64, 40, 24, 64, [64, 64, 65, 300]),
    (32, 8, 128, 96, 32, 48, [48, 129, 200]),
    (16, 4, 64, 64, 0, 33, [33, 97]),                  # no positional slice
    (16, 2, 64, 48, 16, 40, [40, 77]),                 # eight heads per group
    (8, 4, 64, 48, 16, 70, [70, 150]),                 # two heads per group
    (4, 4, 128, 112, 16, 17, [17, 260]),               # one head per group
    (16, 4, 64, 48, 16, 7, [7, 64, 90]),               # few tokens no other kernel takes
    (8, 2, 128, 104, 24, 130, [130, 700]),             # d_h 128 with the 24-wide slice
    (16, 4, 64, 48, 16, 333, [333, 900]),              # several query tiles, ragged tail
])
def test_many_query_tokens(g, gpu, H, G, d_h, d_n, d_r, L, lens):
    """L query tokens per sequence through the blocked (prefill) kernel:
    causal, after a cached prefix of len - L tokens, against the float64
    oracle that materialises every key."""
    cfg, x, h = _multi_case(gpu, H, G, d_h, d_n, d_r, "bfloat16", L, lens=lens)
    announce("many query tokens", H, G, d_h, d_r, "L", L, lens)
    qa = g.absorb_query_multi(x["q_nope"], x["q_rope"], x["M"], x["pos"],
                              rope_base=cfg.rope_base)
    out, lse = g.decode_attention_multi(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                        x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    ref, ref_lse = o.gva_decode_materialized_queries(
        h["q_nope"], h["q_rope"], h["M"], h["v_pool"], h["k_pool"], h["block_table"],
        h["seq_lens"], base=cfg.rope_base)
    assert_bf16_parity(cpu(out).double().numpy(), ref)
    np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, rtol=0, atol=1e-3)


def test_prefill_step_with_append(g, gpu):
    """gva_decode_step_multi with 96 new tokens: all appended (values bit for
    bit), then the causal attention of the 96 queries."""
    L = 96
    lens = [96, 200, 1000]
    cfg, x, h = _multi_case(gpu, 16, 4, 64, 48, 16, "bfloat16", L, lens=lens, append=True)
    announce("prefill step with append")
    out, lse = g.decode_step_multi(x["q_nope"], x["q_rope"], x["M"], x["v_pool"],
                                   x["k_pool"], x["block_table"], x["seq_lens"],
                                   x["max_seq_len"], v_new=x["v_new"], k_new=x["k_new"],
                                   rope_base=cfg.rope_base)
    torch.cuda.synchronize()
    vp, kp = o.append_tokens(h["v_pool"], h["k_pool"], h["v_new"], h["k_new"], h["pos"],
                             h["block_table"], base=cfg.rope_base, cache_dtype="bfloat16")
    for b, n in enumerate(lens):
        for p in range(n - L, n):
            blk, sl = int(h["block_table"][b, p // 64]), p % 64
            np.testing.assert_array_equal(cpu(x["v_pool"][blk, sl]).double().numpy(),
                                          vp[blk, sl])
    ref, ref_lse = o.gva_decode_materialized_queries(
        h["q_nope"], h["q_rope"], h["M"], vp, kp, h["block_table"], h["seq_lens"],
        base=cfg.rope_base)
    assert_bf16_parity(cpu(out).double().numpy(), ref)
    np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, rtol=0, atol=1e-3)


def test_many_query_tokens_invalid_lengths(g, gpu):
    """len = 0: zeros and -inf; 0 < len < L: NaN for that sequence only."""
    L = 32
    cfg, x, h = _multi_case(gpu, 16, 4, 64, 48, 16, "bfloat16", L, lens=[0, 20, 40])
    announce("many query tokens, invalid lengths")
    qa = g.absorb_query_multi(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    out, lse = g.decode_attention_multi(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                        x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    out, lse = cpu(out), cpu(lse)
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(torch.isnan(out[1]))
    ref, _ = o.gva_decode_materialized_queries(
        h["q_nope"], h["q_rope"], h["M"], h["v_pool"], h["k_pool"], h["block_table"],
        h["seq_lens"], base=cfg.rope_base, seqs=[2])
    assert_bf16_parity(out[2:].double().numpy(), ref[2:])


def test_many_query_tokens_out_of_range_device_values(g, gpu):
    """Blocked kernel: a block id past the pool or a length past max_seq_len
    gives NaN rows for that sequence only."""
    L = 40
    cfg, x, h = _multi_case(gpu, 16, 4, 64, 48, 16, "bfloat16", L, lens=[100, 200, 150])
    announce("many query tokens, out-of-range device values")
    qa = g.absorb_query_multi(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    bt = x["block_table"].clone()
    bt[1, 2] = x["num_blocks"] + 7
    sl = x["seq_lens"].clone()
    sl[2] = x["max_seq_len"] + 1
    out, lse = g.decode_attention_multi(qa, x["v_pool"], x["k_pool"], bt, sl, x["max_seq_len"])
    torch.cuda.synchronize()
    out, lse = cpu(out), cpu(lse)
    assert torch.isnan(out[1]).all() and torch.isnan(lse[1]).all()
    assert torch.isnan(out[2]).all() and torch.isnan(lse[2]).all()
    ref, _ = o.gva_decode_materialized_queries(
        h["q_nope"], h["q_rope"], h["M"], h["v_pool"], h["k_pool"], h["block_table"],
        h["seq_lens"], base=cfg.rope_base, seqs=[0])
    assert_bf16_parity(out[:1].double().numpy(), ref[:1])


def test_many_query_tokens_zero_query_is_running_mean(g, gpu):
    """Closed form, no oracle: with qa = 0 every visible key weighs the same,
    so query i (position len - L + i) returns the mean of the values at
    positions 0 .. len - L + i of its group, and lse = ln(len - L + i + 1)."""
    L = 200
    cfg, x, h = _multi_case(gpu, 8, 2, 128, 112, 16, "bfloat16", L, lens=[200, 333])
    announce("many query tokens, zero query")
    qa = torch.zeros((cfg.B, cfg.H, L, cfg.d_h + cfg.d_r), device=gpu)
    out, lse = g.decode_attention_multi(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                        x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    out, lse = cpu(out).double().numpy(), cpu(lse).double().numpy()
    hpg = cfg.H // cfg.G
    for b, n in enumerate([200, 333]):
        V = o.gather_tokens(o.to_f64(h["v_pool"]), h["block_table"][b], n, cfg.block_size)
        csum = np.cumsum(V, axis=0)  # [n, G, d_h]
        pos = np.arange(n - L, n)
        for hh in range(cfg.H):
            ref = csum[pos, hh // hpg] / (pos + 1)[:, None]
            assert_bf16_parity(out[b, hh], ref, what=f"b={b} h={hh}")
            np.testing.assert_allclose(lse[b, hh], np.log(pos + 1.0), rtol=0, atol=1e-4)


def test_prefill_350m_shape_sampled(g, gpu):
    """Prefill of 32 sequences of 4096 tokens at the 350M shape (every token a
    query); the oracle checks two (sequence, head) pairs in full."""
    cfg = syn.get_config("decode_350m")
    L = cfg.T
    announce("prefill 350M shape")
    x = syn.make_gva_multi_inputs(cfg, L, device=gpu)
    qa = g.absorb_query_multi(x["q_nope"], x["q_rope"], x["M"], x["pos"])
    out, lse = g.decode_attention_multi(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                        x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    for b, hh in ((0, 0), (31, 13)):
        sub = seq_subpool(x, b)
        ref, ref_lse = o.gva_decode_materialized_queries(
            cpu(x["q_nope"][b:b + 1]), cpu(x["q_rope"][b:b + 1]), cpu(x["M"]),
            sub["v_pool"], sub["k_pool"], sub["block_table"], sub["seq_lens"],
            base=cfg.rope_base, heads=[hh])
        assert_bf16_parity(cpu(out[b, hh]).double().numpy(), ref[0, hh], what=f"b={b} h={hh}")
        np.testing.assert_allclose(cpu(lse[b, hh]).double().numpy(), ref_lse[0, hh], atol=1e-3)


# ------------------------------- same-shape GQA with many query tokens ----

@pytest.mark.parametrize("H,G,d_h,L,lens", [
    (16, 4, 64, 64, [64, 65, 300]),        # prefill and prefix + chunk
    (32, 8, 128, 40, [40, 129]),           # d_h 128
    (16, 2, 64, 17, [17, 90]),             # eight heads per group
    (4, 4, 128, 100, [100, 230]),          # one head per group
    (16, 4, 64, 5, [5, 70]),               # few tokens (vector or blocked kernel)
])
def test_gqa_many_query_tokens(g, gpu, H, G, d_h, L, lens):
    """gqa_decode_attention_multi against the float64 GQA oracle: query i at
    position len - L + i, causal, keys and values of its group."""
    cfg = syn.with_overrides(syn.get_config("long_ragged"), B=len(lens), H=H, G=G, d_h=d_h,
                             d_n=d_h, d_r=0, cache_dtype="bfloat16", len_range=None,
                             T=None, append=False)
    x = syn.make_gqa_multi_inputs(cfg, L, device=gpu,
                                  seq_lens=torch.tensor(lens, dtype=torch.int32))
    announce("gqa many query tokens", H, G, d_h, "L", L, lens)
    out, lse = g.gqa_decode_attention_multi(x["q"], x["k_pool"], x["v_pool"],
                                            x["block_table"], x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    ref, ref_lse = o.gqa_decode_queries(cpu(x["q"]), cpu(x["k_pool"]), cpu(x["v_pool"]),
                                        cpu(x["block_table"]), cpu(x["seq_lens"]))
    assert_bf16_parity(cpu(out).double().numpy(), ref)
    np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, rtol=0, atol=1e-3)


def test_gqa_many_query_tokens_one_token_is_the_single_query_call(g, gpu):
    cfg = syn.with_overrides(syn.get_config("decode_350m"), B=3, T=300)
    x = syn.make_gqa_multi_inputs(cfg, 1, device=gpu)
    announce("gqa many query tokens, L = 1")
    o1, l1 = g.gqa_decode_attention_multi(x["q"], x["k_pool"], x["v_pool"], x["block_table"],
                                          x["seq_lens"], x["max_seq_len"])
    o0, l0 = g.gqa_decode_attention(x["q"][:, :, 0].contiguous(), x["k_pool"], x["v_pool"],
                                    x["block_table"], x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, 0], o0) and torch.equal(l1[:, :, 0], l0)


@pytest.mark.parametrize("L,lens", [
    (4, [2050]),           # 33 chunks of 64: a third group holding only positions
                           # past some queries' limits (records with max -inf)
    (1, [32 * 64 + 1]),    # 33 chunks, one token in the third group
    (2, [5000, 3000]),     # several groups per sequence, two sequences
    (1, [2048, 700]),      # 32 chunks: one level
])
def test_two_level_merge(g, gpu, L, lens):
    """More than 32 chunks per sequence: chunk records merge per group of 16,
    then the group records; against the float64 oracle."""
    cfg, x, h = _multi_case(gpu, 16, 4, 64, 48, 16, "bfloat16", L, lens=lens)
    announce("two-level merge", L, lens)
    qa = g.absorb_query_multi(x["q_nope"], x["q_rope"], x["M"], x["pos"],
                              rope_base=cfg.rope_base)
    ws = torch.zeros(max(16, g.decode_workspace_bytes_multi(
        cfg.B, cfg.H, L, x["v_pool"], x["k_pool"], x["block_table"], x["max_seq_len"])),
        dtype=torch.uint8, device=gpu)
    out, lse = g.decode_attention_multi(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                        x["seq_lens"], x["max_seq_len"], workspace=ws)
    torch.cuda.synchronize()
    ref, ref_lse = o.gva_decode_materialized_queries(
        h["q_nope"], h["q_rope"], h["M"], h["v_pool"], h["k_pool"], h["block_table"],
        h["seq_lens"], base=cfg.rope_base)
    assert_bf16_parity(cpu(out).double().numpy(), ref)
    np.testing.assert_allclose(cpu(lse).double().numpy(), ref_lse, rtol=0, atol=1e-3)
    # the call left every counter (sequence and group) at zero: a second call
    # on the same workspace gives the same bits
    out2, lse2 = g.decode_attention_multi(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                          x["seq_lens"], x["max_seq_len"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(lse2, lse)


# ---- read-rate probe (measurement helper) ----

@pytest.mark.parametrize("nbytes", [0, 16, 16 * 1023, 16 * 1025 + 16 * 7, (1 << 20) + 48,
                                    71303168])
def test_stream_read_probe_checksum(g, gpu, nbytes):
    """Every byte is read: the XOR of the probe's per-block words equals the
    XOR of all 32-bit words of the buffer (computed on the host), for sizes
    below, at and above one 16-byte unit per block, ragged per-block ranges
    and the 350M-shaped cache size; the output is fully overwritten."""
    announce(f"stream_read_probe bytes={nbytes}")
    gen = torch.Generator(device="cpu").manual_seed(nbytes % 9973)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=gen)
    buf = host.to(gpu)
    from compressed_kv_cache_amd._lib import PROBE_BLOCKS
    out = torch.full((PROBE_BLOCKS,), -1, dtype=torch.int32, device=gpu)
    g.stream_read_probe(buf, out=out)
    torch.cuda.synchronize()
    words = out.cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32)) if nbytes else np.uint32(0)
    assert np.bitwise_xor.reduce(words) == want
    if nbytes == 0:
        assert not words.any()


# ------------------------------------------- scores on the vector units ----
# GVA_DECODE_VALU=1 runs the single-token GVA decode with its scores on the
# vector units (v_dot2_f32_bf16 over the same bf16 high and low query parts),
# the rest of the kernel unchanged: the matrix-core ablation.  It must meet
# the same bars against the oracle.

@pytest.mark.parametrize("name,kw", [
    ("decode_350m", {}),
    ("wide_rope_append", {"B": 16, "T": 3000}),                  # d_r = 24
    ("decode_350m", {"B": 8, "T": 3000, "d_r": 0, "d_n": 64}),
    ("decode_350m", {"B": 8, "T": 3000, "d_r": 32, "d_n": 32}),
    ("decode_350m", {"B": len(EDGE_LENS), "T": None, "len_range": None}),
    ("large_model", {"B": 3, "T": 2000, "with_gqa": False}),     # d_h = 128, d_r = 32
])
def test_vector_unit_scores(g, gpu, monkeypatch, name, kw):
    cfg = syn.with_overrides(syn.get_config(name), **kw)
    monkeypatch.setenv("GVA_DECODE_VALU", "1")
    announce("vector-unit scores", name, kw)
    extra = {}
    if cfg.T is None and cfg.len_range is None:
        extra = {"seq_lens": torch.tensor(EDGE_LENS, dtype=torch.int32), "shuffled": True}
    _check_all(g, gpu, cfg, **extra)


# ------------------------------------------ split planned from host lengths ----
# gva_decode_attention_lens / gva_decode_step_lens: the chunk is sized from
# the host copy of the lengths so that every (sequence, chunk) item holds
# about the same tokens (ragged batches).  Same bars against the oracle; the
# results differ from the max_seq_len split only by summation order.

def _lens_case(gpu, name, kw, lens=None):
    cfg = syn.with_overrides(syn.get_config(name), **kw)
    extra = {}
    if lens is not None:
        extra = {"seq_lens": torch.tensor(lens, dtype=torch.int32), "shuffled": True}
    x, h = gen(cfg, gpu, **extra)
    return cfg, x, h


@pytest.mark.parametrize("name,kw,lens,heads", [
    ("long_ragged", {}, None, [0, 7, 15]),
    ("decode_350m", {"B": len(EDGE_LENS), "T": None, "len_range": None}, EDGE_LENS, None),
    ("decode_350m", {"B": 4, "T": None, "len_range": None}, [0, 5, 0, 1000], None),
    ("decode_350m", {"B": 5, "T": None, "len_range": None}, [70000, 100, 5, 0, 3000], [0, 9]),
    ("decode_350m", {"B": 32, "T": 2048}, None, None),
    # 255 one-token sequences and a long one: the chunk search ends at the long length
    ("decode_350m", {"B": 256, "T": None, "len_range": None}, [1] * 255 + [20000], [0, 5]),
    ("wide_rope_append", {"B": 12, "T": None, "len_range": (1, 6000), "append": False}, None,
     None),
])
def test_decode_with_host_planned_split(g, gpu, name, kw, lens, heads):
    cfg, x, h = _lens_case(gpu, name, kw, lens)
    announce("host-planned split", name, kw, lens)
    qa = g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"], rope_base=cfg.rope_base)
    host = x["seq_lens_host"]
    ws = torch.zeros(g.decode_workspace_bytes_lens(cfg.B, cfg.H, x["v_pool"], x["k_pool"],
                                                   x["block_table"]),
                     dtype=torch.uint8, device=gpu)
    out, lse = g.decode_attention_lens(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                       x["seq_lens"], host, x["max_seq_len"], workspace=ws)
    torch.cuda.synchronize()
    vp, kp = oracle_pools(h, cfg)
    ref, ref_lse = o.gva_decode_materialized(
        h["q_nope"], h["q_rope"], h["M"], vp, kp, h["block_table"], h["seq_lens"],
        base=cfg.rope_base, heads=heads)
    got, got_lse = cpu(out).double().numpy(), cpu(lse).double().numpy()
    sel = np.isfinite(ref_lse)
    assert_bf16_parity(got[sel], ref[sel])
    assert_bf16_split_precision(got[sel], ref[sel])
    np.testing.assert_allclose(got_lse[sel], ref_lse[sel], rtol=0, atol=1e-3)
    for b in range(cfg.B):  # empty sequences: zeros and -inf
        if int(host[b]) == 0:
            assert torch.all(out[b] == 0) and torch.all(lse[b] == -float("inf"))
    # the max_seq_len split: the same up to summation order
    out2, _ = g.decode_attention(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                 x["seq_lens"], x["max_seq_len"])
    torch.cuda.synchronize()
    live = torch.tensor([int(v) > 0 for v in host], device=gpu)
    d = (out - out2)[live].abs().max().item()
    assert d <= 1e-5 * max(1.0, out2[live].abs().max().item())
    # the workspace is reused as is (every counter left zero): same bits
    out3, lse3 = g.decode_attention_lens(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                         x["seq_lens"], host, x["max_seq_len"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out3) and torch.equal(lse.nan_to_num(7), lse3.nan_to_num(7))


def test_host_planned_split_flags_a_length_mismatch(g, gpu):
    """A sequence whose device length gives another chunk count than its
    host length gets NaN; the others are unaffected."""
    lens = [3000, 2000, 500, 64]
    cfg, x, h = _lens_case(gpu, "decode_350m", {"B": 4, "T": None, "len_range": None}, lens)
    qa = g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"], rope_base=cfg.rope_base)
    good, _ = g.decode_attention_lens(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                      x["seq_lens"], lens, x["max_seq_len"])
    wrong = list(lens)
    wrong[0] = 40          # far fewer chunks than the device length needs
    out, lse = g.decode_attention_lens(qa, x["v_pool"], x["k_pool"], x["block_table"],
                                       x["seq_lens"], wrong, x["max_seq_len"])
    torch.cuda.synchronize()
    assert torch.isnan(out[0]).all() and torch.isnan(lse[0]).all()
    # the other sequences see another chunk size, so compare to tolerance
    assert torch.allclose(out[1:], good[1:], rtol=0, atol=1e-5)


def test_step_with_host_planned_split(g, gpu):
    cfg, x, h = _lens_case(gpu, "wide_rope_append", {"B": 10, "T": None, "len_range": (1, 5000)})
    vp0, kp0 = x["v_pool"].clone(), x["k_pool"].clone()
    host = x["seq_lens_host"]
    out, lse = g.decode_step_lens(x["q_nope"], x["q_rope"], x["M"], x["v_pool"], x["k_pool"],
                                  x["block_table"], x["seq_lens"], host, x["max_seq_len"],
                                  v_new=x["v_new"], k_new=x["k_new"], rope_base=cfg.rope_base)
    torch.cuda.synchronize()
    x2 = dict(x)
    x2["v_pool"], x2["k_pool"] = vp0, kp0
    out2, _ = g.decode_step(x2["q_nope"], x2["q_rope"], x2["M"], x2["v_pool"], x2["k_pool"],
                            x2["block_table"], x2["seq_lens"], x2["max_seq_len"],
                            v_new=x2["v_new"], k_new=x2["k_new"], rope_base=cfg.rope_base)
    torch.cuda.synchronize()
    assert torch.equal(x["v_pool"].nan_to_num(7), x2["v_pool"].nan_to_num(7))
    assert torch.allclose(out, out2, rtol=0, atol=1e-5)
    vp, kp = oracle_pools(h, cfg)
    ref, ref_lse = o.gva_decode_materialized(
        h["q_nope"], h["q_rope"], h["M"], vp, kp, h["block_table"], h["seq_lens"],
        base=cfg.rope_base)
    got = cpu(out).double().numpy()
    assert_bf16_parity(got, ref)
    assert_bf16_split_precision(got, ref)


def test_host_planned_split_in_a_graph(g, gpu):
    """The plan travels in the kernel arguments: replays of a captured call
    equal the eager call."""
    cfg, x, h = _lens_case(gpu, "long_ragged", {"len_range": (100, 20000)})
    qa = g.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"], rope_base=cfg.rope_base)
    host = x["seq_lens_host"]
    ws = torch.zeros(g.decode_workspace_bytes_lens(cfg.B, cfg.H, x["v_pool"], x["k_pool"],
                                                   x["block_table"]),
                     dtype=torch.uint8, device=gpu)
    out = torch.empty((cfg.B, cfg.H, cfg.d_h), device=gpu)
    lse = torch.empty((cfg.B, cfg.H), device=gpu)

    def call():
        g.decode_attention_lens(qa, x["v_pool"], x["k_pool"], x["block_table"], x["seq_lens"],
                                host, x["max_seq_len"], workspace=ws, out=out, lse=lse)

    call()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
