"""Pins of the float64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a library
routine (torch's scaled_dot_product_attention in float64, torch's bf16
conversion), a closed form, an invariant, a special case that reduces to a
textbook routine, or brute force on tiny inputs.  The pages print no worked
numeric example; the only stored values are their cache-saving percentages
(tests/golden/cache_savings.json).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

SHAPES = [  # (H, G, d_h, d_n, d_r, T)
    (4, 2, 32, 24, 8, 37),
    (8, 8, 16, 10, 6, 5),
    (8, 2, 16, 16, 2, 64),
    (16, 4, 24, 12, 24, 130),
]


def _rng(seed=0):
    return np.random.default_rng(seed)


def _rope_complex(x, pos, base):
    """RoPE written as complex multiplication: pair (x_2i, x_2i+1) is the
    complex number x_2i + i x_2i+1 multiplied by exp(i * pos * theta_i)."""
    x = np.asarray(x, dtype=np.float64)
    d_r = x.shape[-1]
    theta = base ** (-np.arange(0, d_r, 2, dtype=np.float64) / d_r)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos * theta)
    y = np.empty(x.shape)
    y[..., 0::2] = z.real
    y[..., 1::2] = z.imag
    return y


def _contiguous_pool(V, k, block_size):
    """Pack one sequence [T, ...] into a contiguous paged pool."""
    T = V.shape[0]
    nb = max(1, -(-T // block_size))
    vp = np.full((nb * block_size,) + V.shape[1:], np.nan)
    kp = np.full((nb * block_size,) + k.shape[1:], np.nan)
    vp[:T], kp[:T] = V, k
    vp = vp.reshape((nb, block_size) + V.shape[1:])
    kp = kp.reshape((nb, block_size) + k.shape[1:])
    return vp, kp, np.arange(nb)[None, :]


def _problem(shape, B=2, seed=0, block_size=16):
    H, G, d_h, d_n, d_r, T = shape
    r = _rng(seed)
    q_nope = r.standard_normal((B, H, d_n))
    q_rope = r.standard_normal((B, H, d_r))
    M = r.standard_normal((H, d_h, d_n)) / math.sqrt(d_h)
    lens = np.array([T - (b % 3) for b in range(B)])
    nbs = [-(-int(n) // block_size) for n in lens]
    NB = sum(nbs)
    perm = r.permutation(NB)
    table = np.zeros((B, max(nbs)), dtype=np.int64)
    off = 0
    for b, nb in enumerate(nbs):
        table[b, :nb] = perm[off:off + nb]
        off += nb
    v_pool = r.standard_normal((NB, block_size, G, d_h))
    k_pool = r.standard_normal((NB, block_size, d_r))
    return dict(q_nope=q_nope, q_rope=q_rope, M=M, v_pool=v_pool,
                k_pool=k_pool, block_table=table, seq_lens=lens,
                block_size=block_size, H=H, G=G, d_h=d_h, d_n=d_n, d_r=d_r)


def _sdpa(q, K, V, scale):
    """torch's scaled_dot_product_attention on CPU in float64."""
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, None, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(K))[None, None]
    vt = torch.from_numpy(np.ascontiguousarray(V))[None, None]
    return F.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, 0, 0].numpy()


# ---------------------------------------------------------------- Eq. 7 ----

@pytest.mark.parametrize("shape", SHAPES)
def test_absorbed_equals_materialized(shape):
    """Eq. 7 is exact: attending with the absorbed query over the value cache
    gives the same result as materialising K_h = V M_h (onedev.kr review,
    "How it works"; bisque.today explainer, Equation 7)."""
    p = _problem(shape)
    out_m, lse_m = o.gva_decode_materialized(
        p["q_nope"], p["q_rope"], p["M"], p["v_pool"], p["k_pool"],
        p["block_table"], p["seq_lens"], base=10000.0,
        block_size=p["block_size"])
    qa = o.absorb_query(p["q_nope"], p["q_rope"], p["M"], p["seq_lens"] - 1)
    out_a, lse_a = o.attend_absorbed(qa, p["v_pool"], p["k_pool"],
                                     p["block_table"], p["seq_lens"],
                                     block_size=p["block_size"])
    np.testing.assert_allclose(out_a, out_m, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_a, lse_m, rtol=1e-13, atol=1e-12)


def test_absorbed_score_per_position():
    """Per cached position, <q~, v> equals <q, v M_h> (tiny brute force)."""
    r = _rng(1)
    d_h, d_n = 8, 5
    M = r.standard_normal((1, d_h, d_n))
    q = r.standard_normal((1, 1, d_n))
    qa = o.absorb_query(q, np.zeros((1, 1, 2)), M, [0], scale=1.0)
    for _ in range(10):
        v = r.standard_normal(d_h)
        k_mat = sum(v[e] * M[0, e] for e in range(d_h))  # v M_h, by hand
        s_mat = sum(q[0, 0, n] * k_mat[n] for n in range(d_n))
        s_abs = sum(qa[0, 0, e] * v[e] for e in range(d_h))
        assert abs(s_mat - s_abs) <= 1e-12 * (1 + abs(s_mat))


# --------------------------------------------------- library cross-check ----

@pytest.mark.parametrize("shape", SHAPES)
def test_materialized_matches_sdpa(shape):
    """The oracle equals torch SDPA (float64) on explicitly built full keys
    [V_g M_h | k_rope] and full query [q_nope | R_t q_rope], with RoPE
    written independently as complex multiplication."""
    p = _problem(shape, seed=2)
    H, G = p["H"], p["G"]
    scale = 1.0 / math.sqrt(p["d_n"] + p["d_r"])
    out, lse = o.gva_decode_materialized(
        p["q_nope"], p["q_rope"], p["M"], p["v_pool"], p["k_pool"],
        p["block_table"], p["seq_lens"], block_size=p["block_size"])
    bs = p["block_size"]
    for b, n in enumerate(p["seq_lens"]):
        rows = [(p["block_table"][b, j // bs], j % bs) for j in range(n)]
        Vseq = np.stack([p["v_pool"][blk, s] for blk, s in rows])
        kseq = np.stack([p["k_pool"][blk, s] for blk, s in rows])
        for h in range(H):
            g = h // (H // G)
            Kc = Vseq[:, g, :] @ p["M"][h]
            K = np.concatenate([Kc, kseq], axis=1)
            q = np.concatenate([p["q_nope"][b, h],
                                _rope_complex(p["q_rope"][b, h], n - 1, 1e4)])
            ref = _sdpa(q, K, Vseq[:, g, :], scale)
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)
            s = scale * K @ q
            ref_lse = np.log(np.sum(np.exp(s - s.max()))) + s.max()
            assert abs(lse[b, h] - ref_lse) < 1e-12


def test_textbook_attention_matches_sdpa():
    r = _rng(3)
    for T in (1, 2, 17, 300):
        q = r.standard_normal(12)
        K = r.standard_normal((T, 12)) * 3
        V = r.standard_normal((T, 7))
        out, lse, p, s = o.softmax_attention(q, K, V, 0.4)
        np.testing.assert_allclose(out, _sdpa(q, K, V, 0.4), atol=1e-13)
        assert abs(p.sum() - 1) < 1e-14


def test_gqa_oracle_matches_sdpa():
    r = _rng(4)
    B, H, G, d_h, bs = 2, 8, 2, 16, 8
    lens = np.array([19, 8])
    NB = 3 + 1
    table = np.array([[2, 0, 3], [1, 0, 0]])
    kp = r.standard_normal((NB, bs, G, d_h))
    vp = r.standard_normal((NB, bs, G, d_h))
    q = r.standard_normal((B, H, d_h))
    out, _ = o.gqa_decode(q, kp, vp, table, lens, block_size=bs)
    for b in range(B):
        j = np.arange(lens[b])
        Ks = kp[table[b, j // bs], j % bs]
        Vs = vp[table[b, j // bs], j % bs]
        qt = torch.from_numpy(q[b])[None, :, None, :]            # [1,H,1,d]
        kt = torch.from_numpy(np.ascontiguousarray(Ks.transpose(1, 0, 2)))[None]
        vt = torch.from_numpy(np.ascontiguousarray(Vs.transpose(1, 0, 2)))[None]
        ref = F.scaled_dot_product_attention(qt, kt, vt, enable_gqa=True)
        np.testing.assert_allclose(out[b], ref[0, :, 0].numpy(), atol=1e-12)


# ------------------------------------------------------- special cases ----

def test_uniform_scores_give_mean_of_values():
    """q = 0 makes every score equal: the softmax is flat and the output is
    the plain mean of the group's values (the near-uniform attention the
    pages describe for mis-scaled keys: agihunt.info summary, initialisation
    paragraph; bisque.today explainer, Figure 4)."""
    p = _problem((8, 2, 16, 12, 4, 50), seed=5)
    zeros_n = np.zeros_like(p["q_nope"])
    zeros_r = np.zeros_like(p["q_rope"])
    out, lse = o.gva_decode_materialized(
        zeros_n, zeros_r, p["M"], p["v_pool"], p["k_pool"], p["block_table"],
        p["seq_lens"], block_size=p["block_size"])
    bs = p["block_size"]
    for b, n in enumerate(p["seq_lens"]):
        j = np.arange(n)
        V = p["v_pool"][p["block_table"][b, j // bs], j % bs]
        for h in range(8):
            np.testing.assert_allclose(out[b, h], V[:, h // 4].mean(0), atol=1e-13)
            assert abs(lse[b, h] - math.log(n)) < 1e-13


def test_single_token_returns_its_value():
    p = _problem((4, 2, 8, 6, 2, 1), seed=6, B=1)
    out, lse = o.gva_decode_materialized(
        p["q_nope"], p["q_rope"], p["M"], p["v_pool"], p["k_pool"],
        p["block_table"], np.array([1]), block_size=p["block_size"])
    blk = p["block_table"][0, 0]
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], p["v_pool"][blk, 0, h // 2])


def test_empty_sequence_reading():
    out, lse, pw, _ = o.softmax_attention(np.ones(3), np.zeros((0, 3)),
                                          np.zeros((0, 4)), 1.0)
    assert np.all(out == 0) and lse == -np.inf


def test_kv_equal_special_case():
    """Shared KV (K = V): with d_n = d_h, M_h = I and a zero position query
    the method is plain attention with keys equal to values (agihunt.info
    summary, K=V paragraph; bisque.today explainer, Figure 3)."""
    r = _rng(7)
    H, G, d_h, T, bs = 4, 2, 8, 21, 8
    q_nope = r.standard_normal((1, H, d_h))
    M = np.broadcast_to(np.eye(d_h), (H, d_h, d_h)).copy()
    V = r.standard_normal((T, G, d_h))
    k = r.standard_normal((T, 4))
    vp, kp, table = _contiguous_pool(V, k, bs)
    out, _ = o.gva_decode_materialized(q_nope, np.zeros((1, H, 4)), M, vp, kp,
                                       table, [T], scale=0.3, block_size=bs)
    for h in range(H):
        ref = _sdpa(q_nope[0, h], V[:, h // 2], V[:, h // 2], 0.3)
        np.testing.assert_allclose(out[0, h], ref, atol=1e-13)


# --------------------------------------------------------------- RoPE ----

def test_rope_matches_complex_rotation():
    r = _rng(8)
    for d_r in (2, 8, 16, 24, 32):
        x = r.standard_normal((5, d_r))
        for pos in (0, 1, 7, 4095, 131071):
            np.testing.assert_allclose(o.rope_rotate(x, pos, 1e4),
                                       _rope_complex(x, pos, 1e4), atol=1e-12)


def test_rope_position_zero_is_identity_and_norm_preserving():
    r = _rng(9)
    x = r.standard_normal((3, 16))
    np.testing.assert_array_equal(o.rope_rotate(x, 0, 1e4), x)
    y = o.rope_rotate(x, 12345, 1e4)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1),
                               np.linalg.norm(x, axis=-1), rtol=1e-14)


def test_rope_relative_position():
    """<R_t q, R_j k> depends only on j - t (onedev.kr review, "How it
    differs": nothing learned sits between the two rotations)."""
    r = _rng(10)
    q, k = r.standard_normal(24), r.standard_normal(24)
    for t, j in [(5, 3), (1000, 17), (131071, 4)]:
        a = o.rope_rotate(q, t, 1e4) @ o.rope_rotate(k, j, 1e4)
        b = q @ o.rope_rotate(k, j - t, 1e4)
        assert abs(a - b) < 1e-9


def test_shift_invariance_of_decode():
    """Appending raw keys at positions p0..p0+T-1 with the query at p0+T-1
    gives the same output for every offset p0 (exact float64 caches)."""
    r = _rng(11)
    H, G, d_h, d_n, d_r, T, bs = 4, 2, 8, 6, 8, 40, 16
    q_nope = r.standard_normal((1, H, d_n))
    q_rope = r.standard_normal((1, H, d_r))
    M = r.standard_normal((H, d_h, d_n)) / math.sqrt(d_h)
    V = r.standard_normal((T, G, d_h))
    x = r.standard_normal((T, d_r))  # unrotated positional keys
    outs = []
    for p0 in (0, 3, 1000, 100000):
        P = p0 + T
        nb = -(-P // bs)
        vp = np.zeros((nb, bs, G, d_h))
        kp = np.zeros((nb, bs, d_r))
        table = np.arange(nb)[None, :]
        for j in range(T):
            vp, kp = o.append_token(vp, kp, V[j][None], x[j][None], [p0 + j],
                                    table, block_size=bs, cache_dtype="float64")
        # attend over positions p0..P-1 only: shift the query position via
        # the materialised oracle on the sub-range
        out, _ = _decode_window(q_nope, q_rope, M, vp, kp, table, p0, P, bs)
        outs.append(out)
    for out in outs[1:]:
        np.testing.assert_allclose(out, outs[0], atol=1e-10)


def _decode_window(q_nope, q_rope, M, vp, kp, table, p0, P, bs):
    """Materialised decode over cache positions p0..P-1, query at P-1."""
    H, G = q_nope.shape[1], vp.shape[2]
    j = np.arange(p0, P)
    Vs = vp[table[0, j // bs], j % bs]
    ks = kp[table[0, j // bs], j % bs]
    out = np.zeros((H, vp.shape[3]))
    lse = np.zeros(H)
    scale = 1.0 / math.sqrt(q_nope.shape[2] + q_rope.shape[2])
    for h in range(H):
        g = o.head_group(h, H, G)
        K = np.concatenate([o.reconstruct_keys(Vs[:, g], M[h]), ks], axis=1)
        q = np.concatenate([q_nope[0, h], o.rope_rotate(q_rope[0, h], P - 1, 1e4)])
        out[h], lse[h], _, _ = o.softmax_attention(q, K, Vs[:, g], scale)
    return out, lse


def test_ordinary_rope_blocks_absorption():
    """Negative check: rotating the *reconstructed* key (ordinary RoPE) makes
    the score depend on the relative rotation between q and M^T, so one
    absorbed query cannot serve every cached position (onedev.kr review,
    "How it differs")."""
    r = _rng(12)
    d_h, d = 8, 8
    M = r.standard_normal((d_h, d))
    q = r.standard_normal(d)
    t = 50
    q_abs = o.rope_rotate(q, t, 1e4) @ M.T       # fold once at position t
    errs = []
    for j in range(0, 50):
        v = r.standard_normal(d_h)
        true = o.rope_rotate(q, t, 1e4) @ o.rope_rotate(v @ M, j, 1e4)
        errs.append(abs(true - q_abs @ v))
    assert max(errs) > 1e-2  # absorption fails for j != t


# -------------------------------------------------------- cache counts ----

def test_cache_counts_match_pages():
    with open(os.path.join(GOLDEN, "cache_savings.json")) as f:
        gold = json.load(f)
    for c in gold["cases"]:
        saving = 100.0 * (1.0 - o.cache_ratio(c["G"], c["d_h"], c["d_r"]))
        if "saving_pct_exact" in c:
            assert saving == c["saving_pct_exact"]
        else:
            assert round(saving) == c["saving_pct_approx"]
    # the positional key is shared by all heads: d_r per token, not G*d_r
    assert o.cache_scalars_per_token(4, 64, 16) == 4 * 64 + 16
    assert o.gqa_cache_scalars_per_token(4, 64) == 512


def test_cache_ratio_closed_form():
    for G, d_h, d_r in [(4, 64, 16), (4, 64, 24), (8, 128, 32), (2, 32, 8)]:
        assert o.cache_ratio(G, d_h, d_r) == pytest.approx(
            0.5 + d_r / (2 * G * d_h), abs=1e-15)


# ------------------------------------------------------- bf16 rounding ----

def test_bf16_matches_torch_for_float32_inputs():
    r = _rng(13)
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(2000) * 1e-38).astype(np.float32),  # subnormal
        (r.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.389e38, 3.4e38,
                  -3.4e38, np.inf, -np.inf], dtype=np.float32),
    ])
    # exact ties: integer mantissas with the 9th bit set and nothing below
    ties = (np.arange(256, 512, dtype=np.float32) * 2 + 1) / 512
    x = np.concatenate([x, ties, -ties]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = o.bf16_nearest(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def _bf16_neighbours(x):
    """All bf16 values within a few spacings of x, by enumerating bit
    patterns of the enclosing float32 bf16 grid."""
    b = np.array([x], dtype=np.float32).view(np.uint32)[0] >> 16
    cands = []
    for d in range(-3, 4):
        bits = (int(b) + d) & 0xFFFF
        v = np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]
        if np.isfinite(v):
            cands.append(float(v))
    return cands


def test_bf16_brute_force_float64_inputs():
    """For float64 inputs (single rounding, no float32 step) the result is a
    bf16 value no farther than any other bf16 value; ties go to the even
    bit pattern."""
    r = _rng(14)
    xs = list(r.standard_normal(3000) * np.exp(r.uniform(-30, 30, 3000)))
    # values just beside bf16 ties, which float32 double rounding would spoil
    for m in range(256, 300):
        tie = (2 * m + 1) / 512.0
        xs += [tie + 2.0 ** -40, tie - 2.0 ** -40, tie]
    for x in xs:
        y = float(o.bf16_nearest(np.array([x]))[0])
        cands = _bf16_neighbours(x)
        assert y in cands
        best = min(abs(c - x) for c in cands)
        assert abs(y - x) == best
        near = [c for c in cands if abs(c - x) == best]
        if len(near) == 2:
            bits = np.array([y], dtype=np.float32).view(np.uint32)[0] >> 16
            assert bits % 2 == 0


# -------------------------------------------------------- split / merge ----

def test_merge_of_chunk_partials_equals_full_softmax():
    r = _rng(15)
    for T, chunk in [(100, 7), (64, 64), (1000, 256), (5, 1)]:
        q = r.standard_normal(10)
        K = r.standard_normal((T, 10)) * 2
        V = r.standard_normal((T, 6))
        ms, ls, accs = o.chunk_partials(q, K, V, 0.5, chunk)
        out, lse = o.merge_partials(ms, ls, accs)
        ref, ref_lse, _, _ = o.softmax_attention(q, K, V, 0.5)
        np.testing.assert_allclose(out, ref, atol=1e-13)
        assert abs(lse - ref_lse) < 1e-12


# ------------------------------------------------------------- append ----

def test_append_writes_rounded_rotated_token_in_paged_slot():
    r = _rng(16)
    B, G, d_h, d_r, bs = 3, 2, 8, 6, 4
    NB = 9
    table = np.array([[4, 1, 7], [0, 8, 2], [5, 3, 6]])
    vp = r.standard_normal((NB, bs, G, d_h))
    kp = r.standard_normal((NB, bs, d_r))
    v_new = r.standard_normal((B, G, d_h))
    k_new = r.standard_normal((B, d_r))
    pos = np.array([0, 6, 11])
    vp2, kp2 = o.append_token(vp, kp, v_new, k_new, pos, table, base=1e4,
                              block_size=bs, cache_dtype="bfloat16")
    written = {(4, 0): 0, (8, 2): 1, (6, 3): 2}
    for blk in range(NB):
        for s in range(bs):
            if (blk, s) in written:
                b = written[(blk, s)]
                v_ref = torch.from_numpy(v_new[b].astype(np.float32)).to(
                    torch.bfloat16).double().numpy()
                np.testing.assert_array_equal(vp2[blk, s], v_ref)
                rot = _rope_complex(k_new[b], pos[b], 1e4)
                for i in range(d_r):
                    cands = _bf16_neighbours(rot[i])
                    best = min(abs(c - rot[i]) for c in cands)
                    assert abs(kp2[blk, s, i] - rot[i]) == best
            else:
                np.testing.assert_array_equal(vp2[blk, s], vp[blk, s])
                np.testing.assert_array_equal(kp2[blk, s], kp[blk, s])


# ------------------------------------------- several query tokens (L) ----

def _queries(p, L, seed):
    r = _rng(seed)
    B, H = p["q_nope"].shape[:2]
    return (r.standard_normal((B, H, L, p["d_n"])),
            r.standard_normal((B, H, L, p["d_r"])))


@pytest.mark.parametrize("L", [1, 2, 4])
def test_queries_match_sdpa_with_causal_mask(L):
    """L query tokens per sequence: torch SDPA (float64) over explicitly
    built full keys, with a boolean mask letting query i (position T-L+i)
    see positions 0..T-L+i only; RoPE written as complex multiplication."""
    p = _problem(SHAPES[0], seed=30)
    qn, qr = _queries(p, L, 31)
    H, G, bs = p["H"], p["G"], p["block_size"]
    scale = 1.0 / math.sqrt(p["d_n"] + p["d_r"])
    out, lse = o.gva_decode_materialized_queries(
        qn, qr, p["M"], p["v_pool"], p["k_pool"], p["block_table"],
        p["seq_lens"], block_size=bs)
    for b, n in enumerate(p["seq_lens"]):
        rows = [(p["block_table"][b, j // bs], j % bs) for j in range(n)]
        Vseq = np.stack([p["v_pool"][blk, s] for blk, s in rows])
        kseq = np.stack([p["k_pool"][blk, s] for blk, s in rows])
        allowed = np.arange(n)[None, :] <= (n - L + np.arange(L))[:, None]
        for h in range(H):
            g = h // (H // G)
            K = np.concatenate([Vseq[:, g, :] @ p["M"][h], kseq], axis=1)
            Q = np.stack([np.concatenate([qn[b, h, i],
                                          _rope_complex(qr[b, h, i], n - L + i, 1e4)])
                          for i in range(L)])
            ref = F.scaled_dot_product_attention(
                torch.from_numpy(Q)[None, None], torch.from_numpy(K)[None, None],
                torch.from_numpy(np.ascontiguousarray(Vseq[:, g, :]))[None, None],
                attn_mask=torch.from_numpy(allowed)[None, None], scale=scale)[0, 0].numpy()
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)
            s = scale * Q @ K.T
            s[~allowed] = -np.inf
            m = s.max(axis=1)
            ref_lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
            np.testing.assert_allclose(lse[b, h], ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L", [2, 3])
def test_query_token_i_is_single_query_decode_of_its_prefix(L):
    """Query i equals the (separately pinned) single-query definition on the
    first len-L+i+1 cached positions, with its own q slices."""
    p = _problem(SHAPES[3], seed=32)
    qn, qr = _queries(p, L, 33)
    out, lse = o.gva_decode_materialized_queries(
        qn, qr, p["M"], p["v_pool"], p["k_pool"], p["block_table"],
        p["seq_lens"], block_size=p["block_size"])
    for i in range(L):
        o1, l1 = o.gva_decode_materialized(
            qn[:, :, i], qr[:, :, i], p["M"], p["v_pool"], p["k_pool"],
            p["block_table"], p["seq_lens"] - (L - 1) + i,
            block_size=p["block_size"])
        np.testing.assert_allclose(out[:, :, i], o1, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], l1, rtol=0, atol=1e-13)


@pytest.mark.parametrize("L", [1, 3])
def test_absorbed_queries_equal_materialized(L):
    """Eq. 7 for several query tokens: absorbing each token's query and
    attending over the value cache equals the materialised-key decode."""
    p = _problem(SHAPES[2], seed=34)
    qn, qr = _queries(p, L, 35)
    out_m, lse_m = o.gva_decode_materialized_queries(
        qn, qr, p["M"], p["v_pool"], p["k_pool"], p["block_table"],
        p["seq_lens"], block_size=p["block_size"])
    qa = o.absorb_queries(qn, qr, p["M"], p["seq_lens"] - 1)
    out_a, lse_a = o.attend_absorbed_queries(
        qa, p["v_pool"], p["k_pool"], p["block_table"], p["seq_lens"],
        block_size=p["block_size"])
    np.testing.assert_allclose(out_a, out_m, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_a, lse_m, rtol=0, atol=1e-12)


def test_absorb_queries_rows_are_single_token_absorptions():
    r = _rng(36)
    B, H, L, d_h, d_n, d_r = 3, 4, 3, 8, 6, 4
    qn = r.standard_normal((B, H, L, d_n))
    qr = r.standard_normal((B, H, L, d_r))
    M = r.standard_normal((H, d_h, d_n))
    pos_last = np.array([5, 2, 40])
    qa = o.absorb_queries(qn, qr, M, pos_last, scale=0.3)
    for i in range(L):
        ref = o.absorb_query(qn[:, :, i], qr[:, :, i], M, pos_last - (L - 1) + i,
                             scale=0.3)
        np.testing.assert_allclose(qa[:, :, i], ref, rtol=0, atol=1e-14)
    # the position slice of query i is rotated to its own position
    np.testing.assert_allclose(
        qa[1, 2, 0, d_h:], 0.3 * _rope_complex(qr[1, 2, 0], 0, 1e4), atol=1e-14)


def test_append_tokens_write_each_token_at_its_position():
    r = _rng(37)
    B, L, G, d_h, d_r, bs = 2, 3, 2, 8, 4, 4
    table = np.array([[3, 0, 5], [1, 4, 2]])
    vp = r.standard_normal((6, bs, G, d_h))
    kp = r.standard_normal((6, bs, d_r))
    v_new = r.standard_normal((B, L, G, d_h))
    k_new = r.standard_normal((B, L, d_r))
    pos_last = np.array([5, 9])      # tokens at 3,4,5 and 7,8,9
    vp2, kp2 = o.append_tokens(vp, kp, v_new, k_new, pos_last, table, base=1e4,
                               block_size=bs, cache_dtype="float64")
    written = {}
    for b in range(B):
        for i in range(L):
            pp = pos_last[b] - (L - 1) + i
            written[(table[b, pp // bs], pp % bs)] = (b, i, pp)
    for blk in range(6):
        for s in range(bs):
            if (blk, s) in written:
                b, i, pp = written[(blk, s)]
                np.testing.assert_array_equal(vp2[blk, s], v_new[b, i])
                np.testing.assert_allclose(kp2[blk, s],
                                           _rope_complex(k_new[b, i], pp, 1e4),
                                           atol=1e-14)
            else:
                np.testing.assert_array_equal(vp2[blk, s], vp[blk, s])
                np.testing.assert_array_equal(kp2[blk, s], kp[blk, s])


# --------------------------- ordinary RoPE on the reconstructed key ----

def test_rope_on_keys_matches_sdpa():
    """Keys rebuilt as V_g M_h and rotated at their own positions (complex
    multiplication), query rotated at len-1: torch SDPA in float64."""
    p = _problem((8, 2, 16, 12, 2, 70), seed=40)
    r = _rng(41)
    B, H, G, bs = 2, 8, 2, p["block_size"]
    q = r.standard_normal((B, H, 12))
    out, lse = o.gva_decode_rope_on_keys(q, p["M"], p["v_pool"], p["block_table"],
                                         p["seq_lens"], block_size=bs)
    for b, n in enumerate(p["seq_lens"]):
        rows = [(p["block_table"][b, j // bs], j % bs) for j in range(n)]
        Vseq = np.stack([p["v_pool"][blk, s] for blk, s in rows])
        for h in range(H):
            g = h // (H // G)
            K = np.stack([_rope_complex(Vseq[j, g] @ p["M"][h], j, 1e4) for j in range(n)])
            qr = _rope_complex(q[b, h], n - 1, 1e4)
            ref = _sdpa(qr, K, Vseq[:, g, :], 1.0 / math.sqrt(12))
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)


def test_rope_on_keys_depends_on_relative_positions_only():
    """Shifting every cached position by p0 (keys rebuilt at p0 + j, query at
    p0 + len - 1) leaves the output unchanged: R_t^T R_j = R_(j-t)."""
    r = _rng(42)
    H, G, d_h, d_k, T = 4, 2, 8, 6, 21
    V = r.standard_normal((T, G, d_h))
    M = r.standard_normal((H, d_h, d_k)) / math.sqrt(d_h)
    q = r.standard_normal((1, H, d_k))
    scale = 1.0 / math.sqrt(d_k)
    base_out = None
    for p0 in (0, 7, 1000, 100000):
        outs = []
        for h in range(H):
            g = h // (H // G)
            K = V[:, g] @ M[h]
            Kr = _rope_complex(K, (p0 + np.arange(T))[:, None], 1e4)
            qr = _rope_complex(q[0, h], p0 + T - 1, 1e4)
            outs.append(o.softmax_attention(qr, Kr, V[:, g], scale)[0])
        if base_out is None:
            base_out = outs
            vp, kp, table = _contiguous_pool(V, np.zeros((T, 2)), 8)
            ref, _ = o.gva_decode_rope_on_keys(q, M, vp, table, [T], block_size=8)
            np.testing.assert_allclose(ref[0], np.stack(outs), atol=1e-12)
        else:
            np.testing.assert_allclose(np.stack(outs), np.stack(base_out), atol=1e-9)


def test_rope_on_keys_at_position_zero_is_plain_reconstructed_attention():
    """A length-1 context (query and key at position 0, no rotation) is plain
    attention with the reconstructed key: the output is the value itself."""
    r = _rng(43)
    V = r.standard_normal((1, 2, 8))
    M = r.standard_normal((4, 8, 6))
    q = r.standard_normal((1, 4, 6))
    vp, _, table = _contiguous_pool(V, np.zeros((1, 2)), 4)
    out, lse = o.gva_decode_rope_on_keys(q, M, vp, table, [1], block_size=4)
    for h in range(4):
        g = h // 2
        np.testing.assert_allclose(out[0, h], V[0, g], atol=1e-15)
        s = (q[0, h] @ (V[0, g] @ M[h])) / math.sqrt(6)
        assert abs(lse[0, h] - s) < 1e-12


@pytest.mark.parametrize("L", [1, 3, 8])
def test_gqa_queries_match_sdpa_with_causal_mask(L):
    """Many-token GQA oracle: torch SDPA (float64, enable_gqa) with a boolean
    mask letting query i (position len-L+i) see positions 0..len-L+i only;
    L = 1 is the single-query GQA oracle."""
    r = _rng(40 + L)
    B, H, G, d_h, bs = 2, 8, 2, 16, 8
    lens = np.array([19, 11])
    table = np.array([[2, 0, 3], [1, 4, 0]])
    kp = r.standard_normal((5, bs, G, d_h))
    vp = r.standard_normal((5, bs, G, d_h))
    q = r.standard_normal((B, H, L, d_h))
    out, lse = o.gqa_decode_queries(q, kp, vp, table, lens, block_size=bs)
    for b in range(B):
        n = int(lens[b])
        j = np.arange(n)
        Ks = kp[table[b, j // bs], j % bs]
        Vs = vp[table[b, j // bs], j % bs]
        allowed = j[None, :] <= (n - L + np.arange(L))[:, None]
        kt = torch.from_numpy(np.ascontiguousarray(Ks.transpose(1, 0, 2)))[None]
        vt = torch.from_numpy(np.ascontiguousarray(Vs.transpose(1, 0, 2)))[None]
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q[b])[None], kt, vt,
            attn_mask=torch.from_numpy(allowed)[None, None], enable_gqa=True)
        np.testing.assert_allclose(out[b], ref[0].numpy(), rtol=0, atol=1e-12)
    if L == 1:
        one, one_lse = o.gqa_decode(q[:, :, 0], kp, vp, table, lens, block_size=bs)
        np.testing.assert_array_equal(out[:, :, 0], one)
        np.testing.assert_array_equal(lse[:, :, 0], one_lse)
