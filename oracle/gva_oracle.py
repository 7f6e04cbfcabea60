"""Float64 CPU oracle for Grouped Value Attention (GVA) absorbed decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The
library path (``compressed_kv_cache_amd``, ``libgva``) never calls it, and it
imports nothing from that path: the two share only the seeded input generator
in ``synthetic/``.

Sources (cited by page and section; the pages are summaries of the paper
"Grouped Value Attention: Efficient KV Caching via On-Demand Key
Reconstruction"):

* [review] onedev.kr review "GVA caches only values and restores keys on
  demand, halving the GQA cache", sections "How it works" (key
  reconstruction K_h = V_g(h) M_h and the absorption identity) and "How it
  differs" (decoupled RoPE, the shared positional key, cache-scalar counts,
  the initialisation scale);
* [explainer] bisque.today "Grouped Value Attention matches GQA on a 47%
  smaller KV cache", Equation 7 (absorption is exact) and its section-3
  pointer (fold + shared position key);
* [summary] agihunt.info summary page (Chinese), paragraphs on absorption,
  on decoupled RoPE and on K=V.

Everything here is float64.  The decode oracle *materialises* every content
key ``K_h = V_g(h) M_h`` and runs a textbook softmax over the full keys
``[K_h | k_rope]``; it never uses the absorbed shortcut.  The absorbed
evaluation (``absorb_query`` + ``attend_absorbed``) is a separate definition
used to pin Eq. 7 and to test the library's separate entry points.

Readings of points the pages leave open:

* softmax scale: 1/sqrt(d_n + d_r), the width of the full query/key;
* head -> group map g(h) = h // (H/G) (contiguous groups);
* RoPE: adjacent pairs (2i, 2i+1), angle pos * base**(-2i/d_r), row form
  y = R(pos) x; **parity unpinned** as to the convention itself (the pages
  print no value); pinned only through the relative-rotation property;
* positions are 0-based; the query token sits at position len-1 and attends
  to itself; a sequence of length 0 gives out = 0, lse = -inf;
* appended values are rounded to the cache dtype once, to nearest-even, from
  the exact (float64) rotated key;
* several query tokens per sequence (q_len = L): they are the last L cached
  positions, query i sits at position len-L+i and attends causally to
  positions 0 .. len-L+i (each query token is absorbed separately, once per
  head and token).
"""
import math

import numpy as np

__all__ = [
    "to_f64", "rope_angles", "rope_rotate", "bf16_nearest",
    "cache_scalars_per_token", "gqa_cache_scalars_per_token", "cache_ratio",
    "head_group", "default_scale", "softmax_attention", "gather_tokens",
    "reconstruct_keys", "gva_decode_materialized", "absorb_query",
    "attend_absorbed", "append_token", "gqa_decode", "chunk_partials",
    "merge_partials", "query_positions", "gva_decode_materialized_queries",
    "absorb_queries", "attend_absorbed_queries", "append_tokens",
    "gva_decode_rope_on_keys", "gqa_decode_queries",
]


def to_f64(x):
    """Widen an array-like (numpy array or torch tensor, any float dtype,
    bf16 included) to a float64 numpy array.  Widening is exact."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().cpu()
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()  # exact widening; numpy has no bf16
        return np.asarray(x.numpy(), dtype=np.float64)
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Rotary position encoding of the shared position slice
# --------------------------------------------------------------------------

def rope_angles(d_r, pos, base):
    """Angles pos * theta_i, theta_i = base**(-2i/d_r), i < d_r/2.

    The positional key is rotated by a position-dependent rotation R_j and the
    query's position slice by R_t ([review] "How it differs").  The frequency
    schedule is the reading stated in the module docstring."""
    if d_r % 2:
        raise ValueError("d_r must be even")
    i = np.arange(d_r // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * i / d_r)
    return np.multiply.outer(np.asarray(pos, dtype=np.float64), theta)


def rope_rotate(x, pos, base):
    """Rotate each adjacent pair (x_2i, x_2i+1) of the last axis by angle
    pos * theta_i.  ``pos`` broadcasts against ``x[..., 0]``."""
    x = np.asarray(x, dtype=np.float64)
    d_r = x.shape[-1]
    ang = rope_angles(d_r, pos, base)  # [..., d_r/2]
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    y = np.empty(np.broadcast_shapes(x.shape, c.shape[:-1] + (d_r,)))
    y[..., 0::2] = xe * c - xo * s
    y[..., 1::2] = xe * s + xo * c
    return y


# --------------------------------------------------------------------------
# bf16 storage rounding
# --------------------------------------------------------------------------

_BF16_MANT_BITS = 8          # significant bits incl. the implicit one
_BF16_MIN_EXP = -126         # smallest normal exponent
_BF16_SUB_ULP_EXP = _BF16_MIN_EXP - (_BF16_MANT_BITS - 1)   # 2**-133


def bf16_nearest(x):
    """Nearest bfloat16 value to each float64 ``x`` (ties to even), as float64.

    bf16 keeps 8 significant bits and float32's exponent range.  For |x| in
    [2**(e-1), 2**e) the spacing of bf16 values is 2**(e-8) (never below the
    subnormal spacing 2**-133); the rounded value is rint(x / spacing) *
    spacing with rint rounding half to even; magnitudes reaching 2**128 after
    rounding become infinities.  NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    if np.any(fin):
        xf = x[fin]
        _, e = np.frexp(xf)  # xf = m * 2**e, 0.5 <= |m| < 1
        ulp_exp = np.maximum(e - _BF16_MANT_BITS, _BF16_SUB_ULP_EXP)
        scaled = np.ldexp(xf, -ulp_exp)
        r = np.ldexp(np.rint(scaled), ulp_exp)
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
        out[fin] = r
    return out


def _round_to_cache(x, cache_dtype):
    if cache_dtype == "bfloat16":
        return bf16_nearest(x)
    if cache_dtype == "float32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if cache_dtype == "float64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(cache_dtype)


# --------------------------------------------------------------------------
# Cache accounting
# --------------------------------------------------------------------------

def cache_scalars_per_token(G, d_h, d_r):
    """Persistent scalars per cached token: G grouped value rows of width d_h
    plus one positional key of width d_r shared by all heads
    ([review] "How it differs": N_GVA = T*G*d_h + T*d_r)."""
    return G * d_h + d_r


def gqa_cache_scalars_per_token(G, d_h):
    """Grouped-query attention stores a key and a value row per group:
    N_GQA = 2*T*G*d_h ([review] "How it differs")."""
    return 2 * G * d_h


def cache_ratio(G, d_h, d_r):
    """N_GVA / N_GQA for the same T, G, d_h."""
    return cache_scalars_per_token(G, d_h, d_r) / gqa_cache_scalars_per_token(G, d_h)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def head_group(h, H, G):
    """Value group g(h) of query head h: H/G consecutive heads per group
    (the pages name the map g(h) without fixing it; reading in docstring)."""
    if H % G:
        raise ValueError("H must be a multiple of G")
    return h // (H // G)


def default_scale(d_n, d_r):
    return 1.0 / math.sqrt(d_n + d_r)


def softmax_attention(q, K, Vv, scale):
    """Textbook single-query attention in float64.

    s_j = scale * <q, K_j>;  p = exp(s - max s) / sum exp(s - max s);
    out = sum_j p_j Vv_j;    lse = max s + log sum exp(s - max s).
    Returns (out, lse, p, s).  With no keys: out = 0, lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    Vv = np.asarray(Vv, dtype=np.float64)
    if K.shape[0] == 0:
        return (np.zeros(Vv.shape[1:]), -np.inf, np.zeros(0), np.zeros(0))
    s = scale * (K @ q)
    m = np.max(s)
    e = np.exp(s - m)
    l = np.sum(e)
    p = e / l
    out = p @ Vv
    return out, m + math.log(l), p, s


def gather_tokens(pool, table_row, length, block_size):
    """Rows 0..length-1 of one sequence from a paged pool ``[NB, bs, ...]``:
    token j lives in block table_row[j // bs], slot j % bs."""
    pool = np.asarray(pool)
    j = np.arange(length)
    blocks = np.asarray(table_row)[j // block_size].astype(np.int64)
    return pool[blocks, j % block_size]


def reconstruct_keys(V_g, M_h):
    """Content keys of head h at every cached position: K_h = V_g(h) M_h,
    a [T, d_h] x [d_h, d_n] product ([review] "How it works")."""
    return np.asarray(V_g, dtype=np.float64) @ np.asarray(M_h, dtype=np.float64)


def _select(n, subset):
    return range(n) if subset is None else subset


def gva_decode_materialized(q_nope, q_rope, M, v_pool, k_pool, block_table,
                            seq_lens, scale=None, base=10000.0,
                            block_size=64, seqs=None, heads=None):
    """GVA decode by its plain definition, keys materialised.

    For each sequence b and head h (query at position t = len_b - 1):
      K_h  = V[b, :len, g(h)] @ M[h]                (content keys, [len, d_n])
      q_r  = R_t q_rope[b, h]                       (rotated query slice)
      key_j = [K_h[j] | k_rope[b, j]]               (k_rope stored rotated)
      query = [q_nope[b, h] | q_r]
      out[b, h], lse[b, h] = softmax attention of query over key_j,
                             summing the values V[b, j, g(h)].
    The head is split into an unrotated content slice and a rotated position
    slice whose key is cached once per token and shared by all heads
    ([review] "How it differs"; [summary] decoupled-RoPE paragraph).  Entries
    outside ``seqs`` x ``heads`` are left NaN."""
    q_nope, q_rope, M = to_f64(q_nope), to_f64(q_rope), to_f64(M)
    v_pool, k_pool = to_f64(v_pool), to_f64(k_pool)
    block_table = np.asarray(block_table)
    seq_lens = np.asarray(seq_lens).astype(np.int64)
    B, H, d_n = q_nope.shape
    d_r = q_rope.shape[-1]
    G, d_h = v_pool.shape[2], v_pool.shape[3]
    if scale is None:
        scale = default_scale(d_n, d_r)
    out = np.full((B, H, d_h), np.nan)
    lse = np.full((B, H), np.nan)
    for b in _select(B, seqs):
        n = int(seq_lens[b])
        t = n - 1
        V_all = gather_tokens(v_pool, block_table[b], n, block_size)  # [n,G,d_h]
        k_all = gather_tokens(k_pool, block_table[b], n, block_size)  # [n,d_r]
        for h in _select(H, heads):
            g = head_group(h, H, G)
            Vg = V_all[:, g, :]
            K_h = reconstruct_keys(Vg, M[h])
            q_r = rope_rotate(q_rope[b, h], t, base)
            keys = np.concatenate([K_h, k_all], axis=1)
            query = np.concatenate([q_nope[b, h], q_r])
            o, ls, _, _ = softmax_attention(query, keys, Vg, scale)
            out[b, h], lse[b, h] = o, ls
    return out, lse


def absorb_query(q_nope, q_rope, M, pos, scale=None, base=10000.0):
    """Absorbed query qa[b, h] = scale * [q_nope[b,h] M_h^T | R_pos q_rope[b,h]].

    The fixed map M_h folds into the query once per head and query token:
    q~_h = q_h M_h^T, so that <q_h, v_j M_h> = <q~_h, v_j> exactly
    ([review] "How it works"; [explainer] Equation 7).  The position slice is
    rotated to the query position.  The softmax scale is folded in."""
    q_nope, q_rope, M = to_f64(q_nope), to_f64(q_rope), to_f64(M)
    pos = np.asarray(pos).astype(np.float64)
    B, H, d_n = q_nope.shape
    d_r = q_rope.shape[-1]
    if scale is None:
        scale = default_scale(d_n, d_r)
    # q~[b,h,e] = sum_n q_nope[b,h,n] * M[h,e,n]
    q_tilde = np.einsum("bhn,hen->bhe", q_nope, M)
    q_r = rope_rotate(q_rope, pos[:, None], base)
    return scale * np.concatenate([q_tilde, q_r], axis=-1)


def attend_absorbed(qa, v_pool, k_pool, block_table, seq_lens, H=None,
                    block_size=64, seqs=None, heads=None):
    """Attention of the absorbed query over the value cache itself.

    Score of head h at position j: <qa[b,h], [V[b,j,g(h)] | k_rope[b,j]]>
    (scale already folded into qa); softmax; sum of the same values
    ([review] "How it works": content attention reads only the value
    cache)."""
    qa = to_f64(qa)
    v_pool, k_pool = to_f64(v_pool), to_f64(k_pool)
    block_table = np.asarray(block_table)
    seq_lens = np.asarray(seq_lens).astype(np.int64)
    B, H_, _ = qa.shape
    G, d_h = v_pool.shape[2], v_pool.shape[3]
    out = np.full((B, H_, d_h), np.nan)
    lse = np.full((B, H_), np.nan)
    for b in _select(B, seqs):
        n = int(seq_lens[b])
        V_all = gather_tokens(v_pool, block_table[b], n, block_size)
        k_all = gather_tokens(k_pool, block_table[b], n, block_size)
        for h in _select(H_, heads):
            g = head_group(h, H_, G)
            Vg = V_all[:, g, :]
            keys = np.concatenate([Vg, k_all], axis=1)
            o, ls, _, _ = softmax_attention(qa[b, h], keys, Vg, 1.0)
            out[b, h], lse[b, h] = o, ls
    return out, lse


def append_token(v_pool, k_pool, v_new, k_new, pos, block_table, base=10000.0,
                 block_size=64, cache_dtype="bfloat16"):
    """Write one new token per sequence into copies of the paged caches.

    v_pool[blk, slot, g, :] = round(v_new[b, g, :])
    k_pool[blk, slot, :]    = round(R_pos k_new[b, :])
    with blk = block_table[b, pos // bs], slot = pos % bs.  The positional key
    is stored already rotated, k_rope = (x_j W_r) R_j^T ([review] "How it
    differs"); ``k_new`` is the unrotated x_j W_r.  ``round`` is the cache
    dtype's nearest-even rounding of the exact value (no rounding for
    ``float64``).  Returns (v_pool, k_pool) as float64 arrays."""
    v_pool = np.array(to_f64(v_pool), copy=True)
    k_pool = np.array(to_f64(k_pool), copy=True)
    v_new, k_new = to_f64(v_new), to_f64(k_new)
    pos = np.asarray(pos).astype(np.int64)
    block_table = np.asarray(block_table)
    for b in range(v_new.shape[0]):
        p = int(pos[b])
        blk = int(block_table[b, p // block_size])
        slot = p % block_size
        v_pool[blk, slot] = _round_to_cache(v_new[b], cache_dtype)
        k_pool[blk, slot] = _round_to_cache(rope_rotate(k_new[b], p, base),
                                            cache_dtype)
    return v_pool, k_pool


def gqa_decode(q, k_pool, v_pool, block_table, seq_lens, scale=None,
               block_size=64, seqs=None, heads=None):
    """Grouped-query attention decode: head h scores its (already rotated)
    query against the stored key stream of its group and sums that group's
    values ([review] "What it is": GQA keeps two streams per position)."""
    q = to_f64(q)
    k_pool, v_pool = to_f64(k_pool), to_f64(v_pool)
    block_table = np.asarray(block_table)
    seq_lens = np.asarray(seq_lens).astype(np.int64)
    B, H, d_h = q.shape
    G = v_pool.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d_h)
    out = np.full((B, H, d_h), np.nan)
    lse = np.full((B, H), np.nan)
    for b in _select(B, seqs):
        n = int(seq_lens[b])
        K_all = gather_tokens(k_pool, block_table[b], n, block_size)
        V_all = gather_tokens(v_pool, block_table[b], n, block_size)
        for h in _select(H, heads):
            g = head_group(h, H, G)
            o, ls, _, _ = softmax_attention(q[b, h], K_all[:, g, :],
                                            V_all[:, g, :], scale)
            out[b, h], lse[b, h] = o, ls
    return out, lse


# --------------------------------------------------------------------------
# Several query tokens per sequence
# --------------------------------------------------------------------------

def query_positions(seq_len, q_len):
    """Positions of the q_len query tokens of a sequence whose cache holds
    seq_len tokens: the last q_len positions, seq_len-q_len .. seq_len-1."""
    return np.arange(int(seq_len) - int(q_len), int(seq_len))


def gva_decode_materialized_queries(q_nope, q_rope, M, v_pool, k_pool,
                                    block_table, seq_lens, scale=None,
                                    base=10000.0, block_size=64, seqs=None,
                                    heads=None):
    """GVA decode of L query tokens per sequence, keys materialised.

    q_nope [B, H, L, d_n], q_rope [B, H, L, d_r].  Query token i of sequence
    b sits at position t = len_b - L + i and sees cached positions 0..t
    (causal); for each head h it is the single-query definition of
    ``gva_decode_materialized`` with the context cut at t + 1 and R_t applied
    to its position slice.  Returns out [B, H, L, d_h], lse [B, H, L]."""
    q_nope, q_rope, M = to_f64(q_nope), to_f64(q_rope), to_f64(M)
    v_pool, k_pool = to_f64(v_pool), to_f64(k_pool)
    block_table = np.asarray(block_table)
    seq_lens = np.asarray(seq_lens).astype(np.int64)
    B, H, L, d_n = q_nope.shape
    d_r = q_rope.shape[-1]
    G, d_h = v_pool.shape[2], v_pool.shape[3]
    if scale is None:
        scale = default_scale(d_n, d_r)
    out = np.full((B, H, L, d_h), np.nan)
    lse = np.full((B, H, L), np.nan)
    for b in _select(B, seqs):
        n = int(seq_lens[b])
        V_all = gather_tokens(v_pool, block_table[b], n, block_size)
        k_all = gather_tokens(k_pool, block_table[b], n, block_size)
        for h in _select(H, heads):
            g = head_group(h, H, G)
            K_h = reconstruct_keys(V_all[:, g, :], M[h])
            keys = np.concatenate([K_h, k_all], axis=1)
            for i, t in enumerate(query_positions(n, L)):
                q_r = rope_rotate(q_rope[b, h, i], t, base)
                query = np.concatenate([q_nope[b, h, i], q_r])
                o, ls, _, _ = softmax_attention(query, keys[:t + 1],
                                                V_all[:t + 1, g, :], scale)
                out[b, h, i], lse[b, h, i] = o, ls
    return out, lse


def gqa_decode_queries(q, k_pool, v_pool, block_table, seq_lens, scale=None,
                       block_size=64, seqs=None, heads=None):
    """Grouped-query attention with L query tokens per sequence: the
    comparison the pages draw for prefill ([review] "Premises and limits":
    prefill is bound by matrix products, not by the cache).  q [B, H, L, d_h]
    (already rotated); query token i of sequence b sits at position
    t = len_b - L + i and sees positions 0..t of its group's key and value
    streams.  Returns out [B, H, L, d_h], lse [B, H, L]."""
    q = to_f64(q)
    k_pool, v_pool = to_f64(k_pool), to_f64(v_pool)
    block_table = np.asarray(block_table)
    seq_lens = np.asarray(seq_lens).astype(np.int64)
    B, H, L, d_h = q.shape
    G = v_pool.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d_h)
    out = np.full((B, H, L, d_h), np.nan)
    lse = np.full((B, H, L), np.nan)
    for b in _select(B, seqs):
        n = int(seq_lens[b])
        K_all = gather_tokens(k_pool, block_table[b], n, block_size)
        V_all = gather_tokens(v_pool, block_table[b], n, block_size)
        for h in _select(H, heads):
            g = head_group(h, H, G)
            for i, t in enumerate(query_positions(n, L)):
                o, ls, _, _ = softmax_attention(q[b, h, i], K_all[:t + 1, g, :],
                                                V_all[:t + 1, g, :], scale)
                out[b, h, i], lse[b, h, i] = o, ls
    return out, lse


def absorb_queries(q_nope, q_rope, M, pos_last, scale=None, base=10000.0):
    """Absorbed queries of L tokens per sequence: qa[b, h, i] is
    ``absorb_query`` of token i at position pos_last[b] - L + 1 + i.
    q_nope [B, H, L, d_n], q_rope [B, H, L, d_r] -> qa [B, H, L, d_h+d_r]."""
    q_nope, q_rope, M = to_f64(q_nope), to_f64(q_rope), to_f64(M)
    pos_last = np.asarray(pos_last).astype(np.float64)
    B, H, L, d_n = q_nope.shape
    d_r = q_rope.shape[-1]
    if scale is None:
        scale = default_scale(d_n, d_r)
    q_tilde = np.einsum("bhin,hen->bhie", q_nope, M)
    pos = pos_last[:, None] - (L - 1) + np.arange(L)[None, :]      # [B, L]
    q_r = rope_rotate(q_rope, pos[:, None, :], base)
    return scale * np.concatenate([q_tilde, q_r], axis=-1)


def attend_absorbed_queries(qa, v_pool, k_pool, block_table, seq_lens,
                            block_size=64, seqs=None, heads=None):
    """Causal attention of L absorbed queries per sequence over the value
    cache: query i of sequence b (position len_b - L + i) scores
    <qa[b,h,i], [V[b,j,g(h)] | k_rope[b,j]]> for j <= its position.
    qa [B, H, L, d_h+d_r] -> out [B, H, L, d_h], lse [B, H, L]."""
    qa = to_f64(qa)
    v_pool, k_pool = to_f64(v_pool), to_f64(k_pool)
    block_table = np.asarray(block_table)
    seq_lens = np.asarray(seq_lens).astype(np.int64)
    B, H, L, _ = qa.shape
    G, d_h = v_pool.shape[2], v_pool.shape[3]
    out = np.full((B, H, L, d_h), np.nan)
    lse = np.full((B, H, L), np.nan)
    for b in _select(B, seqs):
        n = int(seq_lens[b])
        V_all = gather_tokens(v_pool, block_table[b], n, block_size)
        k_all = gather_tokens(k_pool, block_table[b], n, block_size)
        for h in _select(H, heads):
            g = head_group(h, H, G)
            keys = np.concatenate([V_all[:, g, :], k_all], axis=1)
            for i, t in enumerate(query_positions(n, L)):
                o, ls, _, _ = softmax_attention(qa[b, h, i], keys[:t + 1],
                                                V_all[:t + 1, g, :], 1.0)
                out[b, h, i], lse[b, h, i] = o, ls
    return out, lse


def append_tokens(v_pool, k_pool, v_new, k_new, pos_last, block_table,
                  base=10000.0, block_size=64, cache_dtype="bfloat16"):
    """Write L new tokens per sequence: token i of sequence b goes to position
    pos_last[b] - L + 1 + i, exactly as ``append_token`` writes one token.
    v_new [B, L, G, d_h], k_new [B, L, d_r] (unrotated)."""
    v_new, k_new = to_f64(v_new), to_f64(k_new)
    pos_last = np.asarray(pos_last).astype(np.int64)
    L = v_new.shape[1]
    for i in range(L):
        v_pool, k_pool = append_token(v_pool, k_pool, v_new[:, i], k_new[:, i],
                                      pos_last - (L - 1) + i, block_table,
                                      base=base, block_size=block_size,
                                      cache_dtype=cache_dtype)
    return v_pool, k_pool


# --------------------------------------------------------------------------
# Ordinary RoPE on the reconstructed keys (the variant that cannot absorb)
# --------------------------------------------------------------------------

def gva_decode_rope_on_keys(q, M, v_pool, block_table, seq_lens, scale=None,
                            base=10000.0, block_size=64, seqs=None, heads=None):
    """GVA decode when ordinary RoPE acts on the whole reconstructed key.

    q [B, H, d_k] (unrotated), M [H, d_h, d_k], cache = values only.  For
    sequence b (query at position t = len_b - 1) and head h:
      K_h[j] = R_j (V[b, j, g(h)] M_h)      (key rebuilt, then rotated at j)
      q_r    = R_t q[b, h]
      out, lse = softmax attention of q_r over K_h (scale 1/sqrt(d_k)),
                 summing the values V[b, j, g(h)].
    The rotation depends on j, so M_h cannot be folded into the query: every
    key is rebuilt at every step (agihunt.info summary and cctest.ai article:
    the best-scoring GVA row keeps ordinary RoPE on the reconstructed key and
    cannot use absorbed decode).  Returns out [B, H, d_h], lse [B, H]."""
    q, M = to_f64(q), to_f64(M)
    v_pool = to_f64(v_pool)
    block_table = np.asarray(block_table)
    seq_lens = np.asarray(seq_lens).astype(np.int64)
    B, H, d_k = q.shape
    G, d_h = v_pool.shape[2], v_pool.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    out = np.full((B, H, d_h), np.nan)
    lse = np.full((B, H), np.nan)
    for b in _select(B, seqs):
        n = int(seq_lens[b])
        V_all = gather_tokens(v_pool, block_table[b], n, block_size)
        for h in _select(H, heads):
            g = head_group(h, H, G)
            K = reconstruct_keys(V_all[:, g, :], M[h])            # [n, d_k]
            K_rot = rope_rotate(K, np.arange(n), base)
            q_r = rope_rotate(q[b, h], n - 1, base)
            o, ls, _, _ = softmax_attention(q_r, K_rot, V_all[:, g, :], scale)
            out[b, h], lse[b, h] = o, ls
    return out, lse


# --------------------------------------------------------------------------
# Split-context partials and their merge
# --------------------------------------------------------------------------

def chunk_partials(q, K, Vv, scale, chunk):
    """Per-chunk softmax partials over consecutive key chunks of ``chunk``
    positions: m_c = max s, l_c = sum exp(s - m_c), acc_c = sum exp(s - m_c) V
    (unnormalised).  Returns lists (m, l, acc)."""
    q, K, Vv = to_f64(q), to_f64(K), to_f64(Vv)
    ms, ls, accs = [], [], []
    for c0 in range(0, K.shape[0], chunk):
        s = scale * (K[c0:c0 + chunk] @ q)
        m = np.max(s)
        e = np.exp(s - m)
        ms.append(m)
        ls.append(np.sum(e))
        accs.append(e @ Vv[c0:c0 + chunk])
    return ms, ls, accs


def merge_partials(ms, ls, accs):
    """Combine chunk partials into the full softmax result:
    m* = max_c m_c, w_c = exp(m_c - m*), L = sum_c w_c l_c,
    out = sum_c w_c acc_c / L, lse = m* + log L."""
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    accs = np.asarray(accs, dtype=np.float64)
    m_star = np.max(ms)
    w = np.exp(ms - m_star)
    L = np.sum(w * ls)
    out = (w @ accs) / L
    return out, m_star + math.log(L)
