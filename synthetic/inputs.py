"""Seeded synthetic inputs for GVA decode, shared by the oracle and the HIP path.

This module draws random tensors and lays them out; it performs none of the
attention arithmetic.  Every array has its own counter-seeded torch generator,
so one array's size never shifts another array's values.

Recipe (Grouped Value Attention pages; the values are standard normal):

* queries ``q_nope[B,H,d_n]`` and ``q_rope[B,H,d_r]`` ~ N(0, 1)  (sigma_Q = 1);
* per-head maps ``M[H,d_h,d_n]`` ~ N(0, sigma_M) with the scale-matched
  initialisation sigma_M = sigma_Q / (sigma_V * sqrt(d_in)), d_in = d_h and
  sigma_Q = sigma_V = 1 (agihunt.info summary, paragraph on initialisation;
  onedev.kr review, section "How it differs", last paragraph);
* value cache ``v_pool[NB,bs,G,d_h]`` and the shared, already-rotated
  positional key cache ``k_pool[NB,bs,d_r]`` ~ N(0, 1), stored in the cache
  dtype (bf16 values are the round-to-nearest-even images of fp32 draws);
* token slots past a sequence's length in its last block hold NaN, so a read
  outside the sequence poisons the result;
* ragged lengths are uniform integers in the inclusive range; blocks are dealt
  to sequences in order from a random permutation (shuffled tables) or from
  ``arange`` (contiguous tables); unused table entries are 0;
* workloads that append draw ``v_new[B,G,d_h]`` and the unrotated
  ``k_new[B,d_r]`` ~ N(0, 1) and poison the slot being appended with NaN;
* with L query tokens per sequence the queries are ``[B,H,L,d_n]`` and
  ``[B,H,L,d_r]``, the new tokens ``[B,L,G,d_h]`` and ``[B,L,d_r]`` (the last
  L positions), all ~ N(0, 1) from their own streams.
"""
import math
from typing import Dict, Optional

import torch

from .configs import GVAConfig

# Per-array generator streams.
_STREAM = {
    "q_nope": 1, "q_rope": 2, "M": 3, "lens": 4, "perm": 5, "v_pool": 6,
    "k_pool": 7, "v_new": 8, "k_new": 9, "gqa_q": 10, "gqa_k": 11,
    "mq_nope": 12, "mq_rope": 13, "mv_new": 14, "mk_new": 15, "gqa_mq": 16,
}

_TORCH_DTYPE = {"float32": torch.float32, "bfloat16": torch.bfloat16}


def _gen(device, seed: int, stream: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + _STREAM[stream])
    return g


def _randn(shape, device, seed, stream, dtype=torch.float32, chunk_rows=None):
    """N(0,1) draw of ``shape``; large arrays are drawn in leading-dim chunks
    (each chunk from the same generator, in order) and cast to ``dtype``."""
    g = _gen(device, seed, stream)
    if chunk_rows is None or shape[0] <= chunk_rows:
        return torch.randn(shape, generator=g, device=device).to(dtype)
    out = torch.empty(shape, dtype=dtype, device=device)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g,
                                 device=device).to(dtype)
    return out


def draw_seq_lens(cfg: GVAConfig, device="cpu", seed: Optional[int] = None):
    seed = cfg.seed if seed is None else seed
    if cfg.len_range is None:
        return torch.full((cfg.B,), cfg.T, dtype=torch.int32, device=device)
    lo, hi = cfg.len_range
    g = _gen("cpu", seed, "lens")
    lens = torch.randint(lo, hi + 1, (cfg.B,), generator=g, dtype=torch.int64)
    return lens.to(torch.int32).to(device)


def block_layout(seq_lens_cpu: torch.Tensor, block_size: int, shuffled: bool,
                 seed: int):
    """Deal cache blocks to sequences.  Returns (block_table[B,max_blocks]
    int32, number of pool blocks)."""
    lens = [int(x) for x in seq_lens_cpu.tolist()]
    nblk = [max(1, -(-n // block_size)) for n in lens]
    total = sum(nblk)
    if shuffled:
        ids = torch.randperm(total, generator=_gen("cpu", seed, "perm"))
    else:
        ids = torch.arange(total)
    max_blocks = max(nblk)
    table = torch.zeros((len(lens), max_blocks), dtype=torch.int32)
    off = 0
    for b, nb in enumerate(nblk):
        table[b, :nb] = ids[off:off + nb].to(torch.int32)
        off += nb
    return table, total


def _poison_tail(pool: torch.Tensor, table_cpu, lens, block_size, extra=None):
    """Write NaN into every token slot at or past each sequence's length in
    its last block (and into the slots listed in ``extra`` as (b, pos))."""
    nan = float("nan")
    for b, n in enumerate(lens):
        last = (max(1, -(-n // block_size))) - 1
        blk = int(table_cpu[b, last])
        start = n - last * block_size
        if start < block_size:
            pool[blk, start:] = nan
    if extra:
        for b, p in extra:
            blk = int(table_cpu[b, p // block_size])
            pool[blk, p % block_size] = nan


def make_gva_inputs(cfg: GVAConfig, device="cpu", seed: Optional[int] = None,
                    seq_lens: Optional[torch.Tensor] = None,
                    shuffled: Optional[bool] = None) -> Dict[str, object]:
    """All inputs of one GVA decode step for workload ``cfg`` on ``device``.

    ``seq_lens`` (host tensor) and ``shuffled`` override the workload's own
    length draw and block-table kind (used for edge-case tests)."""
    seed = cfg.seed if seed is None else seed
    dev = torch.device(device)
    B, H, G, d_h, d_n, d_r, bs = (cfg.B, cfg.H, cfg.G, cfg.d_h, cfg.d_n,
                                  cfg.d_r, cfg.block_size)
    cdt = _TORCH_DTYPE[cfg.cache_dtype]
    lens_cpu = (draw_seq_lens(cfg, "cpu", seed) if seq_lens is None
                else seq_lens.to(torch.int32).cpu())
    lens = [int(x) for x in lens_cpu.tolist()]
    shuffled = cfg.shuffled_blocks if shuffled is None else shuffled
    table_cpu, nb = block_layout(lens_cpu, bs, shuffled, seed)

    sigma_q = 1.0
    sigma_v = 1.0
    sigma_m = sigma_q / (sigma_v * math.sqrt(d_h))  # d_in = d_h

    out = {"cfg": cfg, "seed": seed}
    out["q_nope"] = _randn((B, H, d_n), dev, seed, "q_nope")
    out["q_rope"] = _randn((B, H, d_r), dev, seed, "q_rope")
    out["M"] = _randn((H, d_h, d_n), dev, seed, "M") * sigma_m
    out["sigma_M"] = sigma_m
    # Rows of 64 tokens x G x d_h: draw in chunks of blocks to bound the fp32
    # temporary for the largest pools.
    chunk = max(1, (1 << 27) // (bs * G * d_h))
    v_pool = _randn((nb, bs, G, d_h), dev, seed, "v_pool", cdt, chunk)
    k_pool = _randn((nb, bs, d_r), dev, seed, "k_pool", cdt, chunk)
    extra = None
    if cfg.append:
        out["v_new"] = _randn((B, G, d_h), dev, seed, "v_new")
        out["k_new"] = _randn((B, d_r), dev, seed, "k_new")
        extra = [(b, n - 1) for b, n in enumerate(lens) if n > 0]
    _poison_tail(v_pool, table_cpu, lens, bs, extra)
    _poison_tail(k_pool, table_cpu, lens, bs, extra)
    out["v_pool"] = v_pool
    out["k_pool"] = k_pool
    out["seq_lens"] = lens_cpu.to(dev)
    out["seq_lens_host"] = lens_cpu
    out["pos"] = (lens_cpu - 1).clamp_min(0).to(torch.int32).to(dev)
    out["block_table"] = table_cpu.to(dev)
    out["block_table_host"] = table_cpu
    out["num_blocks"] = nb
    out["max_seq_len"] = max(lens) if lens else 0
    return out


def make_gva_multi_inputs(cfg: GVAConfig, q_len: int, device="cpu",
                          seed: Optional[int] = None,
                          seq_lens: Optional[torch.Tensor] = None,
                          shuffled: Optional[bool] = None) -> Dict[str, object]:
    """Inputs of a decode step with ``q_len`` query tokens per sequence: the
    caches, lengths and maps of ``make_gva_inputs`` (without its one-token
    append), plus ``q_nope[B,H,L,d_n]``, ``q_rope[B,H,L,d_r]`` and, when the
    workload appends, ``v_new[B,L,G,d_h]`` and ``k_new[B,L,d_r]`` for the last
    L positions of each sequence (those slots poisoned with NaN).  ``pos`` is
    the position of each sequence's last token."""
    seed = cfg.seed if seed is None else seed
    dev = torch.device(device)
    base = with_overrides(cfg, append=False)
    out = make_gva_inputs(base, device=device, seed=seed, seq_lens=seq_lens,
                          shuffled=shuffled)
    out["cfg"] = cfg
    B, H, G, d_h, d_n, d_r, bs = (cfg.B, cfg.H, cfg.G, cfg.d_h, cfg.d_n,
                                  cfg.d_r, cfg.block_size)
    L = int(q_len)
    out["q_len"] = L
    out["q_nope"] = _randn((B, H, L, d_n), dev, seed, "mq_nope")
    out["q_rope"] = _randn((B, H, L, d_r), dev, seed, "mq_rope")
    if cfg.append:
        out["v_new"] = _randn((B, L, G, d_h), dev, seed, "mv_new")
        out["k_new"] = _randn((B, L, d_r), dev, seed, "mk_new")
        lens = [int(x) for x in out["seq_lens_host"].tolist()]
        extra = [(b, p) for b, n in enumerate(lens) for p in range(max(0, n - L), n)]
        _poison_tail(out["v_pool"], out["block_table_host"], lens, bs, extra)
        _poison_tail(out["k_pool"], out["block_table_host"], lens, bs, extra)
    return out


def make_gqa_inputs(cfg: GVAConfig, device="cpu", seed: Optional[int] = None,
                    seq_lens: Optional[torch.Tensor] = None) -> Dict[str, object]:
    """Same-shape grouped-query attention decode inputs: one query
    ``q[B,H,d_h]`` (already position-rotated) against key and value caches
    ``k_pool, v_pool[NB,bs,G,d_h]`` (two streams of G*d_h scalars per token)."""
    seed = cfg.seed if seed is None else seed
    dev = torch.device(device)
    B, H, G, d_h, bs = cfg.B, cfg.H, cfg.G, cfg.d_h, cfg.block_size
    cdt = _TORCH_DTYPE[cfg.cache_dtype]
    lens_cpu = (draw_seq_lens(cfg, "cpu", seed) if seq_lens is None
                else seq_lens.to(torch.int32).cpu())
    lens = [int(x) for x in lens_cpu.tolist()]
    table_cpu, nb = block_layout(lens_cpu, bs, cfg.shuffled_blocks, seed)
    chunk = max(1, (1 << 27) // (bs * G * d_h))
    out = {"cfg": cfg, "seed": seed}
    out["q"] = _randn((B, H, d_h), dev, seed, "gqa_q")
    k_pool = _randn((nb, bs, G, d_h), dev, seed, "gqa_k", cdt, chunk)
    v_pool = _randn((nb, bs, G, d_h), dev, seed, "v_pool", cdt, chunk)
    _poison_tail(k_pool, table_cpu, lens, bs)
    _poison_tail(v_pool, table_cpu, lens, bs)
    out["k_pool"] = k_pool
    out["v_pool"] = v_pool
    out["seq_lens"] = lens_cpu.to(dev)
    out["seq_lens_host"] = lens_cpu
    out["block_table"] = table_cpu.to(dev)
    out["block_table_host"] = table_cpu
    out["num_blocks"] = nb
    out["max_seq_len"] = max(lens) if lens else 0
    return out


def make_gqa_multi_inputs(cfg: GVAConfig, q_len: int, device="cpu",
                          seed: Optional[int] = None,
                          seq_lens: Optional[torch.Tensor] = None) -> Dict[str, object]:
    """``make_gqa_inputs`` with ``q_len`` query tokens per sequence:
    ``q[B,H,L,d_h]`` (rotated) for the last L positions of each sequence."""
    out = make_gqa_inputs(cfg, device=device, seed=seed, seq_lens=seq_lens)
    seed = out["seed"]
    out["q_len"] = int(q_len)
    out["q"] = _randn((cfg.B, cfg.H, int(q_len), cfg.d_h), torch.device(device), seed,
                      "gqa_mq")
    return out


def with_overrides(cfg: GVAConfig, **kw) -> GVAConfig:
    """A copy of ``cfg`` with fields replaced (for reduced-size test cases)."""
    d = {k: getattr(cfg, k) for k in cfg.__dataclass_fields__}
    d.update(kw)
    return GVAConfig(**d)
