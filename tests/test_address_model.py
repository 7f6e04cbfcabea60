"""CPU model of the global loads of the cache-reading kernels (no GPU).

The library's contract is that no read leaves the caller's pools, whatever
the device-resident lengths and block ids hold: a length or block id out of
range turns the sequence's output into NaN instead.  The kernels keep that
by construction -- a tile past a wave's range, or behind a bad block id,
reads pool row 0, and every block-table index is clamped into its row -- and
this test restates their index arithmetic in Python and checks every load
of every lane against the pool bounds:

* decode_mfma_kernel: the tiles each wave loads (the register sets' initial
  loads and every reload, including the ones past the wave's last tile), the
  1 KB value pieces of each tile (per lane: row and 16-byte chunk), the
  8-byte positional-key loads (clamped dims), and, for the GQA form, the key
  pieces; for every instance the launcher can pick (groups per head tile,
  d_h, d_r, GQA, waves per block, register sets);
* prefill_kernel: the staged 64-token key blocks (value rows of the block's
  group, positional-key rows);
* rope_keys_kernel: the 16-token tiles of the rotated-key decode.

It is a model: it mirrors the index expressions of the kernel sources (the
same names), so a change there must be carried here.
"""
import itertools

import numpy as np
import pytest

KB = 64          # tokens per cache block
TILE = 16        # tokens per decode tile
EDGE_LENS = [1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 127, 128, 129, 1000]
MULTI_LENS = [4, 5, 63, 64, 65, 66, 67, 128, 129, 1000]


# --------------------------------------------------------------- layouts ----

def make_table(lens, shuffled=True, seed=0, max_blocks=None, spare=0):
    """Block table of a paged pool holding `lens` (shuffled ids), the pool's
    block count (plus `spare` unused blocks) and max_blocks."""
    rng = np.random.default_rng(seed)
    need = [max(1, -(-int(n) // KB)) for n in lens]
    nb = sum(need) + spare
    mb = max_blocks or max(need)
    ids = rng.permutation(nb) if shuffled else np.arange(nb)
    bt = np.zeros((len(lens), mb), dtype=np.int64)
    k = 0
    for b, n in enumerate(need):
        bt[b, :n] = ids[k:k + n]
        k += n
    return bt, nb


# ------------------------------------------------------ decode (split) ----

def plan_mfma(B, max_seq_len, target=256):
    total = B * (max_seq_len if max_seq_len > 0 else 1)
    chunk = -(-total // target)
    chunk = max(KB, -(-chunk // KB) * KB)
    num_chunks = -(-max_seq_len // chunk) if max_seq_len > 0 else 1
    return chunk, num_chunks


def mfma_instance(cols, G, DH, DR, gqa, q_len):
    """(GT, NW, NSET) the launcher picks for `cols` = H * q_len columns, or
    None where the split matrix-core kernel does not take the call."""
    if cols % 16:
        return None
    nht = cols // 16
    if nht & (nht - 1):
        return None
    hpg = cols // G
    eight = not gqa and (DH == 64 or (DH == 128 and hpg == 16))
    if nht > (8 if eight else 4):
        return None
    if gqa:
        if hpg != 4 or q_len != 1 or DH not in (64, 128):
            return None
        GT = 4
    else:
        widths = {(64, 0), (64, 16), (64, 24), (64, 32), (128, 0), (128, 16), (128, 32)}
        if (DH, DR) not in widths:
            return None
        if hpg == 4 and q_len == 1:
            GT = 4
        elif hpg == 8:
            GT = 2
        elif hpg == 16:
            GT = 1
        else:
            return None
    NSET = 3 if (gqa and DH == 64) or GT < 4 else 2
    NW = 4
    if DH == 64 and not gqa and (GT < 4 or nht > 4):
        NW = 8
    if DH == 128 and not gqa and GT == 1 and nht > 4:
        NW = 8
    return GT, NW, NSET


def loaded_tiles(n_my, NSET):
    """Indices i of the tiles tile(i) a wave with n_my tiles loads: the
    initial loads of its register sets and every reload of the loop, the
    ones past n_my included."""
    n_steps = (n_my + 1) // 2
    if NSET == 2:
        idx = {0, 1}
        for i in range(0, 2 * n_steps - 2, 2):
            idx |= {i + 2, i + 3}
        return sorted(idx)
    idx = {0, 1, 2}
    i = 0
    for _ in range(n_steps // 3):
        idx |= {i + 3, i + 4, i + 5, i + 6, i + 7, i + 8}
        i += 6
    if n_steps % 3 == 2:
        idx.add(i + 3)
    return sorted(idx)


def piece_geometry(GT, DH):
    """For the value (and GQA key) pieces of a tile: the largest row offset
    within the tile and the byte range within a token row, over all pieces
    and lanes (relative to the head tile's first group)."""
    ROWB = GT * DH * 2
    NV = GT * (DH // 32)
    rows, lo, hi = [], [], []
    for x, lane in itertools.product(range(NV), range(64)):
        lrow = (16 * lane) // ROWB if ROWB <= 1024 else 0
        lchunk = ((16 * lane) % ROWB) // 16 if ROWB <= 1024 else lane
        prow = x * (1024 // ROWB) if ROWB <= 1024 else x // (ROWB // 1024)
        pchunk = 0 if ROWB <= 1024 else 64 * (x % (ROWB // 1024))
        rows.append(prow + lrow)
        byte = 16 * (pchunk + lchunk)
        lo.append(byte)
        hi.append(byte + 16)
    return max(rows), min(lo), max(hi), ROWB


def plan_lens(lens_host, max_items=256):
    """The split planned from host lengths (gva_decode_attention_lens): the
    smallest chunk, a multiple of the cache block, for which the items (at
    least one per sequence) number at most max_items; items (b, c, nc) in
    sequence order."""
    total = int(sum(int(n) for n in lens_host))
    chunk = max(KB, -(-(-(-total // max_items)) // KB) * KB)

    def count(ch):
        return sum(-(-int(n) // ch) if n > 0 else 1 for n in lens_host)
    while count(chunk) > max_items:
        chunk += KB
    items = []
    for b, n in enumerate(lens_host):
        nc = -(-int(n) // chunk) if n > 0 else 0
        items += [(b, c, nc) for c in range(max(nc, 1))]
    return chunk, items


def decode_reads(lens, bt, nb, G, DH, DR, cols, gqa=False, q_len=1, max_seq_len=None,
                 redirect=True, lens_host=None):
    """Checks every load of one split-decode launch; returns the number of
    tile loads checked.  redirect=False models a kernel without the row-0
    redirect of tiles past the range (the planted mistake of a test below).
    lens_host: the split planned from these host lengths instead (device
    lengths `lens` whose chunk count differs are invalid)."""
    inst = mfma_instance(cols, G, DH, DR, gqa, q_len)
    assert inst is not None, "no split matrix-core instance for this shape"
    GT, NW, NSET = inst
    B, max_blocks = bt.shape
    if max_seq_len is None:
        max_seq_len = int(max(max(lens), 0))
    def valid(n):
        n = int(n)
        bad = n < 0 or n > max_seq_len or n > max_blocks * KB or (0 < n < q_len)
        return 0 if bad else n
    plan_nc = {}
    if lens_host is None:
        chunk, num_chunks = plan_mfma(B, max_seq_len)
        blocks = [(b, c) for b in range(B) for c in range(num_chunks)]
    else:
        chunk, items = plan_lens(lens_host)
        assert len(items) <= 256
        blocks = [(b, c) for b, c, _ in items]
        for p, (b, c, nc) in enumerate(items):
            plan_nc[b] = nc
            # records at p0 + c and p0 + group (after all items), counters at
            # p0 and p0 + 1 + group: inside the shape-only workspace bound
            p0 = p - c
            assert p0 + c < 256 and len(items) + p0 + max(0, -(-nc // 16) - 1) < 2 * 256
            if nc > 32:
                assert -(-nc // 16) < nc and p0 + -(-nc // 16) < 256
    assert chunk % TILE == 0
    nht = cols // 16
    nsub = NW // nht
    vrow_bytes = G * DH * 2
    pool_rows = nb * KB
    max_r, lo, hi, _ = piece_geometry(GT, DH)
    # every lane's piece stays in the 16 rows of its tile and in its group's bytes
    assert max_r <= TILE - 1
    assert lo >= 0 and (nht - 1) * GT * DH * 2 + hi <= vrow_bytes
    NR = (DR + 15) // 16 if not gqa else 0
    for s, q4 in itertools.product(range(NR), range(4)):
        d = min(16 * s + 4 * q4, DR - 4)     # positional-key dims, clamped into the row
        assert 0 <= d and 2 * d + 8 <= 2 * DR
    checked = 0
    for b, c in blocks:
        length = valid(lens[b])
        if lens_host is not None and length and -(-length // chunk) != plan_nc[b]:
            length = 0  # the kernel reports the sequence NaN and loads nothing for it
        j_begin = c * chunk
        active = j_begin < length
        j_end = min(length, j_begin + chunk)
        n_tiles = -(-(j_end - j_begin) // TILE) if active else 0
        for wave in range(NW):
            sub = wave >> (nht.bit_length() - 1)
            n_my = -(-(n_tiles - sub) // nsub) if sub < n_tiles else 0
            for i in loaded_tiles(n_my, NSET):
                k = sub + i * nsub
                idx = min((j_begin + TILE * k) // KB, max_blocks - 1)
                assert 0 <= idx < max_blocks
                blk = int(bt[b, idx])
                real = k < n_tiles
                in_pool = 0 <= blk < nb
                j0 = j_begin + TILE * k
                row0 = blk * KB + (j0 % KB) if (real and in_pool) else 0
                if not redirect:
                    row0 = blk * KB + (j0 % KB)
                assert 0 <= row0 and row0 + max_r < pool_rows, (b, c, wave, k, blk)
                if not gqa and DR > 0:
                    assert row0 + (TILE - 1) < pool_rows  # k_rope rows row0 + li
                checked += 1
    return checked


# ------------------------------------------------------------- prefill ----

def prefill_reads(lens, bt, nb, H, G, DH, DR, L, max_seq_len=None, gqa=False):
    """Checks every staged load of one prefill launch (8 waves per block,
    16 query slots each, 64-token key blocks)."""
    B, max_blocks = bt.shape
    if max_seq_len is None:
        max_seq_len = int(max(lens))
    hpg = H // G
    qw = 8 // hpg
    n_qt = -(-L // (16 * qw))
    vrow_bytes = G * DH * 2
    VLOADS = KB * DH * 2 // 16 // 512
    KIN = DR * 2 // 16
    checked = 0
    for b in range(B):
        length = int(lens[b])
        bad_len = (length < 0 or length > max_seq_len or length > max_blocks * KB
                   or (0 < length < L))
        if bad_len or length == 0:
            continue  # the block writes NaN or zeros and returns before any load
        base = length - L
        for qt in range(n_qt):
            blk_last_slot = min(qt * 16 * qw + 16 * qw, L) - 1
            n_kb = (base + blk_last_slot) // KB + 1
            kbs = set(range(n_kb)) | {min(kb + 1, n_kb - 1) for kb in range(n_kb)}
            for g in range(G):
                for kb in kbs:
                    assert 0 <= kb < n_kb
                    blk = int(bt[b, min(kb, max_blocks - 1)])
                    if blk < 0 or blk >= nb:
                        blk = 0
                    row0 = blk * KB
                    for tid in range(512):
                        for x in range(VLOADS):
                            u = tid + 512 * x
                            r, ch = u // (DH // 8), u % (DH // 8)
                            assert r < KB
                            assert g * DH * 2 + 16 * ch + 16 <= vrow_bytes
                            assert row0 + r < nb * KB
                        if DR > 0 and tid < KB * KIN:
                            r, ch = tid // KIN, tid % KIN
                            assert row0 + r < nb * KB and 16 * ch + 16 <= DR * 2
                    checked += 1
    return checked


# ------------------------------------------------------ rotated-key decode ----

def rope_keys_reads(lens, bt, nb, G, DH, max_seq_len=None, target=1024):
    B, max_blocks = bt.shape
    if max_seq_len is None:
        max_seq_len = int(max(lens))
    total = B * G * max(max_seq_len, 1)
    chunk = max(KB, -(-(-(-total // target)) // KB) * KB)
    num_chunks = -(-max_seq_len // chunk) if max_seq_len > 0 else 1
    checked = 0
    for b in range(B):
        length = int(lens[b])
        if length < 0 or length > max_seq_len or length > max_blocks * KB:
            length = 0
        for c in range(num_chunks):
            j_begin = c * chunk
            if j_begin >= length:
                continue
            j_end = min(length, j_begin + chunk)
            last_j0 = j_begin + ((j_end - j_begin - 1) // TILE) * TILE
            for j0 in list(range(j_begin, j_end, TILE)) + [j_end - 1 + TILE]:
                jj = min(j0, last_j0)
                blk = int(bt[b, min(jj // KB, max_blocks - 1)])
                if blk < 0 or blk >= nb:
                    blk = 0
                row = blk * KB + (jj % KB) + (TILE - 1)  # the largest lane li
                assert row < nb * KB
                # 16 bytes at group g, dims 32 s + 8 q4: inside the group's row
                for s in range(DH // 32):
                    assert (G - 1) * DH * 2 + 2 * (32 * s + 8 * 3) + 16 <= G * DH * 2
                checked += 1
    return checked


# ----------------------------------------------------------------- tests ----

WORKLOADS = [
    # name, B, H, G, d_h, d_r, lens (None: ragged in [1024, 131072])
    ("decode_350m", 32, 16, 4, 64, 16, 4096),
    ("wide_rope_append", 64, 16, 4, 64, 24, 8192),
    ("long_ragged", 8, 16, 4, 64, 16, None),
    ("large_model", 128, 32, 8, 128, 32, 16384),
]


@pytest.mark.parametrize("name,B,H,G,d_h,d_r,T", WORKLOADS)
def test_decode_reads_stay_in_the_pool_on_the_workloads(name, B, H, G, d_h, d_r, T):
    rng = np.random.default_rng(1)
    lens = (rng.integers(1024, 131072, endpoint=True, size=B) if T is None
            else np.full(B, T))
    bt, nb = make_table(lens)
    assert decode_reads(lens, bt, nb, G, d_h, d_r, H) > 0
    if name == "large_model":  # and the same-shape GQA decode
        assert decode_reads(lens, bt, nb, G, d_h, 0, H, gqa=True) > 0


SHAPES = [  # (H, G, d_h, d_r) of the matrix-core ragged-edge cases
    (16, 4, 64, 16), (16, 4, 64, 24), (16, 4, 64, 32), (16, 4, 64, 0),
    (32, 8, 128, 32), (16, 4, 128, 16), (16, 4, 128, 0),
    (64, 16, 64, 16), (128, 32, 64, 16),
]


@pytest.mark.parametrize("H,G,d_h,d_r", SHAPES)
def test_decode_reads_on_ragged_edges_with_bad_entries(H, G, d_h, d_r):
    lens = np.array(EDGE_LENS)
    bt, nb = make_table(lens)
    decode_reads(lens, bt, nb, G, d_h, d_r, H)
    # slack max_seq_len: chunks past every sequence's end
    decode_reads(lens, bt, nb, G, d_h, d_r, H, max_seq_len=KB * bt.shape[1])
    # block ids out of range and lengths past the table: mapped to row 0
    bad_bt = bt.copy()
    for b, n in enumerate(lens):  # unused table entries hold anything
        bad_bt[b, max(1, -(-int(n) // KB)):] = 10 ** 6 + b
    bad_bt[0, 0] = -1
    bad_bt[-1, :] = nb + 5
    bad_lens = lens.copy()
    bad_lens[1] = KB * bt.shape[1] + 1
    bad_lens[2] = -3
    decode_reads(bad_lens, bad_bt, nb, G, d_h, d_r, H, max_seq_len=KB * bt.shape[1])


@pytest.mark.parametrize("H,G,d_h,d_r,L", [
    (16, 4, 64, 16, 2), (16, 4, 64, 16, 4), (16, 4, 64, 24, 4), (16, 4, 64, 0, 4),
    (32, 8, 128, 32, 2), (32, 8, 128, 32, 4), (32, 8, 128, 0, 4),
])
def test_decode_reads_with_several_query_columns(H, G, d_h, d_r, L):
    lens = np.array(MULTI_LENS)
    bt, nb = make_table(lens)
    decode_reads(lens, bt, nb, G, d_h, d_r, H * L, q_len=L)


@pytest.mark.parametrize("B,T", [(1, 70000), (2, 131072), (4, 200000), (1, 524288)])
def test_decode_reads_with_two_level_merges(B, T):
    lens = np.full(B, T)
    bt, nb = make_table(lens)
    chunk, num_chunks = plan_mfma(B, T)
    decode_reads(lens, bt, nb, 4, 64, 16, 16)
    assert num_chunks > 32 or B * T < 256 * 64 * 40


@pytest.mark.parametrize("lens", [
    "long_ragged", EDGE_LENS, [70000, 100, 5, 0, 3000], [0, 0, 1], [131072] * 2,
    list(range(1, 257)),
])
@pytest.mark.parametrize("H,G,d_h,d_r", [(16, 4, 64, 16), (16, 4, 64, 24), (32, 8, 128, 32)])
def test_decode_reads_with_host_planned_split(lens, H, G, d_h, d_r):
    if isinstance(lens, str):
        lens = np.random.default_rng(1).integers(1024, 131072, endpoint=True, size=8)
    lens = np.array(lens)
    bt, nb = make_table(lens)
    ms = int(max(lens.max(), 1))
    assert decode_reads(lens, bt, nb, G, d_h, d_r, H, max_seq_len=ms, lens_host=lens) >= 0
    # device lengths that disagree with the plan (longer and shorter)
    dev = lens.copy()
    dev[0] = min(ms, int(dev[0]) + 5000)
    dev[-1] = max(0, int(dev[-1]) - 3000)
    decode_reads(dev, bt, nb, G, d_h, d_r, H, max_seq_len=ms, lens_host=lens)


def test_host_plan_balances_the_items():
    """Every item holds at most one chunk of tokens, the chunk is the
    smallest multiple of the block with at most 256 items, and a uniform
    batch gets the max_seq_len split."""
    lens = np.random.default_rng(1).integers(1024, 131072, endpoint=True, size=8)
    chunk, items = plan_lens(lens)
    assert len(items) <= 256 and chunk % KB == 0
    assert plan_lens(lens, 256)[0] == chunk
    smaller = chunk - KB
    if smaller >= KB:
        assert sum(-(-int(n) // smaller) for n in lens) > 256
    assert plan_lens(np.full(32, 4096))[0] == plan_mfma(32, 4096)[0]


def test_every_instance_has_in_row_pieces():
    """Piece geometry of every (groups per head tile, d_h, GQA): each lane's
    16-byte piece lies in the 16 rows of its tile and inside its head tile's
    groups of a token row."""
    seen = set()
    for cols, G, d_h, d_r, gqa, q_len in itertools.product(
            (16, 32, 64, 128), (1, 2, 4, 8, 16, 32), (64, 128), (0, 16, 24, 32),
            (False, True), (1, 2, 4)):
        if cols % G or (gqa and d_r):
            continue
        inst = mfma_instance(cols, G, d_h, d_r, gqa, q_len)
        if inst is None:
            continue
        GT, NW, NSET = inst
        seen.add((GT, d_h, d_r, gqa, NW, NSET))
        max_r, lo, hi, rowb = piece_geometry(GT, d_h)
        assert max_r < TILE and lo >= 0 and hi <= rowb
    # the instances the library builds are all reached
    assert len(seen) >= 30, sorted(seen)


def test_loaded_tiles_cover_the_wave_and_at_most_nset_past_it():
    for NSET in (2, 3):
        for n_my in range(0, 40):
            idx = loaded_tiles(n_my, NSET)
            assert set(range(n_my)) <= set(idx)
            assert max(idx) < max(n_my, 1) + NSET + 1


@pytest.mark.parametrize("H,G,d_h,d_r,L,lens", [
    (16, 4, 64, 16, 16, [16, 17, 100, 1000]),
    (16, 4, 64, 24, 64, [64, 65, 700]),
    (32, 8, 128, 32, 16, [16, 300]),
    (16, 4, 64, 16, 512, [512, 4096]),
    (16, 4, 64, 0, 32, [32, 33, 200]),
])
def test_prefill_reads_stay_in_the_pool(H, G, d_h, d_r, L, lens):
    lens = np.array(lens)
    bt, nb = make_table(lens)
    assert prefill_reads(lens, bt, nb, H, G, d_h, d_r, L) > 0
    bad_bt = bt.copy()
    bad_bt[0, :] = -7
    prefill_reads(lens, bad_bt, nb, H, G, d_h, d_r, L)
    prefill_reads(lens, bt, nb, H, G, d_h, 0, L, gqa=True)


@pytest.mark.parametrize("G,d_h,lens", [
    (4, 64, EDGE_LENS), (8, 128, [1, 16, 17, 700, 4096]), (4, 64, [4096] * 32),
])
def test_rope_keys_reads_stay_in_the_pool(G, d_h, lens):
    lens = np.array(lens)
    bt, nb = make_table(lens)
    assert rope_keys_reads(lens, bt, nb, G, d_h) > 0
    bad_bt = bt.copy()
    bad_bt[-1, 0] = nb
    rope_keys_reads(lens, bad_bt, nb, G, d_h, max_seq_len=KB * bt.shape[1])


def test_model_catches_a_planted_overrun():
    """Without the row-0 redirect, a wave's loads past its last tile would
    follow table entries past the sequence's blocks; where those hold
    anything (here: ids past the pool), the model reports the overrun."""
    lens = np.array([100, 33])
    bt, nb = make_table(lens, max_blocks=4)
    for b, n in enumerate(lens):
        bt[b, -(-int(n) // KB):] = nb + 1000  # unused entries: garbage
    decode_reads(lens, bt, nb, 4, 64, 16, 16)  # the kernel as built: fine
    with pytest.raises(AssertionError):
        decode_reads(lens, bt, nb, 4, 64, 16, 16, redirect=False)
