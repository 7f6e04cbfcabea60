"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects bad arguments on the host before any HIP call.

No test here passes a fake pointer through to a launch: every call either
fails validation first or (on a machine with no GPU) reaches the HIP runtime,
which refuses for lack of a device.
"""
import ctypes
import os
import re

import pytest

from conftest import ROOT, gpu_available

HEADER = os.path.join(ROOT, "include", "gva.h")


@pytest.fixture(scope="module")
def g():
    import compressed_kv_cache_amd as pkg
    return pkg


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:gva|gqa)_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = header_functions()
    for n in ("gva_absorb_query", "gva_append_cache", "gva_decode_attention",
              "gva_decode_workspace_size", "gqa_decode_attention",
              "gqa_decode_workspace_size", "gva_cache_scalars_per_token",
              "gva_status_string", "gva_abi_version", "gva_absorb_query_multi",
              "gva_append_cache_multi", "gva_decode_workspace_size_multi",
              "gva_decode_attention_multi", "gva_decode_step_workspace_size_multi",
              "gva_decode_step_multi"):
        assert n in names


def test_library_exports_every_declared_symbol(g):
    lib = ctypes.CDLL(g.LIB_PATH)
    missing = [n for n in header_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding knows every one of them
    from compressed_kv_cache_amd._lib import SIGNATURES
    assert sorted(SIGNATURES) == header_functions()


def test_version_and_status_strings(g):
    assert g.lib.gva_abi_version() == 4
    for code in range(8):
        assert g.lib.gva_status_string(code)
    assert g.lib.gva_status_string(99) == b"unknown status"


def test_cache_scalars_per_token(g):
    assert g.cache_scalars_per_token(4, 64, 16) == 272
    assert g.cache_scalars_per_token(4, 64, 24) == 280
    assert g.cache_scalars_per_token(8, 128, 32) == 1056
    assert g.lib.gva_cache_scalars_per_token(None) == 0


def _shape(g, **kw):
    d = dict(B=2, H=16, G=4, d_h=64, d_n=48, d_r=16, max_blocks=4,
             num_blocks=8, cache_dtype=__import__("torch").bfloat16)
    d.update(kw)
    return g.make_shape(**d)


def _ws(g, s, max_seq_len=256):
    n = ctypes.c_size_t(0)
    st = g.lib.gva_decode_workspace_size(ctypes.byref(s), max_seq_len, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(H=15), 2),                 # H % G != 0
    (dict(G=0), 2),
    (dict(d_h=48), 3),               # unsupported width
    (dict(d_r=15), 3),               # odd position slice
    (dict(d_r=-2), 2),
    (dict(d_r=66), 3),
    (dict(max_blocks=0), 2),
    (dict(num_blocks=0), 2),
    (dict(B=-1), 2),
])
def test_workspace_query_validates_shape(g, kw, code):
    st, _ = _ws(g, _shape(g, **kw))
    assert st == code


def test_no_positional_slice_is_accepted(g):
    """d_r = 0 (no positional slice) is a supported width."""
    st, n = _ws(g, _shape(g, d_r=0))
    assert st == 0 and n > 0


def test_workspace_query_bounds(g):
    s = _shape(g)
    st, n = _ws(g, s, 256)
    assert st == 0 and n > 0
    assert _ws(g, s, 257)[0] == 2      # longer than max_blocks * 64
    assert _ws(g, s, -1)[0] == 2
    assert _ws(g, s, 0)[0] == 0
    bad = _shape(g, cache_dtype=None)
    bad.cache_dtype = 7
    assert _ws(g, bad)[0] == 3
    bs = _shape(g)
    bs.block_size = 32
    assert _ws(g, bs)[0] == 3
    assert g.lib.gva_decode_workspace_size(ctypes.byref(s), 64, None) == 1
    assert g.lib.gva_decode_workspace_size(None, 64, ctypes.byref(ctypes.c_size_t())) == 1


def _decode(g, s, ptrs, ws_bytes=1 << 30, max_seq_len=128):
    P = ctypes.c_void_p
    return g.lib.gva_decode_attention(
        ctypes.byref(s), P(ptrs.get("qa")), P(ptrs.get("v")), P(ptrs.get("k")),
        P(ptrs.get("bt")), P(ptrs.get("sl")), max_seq_len, P(ptrs.get("ws")),
        ws_bytes, P(ptrs.get("out")), P(ptrs.get("lse")), None)


GOOD = dict(qa=0x10000, v=0x20000, k=0x30000, bt=0x40000, sl=0x50000,
            ws=0x60000, out=0x70000, lse=0x80000)


@pytest.mark.parametrize("missing", ["qa", "v", "k", "bt", "sl", "ws", "out"])
def test_decode_null_pointers(g, missing):
    p = dict(GOOD)
    p[missing] = None
    assert _decode(g, _shape(g), p) == 1


@pytest.mark.parametrize("which", ["qa", "v", "k", "ws", "out"])
def test_decode_alignment(g, which):
    p = dict(GOOD)
    p[which] += 8
    assert _decode(g, _shape(g), p) == 4


def test_decode_workspace_too_small(g):
    s = _shape(g)
    _, need = _ws(g, s, 128)
    assert _decode(g, s, GOOD, ws_bytes=need - 1) == 5


def test_decode_empty_batch_is_noop(g):
    s = _shape(g, B=0)
    assert _decode(g, s, {}) == 0


def test_absorb_validation(g):
    P = ctypes.c_void_p
    s = _shape(g)
    args = [P(0x10000)] * 4
    f = g.lib.gva_absorb_query
    assert f(ctypes.byref(s), *args, 0.0, 10000.0, P(None), None) == 1
    assert f(ctypes.byref(s), *args, 0.0, -1.0, P(0x10000), None) == 2
    assert f(ctypes.byref(s), *args, float("nan"), 1e4, P(0x10000), None) == 2
    s2 = _shape(g, d_n=0)
    assert f(ctypes.byref(s2), *args, 0.0, 1e4, P(0x10000), None) == 2
    s3 = _shape(g, d_r=7)
    assert f(ctypes.byref(s3), *args, 0.0, 1e4, P(0x10000), None) == 3
    assert f(None, *args, 0.0, 1e4, P(0x10000), None) == 1


def test_append_validation(g):
    P = ctypes.c_void_p
    f = g.lib.gva_append_cache
    s = _shape(g)
    ptr = [P(0x10000)] * 4
    assert f(ctypes.byref(s), *ptr, 1e4, P(None), P(0x1000), None) == 1
    s2 = _shape(g, G=3)
    assert f(ctypes.byref(s2), *ptr, 1e4, P(0x1000), P(0x1000), None) == 2
    assert f(ctypes.byref(s), *ptr, 0.0, P(0x1000), P(0x1000), None) == 2


def test_gqa_validation(g):
    P = ctypes.c_void_p
    s = _shape(g)
    n = ctypes.c_size_t()
    assert g.lib.gqa_decode_workspace_size(ctypes.byref(s), 128, ctypes.byref(n)) == 0
    assert n.value > 0
    st = g.lib.gqa_decode_attention(
        ctypes.byref(s), P(None), 0.0, P(0x1000), P(0x1000), P(0x1000), P(0x1000),
        128, P(0x1000), n.value, P(0x1000), P(None), None)
    assert st == 1


@pytest.mark.skipif(gpu_available(), reason="only meaningful with no GPU present")
def test_launch_without_device_reports_hip_error(g):
    """With valid arguments and no GPU the HIP runtime refuses the launch."""
    P = ctypes.c_void_p
    s = _shape(g)
    st = g.lib.gva_absorb_query(ctypes.byref(s), P(0x10000), P(0x10000), P(0x10000),
                                P(0x10000), 0.0, 1e4, P(0x10000), None)
    assert st == 6


# ---- several query tokens per sequence ----

def _ws_multi(g, s, q_len, max_seq_len=256):
    n = ctypes.c_size_t(0)
    st = g.lib.gva_decode_workspace_size_multi(ctypes.byref(s), q_len, max_seq_len,
                                               ctypes.byref(n))
    return st, n.value


def test_multi_workspace_validates_q_len(g):
    s = _shape(g)
    assert _ws_multi(g, s, 0)[0] == 2
    assert _ws_multi(g, s, -3)[0] == 2
    assert _ws_multi(g, s, 65536)[0] == 0     # many query tokens: the blocked kernel
    assert _ws_multi(g, s, 65537)[0] == 3
    st1, n1 = _ws_multi(g, s, 1)
    assert (st1, n1) == _ws(g, s)          # q_len = 1 is the single-token call
    st4, n4 = _ws_multi(g, s, 4)
    assert st4 == 0 and n4 > n1            # one partial record per query token


def test_multi_step_workspace_holds_all_absorbed_queries(g):
    s = _shape(g)
    n1, n4 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert g.lib.gva_decode_step_workspace_size_multi(ctypes.byref(s), 1, 256,
                                                      ctypes.byref(n1)) == 0
    n0 = ctypes.c_size_t(0)
    assert g.lib.gva_decode_step_workspace_size(ctypes.byref(s), 256, ctypes.byref(n0)) == 0
    assert n0.value == n1.value
    assert g.lib.gva_decode_step_workspace_size_multi(ctypes.byref(s), 4, 256,
                                                      ctypes.byref(n4)) == 0
    qa4 = s.B * s.H * 4 * (s.d_h + s.d_r) * 4
    assert n4.value >= qa4


def test_multi_entry_points_validate(g):
    P = ctypes.c_void_p
    s = _shape(g)
    args = [P(0x10000)] * 4
    f = g.lib.gva_absorb_query_multi
    assert f(ctypes.byref(s), 0, *args, 0.0, 1e4, P(0x10000), None) == 2
    assert f(ctypes.byref(s), 2, *args, 0.0, 1e4, P(None), None) == 1
    a = g.lib.gva_append_cache_multi
    ptr = [P(0x10000)] * 4
    assert a(ctypes.byref(s), 0, *ptr, 1e4, P(0x1000), P(0x1000), None) == 2
    assert a(ctypes.byref(s), 2, *ptr, 1e4, P(None), P(0x1000), None) == 1
    d = g.lib.gva_decode_attention_multi
    assert d(ctypes.byref(s), 0, P(0x10000), P(0x20000), P(0x30000), P(0x40000),
             P(0x50000), 128, P(0x60000), 1 << 30, P(0x70000), P(None), None) == 2
    assert d(ctypes.byref(s), 4, P(None), P(0x20000), P(0x30000), P(0x40000),
             P(0x50000), 128, P(0x60000), 1 << 30, P(0x70000), P(None), None) == 1
    _, need = _ws_multi(g, s, 4, 128)
    assert d(ctypes.byref(s), 4, P(0x10000), P(0x20000), P(0x30000), P(0x40000),
             P(0x50000), 128, P(0x60000), need - 1, P(0x70000), P(None), None) == 5


# ---- ordinary RoPE on the reconstructed key ----

def test_rope_keys_validation(g):
    P = ctypes.c_void_p
    n = ctypes.c_size_t(0)
    f = g.lib.gva_decode_rope_keys_workspace_size
    assert f(ctypes.byref(_shape(g, d_n=64, d_r=0)), 256, ctypes.byref(n)) == 0 and n.value > 0
    assert f(ctypes.byref(_shape(g, d_n=64, d_r=16)), 256, ctypes.byref(n)) == 2  # no slice
    assert f(ctypes.byref(_shape(g, d_n=63, d_r=0)), 256, ctypes.byref(n)) == 2   # odd width
    assert f(ctypes.byref(_shape(g, d_n=40, d_r=0)), 256, ctypes.byref(n)) == 3   # no kernel
    assert f(ctypes.byref(_shape(g, d_n=64, d_r=0)), 257, ctypes.byref(n)) == 2
    d = g.lib.gva_decode_rope_keys
    s = _shape(g, d_n=64, d_r=0)
    args = [P(0x10000), P(0x20000), 0.0, 1e4, P(0x30000), P(0x40000), P(0x50000), 128,
            P(0x60000), 1 << 30, P(0x70000), P(None), None]
    bad = list(args)
    bad[0] = P(None)
    assert d(ctypes.byref(s), *bad) == 1
    bad = list(args)
    bad[3] = -1.0
    assert d(ctypes.byref(s), *bad) == 2
    bad = list(args)
    bad[9] = 16
    assert d(ctypes.byref(s), *bad) == 5


def test_many_query_tokens_need_no_workspace(g):
    """From 16 query tokens per sequence on, supported shapes go to the
    blocked kernel, which keeps no split records."""
    s = _shape(g)
    assert _ws_multi(g, s, 16) == (0, 0)
    assert _ws_multi(g, s, 256, 256) == (0, 0)
    assert _ws_multi(g, s, 4)[1] > 0          # the split decode kernel
    assert _ws_multi(g, s, 3)[0] == 0         # taken by some kernel
    assert _ws_multi(g, s, 15)[0] == 0
    f32 = _shape(g, cache_dtype=__import__("torch").float32)
    st, n = _ws_multi(g, f32, 16)             # fp32 cache: the vector kernel
    assert st in (0, 3)


def test_many_query_tokens_grid_bound(g):
    """The blocked kernel runs one grid row per (sequence, value group): a
    batch past that bound goes to another kernel or is reported unsupported,
    never launched out of range."""
    ok = _shape(g, B=16383, G=4, H=16)      # 65532 rows
    assert _ws_multi(g, ok, 64, 64) == (0, 0)
    big = _shape(g, B=16384, G=4, H=16)     # 65536 rows
    st, n = _ws_multi(g, big, 64, 64)
    assert st == 3 or n > 0                  # not the blocked kernel


def test_batch_past_grid_bound_is_unsupported(g):
    """B * G beyond the launch grid's y limit is refused up front."""
    assert _ws(g, _shape(g, B=16383, G=4))[0] == 0
    assert _ws(g, _shape(g, B=16384, G=4))[0] == 3
    assert _ws(g, _shape(g, B=70000, G=1, H=4))[0] == 3


def test_stream_read_probe_validation(g):
    """The read-rate probe rejects missing and misaligned buffers before any
    HIP call."""
    P = ctypes.c_void_p
    f = g.lib.gva_stream_read_probe
    assert f(P(0x10000), 16, None, None) == 1           # no output
    assert f(None, 16, P(0x10000), None) == 1           # no buffer for 16 bytes
    assert f(P(0x10008), 16, P(0x10000), None) == 4     # buffer not 16B aligned
    assert f(P(0x10000), 24, P(0x10000), None) == 4     # bytes not a multiple of 16
    assert f(P(0x10000), 16, P(0x10002), None) == 4     # output not 4B aligned
    from compressed_kv_cache_amd._lib import PROBE_BLOCKS
    assert PROBE_BLOCKS == int(re.search(r"#define GVA_PROBE_BLOCKS (\d+)",
                                         open(HEADER).read()).group(1))


def _step_noalloc(g, s, ptrs, max_seq_len=128):
    P = ctypes.c_void_p
    return g.lib.gva_decode_step_noalloc(
        ctypes.byref(s), P(ptrs.get("qn")), P(ptrs.get("qr")), P(ptrs.get("M")), 0.0,
        10000.0, P(ptrs.get("vn")), P(ptrs.get("kn")), P(ptrs.get("v")), P(ptrs.get("k")),
        P(ptrs.get("bt")), P(ptrs.get("sl")), max_seq_len, P(ptrs.get("out")),
        P(ptrs.get("lse")), None)


NOALLOC_GOOD = dict(qn=0x10000, qr=0x20000, M=0x30000, v=0x40000, k=0x50000, bt=0x60000,
                    sl=0x70000, out=0x80000, lse=0x90000)


@pytest.mark.parametrize("missing", ["qn", "qr", "M", "v", "k", "bt", "sl", "out"])
def test_noalloc_step_null_pointers(g, missing):
    ptrs = dict(NOALLOC_GOOD)
    ptrs[missing] = None
    assert _step_noalloc(g, _shape(g), ptrs) == 1


def test_noalloc_step_rejects_a_workspace_past_the_scratch(g):
    """A call whose step workspace exceeds the fixed device scratch is
    refused with GVA_ERR_SCRATCH before any HIP call (fake pointers)."""
    s = _shape(g, B=4096, max_blocks=64, num_blocks=4096 * 64)
    n = ctypes.c_size_t(0)
    assert g.lib.gva_decode_step_workspace_size(ctypes.byref(s), 4096, ctypes.byref(n)) == 0
    assert n.value > g.NOALLOC_SCRATCH_BYTES
    assert _step_noalloc(g, s, NOALLOC_GOOD, max_seq_len=4096) == 7
    small = _shape(g, B=2)
    assert g.lib.gva_decode_step_workspace_size(ctypes.byref(small), 128,
                                                ctypes.byref(n)) == 0
    assert n.value <= g.NOALLOC_SCRATCH_BYTES


def test_noalloc_step_validates_like_the_step(g):
    ptrs = dict(NOALLOC_GOOD)
    ptrs["v"] = 0x40008  # misaligned cache
    assert _step_noalloc(g, _shape(g), ptrs) == 4
    assert _step_noalloc(g, _shape(g, H=15), NOALLOC_GOOD) == 2
    assert _step_noalloc(g, _shape(g), NOALLOC_GOOD, max_seq_len=257) == 2


# ---- the host-planned split (gva_*_lens): argument checks, no GPU ----

def _ws_lens(g, s):
    n = ctypes.c_size_t(0)
    st = g.lib.gva_decode_workspace_size_lens(ctypes.byref(s), ctypes.byref(n))
    return st, n.value


def test_lens_workspace_depends_on_the_shape_only(g):
    st, n = _ws_lens(g, _shape(g, B=8))
    assert st == 0 and n > 0
    # records and counters for 256 items, and as many group records
    assert n >= 256 * 256 + 2 * 256 * 16 * (64 + 4) * 4
    assert _ws_lens(g, _shape(g, B=1)) == (0, n)
    m = ctypes.c_size_t(0)
    assert g.lib.gva_decode_step_workspace_size_lens(ctypes.byref(_shape(g, B=8)),
                                                     ctypes.byref(m)) == 0
    assert m.value >= n + 8 * 16 * (64 + 16) * 4


@pytest.mark.parametrize("kw", [
    dict(B=257),                                   # more sequences than plan items
    dict(G=2),                                     # H = 8 G: not the single-token instances
    dict(cache_dtype=__import__("torch").float32),  # no matrix-core decode
    dict(d_h=32, d_n=24, d_r=8),                   # no matrix-core instance
])
def test_lens_unsupported_shapes(g, kw):
    assert _ws_lens(g, _shape(g, **kw))[0] == 3


def _call_lens(g, s, lens, max_seq_len=256):
    P = ctypes.c_void_p
    host = (ctypes.c_int32 * len(lens))(*lens) if lens is not None else None
    return g.lib.gva_decode_attention_lens(
        ctypes.byref(s), P(0x10000), P(0x10000), P(0x10000), P(0x10000), P(0x10000),
        host, max_seq_len, P(0x10000), 1 << 30, P(0x10000), None, None)


def test_lens_host_lengths_are_checked_before_any_launch(g):
    s = _shape(g, B=3)
    assert _call_lens(g, s, [10, 300, 5]) == 2       # a length past max_seq_len
    assert _call_lens(g, s, [10, -1, 5]) == 2        # a negative length
    assert _call_lens(g, s, None) == 1               # no host lengths
    assert _call_lens(g, _shape(g, B=0), None) == 0  # nothing to do
    assert _call_lens(g, _shape(g, B=257), [1] * 257) == 3
