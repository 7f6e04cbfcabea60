"""Python entry points with the C ABI's names.

Argument marshalling only: each function checks that the torch tensors have
the dtype, device and layout the C ABI documents, builds the size struct and
calls libgva on torch's current HIP stream.  All arithmetic runs in the HIP
kernels; there is no other implementation to fall back to.
"""
import ctypes

import torch

from . import _lib
from ._lib import GvaShape, check

BLOCK_SIZE = 64

_CACHE_DTYPES = {torch.float32: _lib.GVA_F32, torch.bfloat16: _lib.GVA_BF16}


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtype, device, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _cache_dtype(pool, name):
    if pool.dtype not in _CACHE_DTYPES:
        raise TypeError(f"{name} must be float32 or bfloat16, got {pool.dtype}")
    return _CACHE_DTYPES[pool.dtype]


def make_shape(B, H, G, d_h, d_n, d_r, max_blocks=1, num_blocks=1,
               cache_dtype=torch.bfloat16, block_size=BLOCK_SIZE):
    return GvaShape(B, H, G, d_h, d_n, d_r, block_size, max_blocks, num_blocks,
                    _CACHE_DTYPES.get(cache_dtype, -1))


def cache_scalars_per_token(G, d_h, d_r):
    """G*d_h + d_r persistent scalars per cached token (computed by libgva)."""
    s = make_shape(1, G, G, d_h, 1, d_r)
    return int(_lib.load().gva_cache_scalars_per_token(ctypes.byref(s)))


def stream_read_probe(buf, out=None):
    """Plain streaming read of a contiguous device tensor's bytes (a
    calibration of the achievable read rate; gva_stream_read_probe).
    Returns an int32 tensor of PROBE_BLOCKS words on buf's device whose XOR
    is the XOR of every 32-bit word of buf."""
    if not isinstance(buf, torch.Tensor) or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous torch.Tensor")
    dev = buf.device
    if out is None:
        out = torch.empty(_lib.PROBE_BLOCKS, dtype=torch.int32, device=dev)
    _need(out, "out", torch.int32, dev, 1)
    if out.numel() != _lib.PROBE_BLOCKS:
        raise ValueError(f"out must hold {_lib.PROBE_BLOCKS} words")
    nbytes = buf.numel() * buf.element_size()
    check("gva_stream_read_probe",
          _lib.load().gva_stream_read_probe(_ptr(buf), nbytes, _ptr(out), _stream(dev)))
    return out


def absorb_query(q_nope, q_rope, M, pos, softmax_scale=None, rope_base=10000.0,
                 out=None):
    """qa[B,H,d_h+d_r] = s * [q_nope M_h^T | R(pos) q_rope] (gva_absorb_query)."""
    dev = q_nope.device
    _need(q_nope, "q_nope", torch.float32, dev, 3)
    B, H, d_n = q_nope.shape
    _need(q_rope, "q_rope", torch.float32, dev, 3)
    _need(M, "M", torch.float32, dev, 3)
    _need(pos, "pos", torch.int32, dev, 1)
    d_r = q_rope.shape[2]
    d_h = M.shape[1]
    if tuple(q_rope.shape[:2]) != (B, H) or tuple(M.shape) != (H, d_h, d_n) \
            or pos.shape[0] != B:
        raise ValueError("inconsistent shapes for absorb_query")
    if out is None:
        out = torch.empty((B, H, d_h + d_r), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, 3)
    s = make_shape(B, H, 1, d_h, d_n, d_r)
    st = _lib.load().gva_absorb_query(
        ctypes.byref(s), _ptr(q_nope), _ptr(q_rope), _ptr(M), _ptr(pos),
        float(softmax_scale or 0.0), float(rope_base), _ptr(out), _stream(dev))
    check("gva_absorb_query", st)
    return out


def append_cache(v_new, k_new, pos, block_table, v_pool, k_pool,
                 rope_base=10000.0):
    """Write each sequence's new token (values, rotated k_rope) in place."""
    dev = v_pool.device
    _need(v_new, "v_new", torch.float32, dev, 3)
    _need(k_new, "k_new", torch.float32, dev, 2)
    _need(pos, "pos", torch.int32, dev, 1)
    _need(block_table, "block_table", torch.int32, dev, 2)
    cdt = _cache_dtype(v_pool, "v_pool")
    _need(v_pool, "v_pool", v_pool.dtype, dev, 4)
    _need(k_pool, "k_pool", v_pool.dtype, dev, 3)
    NB, bs, G, d_h = v_pool.shape
    B = v_new.shape[0]
    d_r = k_pool.shape[2]
    if tuple(v_new.shape) != (B, G, d_h) or tuple(k_new.shape) != (B, d_r) \
            or k_pool.shape[0] != NB or k_pool.shape[1] != bs \
            or block_table.shape[0] != B or pos.shape[0] != B:
        raise ValueError("inconsistent shapes for append_cache")
    s = GvaShape(B, G, G, d_h, 1, d_r, bs, block_table.shape[1], NB, cdt)
    st = _lib.load().gva_append_cache(
        ctypes.byref(s), _ptr(v_new), _ptr(k_new), _ptr(pos), _ptr(block_table),
        float(rope_base), _ptr(v_pool), _ptr(k_pool), _stream(dev))
    check("gva_append_cache", st)


def _decode_shape(B, H, v_pool, d_r, block_table, keys_separate=False):
    NB, bs, G, d_h = v_pool.shape
    cdt = _cache_dtype(v_pool, "v_pool")
    return GvaShape(B, H, G, d_h, 1, d_r, bs, block_table.shape[1], NB, cdt)


def decode_workspace_bytes(B, H, v_pool, k_pool, block_table, max_seq_len):
    """Workspace size gva_decode_attention needs for these caches.  A
    workspace must be zero-filled once when allocated (torch.zeros)."""
    s = _decode_shape(B, H, v_pool, k_pool.shape[2], block_table)
    n = ctypes.c_size_t(0)
    check("gva_decode_workspace_size", _lib.load().gva_decode_workspace_size(
        ctypes.byref(s), int(max_seq_len), ctypes.byref(n)))
    return n.value


def gqa_decode_workspace_bytes(B, H, k_pool, v_pool, block_table, max_seq_len):
    """Workspace size gqa_decode_attention needs for these caches."""
    s = _decode_shape(B, H, v_pool, 0, block_table, True)
    n = ctypes.c_size_t(0)
    check("gqa_decode_workspace_size", _lib.load().gqa_decode_workspace_size(
        ctypes.byref(s), int(max_seq_len), ctypes.byref(n)))
    return n.value


def _workspace(nbytes, dev, workspace):
    # zero-filled on allocation: the per-sequence counters at its start must
    # be zero before the first call (each call leaves them zero again)
    if workspace is None:
        workspace = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace too small")
    return workspace


def _host_lens(seq_lens_host, B):
    """The host copy of the lengths as a contiguous CPU int32 tensor."""
    t = torch.as_tensor(seq_lens_host, dtype=torch.int32).cpu().contiguous()
    if t.dim() != 1 or t.shape[0] != B:
        raise ValueError("seq_lens_host must hold one length per sequence")
    return t


def _decode(qa, v_pool, k_pool, block_table, seq_lens, max_seq_len, workspace, out, lse,
            want_lse, seq_lens_host):
    dev = qa.device
    _need(qa, "qa", torch.float32, dev, 3)
    _need(v_pool, "v_pool", v_pool.dtype, dev, 4)
    _need(k_pool, "k_pool", v_pool.dtype, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, H, dq = qa.shape
    d_h, d_r = v_pool.shape[3], k_pool.shape[2]
    if dq != d_h + d_r or block_table.shape[0] != B or seq_lens.shape[0] != B \
            or k_pool.shape[:2] != v_pool.shape[:2]:
        raise ValueError("inconsistent shapes for decode_attention")
    s = _decode_shape(B, H, v_pool, d_r, block_table)
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    if seq_lens_host is None:
        check("gva_decode_workspace_size",
              lib.gva_decode_workspace_size(ctypes.byref(s), int(max_seq_len), ctypes.byref(n)))
    else:
        hl = _host_lens(seq_lens_host, B)
        check("gva_decode_workspace_size_lens",
              lib.gva_decode_workspace_size_lens(ctypes.byref(s), ctypes.byref(n)))
    workspace = _workspace(n.value, dev, workspace)
    if out is None:
        out = torch.empty((B, H, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    if seq_lens_host is None:
        st = lib.gva_decode_attention(
            ctypes.byref(s), _ptr(qa), _ptr(v_pool), _ptr(k_pool), _ptr(block_table),
            _ptr(seq_lens), int(max_seq_len), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
            _stream(dev))
        check("gva_decode_attention", st)
    else:
        st = lib.gva_decode_attention_lens(
            ctypes.byref(s), _ptr(qa), _ptr(v_pool), _ptr(k_pool), _ptr(block_table),
            _ptr(seq_lens), hl.data_ptr(), int(max_seq_len), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
            _stream(dev))
        check("gva_decode_attention_lens", st)
    return out, lse


def decode_attention(qa, v_pool, k_pool, block_table, seq_lens, max_seq_len,
                     workspace=None, out=None, lse=None, want_lse=True):
    """out[B,H,d_h] (and lse[B,H]) of the absorbed query over the paged
    value cache and shared positional-key cache (gva_decode_attention)."""
    return _decode(qa, v_pool, k_pool, block_table, seq_lens, max_seq_len, workspace, out,
                   lse, want_lse, None)


def decode_attention_lens(qa, v_pool, k_pool, block_table, seq_lens, seq_lens_host,
                          max_seq_len, workspace=None, out=None, lse=None, want_lse=True):
    """decode_attention with the context split planned from the host copy of
    the lengths (gva_decode_attention_lens; ragged batches).  seq_lens_host:
    the same lengths in host memory (a CPU tensor or a sequence)."""
    return _decode(qa, v_pool, k_pool, block_table, seq_lens, max_seq_len, workspace, out,
                   lse, want_lse, seq_lens_host)


def decode_workspace_bytes_lens(B, H, v_pool, k_pool, block_table):
    """Workspace size gva_decode_attention_lens needs for these caches (any
    lengths; zero-fill once when allocated)."""
    s = _decode_shape(B, H, v_pool, k_pool.shape[2], block_table)
    n = ctypes.c_size_t(0)
    check("gva_decode_workspace_size_lens", _lib.load().gva_decode_workspace_size_lens(
        ctypes.byref(s), ctypes.byref(n)))
    return n.value


def gqa_decode_attention(q, k_pool, v_pool, block_table, seq_lens, max_seq_len,
                         softmax_scale=None, workspace=None, out=None, lse=None,
                         want_lse=True):
    """Same-shape grouped-query attention decode (gqa_decode_attention)."""
    dev = q.device
    _need(q, "q", torch.float32, dev, 3)
    _need(v_pool, "v_pool", v_pool.dtype, dev, 4)
    _need(k_pool, "k_pool", v_pool.dtype, dev, 4)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, H, d_h = q.shape
    if tuple(k_pool.shape) != tuple(v_pool.shape) or v_pool.shape[3] != d_h:
        raise ValueError("inconsistent shapes for gqa_decode_attention")
    s = _decode_shape(B, H, v_pool, 0, block_table, True)
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    check("gqa_decode_workspace_size",
          lib.gqa_decode_workspace_size(ctypes.byref(s), int(max_seq_len), ctypes.byref(n)))
    workspace = _workspace(n.value, dev, workspace)
    if out is None:
        out = torch.empty((B, H, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    st = lib.gqa_decode_attention(
        ctypes.byref(s), _ptr(q), float(softmax_scale or 0.0), _ptr(k_pool),
        _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), int(max_seq_len),
        _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(out), _ptr(lse), _stream(dev))
    check("gqa_decode_attention", st)
    return out, lse


def decode_step_workspace_bytes(q_nope, q_rope, v_pool, k_pool, block_table, max_seq_len):
    """Workspace size gva_decode_step needs (zero-fill it once when allocated)."""
    B, H, d_n = q_nope.shape
    NB, bs, G, d_h = v_pool.shape
    s = GvaShape(B, H, G, d_h, d_n, q_rope.shape[2], bs, block_table.shape[1], NB,
                 _cache_dtype(v_pool, "v_pool"))
    n = ctypes.c_size_t(0)
    check("gva_decode_step_workspace_size", _lib.load().gva_decode_step_workspace_size(
        ctypes.byref(s), int(max_seq_len), ctypes.byref(n)))
    return n.value


def _step(q_nope, q_rope, M, v_pool, k_pool, block_table, seq_lens, max_seq_len, v_new,
          k_new, softmax_scale, rope_base, workspace, out, lse, want_lse, seq_lens_host):
    dev = v_pool.device
    _need(q_nope, "q_nope", torch.float32, dev, 3)
    _need(q_rope, "q_rope", torch.float32, dev, 3)
    _need(M, "M", torch.float32, dev, 3)
    _need(v_pool, "v_pool", v_pool.dtype, dev, 4)
    _need(k_pool, "k_pool", v_pool.dtype, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, H, d_n = q_nope.shape
    NB, bs, G, d_h = v_pool.shape
    d_r = q_rope.shape[2]
    if tuple(q_rope.shape[:2]) != (B, H) or tuple(M.shape) != (H, d_h, d_n) \
            or tuple(k_pool.shape) != (NB, bs, d_r) or block_table.shape[0] != B \
            or seq_lens.shape[0] != B:
        raise ValueError("inconsistent shapes for decode_step")
    if (v_new is None) != (k_new is None):
        raise ValueError("give both v_new and k_new, or neither")
    if v_new is not None:
        _need(v_new, "v_new", torch.float32, dev, 3)
        _need(k_new, "k_new", torch.float32, dev, 2)
        if tuple(v_new.shape) != (B, G, d_h) or tuple(k_new.shape) != (B, d_r):
            raise ValueError("inconsistent shapes for v_new / k_new")
    s = GvaShape(B, H, G, d_h, d_n, d_r, bs, block_table.shape[1], NB,
                 _cache_dtype(v_pool, "v_pool"))
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    if seq_lens_host is None:
        check("gva_decode_step_workspace_size", lib.gva_decode_step_workspace_size(
            ctypes.byref(s), int(max_seq_len), ctypes.byref(n)))
    else:
        hl = _host_lens(seq_lens_host, B)
        check("gva_decode_step_workspace_size_lens", lib.gva_decode_step_workspace_size_lens(
            ctypes.byref(s), ctypes.byref(n)))
    workspace = _workspace(n.value, dev, workspace)
    if out is None:
        out = torch.empty((B, H, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    if seq_lens_host is None:
        st = lib.gva_decode_step(
            ctypes.byref(s), _ptr(q_nope), _ptr(q_rope), _ptr(M), float(softmax_scale or 0.0),
            float(rope_base), _ptr(v_new), _ptr(k_new), _ptr(v_pool), _ptr(k_pool),
            _ptr(block_table), _ptr(seq_lens), int(max_seq_len), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(dev))
        check("gva_decode_step", st)
    else:
        st = lib.gva_decode_step_lens(
            ctypes.byref(s), _ptr(q_nope), _ptr(q_rope), _ptr(M), float(softmax_scale or 0.0),
            float(rope_base), _ptr(v_new), _ptr(k_new), _ptr(v_pool), _ptr(k_pool),
            _ptr(block_table), _ptr(seq_lens), hl.data_ptr(), int(max_seq_len),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
            _stream(dev))
        check("gva_decode_step_lens", st)
    return out, lse


def decode_step(q_nope, q_rope, M, v_pool, k_pool, block_table, seq_lens, max_seq_len,
                v_new=None, k_new=None, softmax_scale=None, rope_base=10000.0,
                workspace=None, out=None, lse=None, want_lse=True):
    """Append (if v_new/k_new are given) + absorb + decode in two launches
    (gva_decode_step).  The new token and the query sit at seq_lens - 1."""
    return _step(q_nope, q_rope, M, v_pool, k_pool, block_table, seq_lens, max_seq_len, v_new,
                 k_new, softmax_scale, rope_base, workspace, out, lse, want_lse, None)


def decode_step_lens(q_nope, q_rope, M, v_pool, k_pool, block_table, seq_lens, seq_lens_host,
                     max_seq_len, v_new=None, k_new=None, softmax_scale=None,
                     rope_base=10000.0, workspace=None, out=None, lse=None, want_lse=True):
    """decode_step with the context split planned from the host copy of the
    lengths (gva_decode_step_lens; ragged batches)."""
    return _step(q_nope, q_rope, M, v_pool, k_pool, block_table, seq_lens, max_seq_len, v_new,
                 k_new, softmax_scale, rope_base, workspace, out, lse, want_lse, seq_lens_host)


def decode_step_workspace_bytes_lens(q_nope, q_rope, v_pool, k_pool, block_table):
    """Workspace size gva_decode_step_lens needs (any lengths; zero-fill once)."""
    B, H, d_n = q_nope.shape
    NB, bs, G, d_h = v_pool.shape
    s = GvaShape(B, H, G, d_h, d_n, q_rope.shape[2], bs, block_table.shape[1], NB,
                 _cache_dtype(v_pool, "v_pool"))
    n = ctypes.c_size_t(0)
    check("gva_decode_step_workspace_size_lens", _lib.load().gva_decode_step_workspace_size_lens(
        ctypes.byref(s), ctypes.byref(n)))
    return n.value


def decode_step_noalloc(q_nope, q_rope, M, v_pool, k_pool, block_table, seq_lens,
                        max_seq_len, v_new=None, k_new=None, softmax_scale=None,
                        rope_base=10000.0, out=None, lse=None, want_lse=True):
    """decode_step with no workspace argument (gva_decode_step_noalloc): the
    library takes its workspace from a fixed device array of
    NOALLOC_SCRATCH_BYTES per GPU.  `out` (and `lse`) are the caller's; pass
    them to make the call allocate nothing at all.  Calls that overlap on
    one GPU race."""
    dev = v_pool.device
    _need(q_nope, "q_nope", torch.float32, dev, 3)
    _need(q_rope, "q_rope", torch.float32, dev, 3)
    _need(M, "M", torch.float32, dev, 3)
    _need(v_pool, "v_pool", v_pool.dtype, dev, 4)
    _need(k_pool, "k_pool", v_pool.dtype, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, H, d_n = q_nope.shape
    NB, bs, G, d_h = v_pool.shape
    d_r = q_rope.shape[2]
    if tuple(q_rope.shape[:2]) != (B, H) or tuple(M.shape) != (H, d_h, d_n) \
            or tuple(k_pool.shape) != (NB, bs, d_r) or block_table.shape[0] != B \
            or seq_lens.shape[0] != B:
        raise ValueError("inconsistent shapes for decode_step_noalloc")
    if (v_new is None) != (k_new is None):
        raise ValueError("give both v_new and k_new, or neither")
    if v_new is not None:
        _need(v_new, "v_new", torch.float32, dev, 3)
        _need(k_new, "k_new", torch.float32, dev, 2)
        if tuple(v_new.shape) != (B, G, d_h) or tuple(k_new.shape) != (B, d_r):
            raise ValueError("inconsistent shapes for v_new / k_new")
    s = GvaShape(B, H, G, d_h, d_n, d_r, bs, block_table.shape[1], NB,
                 _cache_dtype(v_pool, "v_pool"))
    if out is None:
        out = torch.empty((B, H, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    lib = _lib.load()
    st = lib.gva_decode_step_noalloc(
        ctypes.byref(s), _ptr(q_nope), _ptr(q_rope), _ptr(M), float(softmax_scale or 0.0),
        float(rope_base), _ptr(v_new), _ptr(k_new), _ptr(v_pool), _ptr(k_pool),
        _ptr(block_table), _ptr(seq_lens), int(max_seq_len), _ptr(out), _ptr(lse),
        _stream(dev))
    check("gva_decode_step_noalloc", st)
    return out, lse


# ---- several tokens per sequence (q_len = L): the *_multi entry points ----

def absorb_query_multi(q_nope, q_rope, M, pos, softmax_scale=None, rope_base=10000.0,
                       out=None):
    """qa[B,H,L,d_h+d_r] for L query tokens per sequence; pos[b] is the
    position of the last one (gva_absorb_query_multi)."""
    dev = q_nope.device
    _need(q_nope, "q_nope", torch.float32, dev, 4)
    B, H, L, d_n = q_nope.shape
    _need(q_rope, "q_rope", torch.float32, dev, 4)
    _need(M, "M", torch.float32, dev, 3)
    _need(pos, "pos", torch.int32, dev, 1)
    d_r = q_rope.shape[3]
    d_h = M.shape[1]
    if tuple(q_rope.shape[:3]) != (B, H, L) or tuple(M.shape) != (H, d_h, d_n) \
            or pos.shape[0] != B:
        raise ValueError("inconsistent shapes for absorb_query_multi")
    if out is None:
        out = torch.empty((B, H, L, d_h + d_r), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, 4)
    s = make_shape(B, H, 1, d_h, d_n, d_r)
    st = _lib.load().gva_absorb_query_multi(
        ctypes.byref(s), L, _ptr(q_nope), _ptr(q_rope), _ptr(M), _ptr(pos),
        float(softmax_scale or 0.0), float(rope_base), _ptr(out), _stream(dev))
    check("gva_absorb_query_multi", st)
    return out


def append_cache_multi(v_new, k_new, pos, block_table, v_pool, k_pool, rope_base=10000.0):
    """Write L new tokens per sequence (v_new [B,L,G,d_h], k_new [B,L,d_r]);
    pos[b] is the position of the last one (gva_append_cache_multi)."""
    dev = v_pool.device
    _need(v_new, "v_new", torch.float32, dev, 4)
    _need(k_new, "k_new", torch.float32, dev, 3)
    _need(pos, "pos", torch.int32, dev, 1)
    _need(block_table, "block_table", torch.int32, dev, 2)
    cdt = _cache_dtype(v_pool, "v_pool")
    _need(v_pool, "v_pool", v_pool.dtype, dev, 4)
    _need(k_pool, "k_pool", v_pool.dtype, dev, 3)
    NB, bs, G, d_h = v_pool.shape
    B, L = v_new.shape[:2]
    d_r = k_pool.shape[2]
    if tuple(v_new.shape) != (B, L, G, d_h) or tuple(k_new.shape) != (B, L, d_r) \
            or k_pool.shape[0] != NB or k_pool.shape[1] != bs \
            or block_table.shape[0] != B or pos.shape[0] != B:
        raise ValueError("inconsistent shapes for append_cache_multi")
    s = GvaShape(B, G, G, d_h, 1, d_r, bs, block_table.shape[1], NB, cdt)
    st = _lib.load().gva_append_cache_multi(
        ctypes.byref(s), L, _ptr(v_new), _ptr(k_new), _ptr(pos), _ptr(block_table),
        float(rope_base), _ptr(v_pool), _ptr(k_pool), _stream(dev))
    check("gva_append_cache_multi", st)


def decode_workspace_bytes_multi(B, H, q_len, v_pool, k_pool, block_table, max_seq_len):
    """Workspace size gva_decode_attention_multi needs (zero-fill once)."""
    s = _decode_shape(B, H, v_pool, k_pool.shape[2], block_table)
    n = ctypes.c_size_t(0)
    check("gva_decode_workspace_size_multi", _lib.load().gva_decode_workspace_size_multi(
        ctypes.byref(s), int(q_len), int(max_seq_len), ctypes.byref(n)))
    return n.value


def decode_attention_multi(qa, v_pool, k_pool, block_table, seq_lens, max_seq_len,
                           workspace=None, out=None, lse=None, want_lse=True):
    """out[B,H,L,d_h] (and lse[B,H,L]) of L absorbed queries per sequence,
    query i at position seq_lens-L+i attending causally
    (gva_decode_attention_multi)."""
    dev = qa.device
    _need(qa, "qa", torch.float32, dev, 4)
    _need(v_pool, "v_pool", v_pool.dtype, dev, 4)
    _need(k_pool, "k_pool", v_pool.dtype, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, H, L, dq = qa.shape
    d_h, d_r = v_pool.shape[3], k_pool.shape[2]
    if dq != d_h + d_r or block_table.shape[0] != B or seq_lens.shape[0] != B \
            or k_pool.shape[:2] != v_pool.shape[:2]:
        raise ValueError("inconsistent shapes for decode_attention_multi")
    s = _decode_shape(B, H, v_pool, d_r, block_table)
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    check("gva_decode_workspace_size_multi", lib.gva_decode_workspace_size_multi(
        ctypes.byref(s), L, int(max_seq_len), ctypes.byref(n)))
    workspace = _workspace(n.value, dev, workspace)
    if out is None:
        out = torch.empty((B, H, L, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    st = lib.gva_decode_attention_multi(
        ctypes.byref(s), L, _ptr(qa), _ptr(v_pool), _ptr(k_pool), _ptr(block_table),
        _ptr(seq_lens), int(max_seq_len), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(dev))
    check("gva_decode_attention_multi", st)
    return out, lse


def decode_step_multi(q_nope, q_rope, M, v_pool, k_pool, block_table, seq_lens, max_seq_len,
                      v_new=None, k_new=None, softmax_scale=None, rope_base=10000.0,
                      workspace=None, out=None, lse=None, want_lse=True):
    """Append L new tokens (if v_new/k_new are given) + absorb L queries +
    causal decode (gva_decode_step_multi); seq_lens counts the new tokens."""
    dev = v_pool.device
    _need(q_nope, "q_nope", torch.float32, dev, 4)
    _need(q_rope, "q_rope", torch.float32, dev, 4)
    _need(M, "M", torch.float32, dev, 3)
    _need(v_pool, "v_pool", v_pool.dtype, dev, 4)
    _need(k_pool, "k_pool", v_pool.dtype, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, H, L, d_n = q_nope.shape
    NB, bs, G, d_h = v_pool.shape
    d_r = q_rope.shape[3]
    if tuple(q_rope.shape[:3]) != (B, H, L) or tuple(M.shape) != (H, d_h, d_n) \
            or tuple(k_pool.shape) != (NB, bs, d_r) or block_table.shape[0] != B \
            or seq_lens.shape[0] != B:
        raise ValueError("inconsistent shapes for decode_step_multi")
    if (v_new is None) != (k_new is None):
        raise ValueError("give both v_new and k_new, or neither")
    if v_new is not None:
        _need(v_new, "v_new", torch.float32, dev, 4)
        _need(k_new, "k_new", torch.float32, dev, 3)
        if tuple(v_new.shape) != (B, L, G, d_h) or tuple(k_new.shape) != (B, L, d_r):
            raise ValueError("inconsistent shapes for v_new / k_new")
    s = GvaShape(B, H, G, d_h, d_n, d_r, bs, block_table.shape[1], NB,
                 _cache_dtype(v_pool, "v_pool"))
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    check("gva_decode_step_workspace_size_multi", lib.gva_decode_step_workspace_size_multi(
        ctypes.byref(s), L, int(max_seq_len), ctypes.byref(n)))
    workspace = _workspace(n.value, dev, workspace)
    if out is None:
        out = torch.empty((B, H, L, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    st = lib.gva_decode_step_multi(
        ctypes.byref(s), L, _ptr(q_nope), _ptr(q_rope), _ptr(M), float(softmax_scale or 0.0),
        float(rope_base), _ptr(v_new), _ptr(k_new), _ptr(v_pool), _ptr(k_pool),
        _ptr(block_table), _ptr(seq_lens), int(max_seq_len), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(dev))
    check("gva_decode_step_multi", st)
    return out, lse


def gqa_decode_attention_multi(q, k_pool, v_pool, block_table, seq_lens, max_seq_len,
                               softmax_scale=None, workspace=None, out=None, lse=None,
                               want_lse=True):
    """Same-shape GQA with L query tokens per sequence, query i at position
    seq_lens-L+i attending causally (gqa_decode_attention_multi); q[B,H,L,d_h]
    rotated."""
    dev = q.device
    _need(q, "q", torch.float32, dev, 4)
    _need(v_pool, "v_pool", v_pool.dtype, dev, 4)
    _need(k_pool, "k_pool", v_pool.dtype, dev, 4)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, H, L, d_h = q.shape
    if tuple(k_pool.shape) != tuple(v_pool.shape) or v_pool.shape[3] != d_h:
        raise ValueError("inconsistent shapes for gqa_decode_attention_multi")
    s = _decode_shape(B, H, v_pool, 0, block_table, True)
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    check("gqa_decode_workspace_size_multi", lib.gqa_decode_workspace_size_multi(
        ctypes.byref(s), L, int(max_seq_len), ctypes.byref(n)))
    workspace = _workspace(n.value, dev, workspace)
    if out is None:
        out = torch.empty((B, H, L, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    st = lib.gqa_decode_attention_multi(
        ctypes.byref(s), L, _ptr(q), float(softmax_scale or 0.0), _ptr(k_pool), _ptr(v_pool),
        _ptr(block_table), _ptr(seq_lens), int(max_seq_len), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(dev))
    check("gqa_decode_attention_multi", st)
    return out, lse


# ---- ordinary RoPE on the reconstructed key (no absorption) ----

def decode_rope_keys(q, M, v_pool, block_table, seq_lens, max_seq_len, softmax_scale=None,
                     rope_base=10000.0, workspace=None, out=None, lse=None, want_lse=True):
    """out[B,H,d_h] (and lse[B,H]) of the variant whose keys R_j (v_j M_h)
    are rebuilt and rotated per token (gva_decode_rope_keys); q[B,H,d_k]
    unrotated, M[H,d_h,d_k]."""
    dev = q.device
    _need(q, "q", torch.float32, dev, 3)
    _need(M, "M", torch.float32, dev, 3)
    _need(v_pool, "v_pool", v_pool.dtype, dev, 4)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    B, H, d_k = q.shape
    NB, bs, G, d_h = v_pool.shape
    if tuple(M.shape) != (H, d_h, d_k) or block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("inconsistent shapes for decode_rope_keys")
    s = GvaShape(B, H, G, d_h, d_k, 0, bs, block_table.shape[1], NB,
                 _cache_dtype(v_pool, "v_pool"))
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    check("gva_decode_rope_keys_workspace_size", lib.gva_decode_rope_keys_workspace_size(
        ctypes.byref(s), int(max_seq_len), ctypes.byref(n)))
    if workspace is None:
        workspace = torch.empty(max(n.value, 16), dtype=torch.uint8, device=dev)
    if workspace.numel() * workspace.element_size() < n.value:
        raise ValueError("workspace too small")
    if out is None:
        out = torch.empty((B, H, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    st = lib.gva_decode_rope_keys(
        ctypes.byref(s), _ptr(q), _ptr(M), float(softmax_scale or 0.0), float(rope_base),
        _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), int(max_seq_len), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(dev))
    check("gva_decode_rope_keys", st)
    return out, lse
