"""Loader for libgva.so and its C signatures (ctypes)."""
import ctypes
import os

# torch first: its HIP runtime (soname libamdhip64.so.7) is then the one
# libgva binds to, so device pointers and streams are shared.
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgva.so")


class GvaShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "B", "H", "G", "d_h", "d_n", "d_r", "block_size", "max_blocks",
        "num_blocks", "cache_dtype")]


GVA_F32 = 0
GVA_BF16 = 1
STATUS = {0: "GVA_OK", 1: "GVA_ERR_NULL", 2: "GVA_ERR_SHAPE",
          3: "GVA_ERR_UNSUPPORTED", 4: "GVA_ERR_ALIGN",
          5: "GVA_ERR_WORKSPACE", 6: "GVA_ERR_HIP", 7: "GVA_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 16 << 20  # GVA_NOALLOC_SCRATCH_BYTES

_P = ctypes.c_void_p
_SHAPE = ctypes.POINTER(GvaShape)
_I32 = ctypes.c_int32
_F32 = ctypes.c_float
_SIZE = ctypes.c_size_t

PROBE_BLOCKS = 1024  # GVA_PROBE_BLOCKS: words written by gva_stream_read_probe

SIGNATURES = {
    "gva_abi_version": (_I32, []),
    "gva_status_string": (ctypes.c_char_p, [_I32]),
    "gva_cache_scalars_per_token": (ctypes.c_uint64, [_SHAPE]),
    "gva_stream_read_probe": (_I32, [_P, ctypes.c_uint64, _P, _P]),
    "gva_absorb_query": (_I32, [_SHAPE, _P, _P, _P, _P, _F32, _F32, _P, _P]),
    "gva_append_cache": (_I32, [_SHAPE, _P, _P, _P, _P, _F32, _P, _P, _P]),
    "gva_decode_workspace_size": (_I32, [_SHAPE, _I32, ctypes.POINTER(_SIZE)]),
    "gva_decode_attention": (_I32, [_SHAPE, _P, _P, _P, _P, _P, _I32, _P, _SIZE,
                                    _P, _P, _P]),
    "gva_decode_step_workspace_size": (_I32, [_SHAPE, _I32, ctypes.POINTER(_SIZE)]),
    "gva_decode_step": (_I32, [_SHAPE, _P, _P, _P, _F32, _F32, _P, _P, _P, _P, _P, _P, _I32,
                               _P, _SIZE, _P, _P, _P]),
    "gva_decode_step_noalloc": (_I32, [_SHAPE, _P, _P, _P, _F32, _F32, _P, _P, _P, _P, _P,
                                       _P, _I32, _P, _P, _P]),
    "gva_decode_workspace_size_lens": (_I32, [_SHAPE, ctypes.POINTER(_SIZE)]),
    "gva_decode_attention_lens": (_I32, [_SHAPE, _P, _P, _P, _P, _P, _P, _I32, _P, _SIZE,
                                         _P, _P, _P]),
    "gva_decode_step_workspace_size_lens": (_I32, [_SHAPE, ctypes.POINTER(_SIZE)]),
    "gva_decode_step_lens": (_I32, [_SHAPE, _P, _P, _P, _F32, _F32, _P, _P, _P, _P, _P, _P, _P,
                                    _I32, _P, _SIZE, _P, _P, _P]),
    "gva_absorb_query_multi": (_I32, [_SHAPE, _I32, _P, _P, _P, _P, _F32, _F32, _P, _P]),
    "gva_append_cache_multi": (_I32, [_SHAPE, _I32, _P, _P, _P, _P, _F32, _P, _P, _P]),
    "gva_decode_workspace_size_multi": (_I32, [_SHAPE, _I32, _I32, ctypes.POINTER(_SIZE)]),
    "gva_decode_attention_multi": (_I32, [_SHAPE, _I32, _P, _P, _P, _P, _P, _I32, _P, _SIZE,
                                          _P, _P, _P]),
    "gva_decode_step_workspace_size_multi": (_I32, [_SHAPE, _I32, _I32,
                                                    ctypes.POINTER(_SIZE)]),
    "gva_decode_step_multi": (_I32, [_SHAPE, _I32, _P, _P, _P, _F32, _F32, _P, _P, _P, _P, _P,
                                     _P, _I32, _P, _SIZE, _P, _P, _P]),
    "gva_decode_rope_keys_workspace_size": (_I32, [_SHAPE, _I32, ctypes.POINTER(_SIZE)]),
    "gva_decode_rope_keys": (_I32, [_SHAPE, _P, _P, _F32, _F32, _P, _P, _P, _I32, _P, _SIZE,
                                    _P, _P, _P]),
    "gqa_decode_workspace_size": (_I32, [_SHAPE, _I32, ctypes.POINTER(_SIZE)]),
    "gqa_decode_attention": (_I32, [_SHAPE, _P, _F32, _P, _P, _P, _P, _I32, _P,
                                    _SIZE, _P, _P, _P]),
    "gqa_decode_workspace_size_multi": (_I32, [_SHAPE, _I32, _I32, ctypes.POINTER(_SIZE)]),
    "gqa_decode_attention_multi": (_I32, [_SHAPE, _I32, _P, _F32, _P, _P, _P, _P, _I32, _P,
                                          _SIZE, _P, _P, _P]),
}

_lib = None


def load(path=None):
    """Load libgva.so once; raise if it is missing (no fallback exists)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"libgva.so not found at {p}; build it with "
            "`python compressed_kv_cache_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


class GvaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        lib = load()
        msg = lib.gva_status_string(status).decode()
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")


def check(fn, status):
    if status != 0:
        raise GvaError(fn, status)
