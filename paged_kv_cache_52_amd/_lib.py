"""ctypes loader for libpagedattn.so (built in-tree by build.py).

There is no fallback: if the library is missing or does not load, importing
the binding raises, so no other code path can silently stand in for the HIP
kernels.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# PAGEDATTN_LIB names another build of the same library (the sanitizer build
# of tests/sanitize_host.py); by default the in-tree build.
LIB_PATH = os.environ.get("PAGEDATTN_LIB") or os.path.join(PKG, "libpagedattn.so")

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

# Exported symbol -> (restype, argtypes); mirrors include/pagedattn.h.
SIGNATURES = {
    "pa_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_num_splits": (_I32, [_I32, _I32]),
    "pa_max_splits": (_I32, [_I32, _I32, _I32, _I32]),
    "pa_default_split_tokens": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pa_sched_bytes": (_SZ, [_I32, _I32]),
    "pa_sched_bytes_packed": (_SZ, [_I32, _I32, _I32, _I32]),
    "pa_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "pa_workspace_bytes_packed": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "paged_kv_write": (ctypes.c_int, [_P, _P, _I32, _P, _I64, _I32, _I32, _P, _P, _P, _P, _I64,
                                      _I32, _P]),
    # q, q_dtype, B, Q, Hq, D, kc, vc, ks, vs, cache_dtype, NB, Hkv, tables, mb,
    # context_lens, query_start, mcl, W, scale, T, S, m, l, acc, sched, stream
    "paged_attn_decode_partial": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P,
                                                 _P, _I32, _I64, _I32, _P, _I32, _P, _P, _I32,
                                                 _I32, _F32, _I32, _I32, _P, _P, _P, _P, _P]),
    # context_lens, query_start, tables, B, mb, mcl, Q, g, W, T, group_members, sched, stream
    "paged_attn_plan": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                       _I32, _P, _P]),
    "paged_decode_prepare": (ctypes.c_int, [_P, _P, _I32, _P, _I64, _I32, _I32, _P, _P, _P, _P,
                                            _I64, _I32, _P, _P, _P, _I32, _I32, _I32, _I32,
                                            _I32, _I32, _I32, _I32, _P, _P]),
    # m, l, acc, context_lens, query_start, B, Q, Hq, D, mb, mcl, W, T, S, out, out_dtype,
    # stream
    "paged_attn_reduce": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                         _I32, _I32, _I32, _P, _I32, _P]),
    "pa_hbm_read_probe": (ctypes.c_int, [_P, _SZ, _P, _I32, _P]),
    "paged_attn_decode": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _I32,
                                         _I64, _I32, _P, _I32, _P, _P, _I32, _I32, _F32, _I32,
                                         _P, _P, _SZ, _P]),
    "paged_attn_decode_noalloc": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P,
                                                 _P, _I32, _I64, _I32, _P, _I32, _P, _P, _I32,
                                                 _I32, _F32, _I32, _P, _P]),
}

_lib = None


def load():
    """Load the library once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                "g.build()'` (hipcc, gfx950). There is no fallback implementation.")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
