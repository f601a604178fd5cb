"""CPU oracle for paged-KV decode attention. TEST INFRASTRUCTURE ONLY.

A thin ctypes wrapper over ``oracle.c`` (plain C, fp64). Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import this package; the
HIP library never does, and this package never imports the HIP library.

Arrays are NumPy arrays on the host. dtype codes follow the element type:
``np.float32`` is fp32, ``np.uint16``/``np.int16`` hold bf16 bit patterns,
``np.int8`` is the INT8 cache and ``np.uint8`` holds OCP FP8 E4M3 codes.
Shapes:

* q            [num_seqs][num_q_heads][head_dim], or
               [num_seqs][num_query_tokens][num_q_heads][head_dim] (several query
               tokens per sequence: the last num_query_tokens tokens of its context),
               or, with query_start [num_seqs + 1], the packed
               [query_start[-1]][num_q_heads][head_dim] (sequence s owns rows
               query_start[s] .. query_start[s+1]-1, its last tokens)
* k/v cache    [num_blocks][num_kv_heads][16][head_dim]
* k/v scale    [num_blocks][num_kv_heads][16] float32 (INT8 / FP8 caches only)
* block_tables [num_seqs][max_blocks_per_seq] int32
* context_lens [num_seqs] int32
* slot_mapping [num_tokens] int64 (negative = skip)

What each function computes, and which page it follows, is stated in
``oracle.c``.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_ORACLE_LIB names another build of oracle.c (the sanitizer build of
# tests/sanitize_host.py); by default the in-tree build.
_LIB_PATH = os.environ.get("PA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

BLOCK_SIZE = 16
F32, BF16, I8, FP8 = 0, 1, 2, 3


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_kv_write.argtypes = [P, P, I, P, L, I, I, P, P, P, P, L, I]
        lib.oracle_kv_write.restype = I
        lib.oracle_decode.argtypes = [P, I, I, I, I, P, P, P, P, P, I, I, I, P, I, P, D, P, P,
                                      P, L, P]
        lib.oracle_decode.restype = None
        lib.oracle_decode_split.argtypes = [P, I, I, I, I, I, P, P, P, P, P, I, I, I, P, I, P, D,
                                            I, I, P, P, P]
        lib.oracle_decode_split.restype = None
        lib.oracle_merge.argtypes = [P, P, P, L, I, I, P]
        lib.oracle_merge.restype = None
        lib.oracle_num_splits.argtypes = [I, I]
        lib.oracle_num_splits.restype = I
        lib.oracle_split_base.argtypes = [I, I, I]
        lib.oracle_split_base.restype = I
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_decode.restype = D
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = I
        lib.oracle_proc_bind.argtypes = []
        lib.oracle_proc_bind.restype = I
        lib.oracle_interleave.argtypes = [P, ctypes.c_size_t, I]
        lib.oracle_interleave.restype = I
        _lib = lib
    return _lib


def _code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype in (np.uint16, np.int16):
        return BF16
    if a.dtype == np.int8:
        return I8
    if a.dtype == np.uint8:
        return FP8
    raise TypeError(f"unsupported dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.asarray(a)
    if dtype is not None and a.dtype != dtype:
        a = a.astype(dtype)
    return np.ascontiguousarray(a)


def e4m3_decode(code: int) -> float:
    """Value of one OCP FP8 E4M3 code."""
    return float(_load().oracle_e4m3_decode(int(code)))


def e4m3_encode(x: float) -> int:
    """E4M3 code of an fp32 value (nearest, ties to even, saturating at 448)."""
    return int(_load().oracle_e4m3_encode(float(np.float32(x))))


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def proc_bind() -> str:
    """Thread binding of the oracle's OpenMP loops (omp_get_proc_bind)."""
    v = int(_load().oracle_proc_bind())
    return {0: "false", 1: "true", 2: "primary", 3: "close", 4: "spread"}.get(v, str(v))


def interleave(a: np.ndarray, nodes: int) -> int:
    """Spread the pages of array a over NUMA nodes 0 .. nodes-1 (0 or an errno)."""
    return int(_load().oracle_interleave(_ptr(a), a.nbytes, int(nodes)))


def split_base(context_len: int, num_query_tokens: int = 1, window: int = 0) -> int:
    """First token of a sequence's split range (0 without a window)."""
    return int(_load().oracle_split_base(int(context_len), int(num_query_tokens), int(window)))


def num_splits(context_len: int, split_tokens: int, num_query_tokens: int = 1,
               window: int = 0) -> int:
    """max(1, ceil((L - base) / T)) with base = split_base(L, Q, W)."""
    base = split_base(context_len, num_query_tokens, window)
    return int(_load().oracle_num_splits(int(context_len) - base, int(split_tokens)))


def kv_write(k, v, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None):
    """Write new K/V rows into the pool in place (k_cache etc. are modified)."""
    k, v = _c(k), _c(v)
    slot_mapping = _c(slot_mapping, np.int64)
    for a in (k_cache, v_cache, k_scale, v_scale):
        if a is not None and not a.flags.c_contiguous:
            raise ValueError("cache arrays must be C-contiguous")
    num_blocks, num_kv_heads, bs, head_dim = k_cache.shape
    assert bs == BLOCK_SIZE and k.shape[1:] == (num_kv_heads, head_dim)
    rc = _load().oracle_kv_write(_ptr(k), _ptr(v), _code(k), _ptr(slot_mapping), k.shape[0],
                                 num_kv_heads, head_dim, _ptr(k_cache), _ptr(v_cache),
                                 _ptr(k_scale), _ptr(v_scale), num_blocks, _code(k_cache))
    if rc != 0:
        raise ValueError("oracle_kv_write rejected its arguments")


def _decode_common(q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale, window,
                   query_start=None):
    q, k_cache, v_cache = _c(q), _c(k_cache), _c(v_cache)
    k_scale, v_scale = _c(k_scale, np.float32), _c(v_scale, np.float32)
    block_tables, context_lens = _c(block_tables, np.int32), _c(context_lens, np.int32)
    num_seqs = len(context_lens)
    if query_start is not None:
        query_start = _c(query_start, np.int32)
        assert q.ndim == 3 and query_start.shape == (num_seqs + 1,) and query_start[0] == 0
        assert (np.diff(query_start) >= 0).all() and query_start[-1] == q.shape[0]
        counts = np.diff(query_start)
    else:
        if q.ndim == 3:
            q = q.reshape(q.shape[0], 1, q.shape[1], q.shape[2])
        assert q.shape[0] == num_seqs and q.shape[1] >= 1
        counts = np.full(num_seqs, q.shape[1])
    num_q_heads, head_dim = q.shape[-2], q.shape[-1]
    num_blocks, num_kv_heads, bs, hd = k_cache.shape
    assert bs == BLOCK_SIZE and hd == head_dim and num_q_heads % num_kv_heads == 0
    assert window >= 0
    if _code(k_cache) in (I8, FP8):
        assert k_scale is not None and v_scale is not None
    # Every block the definition will read must exist in the pool (blocks
    # before a sliding window's reach are never read).
    for s in range(num_seqs):
        L = int(context_lens[s])
        nb = -(-L // BLOCK_SIZE)
        assert nb <= block_tables.shape[1]
        ids = block_tables[s, split_base(L, int(counts[s]), window) // BLOCK_SIZE:nb]
        assert (ids >= 0).all() and (ids < num_blocks).all()
    return q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, query_start, counts


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale=None, v_scale=None,
           rows=None, window=0, query_start=None):
    """Decode attention by definition, in fp64.

    q is [B][Hq][D] (one query token per sequence) or [B][Q][Hq][D], or with
    query_start ([B + 1] offsets) the packed [N][Hq][D]; window is the sliding
    window in tokens (0: none). rows: optional (seq_ids, head_ids) pair, or
    (seq_ids, query_token_ids, head_ids) triple, of equal-length int arrays
    (query_token_ids count within the sequence); the result is then
    [n_rows][head_dim]. Without rows it has q's shape.
    """
    shape = np.shape(q)
    (q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, query_start,
     counts) = _decode_common(q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                              window, query_start)
    num_seqs = len(context_lens)
    num_q_heads, head_dim = q.shape[-2], q.shape[-1]
    nqt = 0 if query_start is not None else q.shape[1]
    if rows is None:
        seq_ids = np.repeat(np.arange(num_seqs, dtype=np.int32), counts * num_q_heads)
        tok_ids = np.concatenate([np.repeat(np.arange(c, dtype=np.int32), num_q_heads)
                                  for c in counts] or [np.zeros(0, np.int32)])
        head_ids = np.tile(np.arange(num_q_heads, dtype=np.int32), int(counts.sum()))
    elif len(rows) == 2:
        seq_ids, head_ids = _c(rows[0], np.int32), _c(rows[1], np.int32)
        tok_ids = np.zeros_like(seq_ids)
    else:
        seq_ids, tok_ids, head_ids = (_c(r, np.int32) for r in rows)
    out = np.zeros((len(seq_ids), head_dim), dtype=np.float64)
    _load().oracle_decode(_ptr(q), _code(q), num_q_heads, nqt, int(window), _ptr(query_start),
                          _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                          _code(k_cache),
                          k_cache.shape[1], head_dim, _ptr(block_tables), block_tables.shape[1],
                          _ptr(context_lens), float(scale), _ptr(seq_ids), _ptr(tok_ids),
                          _ptr(head_ids), len(seq_ids), _ptr(out))
    if rows is None:
        out = out.reshape(shape[:-1] + (head_dim,))
    return out


def decode_split(q, k_cache, v_cache, block_tables, context_lens, scale, split_tokens,
                 max_splits=None, k_scale=None, v_scale=None, window=0, query_start=None):
    """Split-K partials (m, l, acc) in fp64; acc is not divided by l. Shapes:
    m, l [B](+[Q])[Hq][S], acc [B](+[Q])[Hq][S][D], following q ([N][Hq][S]
    and [N][Hq][S][D] with query_start)."""
    lead = np.shape(q)[:-1]
    (q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, query_start,
     counts) = _decode_common(q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                              window, query_start)
    num_seqs = len(context_lens)
    num_q_heads, head_dim = q.shape[-2], q.shape[-1]
    nqt = 0 if query_start is not None else q.shape[1]
    if max_splits is None:
        max_splits = max([num_splits(int(L), split_tokens, int(c), window)
                          for L, c in zip(context_lens, counts)] or [1])
    m = np.zeros(lead + (max_splits,), dtype=np.float64)
    l = np.zeros_like(m)
    acc = np.zeros(lead + (max_splits, head_dim), dtype=np.float64)
    _load().oracle_decode_split(_ptr(q), _code(q), num_seqs, num_q_heads, nqt, int(window),
                                _ptr(query_start), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                _ptr(v_scale),
                                _code(k_cache), k_cache.shape[1], head_dim, _ptr(block_tables),
                                block_tables.shape[1], _ptr(context_lens), float(scale),
                                int(split_tokens), int(max_splits), _ptr(m), _ptr(l), _ptr(acc))
    return m, l, acc


def merge(m, l, acc):
    """Reduce split partials to the attention output, in fp64."""
    m, l, acc = _c(m, np.float64), _c(l, np.float64), _c(acc, np.float64)
    max_splits, head_dim = acc.shape[-2], acc.shape[-1]
    lead = m.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    out = np.zeros(lead + (head_dim,), dtype=np.float64)
    _load().oracle_merge(_ptr(m), _ptr(l), _ptr(acc), rows, max_splits, head_dim, _ptr(out))
    return out
