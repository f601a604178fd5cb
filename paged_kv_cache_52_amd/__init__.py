"""Paged-KV decode attention for MI355X: Python binding of libpagedattn.

Every function here only checks and marshals arguments (torch tensors ->
device pointers, torch's current stream) and calls the C ABI declared in
include/pagedattn.h; all arithmetic runs in the library's HIP kernels. The
library must be built (``__graft_entry__.build()``); there is no fallback.

Tensor layouts (block size 16):

* q, out          [num_seqs][num_q_heads][head_dim] (one query token per
                  sequence) or [num_seqs][Q][num_q_heads][head_dim] (Q query
                  tokens: the sequence's last Q positions), fp32 or bf16; with
                  ``query_start`` ([num_seqs + 1] int32 offsets, a batch whose
                  sequences have their own query counts, e.g. decodes mixed
                  with prefill chunks) the packed [N][num_q_heads][head_dim],
                  sequence s owning rows query_start[s] .. query_start[s+1]-1
* k_cache, v_cache [num_blocks][num_kv_heads][16][head_dim], fp32/bf16/int8/
                  float8_e4m3fn (OCP FP8 E4M3)
* k_scale, v_scale [num_blocks][num_kv_heads][16] fp32 (int8 and fp8 caches only)
* block_tables    [num_seqs][max_blocks_per_seq] int32
* context_lens    [num_seqs] int32
* slot_mapping    [num_tokens] int64 (negative = skip)

``sliding_window`` (tokens, 0 = none) limits each query token to its W most
recent positions.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _lib

BLOCK_SIZE = 16
MAX_QUERY_TOKENS = 4096
_INT32_MAX = 2**31 - 1
PA_F32, PA_BF16, PA_I8, PA_FP8 = 0, 1, 2, 3
_DTYPE_CODES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.int8: PA_I8,
                torch.float8_e4m3fn: PA_FP8}
_QUANTISED = (torch.int8, torch.float8_e4m3fn)  # caches that carry per-token scales


class PagedAttnError(RuntimeError):
    pass


def _check(status: int) -> None:
    if status != 0:
        msg = _lib.load().pa_strerror(status).decode()
        raise PagedAttnError(f"libpagedattn status {status}: {msg}")


def _code(t: torch.Tensor) -> int:
    try:
        return _DTYPE_CODES[t.dtype]
    except KeyError:
        raise PagedAttnError(f"unsupported dtype {t.dtype}") from None


def _dev(t: Optional[torch.Tensor], name: str, dtype=None) -> int:
    if t is None:
        return None
    if not t.is_cuda:
        raise PagedAttnError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise PagedAttnError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise PagedAttnError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def num_splits(context_len: int, split_tokens: int) -> int:
    """max(1, ceil(context_len / split_tokens))."""
    return int(_lib.load().pa_num_splits(int(context_len), int(split_tokens)))


def max_splits(max_context_len: int, split_tokens: int, num_query_tokens: int = 1,
               sliding_window: int = 0) -> int:
    """Splits of the longest split range under the bound (the partials' stride)."""
    return int(_lib.load().pa_max_splits(int(max_context_len), int(num_query_tokens),
                                         int(sliding_window), int(split_tokens)))


def default_split_tokens(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                         cache_dtype, max_context_len: int, num_query_tokens: int = 1,
                         sliding_window: int = 0) -> int:
    """Split size the library picks for split_tokens=None (cache_dtype: a torch
    dtype or a PA_* code)."""
    code = _DTYPE_CODES.get(cache_dtype, cache_dtype)
    if not isinstance(code, int):
        raise PagedAttnError(f"unsupported cache dtype {cache_dtype}")
    return int(_lib.load().pa_default_split_tokens(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                   code, max_context_len, num_query_tokens,
                                                   sliding_window))


def sched_bytes(num_seqs: int, max_splits: int, total_query_tokens: Optional[int] = None,
                q_heads_per_kv: int = 1) -> int:
    """Plan scratch bytes; pass total_query_tokens (and g) for packed queries."""
    if total_query_tokens is None:
        return int(_lib.load().pa_sched_bytes(num_seqs, max_splits))
    return int(_lib.load().pa_sched_bytes_packed(num_seqs, max_splits, int(total_query_tokens),
                                                 int(q_heads_per_kv)))


def workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, max_splits: int,
                    num_query_tokens: int = 1, num_kv_heads: Optional[int] = None,
                    packed: bool = False) -> int:
    """paged_attn_decode workspace; with packed=True num_query_tokens is the
    total N and num_kv_heads is required."""
    if packed:
        return int(_lib.load().pa_workspace_bytes_packed(num_seqs, num_query_tokens, num_q_heads,
                                                         num_kv_heads, head_dim, max_splits))
    return int(_lib.load().pa_workspace_bytes(num_seqs, num_query_tokens, num_q_heads, head_dim,
                                              max_splits))


def _query_bound(num_query_tokens: int, packed: bool) -> int:
    """Largest query count of one sequence: Q, or min(N, MAX_QUERY_TOKENS)."""
    return max(1, min(num_query_tokens, MAX_QUERY_TOKENS)) if packed else num_query_tokens


def paged_kv_write(k, v, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None) -> None:
    """Write one step's new K/V rows into the pool at their slots (in place)."""
    T, Hkv, D = k.shape
    NB = k_cache.shape[0]
    if k_cache.shape != (NB, Hkv, BLOCK_SIZE, D) or v_cache.shape != k_cache.shape:
        raise PagedAttnError("cache shape must be [num_blocks][num_kv_heads][16][head_dim]")
    if v.shape != k.shape or slot_mapping.shape != (T,):
        raise PagedAttnError("k, v must be [T][Hkv][D] and slot_mapping [T]")
    if k_cache.dtype in _QUANTISED and (k_scale is None or v_scale is None):
        raise PagedAttnError("an int8 or fp8 cache needs k_scale and v_scale")
    for sc in (k_scale, v_scale):
        if sc is not None and sc.shape != (NB, Hkv, BLOCK_SIZE):
            raise PagedAttnError("scales must be [num_blocks][num_kv_heads][16]")
    lib = _lib.load()
    _check(lib.paged_kv_write(
        _dev(k, "k"), _dev(v, "v", k.dtype), _code(k), _dev(slot_mapping, "slot_mapping",
                                                            torch.int64),
        T, Hkv, D, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache", k_cache.dtype),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32), NB,
        _code(k_cache), _stream(k.device)))


@dataclasses.dataclass
class Plan:
    """Split list of one decode step (see paged_attn_plan); it depends only on
    the lengths, bounds, query-token count and window, so every layer of the
    step with the same window can reuse it."""
    sched: torch.Tensor         # int32 scratch, pa_sched_bytes(num_seqs, max_splits)
    context_lens: torch.Tensor  # [B] int32 the plan was made from
    max_blocks_per_seq: int
    max_context_len: int
    split_tokens: int
    max_splits: int
    num_query_tokens: int = 1   # per sequence, or the packed total N
    sliding_window: int = 0
    group_members: int = 1
    query_start: Optional[torch.Tensor] = None  # [B+1] int32 with packed queries


@dataclasses.dataclass
class Partials:
    """Split-K partials of one decode call (see paged_attn_decode_partial)."""
    m: torch.Tensor             # [B][Q][Hq][max_splits] fp32 (packed: [N][Hq][max_splits])
    l: torch.Tensor             # same shape as m
    acc: torch.Tensor           # m's shape + [D] fp32, not divided by l
    context_lens: torch.Tensor  # [B] int32
    split_tokens: int
    sliding_window: int = 0
    query_start: Optional[torch.Tensor] = None  # [B+1] int32 with packed queries
    # Bounds of the decode call that wrote the partials: the reduce clamps each
    # context length to min(max_context_len, 16 * max_blocks_per_seq) as the
    # split kernel did (None: no bound beyond the int32 range).
    max_context_len: Optional[int] = None
    max_blocks_per_seq: Optional[int] = None

    @property
    def max_splits(self) -> int:
        return self.m.shape[-1]

    @property
    def num_query_tokens(self) -> int:
        """Per sequence, or the packed total N."""
        return self.m.shape[0] if self.query_start is not None else self.m.shape[1]


def _q_shape(q, query_start=None, context_lens=None):
    """(B, Q, Hq, D) of a [B][Hq][D] or [B][Q][Hq][D] query tensor, or
    (B, N, Hq, D) of a packed [N][Hq][D] one (B from context_lens)."""
    if query_start is not None:
        if q.dim() != 3:
            raise PagedAttnError("packed q must be [N][Hq][D]")
        B = context_lens.shape[0]
        if query_start.shape != (B + 1,):
            raise PagedAttnError("query_start must be [num_seqs + 1]")
        return B, q.shape[0], q.shape[1], q.shape[2]
    if q.dim() == 3:
        return q.shape[0], 1, q.shape[1], q.shape[2]
    if q.dim() == 4:
        B, Q, Hq, D = q.shape
        if not 1 <= Q <= MAX_QUERY_TOKENS:
            raise PagedAttnError(f"1..{MAX_QUERY_TOKENS} query tokens per sequence, got {Q}")
        return B, Q, Hq, D
    raise PagedAttnError("q must be [B][Hq][D] or [B][Q][Hq][D]")


def _max_len(context_lens, max_context_len):
    if max_context_len is None:
        return int(context_lens.max().item()) if context_lens.numel() else 0
    return int(max_context_len)


def _plan_sizes(context_lens, max_blocks_per_seq, max_context_len, split_tokens, sched, Q, W,
                cache=None, packed_g=None):
    """cache = (num_q_heads, num_kv_heads, head_dim, cache dtype) picks the
    default split size when split_tokens is None; without it split_tokens is
    required. packed_g = g for packed queries (Q is then the total N; the
    default split size is taken for the mean count per sequence)."""
    B = context_lens.shape[0]
    mcl = _max_len(context_lens, max_context_len)
    packed = packed_g is not None
    Qb = _query_bound(Q, packed)
    if split_tokens:
        T = int(split_tokens)
    elif cache is not None:
        Qd = max(1, min(MAX_QUERY_TOKENS, -(-Q // max(B, 1)))) if packed else Q
        T = default_split_tokens(B, cache[0], cache[1], cache[2], cache[3], mcl, Qd, W)
    else:
        raise PagedAttnError("paged_attn_plan needs split_tokens (see default_split_tokens)")
    S = max(1, max_splits(min(mcl, int(max_blocks_per_seq) * BLOCK_SIZE), T, Qb, W))
    need = sched_bytes(B, S, Q if packed else None, packed_g or 1)
    if sched is None or sched.numel() * sched.element_size() < need:
        sched = torch.empty(max(need, 16) // 4, dtype=torch.int32, device=context_lens.device)
    return B, mcl, T, S, sched


def paged_attn_plan(context_lens, max_blocks_per_seq: int, *, max_context_len=None,
                    split_tokens=None, num_query_tokens: int = 1, sliding_window: int = 0,
                    block_tables=None, group_members: int = 1, query_start=None,
                    q_heads_per_kv: Optional[int] = None,
                    sched: Optional[torch.Tensor] = None, _cache=None) -> Plan:
    """Plan kernel: list every split of the batch (on the device, from
    context_lens) for the split kernel. split_tokens is required. With
    group_members > 1 (and block_tables), splits of consecutive sequences that
    start on the same physical block become shared work items. With
    query_start (packed queries) num_query_tokens is the total N and
    q_heads_per_kv (g = Hq / Hkv) is required."""
    Q, W = int(num_query_tokens), int(sliding_window)
    g = None
    if query_start is not None:
        if q_heads_per_kv is None:
            raise PagedAttnError("a packed plan needs q_heads_per_kv")
        g = int(q_heads_per_kv)
    B, mcl, T, S, sched = _plan_sizes(context_lens, max_blocks_per_seq, max_context_len,
                                      split_tokens, sched, Q, W, _cache, g)
    _check(_lib.load().paged_attn_plan(_dev(context_lens, "context_lens", torch.int32),
                                       _dev(query_start, "query_start", torch.int32),
                                       _dev(block_tables, "block_tables", torch.int32), B,
                                       max_blocks_per_seq, mcl, Q, g or 1, W, T,
                                       int(group_members), _dev(sched, "sched", torch.int32),
                                       _stream(context_lens.device)))
    return Plan(sched, context_lens, max_blocks_per_seq, mcl, T, S, Q, W, int(group_members),
                query_start)


def paged_decode_prepare(k, v, slot_mapping, k_cache, v_cache, context_lens,
                         max_blocks_per_seq: int, k_scale=None, v_scale=None, *,
                         max_context_len=None, split_tokens=None, num_query_tokens: int = 1,
                         sliding_window: int = 0, num_q_heads: Optional[int] = None,
                         block_tables=None, group_members: int = 1, query_start=None,
                         sched: Optional[torch.Tensor] = None) -> Plan:
    """paged_kv_write + paged_attn_plan in one launch; returns the plan.
    Without split_tokens the default is taken for num_q_heads query heads.
    With query_start (packed queries) num_query_tokens is the total N and
    num_q_heads is required."""
    T_tok, Hkv, D = k.shape
    NB = k_cache.shape[0]
    if k_cache.shape != (NB, Hkv, BLOCK_SIZE, D) or v_cache.shape != k_cache.shape:
        raise PagedAttnError("cache shape must be [num_blocks][num_kv_heads][16][head_dim]")
    if v.shape != k.shape or slot_mapping.shape != (T_tok,):
        raise PagedAttnError("k, v must be [T][Hkv][D] and slot_mapping [T]")
    if k_cache.dtype in _QUANTISED and (k_scale is None or v_scale is None):
        raise PagedAttnError("an int8 or fp8 cache needs k_scale and v_scale")
    Q, W = int(num_query_tokens), int(sliding_window)
    cache = None if num_q_heads is None else (int(num_q_heads), Hkv, D, k_cache.dtype)
    g = None
    if query_start is not None:
        if num_q_heads is None:
            raise PagedAttnError("a packed plan needs num_q_heads")
        g = int(num_q_heads) // Hkv
    B, mcl, T, S, sched = _plan_sizes(context_lens, max_blocks_per_seq, max_context_len,
                                      split_tokens, sched, Q, W, cache, g)
    _check(_lib.load().paged_decode_prepare(
        _dev(k, "k"), _dev(v, "v", k.dtype), _code(k),
        _dev(slot_mapping, "slot_mapping", torch.int64), T_tok, Hkv, D, _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache", k_cache.dtype), _dev(k_scale, "k_scale", torch.float32),
        _dev(v_scale, "v_scale", torch.float32), NB, _code(k_cache),
        _dev(context_lens, "context_lens", torch.int32),
        _dev(query_start, "query_start", torch.int32),
        _dev(block_tables, "block_tables", torch.int32), B, max_blocks_per_seq, mcl, Q, g or 1,
        W, T, int(group_members), _dev(sched, "sched", torch.int32), _stream(k.device)))
    return Plan(sched, context_lens, max_blocks_per_seq, mcl, T, S, Q, W, int(group_members),
                query_start)


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                 query_start=None):
    B, Q, Hq, D = _q_shape(q, query_start, context_lens)
    NB, Hkv, bs, Dk = k_cache.shape
    if bs != BLOCK_SIZE or Dk != D or v_cache.shape != k_cache.shape:
        raise PagedAttnError("cache shape must be [num_blocks][num_kv_heads][16][head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise PagedAttnError("block_tables must be [B][max_blocks], context_lens [B]")
    if k_cache.dtype in _QUANTISED and (k_scale is None or v_scale is None):
        raise PagedAttnError("an int8 or fp8 cache needs k_scale and v_scale")
    return (_dev(q, "q"), _code(q), B, Q, Hq, D, _dev(k_cache, "k_cache"),
            _dev(v_cache, "v_cache", k_cache.dtype), _dev(k_scale, "k_scale", torch.float32),
            _dev(v_scale, "v_scale", torch.float32), _code(k_cache), NB, Hkv,
            _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
            _dev(context_lens, "context_lens", torch.int32),
            _dev(query_start, "query_start", torch.int32))


def paged_attn_decode_partial(q, k_cache, v_cache, block_tables, context_lens, scale,
                              k_scale=None, v_scale=None, *, max_context_len=None,
                              split_tokens=None, sliding_window: int = 0,
                              plan: Optional[Plan] = None, query_start=None,
                              partials: Optional[Partials] = None) -> Partials:
    """Split kernel: returns the per-split (m, l, acc). Without `plan`, the
    plan kernel runs first. With query_start, q is the packed [N][Hq][D]."""
    lib = _lib.load()
    B, Q, Hq, D = _q_shape(q, query_start, context_lens)
    Hkv = k_cache.shape[1]
    W = int(sliding_window)
    mb = block_tables.shape[1]
    packed = query_start is not None
    if plan is None:
        plan = paged_attn_plan(context_lens, mb, max_context_len=max_context_len,
                               split_tokens=split_tokens, num_query_tokens=Q, sliding_window=W,
                               query_start=query_start, q_heads_per_kv=Hq // Hkv,
                               _cache=(Hq, Hkv, D, k_cache.dtype))
    elif (plan.max_blocks_per_seq != mb or plan.context_lens is not context_lens or
          (split_tokens and int(split_tokens) != plan.split_tokens) or
          (max_context_len is not None and int(max_context_len) != plan.max_context_len) or
          plan.num_query_tokens != Q or plan.sliding_window != W or
          plan.query_start is not query_start):
        raise PagedAttnError("plan was made for other arguments")
    if plan.group_members > 1:
        # Group entries put each member's rows in one wave: all Q*g rows of a
        # KV head must fit one row group of the engine that runs.
        mfma = q.dtype == torch.bfloat16 and D == 128 and k_cache.dtype != torch.float32
        if Q * (Hq // Hkv) > (16 if mfma else 8):
            raise PagedAttnError("a plan with group entries needs num_query_tokens * "
                                 f"(Hq / Hkv) <= {16 if mfma else 8} here")
    T, S = plan.split_tokens, plan.max_splits
    lead = (Q, Hq) if packed else (B, Q, Hq)
    if partials is None:
        partials = Partials(m=torch.empty(lead + (S,), dtype=torch.float32, device=q.device),
                            l=torch.empty(lead + (S,), dtype=torch.float32, device=q.device),
                            acc=torch.empty(lead + (S, D), dtype=torch.float32,
                                            device=q.device),
                            context_lens=context_lens, split_tokens=T, sliding_window=W,
                            query_start=query_start)
    else:
        if tuple(partials.m.shape[:-1]) != lead:
            raise PagedAttnError("partials must be [B][Q][Hq][max_splits](...), or "
                                 "[N][Hq][max_splits](...) with packed queries")
        partials.context_lens, partials.split_tokens = context_lens, T
        partials.sliding_window, partials.query_start = W, query_start
    partials.max_context_len, partials.max_blocks_per_seq = plan.max_context_len, mb
    args = _decode_args(q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                        query_start)
    _check(lib.paged_attn_decode_partial(
        *args, plan.max_context_len, W, float(scale), T, partials.max_splits,
        _dev(partials.m, "m", torch.float32), _dev(partials.l, "l", torch.float32),
        _dev(partials.acc, "acc", torch.float32), _dev(plan.sched, "sched", torch.int32),
        _stream(q.device)))
    return partials


def paged_attn_reduce(partials: Partials, out: torch.Tensor) -> torch.Tensor:
    """Reduce kernel: merge the partials into out ([B][Hq][D] or [B][Q][Hq][D],
    or [N][Hq][D] with packed queries; fp32 or bf16)."""
    lib = _lib.load()
    D = partials.acc.shape[-1]
    if partials.query_start is not None:
        N, Hq, S = partials.m.shape
        B, Q = partials.context_lens.shape[0], N
        if out.shape != (N, Hq, D):
            raise PagedAttnError("out must be [N][Hq][D] with packed queries")
    else:
        B, Q, Hq, S = partials.m.shape
        if out.shape not in ((B, Q, Hq, D),) + (((B, Hq, D),) if Q == 1 else ()):
            raise PagedAttnError("out must be [B][Hq][D] or [B][Q][Hq][D]")
    mcl = _INT32_MAX if partials.max_context_len is None else int(partials.max_context_len)
    mb = (_INT32_MAX // BLOCK_SIZE if partials.max_blocks_per_seq is None
          else int(partials.max_blocks_per_seq))
    _check(lib.paged_attn_reduce(
        _dev(partials.m, "m", torch.float32), _dev(partials.l, "l", torch.float32),
        _dev(partials.acc, "acc", torch.float32),
        _dev(partials.context_lens, "context_lens", torch.int32),
        _dev(partials.query_start, "query_start", torch.int32), B, Q, Hq, D, mb, mcl,
        partials.sliding_window, partials.split_tokens, S, _dev(out, "out"), _code(out),
        _stream(out.device)))
    return out


def paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out=None,
                      k_scale=None, v_scale=None, *, max_context_len=None, split_tokens=None,
                      sliding_window: int = 0, query_start=None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Whole decode step: split kernel then reduce kernel, out in q's dtype and
    shape (q packed [N][Hq][D] with query_start)."""
    lib = _lib.load()
    B, Q, Hq, D = _q_shape(q, query_start, context_lens)
    W = int(sliding_window)
    packed = query_start is not None
    Hkv = k_cache.shape[1]
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise PagedAttnError("out must match q's shape and dtype")
    mcl = _max_len(context_lens, max_context_len)
    mb = block_tables.shape[1]
    Qb = _query_bound(Q, packed)
    Qd = max(1, min(MAX_QUERY_TOKENS, -(-Q // max(B, 1)))) if packed else Q
    T = (int(split_tokens) if split_tokens else
         default_split_tokens(B, Hq, Hkv, D, k_cache.dtype, mcl, Qd, W))
    S = max(1, max_splits(min(mcl, mb * BLOCK_SIZE), T, Qb, W))
    need = workspace_bytes(B, Hq, D, S, Q, Hkv, packed)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    args = _decode_args(q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                        query_start)
    _check(lib.paged_attn_decode(*args, mcl, W, float(scale), T, _dev(out, "out"),
                                 _dev(workspace, "workspace"), workspace.numel(),
                                 _stream(q.device)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # PA_NOALLOC_SCRATCH_BYTES


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                              k_scale=None, v_scale=None, *, max_context_len=None,
                              split_tokens=None, sliding_window: int = 0,
                              query_start=None) -> torch.Tensor:
    """paged_attn_decode with no workspace: the library's fixed per-GPU
    scratch holds the plan and partials (calls on one GPU must not overlap).
    out (q's shape and dtype) is required; nothing is allocated. A call that
    needs more than NOALLOC_SCRATCH_BYTES raises."""
    lib = _lib.load()
    B, Q, Hq, D = _q_shape(q, query_start, context_lens)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise PagedAttnError("out must match q's shape and dtype")
    args = _decode_args(q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                        query_start)
    _check(lib.paged_attn_decode_noalloc(*args, _max_len(context_lens, max_context_len),
                                         int(sliding_window), float(scale),
                                         int(split_tokens or 0), _dev(out, "out"),
                                         _stream(q.device)))
    return out


def hbm_read_probe(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Read all of `buf` once (measurement aid: practical HBM read bandwidth)."""
    if buf.numel() * buf.element_size() % 16:
        raise PagedAttnError("probe buffer size must be a multiple of 16 bytes")
    _check(_lib.load().pa_hbm_read_probe(
        _dev(buf, "buf"), buf.numel() * buf.element_size(), _dev(sink, "sink", torch.int32),
        sink.numel(), _stream(buf.device)))


__all__ = [
    "BLOCK_SIZE", "MAX_QUERY_TOKENS", "PagedAttnError", "Plan", "Partials", "num_splits",
    "max_splits", "default_split_tokens", "sched_bytes", "workspace_bytes", "paged_kv_write",
    "paged_attn_plan", "paged_decode_prepare", "paged_attn_decode_partial", "paged_attn_reduce",
    "paged_attn_decode", "paged_attn_decode_noalloc", "NOALLOC_SCRATCH_BYTES", "hbm_read_probe",
]
