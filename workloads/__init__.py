"""Seeded synthetic decode batches for paged-KV attention.

This module only draws inputs: sequence lengths, block tables, pool contents,
queries and the new token of the decode step. It holds none of the attention
arithmetic, and both the HIP library's tests and the CPU oracle's tests take
their inputs from here.

Recipe (every draw is seeded):

* Sequence-level structure (context lengths, block-table permutations, the
  shared-prefix grouping) comes from ``numpy.random.default_rng(seed)``
  (PCG64), so it is the same on every machine and device.
* Tensor values (q, the pool, the new token's K/V) are N(0, 1) float32 draws
  from ``torch.Generator(device).manual_seed(seed)`` on the requested device,
  rounded to nearest-even bf16 where the workload is bf16. CPU and GPU
  generators give different (each reproducible) value streams.
* The pool has num_blocks = max(ceil(1.1 * sum(L) / 16), blocks needed + 1)
  blocks (the tiny workload fixes 64). The blocks used by the sequences are a
  seeded random permutation of the pool, so logically adjacent blocks are
  physically scattered; one more block is the "pad" block. Table entries past a
  sequence's last block point at the pad block.
* The decode step's new token of sequence s sits at position L_s - 1; its slot
  is ``slot_mapping[s]`` and its K/V rows are ``new_k[s]``/``new_v[s]``. With
  Q = ``query_tokens`` > 1 (multi-token decode) the step's Q new tokens are
  positions L_s - Q .. L_s - 1, q is [B][Q][Hq][D] and slot_mapping, new_k,
  new_v hold B*Q rows, sequence-major.
* With a sliding window W > 0 only the blocks from the one holding token
  max(0, L_s - Q - W + 1) on are allocated (as a cache that frees blocks
  behind the window would); earlier table entries are -1.
* ``poison=True`` fills every pool slot that no sequence attends (tail slots of
  last blocks, tokens before a window's reach, unused blocks, the pad block)
  with NaN (INT8 pools: NaN scales).

Workloads (block size 16 throughout):

* ``tiny_fp32``: 4 seqs, 8 q / 2 KV heads, head_dim 64, fp32, pool 64 blocks,
  L uniform in [1, 128].
* ``llama8b_bf16``: 64 seqs, 32 q / 8 KV heads, head_dim 128, bf16,
  L uniform in [512, 4096].
* ``long_bf16``: 8 seqs, 32 q / 8 KV heads, head_dim 128, bf16,
  L uniform in [32768, 131072], splits of 512 tokens.
* ``int8_kv``: 128 seqs, 32 q / 8 KV heads, head_dim 128, INT8 cache with
  per-token fp32 scales, bf16 q/out, L uniform in [1024, 8192]. The pool is
  filled by writing bf16 N(0, 1) K/V for every context token through the KV
  write (``fill_k``/``fill_v``/``fill_slots``).
* ``shared_prefix_bf16``: 32 prompts x 8 samples (256 seqs), 64 q / 4 KV heads,
  head_dim 128, bf16. Each group's 2000-token prefix (125 full blocks) is
  mapped to the same physical blocks; each sample's private suffix length is
  clip(rint(exp(N(ln 300, 1))), 1, 16384) and L = 2000 + suffix + 1.
* ``fp8_kv``: the INT8 batch's shape with an FP8 (OCP E4M3) cache, per-token
  fp32 scales, filled through the KV write.
* ``mtp4_llama8b_bf16``: the 8B-shaped batch with 4 query tokens per sequence
  (3 draft tokens and the target token of MTP speculative decoding).
* ``swa4k_bf16``: 64 seqs, 32 q / 8 KV heads, head_dim 128, bf16, L uniform in
  [8192, 65536], sliding window of 4096 tokens.
* ``prefill512_bf16``: chunked prefill, 8 seqs, 32 q / 8 KV heads, head_dim 128,
  bf16, L uniform in [2048, 8192] including a 512-token chunk whose tokens are
  the step's query tokens (written through the KV write first).
* ``mixed_llama8b_bf16``: one call mixing decode and chunked prefill: the
  8B-shaped batch's 64 decode sequences (one query token, L uniform in
  [512, 4096]) followed by 2 sequences each carrying a 512-token prefill chunk
  (L uniform in [2048, 8192], chunk included).

Per-sequence query counts (``query_counts``, or a workload with prefill
chunks): sequence s has Q_s query tokens, its last Q_s positions; q is packed
as [N][Hq][D] with N = sum Q_s, sequence s owning rows query_start[s] ..
query_start[s+1]-1 (``Batch.query_start``, [B+1] int32), and slot_mapping,
new_k, new_v hold the same N rows.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

BLOCK_SIZE = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                 # q / out / source K,V: "fp32" | "bf16"
    cache_dtype: str           # "fp32" | "bf16" | "int8" | "fp8" (OCP E4M3)
    ctx_lo: int = 0
    ctx_hi: int = 0
    fixed_pool_blocks: int = 0  # 0: 1.1x the attended tokens
    split_tokens: int = 512
    query_tokens: int = 1      # query tokens per sequence (mtp_k + 1)
    window: int = 0            # sliding window in tokens, 0 = none
    # mixed batches: chunk_seqs more sequences with chunk_tokens query tokens
    chunk_seqs: int = 0
    chunk_tokens: int = 0
    chunk_lo: int = 0
    chunk_hi: int = 0
    # shared-prefix workloads
    groups: int = 0
    samples: int = 0
    prefix_len: int = 0
    suffix_median: float = 0.0
    suffix_sigma: float = 0.0
    suffix_max: int = 0


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 4, 8, 2, 64, "fp32", "fp32", 1, 128, fixed_pool_blocks=64),
        Workload("llama8b_bf16", 64, 32, 8, 128, "bf16", "bf16", 512, 4096),
        Workload("long_bf16", 8, 32, 8, 128, "bf16", "bf16", 32768, 131072),
        Workload("int8_kv", 128, 32, 8, 128, "bf16", "int8", 1024, 8192),
        Workload("shared_prefix_bf16", 256, 64, 4, 128, "bf16", "bf16", groups=32, samples=8,
                 prefix_len=2000, suffix_median=300.0, suffix_sigma=1.0, suffix_max=16384),
        Workload("fp8_kv", 128, 32, 8, 128, "bf16", "fp8", 1024, 8192),
        Workload("mtp4_llama8b_bf16", 64, 32, 8, 128, "bf16", "bf16", 512, 4096,
                 query_tokens=4),
        Workload("swa4k_bf16", 64, 32, 8, 128, "bf16", "bf16", 8192, 65536, window=4096),
        Workload("prefill512_bf16", 8, 32, 8, 128, "bf16", "bf16", 2048, 8192,
                 query_tokens=512),
        Workload("mixed_llama8b_bf16", 64, 32, 8, 128, "bf16", "bf16", 512, 4096,
                 chunk_seqs=2, chunk_tokens=512, chunk_lo=2048, chunk_hi=8192),
    ]
}

TORCH_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16, "int8": torch.int8,
                "fp8": torch.float8_e4m3fn}
QUANTISED = ("int8", "fp8")  # caches filled through the quantising KV write


@dataclasses.dataclass
class Batch:
    workload: Workload
    q: torch.Tensor               # [B][Hq][D], or [B][Q][Hq][D] with Q query tokens, or
                                  # [N][Hq][D] with per-sequence counts (query_start)
    k_cache: torch.Tensor         # [NB][Hkv][16][D]
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]  # [NB][Hkv][16] float32 (INT8 / FP8 only)
    v_scale: Optional[torch.Tensor]
    block_tables: torch.Tensor    # [B][max_blocks] int32
    context_lens: torch.Tensor    # [B] int32
    slot_mapping: torch.Tensor    # [B*Q] int64, slots of positions L-Q .. L-1
    new_k: torch.Tensor           # [B*Q][Hkv][D]
    new_v: torch.Tensor
    scale: float
    max_context_len: int
    pad_block: int
    fill_k: Optional[torch.Tensor] = None      # INT8: every context token's K/V
    fill_v: Optional[torch.Tensor] = None
    fill_slots: Optional[torch.Tensor] = None
    num_blocks_shared: int = 0    # physical blocks referenced (shared counted once)
    num_blocks_logical: int = 0   # sum over seqs of ceil(L/16)
    query_tokens: int = 1         # Q, or with query_start the largest Q_s
    window: int = 0
    query_start: Optional[torch.Tensor] = None  # [B+1] int32 (per-sequence counts)

    @property
    def num_seqs(self) -> int:
        return self.context_lens.shape[0]


def _lengths(w: Workload, rng: np.random.Generator, num_seqs: int, ctx_lo: int, ctx_hi: int):
    if w.groups:
        mu = math.log(w.suffix_median)
        suffix = np.clip(np.rint(np.exp(rng.normal(mu, w.suffix_sigma, size=num_seqs))), 1,
                         w.suffix_max).astype(np.int64)
        return (w.prefix_len + suffix + 1).astype(np.int64), suffix
    return rng.integers(ctx_lo, ctx_hi + 1, size=num_seqs).astype(np.int64), None


def reach_start(L, query_tokens: int = 1, window: int = 0):
    """Earliest position any query token of a sequence attends (elementwise)."""
    L = np.asarray(L, dtype=np.int64)
    if window <= 0:
        return np.zeros_like(L)
    return np.maximum(L - query_tokens - window + 1, 0)


def attended_slots(tables: np.ndarray, L: np.ndarray, lo: Optional[np.ndarray] = None):
    """Physical slot of every (sequence, lo <= position < L) pair, sequence-major."""
    if len(L) == 0:
        return np.zeros(0, np.int64)
    lo = np.zeros_like(L) if lo is None else lo
    n = L - lo
    seq = np.repeat(np.arange(len(L)), n)
    starts = np.cumsum(n) - n
    pos = np.arange(int(n.sum())) - np.repeat(starts, n) + np.repeat(lo, n)
    return tables[seq, pos // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + pos % BLOCK_SIZE


def _randn(shape, gen: torch.Generator, device, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(dtype)


def make_batch(name, seed: int, device="cpu", *, num_seqs: Optional[int] = None,
               ctx_range: Optional[tuple] = None, poison: bool = False,
               contiguous_tables: bool = False, groups: Optional[int] = None,
               suffix_max: Optional[int] = None, query_tokens: Optional[int] = None,
               window: Optional[int] = None, lengths=None, query_counts=None) -> Batch:
    """Draw one decode batch of workload ``name`` (a key of WORKLOADS or a
    Workload).

    num_seqs / ctx_range / groups / suffix_max shrink a workload for tests;
    query_tokens / window override the workload's; lengths fixes the context
    lengths (one per sequence); query_counts gives every sequence its own number
    of query tokens (a packed q with query_start); contiguous_tables assigns
    physical blocks in logical order instead of a random permutation (the
    "contiguous slice" layout).
    """
    w = name if isinstance(name, Workload) else WORKLOADS[name]
    if groups is not None or suffix_max is not None:
        w = dataclasses.replace(w, groups=groups or w.groups, suffix_max=suffix_max or w.suffix_max)
    if query_tokens is not None or window is not None:
        w = dataclasses.replace(w, query_tokens=w.query_tokens if query_tokens is None else query_tokens,
                                window=w.window if window is None else window)
    Q, W = w.query_tokens, w.window
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device).manual_seed(seed)
    if w.groups:
        B = w.groups * w.samples
    else:
        B = num_seqs or w.num_seqs
    lo, hi = ctx_range if ctx_range is not None else (w.ctx_lo, w.ctx_hi)
    L, suffix = _lengths(w, rng, B, lo, hi)
    if w.chunk_seqs and lengths is None and query_counts is None:
        Lc = rng.integers(w.chunk_lo, w.chunk_hi + 1, size=w.chunk_seqs).astype(np.int64)
        L = np.concatenate([L, Lc])
        query_counts = [Q] * B + [w.chunk_tokens] * w.chunk_seqs
        B = len(L)
    if lengths is not None:
        L = np.asarray(lengths, dtype=np.int64)
        B = len(L)
    varlen = query_counts is not None
    if varlen:
        Qs = np.asarray(query_counts, dtype=np.int64)
        assert Qs.shape == (B,) and (Qs >= 0).all()
        Q = int(Qs.max()) if B else 0
    else:
        Qs = np.full(B, Q, dtype=np.int64)
    nblk = -(-L // BLOCK_SIZE)
    max_blocks = int(nblk.max()) if B else 1
    first_blk = reach_start(L, Qs, W) // BLOCK_SIZE  # blocks before it are never read
    nalloc = nblk - first_blk

    # Physical block assignment.
    if w.groups:
        pre_blocks = w.prefix_len // BLOCK_SIZE
        assert pre_blocks * BLOCK_SIZE == w.prefix_len
        priv = nblk - pre_blocks
        needed = w.groups * pre_blocks + int(priv.sum())
        unique_tokens = w.groups * w.prefix_len + int((L - w.prefix_len).sum())
    else:
        needed = int(nalloc.sum())
        unique_tokens = int((L - first_blk * BLOCK_SIZE).sum())
    if w.fixed_pool_blocks:
        num_blocks = w.fixed_pool_blocks
        assert num_blocks >= needed + 1
    else:
        num_blocks = max(math.ceil(1.1 * unique_tokens / BLOCK_SIZE), needed + 1)
    order = np.arange(num_blocks) if contiguous_tables else rng.permutation(num_blocks)
    pad_block = int(order[needed])
    tables = np.full((B, max_blocks), pad_block, dtype=np.int32)
    for s in range(B):
        tables[s, :first_blk[s]] = -1  # freed behind the window
    cursor = 0
    if w.groups:
        prefix_ids = []
        for g in range(w.groups):
            prefix_ids.append(order[cursor:cursor + pre_blocks])
            cursor += pre_blocks
        for s in range(B):
            g = s // w.samples
            tables[s, :pre_blocks] = prefix_ids[g]
            tables[s, pre_blocks:nblk[s]] = order[cursor:cursor + priv[s]]
            cursor += priv[s]
    else:
        for s in range(B):
            tables[s, first_blk[s]:nblk[s]] = order[cursor:cursor + nalloc[s]]
            cursor += nalloc[s]
    assert cursor == needed

    D, Hq, Hkv = w.head_dim, w.num_q_heads, w.num_kv_heads
    in_dt = TORCH_DTYPES[w.dtype]
    N = int(Qs.sum())
    if varlen:
        q = _randn((N, Hq, D), gen, device, in_dt)
    else:
        q = _randn((B, Hq, D) if Q == 1 else (B, Q, Hq, D), gen, device, in_dt)
    new_k = _randn((N, Hkv, D), gen, device, in_dt)
    new_v = _randn((N, Hkv, D), gen, device, in_dt)
    # Positions L-Q_s .. L-1 of every sequence, sequence-major (negative
    # positions, for L < Q_s, get slot -1: nothing to write).
    seq = np.repeat(np.arange(B), Qs)
    starts = np.concatenate([[0], np.cumsum(Qs)]).astype(np.int64)
    pos = L[seq] - Qs[seq] + (np.arange(N) - starts[seq])
    ok = pos >= 0
    pos_c = np.maximum(pos, 0)
    slot_mapping = np.where(ok, tables[seq, pos_c // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE
                            + pos_c % BLOCK_SIZE, -1).astype(np.int64)

    k_scale = v_scale = fill_k = fill_v = fill_slots = None
    cache_shape = (num_blocks, Hkv, BLOCK_SIZE, D)
    if w.cache_dtype in QUANTISED:
        cdt = TORCH_DTYPES[w.cache_dtype]
        k_cache = torch.zeros(cache_shape, dtype=cdt, device=device)
        v_cache = torch.zeros(cache_shape, dtype=cdt, device=device)
        fill = torch.nan if poison else 0.0
        k_scale = torch.full(cache_shape[:3], fill, dtype=torch.float32, device=device)
        v_scale = torch.full(cache_shape[:3], fill, dtype=torch.float32, device=device)
        # Every attended token's K/V, to be written through the KV write.
        fill_slots_np = np.unique(attended_slots(tables, L, reach_start(L, Qs, W)))
        fill_slots = torch.from_numpy(fill_slots_np).to(device)
        fill_k = _randn((len(fill_slots_np), Hkv, D), gen, device, in_dt)
        fill_v = _randn((len(fill_slots_np), Hkv, D), gen, device, in_dt)
    else:
        cdt = TORCH_DTYPES[w.cache_dtype]
        k_cache = _randn(cache_shape, gen, device, cdt)
        v_cache = _randn(cache_shape, gen, device, cdt)
        if poison:
            live = torch.zeros(num_blocks * BLOCK_SIZE, dtype=torch.bool)
            live[torch.from_numpy(attended_slots(tables, L, reach_start(L, Qs, W)))] = True
            dead = (~live).view(num_blocks, 1, BLOCK_SIZE, 1).expand(cache_shape).to(device)
            k_cache.masked_fill_(dead, float("nan"))
            v_cache.masked_fill_(dead, float("nan"))

    logical = int(nblk.sum())
    return Batch(
        workload=w, q=q, k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale,
        block_tables=torch.from_numpy(tables).to(device),
        context_lens=torch.from_numpy(L.astype(np.int32)).to(device),
        slot_mapping=torch.from_numpy(slot_mapping).to(device),
        new_k=new_k, new_v=new_v, scale=1.0 / math.sqrt(D),
        max_context_len=int(L.max()) if B else 0, pad_block=pad_block,
        fill_k=fill_k, fill_v=fill_v, fill_slots=fill_slots,
        num_blocks_shared=needed, num_blocks_logical=logical, query_tokens=Q, window=W,
        query_start=(torch.from_numpy(starts.astype(np.int32)).to(device) if varlen else None))


def kv_token_slots(prefix_len: int, gen_lens, shared: bool) -> int:
    """Token slots a batch of samples of one prompt occupies.

    Each sample holds the prompt plus its own generated tokens; with shared
    (reference-counted) prefix blocks the prompt is stored once.
    """
    gen_lens = [int(g) for g in gen_lens]
    if shared:
        return prefix_len + sum(gen_lens)
    return sum(prefix_len + g for g in gen_lens)


def kv_blocks(prefix_len: int, gen_lens, shared: bool, block_size: int = BLOCK_SIZE) -> int:
    """Physical blocks for the same batch (prompt a whole number of blocks when shared)."""
    gen_lens = [int(g) for g in gen_lens]
    if shared:
        assert prefix_len % block_size == 0
        return prefix_len // block_size + sum(-(-g // block_size) for g in gen_lens)
    return sum(-(-(prefix_len + g) // block_size) for g in gen_lens)


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, cache_dtype: str) -> int:
    """KV bytes one token occupies in the pool (K and V rows, plus INT8/FP8 scales)."""
    elt = {"fp32": 4, "bf16": 2, "int8": 1, "fp8": 1}[cache_dtype]
    extra = 2 * num_kv_heads * 4 if cache_dtype in QUANTISED else 0
    return 2 * num_kv_heads * head_dim * elt + extra


def fragmentation(context_lens, block_size: int = BLOCK_SIZE) -> float:
    """Fraction of allocated block slots that hold no token (tail waste)."""
    L = np.asarray(context_lens, dtype=np.int64)
    alloc = int((-(-L // block_size)).sum()) * block_size
    return 0.0 if alloc == 0 else 1.0 - float(L.sum()) / alloc
