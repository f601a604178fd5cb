"""The synthetic batches' new-token slots. paged_kv_write leaves duplicate slots
in one call as a race (unspecified winner), so every batch the tests and the
benchmark write must give each new token its own slot: unique among the
written ones, inside the pool, and in the block the token's own table names
for its position (skipped slots, -1, only for positions before the sequence
starts)."""
import numpy as np
import pytest

import workloads


def _small(name):
    w = workloads.WORKLOADS[name]
    kw = {"num_seqs": min(w.num_seqs, 16)}
    if w.groups:
        kw = {"groups": 2, "suffix_max": 600}
    if getattr(w, "chunk_seqs", 0):
        kw = {}
    if w.query_tokens > 64:
        kw = {"num_seqs": 2}
    if w.ctx_hi > 16384:  # long contexts: the same generator on shorter ones
        kw["ctx_range"] = (w.ctx_lo // 16, w.ctx_hi // 16)
    return workloads.make_batch(name, 3, "cpu", **kw)


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_new_token_slots_are_unique_and_own(name):
    b = _small(name)
    slots = b.slot_mapping.numpy()
    L = b.context_lens.numpy().astype(np.int64)
    tables = b.block_tables.numpy()
    B = len(L)
    if b.query_start is not None:
        qs = b.query_start.numpy().astype(np.int64)
        counts = np.diff(qs)
    else:
        counts = np.full(B, b.query_tokens, np.int64)
    assert len(slots) == counts.sum()
    seq = np.repeat(np.arange(B), counts)
    first = np.concatenate([[0], np.cumsum(counts)])[:-1]
    pos = L[seq] - counts[seq] + (np.arange(len(slots)) - first[seq])
    written = slots >= 0
    assert np.array_equal(written, pos >= 0)
    s = slots[written]
    assert len(np.unique(s)) == len(s), "two new tokens share a slot"
    num_blocks = b.k_cache.shape[0]
    assert (s < num_blocks * 16).all()
    p = pos[written]
    assert np.array_equal(s // 16, tables[seq[written], p // 16])
    assert np.array_equal(s % 16, p % 16)
