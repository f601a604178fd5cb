"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle (oracle/oracle.c) against something fixed by the
pages or by mathematics: a library attention routine on contiguous data, a
closed form, an invariance of the definition, or a hand-worked example.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(t):
    """Host NumPy view of a batch tensor (bf16 as its uint16 bit pattern, FP8
    as its uint8 codes)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def _f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def _small(name, seed, **kw):
    return workloads.make_batch(name, seed, "cpu", **kw)


def _decode(b, rows=None, **kw):
    return oracle.decode(_np(b.q), _np(b.k_cache), _np(b.v_cache), _np(b.block_tables),
                         _np(b.context_lens), b.scale,
                         None if b.k_scale is None else _np(b.k_scale),
                         None if b.v_scale is None else _np(b.v_scale), rows=rows, **kw)


# ---------------------------------------------------------------- library pin

@pytest.mark.parametrize("name,kw", [
    ("tiny_fp32", {}),
    ("llama8b_bf16", dict(num_seqs=3, ctx_range=(1, 100))),
    ("shared_prefix_bf16", dict(groups=1, suffix_max=40)),
])
def test_matches_sdpa_on_contiguous_tables(name, kw):
    """With blocks laid out in logical order, sequence s's K/V form one
    contiguous slice of the pool; torch's scaled_dot_product_attention (fp64,
    grouped heads) on that slice is the textbook softmax attention."""
    b = _small(name, 11, contiguous_tables=True, **kw)
    out = _decode(b)
    k, v, q = _f64(b.k_cache), _f64(b.v_cache), _f64(b.q)
    Hq, Hkv = b.q.shape[1], b.k_cache.shape[1]
    tables = b.block_tables.numpy()
    for s in range(b.num_seqs):
        L = int(b.context_lens[s])
        nb = -(-L // 16)
        first = int(tables[s, 0])
        if name != "shared_prefix_bf16":
            assert (tables[s, :nb] == np.arange(first, first + nb)).all()
            ks = torch.from_numpy(k[first:first + nb]).permute(1, 0, 2, 3).reshape(Hkv, nb * 16, -1)[:, :L]
            vs = torch.from_numpy(v[first:first + nb]).permute(1, 0, 2, 3).reshape(Hkv, nb * 16, -1)[:, :L]
        else:
            # Shared prefix blocks come first in the pool, so a sample's own
            # blocks are not adjacent to them: gather logical token t from
            # block tables[s, t // 16], row t % 16.
            t = np.arange(L)
            ks = torch.from_numpy(k[tables[s, t // 16], :, t % 16]).permute(1, 0, 2)
            vs = torch.from_numpy(v[tables[s, t // 16], :, t % 16]).permute(1, 0, 2)
        qs = torch.from_numpy(q[s]).reshape(1, Hq, 1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qs, ks.unsqueeze(0).contiguous(), vs.unsqueeze(0).contiguous(), scale=b.scale,
            enable_gqa=(Hq != Hkv))
        np.testing.assert_allclose(out[s], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariances

def _permute_pool(b, seed):
    """Relocate every physical block b to perm[b] and rewrite the tables."""
    rng = np.random.default_rng(seed)
    nb = b.k_cache.shape[0]
    perm = rng.permutation(nb)
    k2 = np.empty_like(_np(b.k_cache))
    v2 = np.empty_like(_np(b.v_cache))
    k2[perm] = _np(b.k_cache)
    v2[perm] = _np(b.v_cache)
    ks2 = vs2 = None
    if b.k_scale is not None:
        ks2 = np.empty_like(_np(b.k_scale))
        vs2 = np.empty_like(_np(b.v_scale))
        ks2[perm] = _np(b.k_scale)
        vs2[perm] = _np(b.v_scale)
    tables2 = perm[b.block_tables.numpy()].astype(np.int32)
    return k2, v2, ks2, vs2, tables2


@pytest.mark.parametrize("name", ["tiny_fp32", "llama8b_bf16"])
def test_physical_placement_invariance(name):
    """Moving blocks around the pool and rewriting the tables leaves every
    output bitwise unchanged (the gather is by logical position only)."""
    b = _small(name, 3, num_seqs=4, ctx_range=(1, 130))
    ref = _decode(b)
    k2, v2, _, _, t2 = _permute_pool(b, 99)
    out = oracle.decode(_np(b.q), k2, v2, t2, _np(b.context_lens), b.scale)
    assert np.array_equal(out, ref)


def test_physical_placement_invariance_int8():
    b = _int8_batch(5)
    ref = _decode(b)
    k2, v2, ks2, vs2, t2 = _permute_pool(b, 7)
    out = oracle.decode(_np(b.q), k2, v2, t2, _np(b.context_lens), b.scale, ks2, vs2)
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("split_tokens", [16, 32, 64, 48, 512, 100000])
def test_split_count_invariance(split_tokens):
    """Split-K partials merged by the reduce equal the unsplit softmax for any
    split size (the merge is exact up to rounding)."""
    b = _small("tiny_fp32", 21)
    ref = _decode(b)
    m, l, acc = oracle.decode_split(_np(b.q), _np(b.k_cache), _np(b.v_cache),
                                    _np(b.block_tables), _np(b.context_lens), b.scale,
                                    split_tokens)
    out = oracle.merge(m, l, acc)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # Empty splits are exactly (-inf, 0, 0), and the count per sequence is
    # max(1, ceil(L / split_tokens)).
    for s, L in enumerate(b.context_lens.tolist()):
        n = max(1, -(-L // split_tokens))
        assert oracle.num_splits(L, split_tokens) == n
        assert np.all(l[s, :, :n] >= 1.0)
        assert np.all(np.isneginf(m[s, :, n:])) and np.all(l[s, :, n:] == 0)
        assert np.all(acc[s, :, n:] == 0)


def test_merge_single_split_and_ignores_empty():
    rng = np.random.default_rng(0)
    m = np.array([[1.5, -np.inf, -np.inf]])
    l = np.array([[2.0, 0.0, 0.0]])
    acc = rng.normal(size=(1, 3, 8))
    acc[0, 1:] = np.nan  # contents of empty splits must never be read
    out = oracle.merge(m, l, acc)
    np.testing.assert_allclose(out[0], acc[0, 0] / 2.0, rtol=0, atol=0)


def test_merge_two_splits_worked_example():
    """Two splits with maxima 0 and ln 2: weights 1/2 and 1 relative to the
    larger one, so out = (acc0/2 + acc1) / (l0/2 + l1)."""
    m = np.array([[0.0, math.log(2.0)]])
    l = np.array([[3.0, 5.0]])
    acc = np.array([[[1.0, -2.0], [4.0, 8.0]]])
    out = oracle.merge(m, l, acc)
    expect = (acc[0, 0] / 2 + acc[0, 1]) / (3.0 / 2 + 5.0)
    np.testing.assert_allclose(out[0], expect, rtol=1e-15, atol=0)


# ---------------------------------------------------------------- closed forms

def test_single_token_returns_v():
    """L = 1: the softmax has one term, so out is that token's V row exactly."""
    b = _small("llama8b_bf16", 4, num_seqs=5, ctx_range=(1, 1))
    out = _decode(b)
    v = _f64(b.v_cache)
    Hq, Hkv = b.q.shape[1], b.k_cache.shape[1]
    g = Hq // Hkv
    for s in range(5):
        blk = int(b.block_tables[s, 0])
        for h in range(Hq):
            assert np.array_equal(out[s, h], v[blk, h // g, 0])


@pytest.mark.parametrize("how", ["zero_q", "zero_scale", "equal_keys"])
def test_uniform_weights_give_mean_of_v(how):
    """Equal logits make every weight equal, so out is the mean of V."""
    b = _small("tiny_fp32", 8)
    q, k = _np(b.q).copy(), _np(b.k_cache).copy()
    scale = b.scale
    if how == "zero_q":
        q[:] = 0
    elif how == "zero_scale":
        scale = 0.0
    else:
        k[:] = k[0, 0, 0]  # every key row identical
    out = oracle.decode(q, k, _np(b.v_cache), _np(b.block_tables), _np(b.context_lens), scale)
    v = _f64(b.v_cache)
    g = b.q.shape[1] // b.k_cache.shape[1]
    for s, L in enumerate(b.context_lens.tolist()):
        t = np.arange(L)
        blocks = b.block_tables[s].numpy()[t // 16]
        for h in range(b.q.shape[1]):
            rows = v[blocks, h // g, t % 16]
            np.testing.assert_allclose(out[s, h], rows.mean(axis=0), rtol=0, atol=1e-12)


def test_two_token_worked_example():
    """Hand-worked: q = (1, 0), keys (ln 3, 0) and (0, 0), scale 1: weights
    3/4 and 1/4, so out = 3/4 v0 + 1/4 v1."""
    D = 2
    q = np.array([[[1.0, 0.0]]], dtype=np.float32)
    k = np.zeros((2, 1, 16, D), dtype=np.float32)
    v = np.zeros_like(k)
    k[1, 0, 0] = [np.float32(math.log(3.0)), 0.0]
    v[1, 0, 0] = [4.0, -8.0]
    v[1, 0, 1] = [0.0, 16.0]
    out = oracle.decode(q, k, v, np.array([[1]], np.int32), np.array([2], np.int32), 1.0)
    w0 = math.exp(float(np.float32(math.log(3.0))))  # 3 up to the fp32 rounding of ln 3
    expect = (w0 * np.array([4.0, -8.0]) + np.array([0.0, 16.0])) / (w0 + 1.0)
    np.testing.assert_allclose(out[0, 0], expect, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(out[0, 0], [3.0, -2.0], atol=1e-6)


def test_zero_length_context():
    b = _small("tiny_fp32", 2)
    lens = _np(b.context_lens).copy()
    lens[1] = 0
    out = oracle.decode(_np(b.q), _np(b.k_cache), _np(b.v_cache), _np(b.block_tables), lens,
                        b.scale)
    assert np.all(out[1] == 0)
    m, l, acc = oracle.decode_split(_np(b.q), _np(b.k_cache), _np(b.v_cache),
                                    _np(b.block_tables), lens, b.scale, 16)
    assert np.all(np.isneginf(m[1])) and np.all(l[1] == 0) and np.all(acc[1] == 0)
    assert np.all(oracle.merge(m, l, acc)[1] == 0)


def test_gqa_equals_mha_with_repeated_kv_heads():
    """Query head h of a g-group reads KV head h // g: the same as multi-head
    attention over a pool whose KV heads are each repeated g times."""
    b = _small("llama8b_bf16", 6, num_seqs=3, ctx_range=(1, 70))
    g = b.q.shape[1] // b.k_cache.shape[1]
    k_mha = np.ascontiguousarray(np.repeat(_np(b.k_cache), g, axis=1))
    v_mha = np.ascontiguousarray(np.repeat(_np(b.v_cache), g, axis=1))
    ref = oracle.decode(_np(b.q), k_mha, v_mha, _np(b.block_tables), _np(b.context_lens),
                        b.scale)
    assert np.array_equal(_decode(b), ref)


def test_poisoned_unattended_slots_do_not_leak():
    """NaN in every slot no sequence attends leaves the output finite and equal
    to the unpoisoned result."""
    clean = _small("tiny_fp32", 31)
    dirty = _small("tiny_fp32", 31, poison=True)
    assert torch.isnan(dirty.k_cache).any()
    out = _decode(dirty)
    assert np.isfinite(out).all()
    assert np.array_equal(out, _decode(clean))


def test_row_subset_matches_full():
    b = _small("llama8b_bf16", 9, num_seqs=4, ctx_range=(1, 90))
    full = _decode(b)
    seqs = np.array([3, 0, 2], np.int32)
    heads = np.array([31, 5, 0], np.int32)
    sub = _decode(b, rows=(seqs, heads))
    assert np.array_equal(sub, full[seqs, heads])


# ---------------------------------------------------------------- KV write

@pytest.mark.parametrize("name", ["tiny_fp32", "llama8b_bf16"])
def test_kv_write_readback(name):
    b = _small(name, 12, num_seqs=6, ctx_range=(1, 60))
    k_cache, v_cache = _np(b.k_cache).copy(), _np(b.v_cache).copy()
    before_k, before_v = k_cache.copy(), v_cache.copy()
    slots = _np(b.slot_mapping).copy()
    slots[2] = -1  # skipped token
    oracle.kv_write(_np(b.new_k), _np(b.new_v), slots, k_cache, v_cache)
    nk, nv = _np(b.new_k), _np(b.new_v)
    touched = np.zeros(k_cache.shape[:1] + k_cache.shape[2:3], bool)
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        blk, off = divmod(int(sl), 16)
        assert np.array_equal(k_cache[blk, :, off], nk[t])
        assert np.array_equal(v_cache[blk, :, off], nv[t])
        touched[blk, off] = True
    untouched = ~touched
    assert np.array_equal(k_cache.transpose(0, 2, 1, 3)[untouched],
                          before_k.transpose(0, 2, 1, 3)[untouched])
    assert np.array_equal(v_cache.transpose(0, 2, 1, 3)[untouched],
                          before_v.transpose(0, 2, 1, 3)[untouched])
    # Writing the same tokens again changes nothing.
    k2, v2 = k_cache.copy(), v_cache.copy()
    oracle.kv_write(nk, nv, slots, k2, v2)
    assert np.array_equal(k2, k_cache) and np.array_equal(v2, v_cache)


def test_kv_write_then_decode_sees_new_token():
    """The new token lands at position L-1 and decode over a 1-token context
    returns exactly its V."""
    b = _small("tiny_fp32", 13, ctx_range=(1, 1))
    k_cache, v_cache = _np(b.k_cache).copy(), _np(b.v_cache).copy()
    oracle.kv_write(_np(b.new_k), _np(b.new_v), _np(b.slot_mapping), k_cache, v_cache)
    out = oracle.decode(_np(b.q), k_cache, v_cache, _np(b.block_tables), _np(b.context_lens),
                        b.scale)
    g = b.q.shape[1] // b.k_cache.shape[1]
    for s in range(b.num_seqs):
        for h in range(b.q.shape[1]):
            assert np.array_equal(out[s, h], _np(b.new_v)[s, h // g].astype(np.float64))


# ---------------------------------------------------------------- INT8

def _bf16_bits(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _quantise_rows(x_bf16_bits):
    """Run rows [T][D] through the oracle's INT8 write (one KV head)."""
    T, D = x_bf16_bits.shape
    nblocks = -(-T // 16)
    kc = np.zeros((nblocks, 1, 16, D), np.int8)
    vc = np.zeros_like(kc)
    ks = np.full((nblocks, 1, 16), np.nan, np.float32)
    vs = np.full_like(ks, np.nan)
    src = np.ascontiguousarray(x_bf16_bits.reshape(T, 1, D))
    oracle.kv_write(src, src, np.arange(T, dtype=np.int64), kc, vc, ks, vs)
    codes = kc.reshape(-1, D)[:T]
    scales = ks.reshape(-1)[:T]
    assert np.array_equal(codes, vc.reshape(-1, D)[:T])
    assert np.array_equal(scales, vs.reshape(-1)[:T], equal_nan=True)
    return codes, scales


def test_int8_quantiser_worked_examples():
    with open(os.path.join(GOLDEN, "int8_quant_rows.json")) as f:
        fx = json.load(f)
    x = np.array([r["x"] for r in fx["rows"]], dtype=np.float32)
    codes, scales = _quantise_rows(_bf16_bits(x))
    for i, r in enumerate(fx["rows"]):
        assert scales[i] == np.float32(r["scale"])
        assert codes[i].tolist() == r["code"]


def _numpy_quantiser(x32):
    """Independent float32 NumPy quantiser: IEEE divide, ties-to-even rint."""
    a = np.max(np.abs(x32), axis=1)
    sc = (a / np.float32(127.0)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.rint(x32 / sc[:, None])
    r = np.where(a[:, None] == 0, 0, np.clip(r, -127, 127))
    return r.astype(np.int8), sc


def test_int8_quantiser_properties_and_independent_implementation():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(300, 128)).astype(np.float32)
    x[7] = 0.0
    x[8] *= 1e-30
    x[9] *= 1e30
    bits = _bf16_bits(x)
    codes, scales = _quantise_rows(bits)
    xw = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    ref_codes, ref_scales = _numpy_quantiser(xw)
    assert np.array_equal(codes, ref_codes)
    assert np.array_equal(scales, ref_scales)
    assert codes.min() >= -127 and codes.max() <= 127
    nz = np.max(np.abs(xw), axis=1) > 0
    # The absmax element maps to +-127 and the error is at most half a step
    # (plus fp32 rounding of the scale and the quotient).
    am = np.argmax(np.abs(xw), axis=1)
    assert np.all(np.abs(codes[nz, am[nz]]) == 127)
    err = np.abs(xw - codes.astype(np.float64) * scales[:, None])
    assert np.all(err[nz] <= scales[nz, None] * (0.5 + 1e-5))
    assert np.all(codes[~nz] == 0) and np.all(scales[~nz] == 0)


def _int8_batch(seed):
    b = workloads.make_batch("int8_kv", seed, "cpu", num_seqs=4, ctx_range=(1, 70))
    kc, vc = _np(b.k_cache).copy(), _np(b.v_cache).copy()
    ks, vs = _np(b.k_scale).copy(), _np(b.v_scale).copy()
    oracle.kv_write(_np(b.fill_k), _np(b.fill_v), _np(b.fill_slots), kc, vc, ks, vs)
    b.k_cache, b.v_cache = torch.from_numpy(kc), torch.from_numpy(vc)
    b.k_scale, b.v_scale = torch.from_numpy(ks), torch.from_numpy(vs)
    return b


def test_int8_dequant_uses_per_token_scales():
    """An INT8 pool whose per-token scales are distinct powers of two equals,
    exactly, an fp32 pool holding code * scale (the products are exact)."""
    b = _int8_batch(3)
    rng = np.random.default_rng(1)
    ks = np.ldexp(1.0, rng.integers(-6, 6, size=b.k_scale.shape)).astype(np.float32)
    vs = np.ldexp(1.0, rng.integers(-6, 6, size=b.v_scale.shape)).astype(np.float32)
    kc, vc = _np(b.k_cache), _np(b.v_cache)
    k32 = (kc.astype(np.float32) * ks[..., None]).astype(np.float32)
    v32 = (vc.astype(np.float32) * vs[..., None]).astype(np.float32)
    q32 = torch.from_numpy(_np(b.q)).view(torch.bfloat16).float().numpy()
    q16 = _np(b.q)
    out_i8 = oracle.decode(q16, kc, vc, _np(b.block_tables), _np(b.context_lens), b.scale, ks, vs)
    out_32 = oracle.decode(q32, k32, v32, _np(b.block_tables), _np(b.context_lens), b.scale)
    assert np.array_equal(out_i8, out_32)


# ---------------------------------------------------------------- FP8 (E4M3)
#
# [ATOM 3] runs with --kv_cache_dtype fp8. Read as OCP FP8 E4M3 (bias 7, no
# infinities, S.1111.111 = NaN, largest finite 448) with the INT8 recipe's
# per-(token, KV head) scale, absmax / 448.

def test_e4m3_decoding_worked_values():
    """Codes worked by hand from the OCP E4M3 layout (tests/golden/fp8_e4m3.json)."""
    fx = json.load(open(os.path.join(GOLDEN, "fp8_e4m3.json")))
    for c in fx["codes"]:
        v = oracle.e4m3_decode(int(c["code"], 16))
        if c["value"] == "nan":
            assert math.isnan(v), c
        else:
            assert v == float(c["value"]) and math.copysign(1, v) == math.copysign(1, float(c["value"])), c


def test_e4m3_decoding_matches_torch_float8():
    """Every code decodes as torch's float8_e4m3fn (a library rendering of
    the same OCP format), NaN codes included."""
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_decode(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_e4m3_encoding_round_trip_ties_and_saturation():
    # Every finite code is its own value's code.
    for c in range(256):
        if (c & 0x7F) != 0x7F:
            assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c
    # Midpoints between neighbouring codes go to the even mantissa.
    for c in range(0, 0x7E):
        lo, hi = oracle.e4m3_decode(c), oracle.e4m3_decode(c + 1)
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2  # exact in fp32
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == want, hex(c)
        assert oracle.e4m3_encode(-mid) == want | 0x80
    # Past the largest code: saturation; NaN stays NaN.
    for x in (448.0, 463.9, 464.0, 1e6, 3.4e38, float("inf")):
        assert oracle.e4m3_encode(x) == 0x7E and oracle.e4m3_encode(-x) == 0xFE
    assert oracle.e4m3_encode(float("nan")) & 0x7F == 0x7F


def test_e4m3_encoding_matches_torch_float8_in_range():
    """Inside the finite range torch's float8_e4m3fn conversion rounds to
    nearest even too: agreement on random fp32 values of every magnitude."""
    rng = np.random.default_rng(13)
    x = (rng.uniform(-1, 1, 20000) * np.exp2(rng.uniform(-12, 8.8, 20000))).astype(np.float32)
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(v) for v in x], dtype=np.uint8)
    assert np.array_equal(got, ref)


def _quantise_rows_fp8(x_bf16_bits):
    """Run rows [T][D] through the oracle's FP8 write (one KV head)."""
    T, D = x_bf16_bits.shape
    nblocks = -(-T // 16)
    kc = np.zeros((nblocks, 1, 16, D), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.full((nblocks, 1, 16), np.nan, np.float32)
    vs = np.full_like(ks, np.nan)
    src = np.ascontiguousarray(x_bf16_bits.reshape(T, 1, D))
    oracle.kv_write(src, src, np.arange(T, dtype=np.int64), kc, vc, ks, vs)
    return kc.reshape(-1, D)[:T], ks.reshape(-1)[:T]


def test_fp8_quantiser_properties_and_independent_implementation():
    """The FP8 write against an independent quantiser (NumPy fp32 scale and
    divide, torch's float8_e4m3fn rounding): bitwise; the absmax element is
    +-448; the error is within half an E4M3 step of the scaled value."""
    rng = np.random.default_rng(17)
    x = rng.normal(size=(300, 128)).astype(np.float32)
    x[7] = 0.0
    x[8] *= 1e-30
    x[9] *= 1e30
    x[10, :4] = [3.0, -3.0, 1.5, 0.0]  # ties after scaling
    x[10, 4:] = 0.0
    bits = _bf16_bits(x)
    codes, scales = _quantise_rows_fp8(bits)
    xw = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    a = np.max(np.abs(xw), axis=1)
    sc = (a / np.float32(448.0)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        y = (xw / sc[:, None]).astype(np.float32)
    ref = torch.from_numpy(np.where(a[:, None] == 0, 0, y).astype(np.float32))
    ref = ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales, sc) and np.array_equal(codes, ref)
    nz = a > 0
    am = np.argmax(np.abs(xw), axis=1)
    assert np.all(codes[nz, am[nz]] & 0x7F == 0x7E)
    val = np.vectorize(oracle.e4m3_decode)(codes)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))) - 3)
    assert np.all(np.abs(y - val)[nz] <= 0.5 * ulp[nz] * (1 + 1e-6))
    assert np.all(codes[~nz] == 0) and np.all(scales[~nz] == 0)


def test_fp8_dequant_uses_per_token_scales():
    """An FP8 pool whose per-token scales are powers of two equals, exactly,
    an fp32 pool holding value(code) * scale."""
    b = workloads.make_batch("fp8_kv", 3, "cpu", num_seqs=4, ctx_range=(1, 70))
    kc, vc = _np(b.k_cache).copy(), _np(b.v_cache).copy()
    ks, vs = _np(b.k_scale).copy(), _np(b.v_scale).copy()
    oracle.kv_write(_np(b.fill_k), _np(b.fill_v), _np(b.fill_slots), kc, vc, ks, vs)
    rng = np.random.default_rng(1)
    ks = np.ldexp(1.0, rng.integers(-6, 6, size=ks.shape)).astype(np.float32)
    vs = np.ldexp(1.0, rng.integers(-6, 6, size=vs.shape)).astype(np.float32)
    dec = np.vectorize(oracle.e4m3_decode)
    k32 = (dec(kc) * ks[..., None]).astype(np.float32)
    v32 = (dec(vc) * vs[..., None]).astype(np.float32)
    q32 = torch.from_numpy(_np(b.q)).view(torch.bfloat16).float().numpy()
    out_8 = oracle.decode(_np(b.q), kc, vc, _np(b.block_tables), _np(b.context_lens), b.scale, ks, vs)
    out_32 = oracle.decode(q32, k32, v32, _np(b.block_tables), _np(b.context_lens), b.scale)
    assert np.array_equal(out_8, out_32)


# ---------------------------------------------------------------- harness pins

def test_prefix_sharing_example():
    with open(os.path.join(GOLDEN, "prefix_sharing.json")) as f:
        fx = json.load(f)
    gens = [fx["generated_per_sample"]] * fx["samples"]
    assert workloads.kv_token_slots(fx["prompt_len"], gens, shared=False) == fx["unshared_slots"]
    assert workloads.kv_token_slots(fx["prompt_len"], gens, shared=True) == fx["shared_slots"]


def test_shared_prefix_batch_accounting():
    b = workloads.make_batch("shared_prefix_bf16", 5, "cpu", groups=2, suffix_max=64)
    L = b.context_lens.numpy().astype(np.int64)
    pre = 2000 // 16
    # Physical blocks: each group's prefix once plus private blocks per sample.
    expect = 2 * pre + int((-(-(L - 2000) // 16)).sum())
    assert b.num_blocks_shared == expect
    assert b.num_blocks_logical == int((-(-L // 16)).sum())
    t = b.block_tables.numpy()
    for s in range(16):
        assert np.array_equal(t[s, :pre], t[(s // 8) * 8, :pre])
    # Private blocks are never shared.
    priv = np.concatenate([t[s, pre:-(-int(L[s]) // 16)] for s in range(16)])
    assert len(np.unique(priv)) == len(priv)
    assert not set(priv) & set(t[:, :pre].ravel())


def test_kv_bytes_per_token_matches_page_size_example():
    with open(os.path.join(GOLDEN, "kv_size.json")) as f:
        fx = json.load(f)
    per_layer = workloads.kv_bytes_per_token(fx["kv_heads"], fx["head_dim"], fx["dtype"])
    total = per_layer * fx["layers"] * fx["tokens"]
    assert abs(total / 1e9 - fx["page_gigabytes"]) / fx["page_gigabytes"] <= fx["rel_tol"]
    assert workloads.kv_bytes_per_token(8, 128, "bf16") == 4096
    assert workloads.kv_bytes_per_token(8, 128, "int8") == 2112
    assert workloads.kv_bytes_per_token(8, 128, "fp8") == 2112


def test_fragmentation_one_tail_block():
    # Every sequence wastes at most one partial block.
    L = np.array([17, 32, 1, 100])
    waste = (-(-L // 16)) * 16 - L
    assert workloads.fragmentation(L) == pytest.approx(waste.sum() / ((-(-L // 16)) * 16).sum())
    assert np.all(waste < 16)


# ------------------------------------------------ several query tokens, windows
#
# [ATOM 4.2]: with MTP speculative decoding a decode step carries mtp_k + 1 new
# tokens per sequence; read as the last Q tokens of the context, each attending
# causally. [Echo 4] / ATOM's model table: sliding-window attention, read as
# "the W most recent positions, the query's own included".

def _mtp(Q, W=0, seed=21, **kw):
    kw.setdefault("num_seqs", 4)
    kw.setdefault("ctx_range", (Q, 150))
    return _small("llama8b_bf16", seed, query_tokens=Q, window=W, **kw)


@pytest.mark.parametrize("Q", [2, 4])
def test_multi_token_rows_equal_prefix_decodes(Q):
    """Query token i of a sequence of length L is an ordinary one-token decode
    of the length-(L - Q + i + 1) prefix: same tokens in the same order, so the
    outputs agree bitwise."""
    b = _mtp(Q)
    out = _decode(b)
    assert out.shape == tuple(b.q.shape)
    L = _np(b.context_lens)
    for i in range(Q):
        prefix = (L - Q + i + 1).astype(np.int32)
        ref = oracle.decode(_np(b.q)[:, i], _np(b.k_cache), _np(b.v_cache), _np(b.block_tables),
                            prefix, b.scale)
        assert np.array_equal(out[:, i], ref), i


def _dense(b, s):
    """K, V of sequence s as [Hkv][L][D] fp64 tensors, gathered with NumPy."""
    L = int(b.context_lens[s])
    t = np.arange(L)
    tab = b.block_tables.numpy()[s]
    k = torch.from_numpy(_f64(b.k_cache)[tab[t // 16], :, t % 16]).permute(1, 0, 2)
    v = torch.from_numpy(_f64(b.v_cache)[tab[t // 16], :, t % 16]).permute(1, 0, 2)
    return k, v


@pytest.mark.parametrize("Q,W", [(4, 0), (1, 37), (4, 37), (3, 16), (2, 1), (40, 0), (24, 50)])
def test_query_ranges_match_masked_sdpa(Q, W):
    """Textbook masked attention: torch SDPA in fp64 with a boolean mask that
    lets query i (position p = L - Q + i) see t <= p and, with a window W,
    t > p - W."""
    b = _mtp(Q, W, seed=23, ctx_range=(max(Q, 1), 120))
    out = _decode(b, window=W)
    q = _f64(b.q).reshape(b.num_seqs, Q, b.q.shape[-2], -1)
    Hq, Hkv = q.shape[2], b.k_cache.shape[1]
    for s in range(b.num_seqs):
        L = int(b.context_lens[s])
        k, v = _dense(b, s)
        p = L - Q + np.arange(Q)
        t = np.arange(L)
        mask = t[None, :] <= p[:, None]
        if W:
            mask &= t[None, :] > (p[:, None] - W)
        qs = torch.from_numpy(q[s]).permute(1, 0, 2).unsqueeze(0)       # [1][Hq][Q][D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qs, k.unsqueeze(0).contiguous(), v.unsqueeze(0).contiguous(),
            attn_mask=torch.from_numpy(mask), scale=b.scale, enable_gqa=(Hq != Hkv))
        np.testing.assert_allclose(out[s].reshape(Q, Hq, -1), ref[0].permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)


def test_window_at_least_the_context_changes_nothing():
    b = _mtp(1, seed=25, ctx_range=(1, 200))
    ref = _decode(b)
    for W in (200, 201, 10 ** 6):
        assert np.array_equal(_decode(b, window=W), ref)


def test_window_of_one_returns_own_value():
    """W = 1: each query token sees only its own position, so out = that
    token's V row exactly (bf16 values are exact in fp64)."""
    b = _mtp(3, W=1, seed=27, ctx_range=(3, 90))
    out = _decode(b, window=1)
    L = _np(b.context_lens)
    tab, v = b.block_tables.numpy(), _f64(b.v_cache)
    g = b.q.shape[2] // b.k_cache.shape[1]
    for s in range(b.num_seqs):
        for i in range(3):
            p = int(L[s]) - 3 + i
            row = v[tab[s, p // 16], :, p % 16]                         # [Hkv][D]
            assert np.array_equal(out[s, i], np.repeat(row, g, axis=0))


def test_query_before_the_sequence_start_is_zero():
    """L < Q: query tokens at negative positions attend nothing (zero output);
    the others are ordinary."""
    b = _small("llama8b_bf16", 29, lengths=[2, 1, 5], query_tokens=4)
    out = _decode(b)
    assert np.all(out[0, :2] == 0) and np.all(out[1, :3] == 0)
    assert np.all(np.isfinite(out)) and np.any(out[2] != 0) and np.any(out[0, 2:] != 0)


@pytest.mark.parametrize("Q,W", [(4, 0), (1, 100), (4, 100), (2, 33)])
def test_split_invariance_with_query_ranges(Q, W):
    b = _mtp(Q, W, seed=31, ctx_range=(Q, 400))
    ref = _decode(b, window=W)
    for T in (16, 32, 64, 512):
        m, l, acc = oracle.decode_split(_np(b.q), _np(b.k_cache), _np(b.v_cache),
                                        _np(b.block_tables), _np(b.context_lens), b.scale, T,
                                        window=W)
        np.testing.assert_allclose(oracle.merge(m, l, acc), ref, rtol=0, atol=1e-12)


def test_poison_outside_the_reach_changes_nothing():
    """NaN in every slot no query token attends (before the window, in the
    first block's leading rows, past L) and freed table entries (-1) before
    the window leave the result unchanged."""
    kw = dict(num_seqs=5, ctx_range=(40, 300))
    clean = _mtp(4, 45, seed=33, **kw)
    dirty = _mtp(4, 45, seed=33, poison=True, **kw)
    assert (dirty.block_tables.numpy() == -1).any()
    assert np.array_equal(_decode(dirty, window=45), _decode(clean, window=45))
    m, l, acc = oracle.decode_split(_np(dirty.q), _np(dirty.k_cache), _np(dirty.v_cache),
                                    _np(dirty.block_tables), _np(dirty.context_lens),
                                    dirty.scale, 16, window=45)
    assert np.all(np.isfinite(acc)) and np.all(np.isfinite(l))


def test_split_layout_with_windows_hand_worked():
    """Hand-worked split layouts: base = start of the block holding
    max(0, L - Q - W + 1); splits = max(1, ceil((L - base) / T))."""
    cases = json.load(open(os.path.join(GOLDEN, "split_layout.json")))["cases"]
    for c in cases:
        assert oracle.split_base(c["L"], c["Q"], c["W"]) == c["base"], c
        assert oracle.num_splits(c["L"], c["T"], c["Q"], c["W"]) == c["splits"], c


def test_empty_splits_and_rows_in_multi_token_partials():
    """With Q = 4 and T = 16 the last split of a sequence whose length is
    16k + 1 holds only position L - 1: query tokens 0..2 attend none of it and
    get (-inf, 0, 0) there, token 3 gets one token with l = 1."""
    b = _small("llama8b_bf16", 35, lengths=[33, 17], query_tokens=4)
    m, l, acc = oracle.decode_split(_np(b.q), _np(b.k_cache), _np(b.v_cache),
                                    _np(b.block_tables), _np(b.context_lens), b.scale, 16)
    for s, last in ((0, 2), (1, 1)):
        assert np.all(m[s, :3, :, last] == -np.inf) and np.all(l[s, :3, :, last] == 0)
        assert np.all(acc[s, :3, :, last] == 0)
        assert np.all(l[s, 3, :, last] == 1.0)


# ------------------------------------------------ per-sequence query counts
#
# [Echo 3, chunked prefill]: a batch may mix prefill chunks with decodes in one
# call, a decode being a prefill of length 1. Read as: sequence s has its own
# count Q_s (0 allowed) of query tokens, its last Q_s positions, packed as
# rows query_start[s] .. query_start[s+1]-1 of q.

MIXED_LENS = [40, 1, 100, 17, 70, 5, 33]
MIXED_COUNTS = [3, 1, 0, 17, 1, 8, 33]   # L < Q_s for the sixth sequence


def _mixed(seed, **kw):
    kw.setdefault("lengths", MIXED_LENS)
    kw.setdefault("query_counts", MIXED_COUNTS)
    return _small("llama8b_bf16", seed, **kw)


def _decode_mixed(b, **kw):
    return _decode(b, query_start=_np(b.query_start), **kw)


@pytest.mark.parametrize("W", [0, 20])
def test_packed_queries_match_masked_sdpa(W):
    """Every sequence against torch SDPA in fp64 on its own dense K/V, with the
    causal (and window) mask of its own Q_s; rows of query tokens before the
    sequence start are zero."""
    b = _mixed(41, window=W)
    qs = _np(b.query_start)
    out = _decode_mixed(b, window=W)
    assert out.shape == tuple(b.q.shape)
    q = _f64(b.q)
    Hq, Hkv = q.shape[1], b.k_cache.shape[1]
    for s, (L, Q) in enumerate(zip(MIXED_LENS, MIXED_COUNTS)):
        rows = out[qs[s]:qs[s + 1]]
        assert rows.shape[0] == Q
        if Q == 0:
            continue
        p = L - Q + np.arange(Q)
        live = p >= 0
        assert np.all(rows[~live] == 0)
        k, v = _dense(b, s)
        t = np.arange(L)
        mask = t[None, :] <= p[live, None]
        if W:
            mask &= t[None, :] > (p[live, None] - W)
        qq = torch.from_numpy(q[qs[s]:qs[s + 1]][live]).permute(1, 0, 2).unsqueeze(0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, k.unsqueeze(0).contiguous(), v.unsqueeze(0).contiguous(),
            attn_mask=torch.from_numpy(mask), scale=b.scale, enable_gqa=(Hq != Hkv))
        np.testing.assert_allclose(rows[live], ref[0].permute(1, 0, 2).numpy(), rtol=0,
                                   atol=1e-12)


def test_packed_queries_with_equal_counts_equal_the_batched_layout():
    """Q_s = Q for every sequence is the [B][Q][Hq][D] layout flattened: the
    same rows, bitwise, for decode and for the split partials."""
    b = _small("llama8b_bf16", 43, num_seqs=5, ctx_range=(3, 120), query_tokens=3)
    ref = _decode(b)
    flat = _np(b.q).reshape(-1, *b.q.shape[2:])
    qs = np.arange(0, 16, 3, dtype=np.int32)
    args = (_np(b.k_cache), _np(b.v_cache), _np(b.block_tables), _np(b.context_lens), b.scale)
    out = oracle.decode(flat, *args, query_start=qs)
    assert np.array_equal(out.reshape(ref.shape), ref)
    m, l, acc = oracle.decode_split(_np(b.q), *args, 32)
    m2, l2, acc2 = oracle.decode_split(flat, *args, 32, query_start=qs)
    assert np.array_equal(m2.reshape(m.shape), m) and np.array_equal(l2.reshape(l.shape), l)
    assert np.array_equal(acc2.reshape(acc.shape), acc)


@pytest.mark.parametrize("W", [0, 20])
def test_split_invariance_with_packed_queries(W):
    b = _mixed(45, window=W)
    ref = _decode_mixed(b, window=W)
    for T in (16, 48, 512):
        m, l, acc = oracle.decode_split(_np(b.q), _np(b.k_cache), _np(b.v_cache),
                                        _np(b.block_tables), _np(b.context_lens), b.scale, T,
                                        window=W, query_start=_np(b.query_start))
        assert m.shape[:2] == tuple(b.q.shape[:2])
        np.testing.assert_allclose(oracle.merge(m, l, acc), ref, rtol=0, atol=1e-12)


def test_one_query_token_per_sequence_is_plain_decode():
    """Q_s = 1 everywhere (a decode batch in the packed layout) is the
    one-token decode, bitwise."""
    b = _small("tiny_fp32", 47, ctx_range=(1, 128))
    ref = _decode(b)
    qs = np.arange(b.num_seqs + 1, dtype=np.int32)
    assert np.array_equal(_decode(b, query_start=qs), ref)
