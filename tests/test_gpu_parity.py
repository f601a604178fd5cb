"""GPU parity: libpagedattn (HIP, through its C ABI) against the CPU oracle.

Gates:
* KV write: bit-exact (whole pool, and the INT8 scales), compared as bytes.
* Attention, fp32 accumulation: max-abs error <= 2e-3 for bf16 inputs and
  <= 1e-5 for fp32 inputs, on an fp32 output (the reduce writes fp32).
* Attention with a bf16 output: the exact result is rounded to bf16 (relative
  error up to 2^-8: bf16 keeps 8 significant bits, so half an ulp is 2^-8 of
  a value just above a power of two), so the bound is
  2e-3 + 2^-8 * (|oracle| + 2e-3).
* INT8: the oracle dequantises the pool the GPU wrote (after checking it
  bit-exact against the oracle's own write), in fp64.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-3
TOL_F32 = 1e-5
BF16_REL = 2.0 ** -8


def pa():
    import paged_kv_cache_52_amd as m
    return m


def _np(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def _to(b, device):
    """Copy every tensor of a Batch to device."""
    out = workloads.Batch(**{f: getattr(b, f) for f in b.__dataclass_fields__})
    for f in b.__dataclass_fields__:
        v = getattr(b, f)
        if isinstance(v, torch.Tensor):
            setattr(out, f, v.to(device))
    return out


def _oracle_decode(b, rows=None):
    return oracle.decode(_np(b.q), _np(b.k_cache), _np(b.v_cache), _np(b.block_tables),
                         _np(b.context_lens), b.scale,
                         None if b.k_scale is None else _np(b.k_scale),
                         None if b.v_scale is None else _np(b.v_scale), rows=rows,
                         window=b.window,
                         query_start=None if b.query_start is None else _np(b.query_start))


def _tol(b):
    return TOL_F32 if b.q.dtype == torch.float32 else TOL_BF16


def _gpu_fp32_out(g, split_tokens=None):
    """Split kernel + reduce into an fp32 output (the accumulation precision)."""
    parts = pa().paged_attn_decode_partial(g.q, g.k_cache, g.v_cache, g.block_tables,
                                           g.context_lens, g.scale, g.k_scale, g.v_scale,
                                           max_context_len=g.max_context_len,
                                           split_tokens=split_tokens, sliding_window=g.window,
                                           query_start=g.query_start)
    out = torch.empty(g.q.shape, dtype=torch.float32, device=g.q.device)
    pa().paged_attn_reduce(parts, out)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), parts


def _from_np(a, dtype):
    if dtype == torch.bfloat16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(a)


def _write_new_tokens(b, g):
    """Decode step: write the new token of every sequence on both sides (the
    oracle into the CPU batch b, the library into the GPU batch g) and check
    the two pools are bitwise equal."""
    kc, vc = _np(b.k_cache).copy(), _np(b.v_cache).copy()
    ks = vs = None
    if b.k_scale is not None:
        ks, vs = _np(b.k_scale).copy(), _np(b.v_scale).copy()
    oracle.kv_write(_np(b.new_k), _np(b.new_v), _np(b.slot_mapping), kc, vc, ks, vs)
    b.k_cache, b.v_cache = _from_np(kc, b.k_cache.dtype), _from_np(vc, b.v_cache.dtype)
    if ks is not None:
        b.k_scale, b.v_scale = torch.from_numpy(ks), torch.from_numpy(vs)
    pa().paged_kv_write(g.new_k, g.new_v, g.slot_mapping, g.k_cache, g.v_cache, g.k_scale,
                        g.v_scale)
    torch.cuda.synchronize()
    assert np.array_equal(_np(g.k_cache).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(_np(g.v_cache).view(np.uint8), vc.view(np.uint8))
    if ks is not None:
        assert np.array_equal(_np(g.k_scale).view(np.uint32), ks.view(np.uint32))
        assert np.array_equal(_np(g.v_scale).view(np.uint32), vs.view(np.uint32))


def _fill_quantised(b, g):
    """Fill an INT8 / FP8 pool through the KV write on both sides; check
    bit-exact."""
    kc, vc = _np(b.k_cache).copy(), _np(b.v_cache).copy()
    ks, vs = _np(b.k_scale).copy(), _np(b.v_scale).copy()
    oracle.kv_write(_np(b.fill_k), _np(b.fill_v), _np(b.fill_slots), kc, vc, ks, vs)
    pa().paged_kv_write(g.fill_k, g.fill_v, g.fill_slots, g.k_cache, g.v_cache, g.k_scale,
                        g.v_scale)
    torch.cuda.synchronize()
    assert np.array_equal(_np(g.k_cache), kc)
    assert np.array_equal(_np(g.v_cache), vc)
    assert np.array_equal(_np(g.k_scale).view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(_np(g.v_scale).view(np.uint32), vs.view(np.uint32))
    b.k_cache, b.v_cache = torch.from_numpy(kc), torch.from_numpy(vc)
    b.k_scale, b.v_scale = torch.from_numpy(ks), torch.from_numpy(vs)


def _check_out(gpu, ref, tol, what=""):
    err = np.abs(gpu - ref)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    assert err.max() <= tol, f"{what}: max abs err {err.max():.3e} > {tol}"


def _check_bf16_out(gpu_bf16, ref, what=""):
    gpu = gpu_bf16.float().cpu().double().numpy()
    bound = TOL_BF16 + BF16_REL * (np.abs(ref) + TOL_BF16)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    bad = np.abs(gpu - ref) > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond 2e-3 + 2^-8(|ref| + 2e-3)"


# ------------------------------------------------------------------ KV write

@pytest.mark.parametrize("name,kw", [
    ("tiny_fp32", {}),
    ("llama8b_bf16", dict(num_seqs=19, ctx_range=(1, 300))),
    ("llama8b_bf16", dict(num_seqs=3, ctx_range=(1, 300))),
])
def test_kv_write_bit_exact(name, kw):
    print(f"[case] kv_write {name} {kw}", flush=True)
    b = workloads.make_batch(name, 41, "cpu", **kw)
    b.slot_mapping[1] = -1  # skipped token
    g = _to(b, "cuda")
    before = _np(b.k_cache).copy()
    _write_new_tokens(b, g)  # asserts the two pools are bitwise equal
    assert not np.array_equal(_np(b.k_cache).view(np.uint8), before.view(np.uint8))


@pytest.mark.parametrize("cache", ["int8", "fp8"])
def test_kv_write_quantised_bit_exact_with_edge_rows(cache):
    print(f"[case] kv_write {cache} edge rows", flush=True)
    np_dt, t_dt = {"int8": (np.int8, torch.int8), "fp8": (np.uint8, torch.float8_e4m3fn)}[cache]
    rng = np.random.default_rng(3)
    D, Hkv, T = 128, 2, 64
    x = rng.normal(size=(T, Hkv, D)).astype(np.float32)
    x[0, 0] = 0.0                        # zero row
    x[1, 0, :8] = [127.0, 2.5, 3.5, -2.5, 126.5, 0.5, 1.5, -0.5]  # ties at scale 1
    x[1, 0, 8:] = 0.0
    x[2] *= 1e-36                        # subnormal scales
    x[3] *= 1e30                         # large values
    x[4, 1] = -7.0                       # constant row
    x[5, 0, :4] = [448.0, 3.0, 1.5, -0.75]  # FP8 ties after scaling by 1
    x[5, 0, 4:] = 0.0
    k = torch.from_numpy(x).to(torch.bfloat16)
    v = torch.from_numpy(-x[::-1].copy()).to(torch.bfloat16)
    for dt in (torch.bfloat16, torch.float32):
        kk, vv = k.to(dt), v.to(dt)
        NB = 6
        slots = torch.from_numpy(rng.permutation(NB * 16)[:T].astype(np.int64))
        slots[5] = -1
        kc = np.zeros((NB, Hkv, 16, D), np_dt)
        vc = np.zeros_like(kc)
        ks = np.zeros((NB, Hkv, 16), np.float32)
        vs = np.zeros_like(ks)
        oracle.kv_write(_np(kk), _np(vv), _np(slots), kc, vc, ks, vs)
        gk = torch.zeros(kc.shape, dtype=t_dt, device="cuda")
        gv = torch.zeros_like(gk)
        gks = torch.zeros(ks.shape, dtype=torch.float32, device="cuda")
        gvs = torch.zeros_like(gks)
        pa().paged_kv_write(kk.cuda(), vv.cuda(), slots.cuda(), gk, gv, gks, gvs)
        torch.cuda.synchronize()
        assert np.array_equal(_np(gk), kc) and np.array_equal(_np(gv), vc)
        assert np.array_equal(_np(gks).view(np.uint32), ks.view(np.uint32))
        assert np.array_equal(_np(gvs).view(np.uint32), vs.view(np.uint32))


# ------------------------------------------------------------------ decode

SMALL = {
    "tiny_fp32": {},
    "llama8b_bf16": dict(num_seqs=7, ctx_range=(1, 700)),
    "long_bf16": dict(num_seqs=2, ctx_range=(1500, 2600)),
    "shared_prefix_bf16": dict(groups=1, suffix_max=200),
}


@pytest.mark.parametrize("split_tokens", [16, 64, 512])
@pytest.mark.parametrize("name", list(SMALL))
def test_decode_matches_oracle(name, split_tokens):
    print(f"[case] decode {name} split {split_tokens}", flush=True)
    b = workloads.make_batch(name, 51, "cpu", **SMALL[name])
    g = _to(b, "cuda")
    _write_new_tokens(b, g)
    ref = _oracle_decode(b)
    out32, parts = _gpu_fp32_out(g, split_tokens)
    _check_out(out32, ref, _tol(b), f"{name}/fp32-out")
    # Whole step (split + reduce) with the output in q's dtype.
    out = pa().paged_attn_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                                 g.scale, max_context_len=g.max_context_len,
                                 split_tokens=split_tokens)
    torch.cuda.synchronize()
    if b.q.dtype == torch.bfloat16:
        _check_bf16_out(out, ref, f"{name}/bf16-out")
    else:
        _check_out(out.cpu().double().numpy(), ref, TOL_F32, f"{name}/out")


@pytest.mark.parametrize("name", ["tiny_fp32", "llama8b_bf16"])
def test_partials_match_oracle_splits(name):
    """Per-split (m, l, acc) of the split kernel against the oracle's splits."""
    print(f"[case] partials {name}", flush=True)
    b = workloads.make_batch(name, 61, "cpu", **SMALL[name])
    g = _to(b, "cuda")
    T = 32
    _, parts = _gpu_fp32_out(g, T)
    m, l, acc = oracle.decode_split(_np(b.q), _np(b.k_cache), _np(b.v_cache),
                                    _np(b.block_tables), _np(b.context_lens), b.scale, T,
                                    max_splits=parts.max_splits)
    gm = parts.m.cpu().double().numpy().reshape(m.shape)
    gl = parts.l.cpu().double().numpy().reshape(l.shape)
    ga = parts.acc.cpu().double().numpy().reshape(acc.shape)
    for s, L in enumerate(b.context_lens.tolist()):
        n = oracle.num_splits(L, T)
        np.testing.assert_allclose(gm[s, :, :n], m[s, :, :n], rtol=0, atol=1e-4)
        # l and acc are relative to each side's own max: compare l*e^m and acc/l.
        np.testing.assert_allclose(gl[s, :, :n] * np.exp(gm[s, :, :n]),
                                   l[s, :, :n] * np.exp(m[s, :, :n]), rtol=1e-4)
        np.testing.assert_allclose(ga[s, :, :n] / gl[s, :, :n, None],
                                   acc[s, :, :n] / l[s, :, :n, None], rtol=0, atol=_tol(b))


def test_reduce_alone_against_oracle_merge():
    """The reduce kernel on oracle-made partials equals the oracle's merge."""
    print("[case] reduce alone", flush=True)
    b = workloads.make_batch("llama8b_bf16", 71, "cpu", num_seqs=5, ctx_range=(1, 1200))
    T = 64
    m, l, acc = oracle.decode_split(_np(b.q), _np(b.k_cache), _np(b.v_cache),
                                    _np(b.block_tables), _np(b.context_lens), b.scale, T)
    ref = oracle.merge(m, l, acc)
    parts = pa().Partials(m=torch.from_numpy(m).float().cuda().unsqueeze(1),
                          l=torch.from_numpy(l).float().cuda().unsqueeze(1),
                          acc=torch.from_numpy(acc).float().cuda().unsqueeze(1),
                          context_lens=b.context_lens.cuda(), split_tokens=T)
    out = torch.empty(b.q.shape, dtype=torch.float32, device="cuda")
    pa().paged_attn_reduce(parts, out)
    torch.cuda.synchronize()
    _check_out(out.cpu().double().numpy(), ref, 1e-5, "reduce")


@pytest.mark.parametrize("packed", [False, True])
def test_reduce_many_rows_against_oracle_merge(packed):
    """Batches of 16384 rows or more (each reduce wave then merges four rows):
    the reduce on synthetic partials equals the oracle's merge. Some splits
    inside a row's split count are empty; entries past it hold large finite
    values that must not be used."""
    print(f"[case] reduce many rows packed={packed}", flush=True)
    rng = np.random.default_rng(321)
    Hq, D, T = 32, 128, 512
    B = 300 if packed else 600
    lens = rng.integers(0, 3000, size=B).astype(np.int32)
    lens[:3] = [0, 1, 512]
    S = max(oracle.num_splits(int(L), T) for L in lens)
    if packed:
        counts = rng.integers(0, 5, size=B)
        counts[:2] = [0, 3]
        qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        N = int(qs[-1])
        lead = (N, Hq)
        tok_seq = np.repeat(np.arange(B), counts)
        ns = np.array([oracle.num_splits(int(lens[s]), T, int(counts[s])) for s in tok_seq])
        ns_rows = np.repeat(ns, Hq)
    else:
        lead = (B, 1, Hq)
        ns_rows = np.repeat([oracle.num_splits(int(L), T) for L in lens], Hq)
    assert ns_rows.size >= 16384
    m = rng.normal(0.0, 2.0, lead + (S,))
    l = rng.uniform(1.0, 100.0, lead + (S,))
    acc = rng.normal(0.0, 1.0, lead + (S, D)) * l[..., None]
    empty = rng.random(lead + (S,)) < 0.2
    m[empty], l[empty], acc[empty] = -np.inf, 0.0, 0.0
    past = (np.arange(S)[None, :] >= ns_rows[:, None]).reshape(lead + (S,))
    ref = oracle.merge(np.where(past, -np.inf, m), np.where(past, 0.0, l),
                       np.where(past[..., None], 0.0, acc))
    m_g, l_g, acc_g = np.where(past, 50.0, m), np.where(past, 1e3, l), np.where(past[..., None], 1e6, acc)
    cuda = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    parts = pa().Partials(m=cuda(m_g), l=cuda(l_g), acc=cuda(acc_g),
                          context_lens=torch.from_numpy(lens).cuda(), split_tokens=T,
                          query_start=torch.from_numpy(qs).cuda() if packed else None)
    out = torch.empty(((N,) if packed else (B,)) + (Hq, D), dtype=torch.float32, device="cuda")
    pa().paged_attn_reduce(parts, out)
    torch.cuda.synchronize()
    _check_out(out.cpu().double().numpy(), ref.reshape(out.shape), 1e-5, "reduce many rows")


@pytest.mark.parametrize("name", ["tiny_fp32", "llama8b_bf16"])
def test_poisoned_slots_do_not_leak(name):
    """NaN in every unattended slot, the pad block and past-the-end table
    entries: output stays finite and equal to the oracle."""
    print(f"[case] poison {name}", flush=True)
    b = workloads.make_batch(name, 81, "cpu", poison=True, **SMALL[name])
    g = _to(b, "cuda")
    ref = _oracle_decode(b)
    assert np.isfinite(ref).all()
    for T in (16, 512):
        out32, _ = _gpu_fp32_out(g, T)
        _check_out(out32, ref, _tol(b), f"poison/{T}")


def test_reduce_clamps_lengths_like_the_split_kernel():
    """Lengths past 16 * max_blocks_per_seq are clamped by the split kernel;
    the reduce clamps them the same way, so it merges exactly the splits the
    kernel wrote even when the partials have room for more (here filled with
    stale values that would spoil the result if merged)."""
    print("[case] reduce length clamp", flush=True)
    b = workloads.make_batch("llama8b_bf16", 291, "cpu", lengths=[128, 128, 64])
    assert b.block_tables.shape[1] == 8
    g = _to(b, "cuda")
    g.context_lens = torch.tensor([300, 129, 64], dtype=torch.int32, device="cuda")
    ref = _oracle_decode(b)  # the lengths the clamp leaves: 128, 128, 64
    B, Hq, D = g.q.shape
    S = 40  # 16-token splits: the clamped bound needs 8, the raw lengths up to 19
    parts = pa().Partials(
        m=torch.full((B, 1, Hq, S), 50.0, device="cuda"),
        l=torch.ones((B, 1, Hq, S), device="cuda"),
        acc=torch.full((B, 1, Hq, S, D), 1e3, device="cuda"),
        context_lens=g.context_lens, split_tokens=16)
    pa().paged_attn_decode_partial(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                                   g.scale, max_context_len=300, split_tokens=16,
                                   partials=parts)
    out = torch.empty(g.q.shape, dtype=torch.float32, device="cuda")
    pa().paged_attn_reduce(parts, out)
    torch.cuda.synchronize()
    assert parts.max_context_len == 300 and parts.max_blocks_per_seq == 8
    _check_out(out.cpu().double().numpy(), ref, TOL_BF16, "clamped lengths")


def test_edge_lengths():
    """L = 0, 1, block and split boundaries in one ragged batch."""
    print("[case] edge lengths", flush=True)
    lens = [0, 1, 15, 16, 17, 511, 512, 513, 1024, 31, 2]
    b = workloads.make_batch("llama8b_bf16", 91, "cpu", num_seqs=len(lens), ctx_range=(1024, 1024))
    b.context_lens = torch.tensor(lens, dtype=torch.int32)
    g = _to(b, "cuda")
    ref = _oracle_decode(b)
    for T in (16, 512):
        out32, _ = _gpu_fp32_out(g, T)
        _check_out(out32, ref, TOL_BF16, f"edges/{T}")
        assert np.all(out32[0] == 0)
    # L = 1: the output is that token's V exactly (bf16 values, exact in fp32).
    out = pa().paged_attn_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                                 g.scale, max_context_len=1024)
    torch.cuda.synchronize()
    blk = int(b.block_tables[1, 0])
    gsz = b.q.shape[1] // b.k_cache.shape[1]
    vrow = b.v_cache[blk, :, 0].float()
    assert torch.equal(out[1].float().cpu(), vrow.repeat_interleave(gsz, dim=0))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (6, 6), (4, 4), (8, 4), (16, 4), (16, 2), (32, 2)])
def test_gqa_group_sizes(Hq, Hkv, D, dtype):
    print(f"[case] gqa Hq={Hq} Hkv={Hkv} D={D} {dtype}", flush=True)
    name = "tiny_fp32" if dtype == "fp32" else "llama8b_bf16"
    w = dataclasses.replace(workloads.WORKLOADS[name], num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim=D, fixed_pool_blocks=0)
    b = workloads.make_batch(w, 101, "cpu", num_seqs=5, ctx_range=(1, 600))
    g = _to(b, "cuda")
    ref = _oracle_decode(b)
    out32, _ = _gpu_fp32_out(g, 128)
    _check_out(out32, ref, _tol(b), f"gqa {Hq}/{Hkv}/{D}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("qdt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("name", ["int8_kv", "fp8_kv"])
def test_quantised_decode_matches_oracle(name, qdt, D):
    print(f"[case] {name} decode q={qdt} D={D}", flush=True)
    w = dataclasses.replace(workloads.WORKLOADS[name], head_dim=D)
    b = workloads.make_batch(w, 111, "cpu", num_seqs=6, ctx_range=(1, 900), poison=True)
    b.q = b.q.to(qdt)
    g = _to(b, "cuda")
    _fill_quantised(b, g)
    ref = _oracle_decode(b)
    for T in (16, 512):
        out32, _ = _gpu_fp32_out(g, T)
        _check_out(out32, ref, TOL_BF16, f"{name}/{T}")


# Per-sequence V magnitudes (a factor on the V rows of even blocks, another on
# odd blocks): INT8 V scales from about 2^-18 to 2^3, alone and mixed within
# one sequence, so that weights p * vscale span a wide range.
V_SCALE_FACTORS = [(1.0, 1.0), (16.0, 16.0), (2.0 ** -8, 2.0 ** -8), (1.0, 64.0),
                   (1.0, 2.0 ** -10), (2.0 ** -12, 2.0 ** -12), (2.0 ** 8, 1.0)]


@pytest.mark.parametrize("T", [16, 512])
def test_int8_v_scale_range(T):
    """INT8 decode with V rows scaled by powers of two over a wide range: the
    error bound scales with the sequence's largest factor (the result is
    linear in V)."""
    print(f"[case] int8 V scale range T={T}", flush=True)
    n = len(V_SCALE_FACTORS)
    b = workloads.make_batch("int8_kv", 113, "cpu", num_seqs=n, ctx_range=(200, 1500),
                             poison=True)
    owner = {}
    for s in range(n):
        nblk = -(-int(b.context_lens[s]) // 16)
        for j, blk in enumerate(b.block_tables[s, :nblk].tolist()):
            owner[blk] = (s, j)
    f = np.ones(len(b.fill_slots))
    for i, slot in enumerate(b.fill_slots.tolist()):
        s, j = owner[slot // 16]
        f[i] = V_SCALE_FACTORS[s][j % 2]
    b.fill_v = (b.fill_v.double() * torch.from_numpy(f)[:, None, None]).to(b.fill_v.dtype)
    g = _to(b, "cuda")
    _fill_quantised(b, g)
    vs = _np(b.v_scale)
    assert (vs[vs > 0] > 0.5).any() and (vs[vs > 0] < 2.0 ** -14).any()
    ref = _oracle_decode(b)
    out32, _ = _gpu_fp32_out(g, T)
    for s in range(n):
        tol = TOL_BF16 * max(V_SCALE_FACTORS[s])
        _check_out(out32[s], ref[s], tol, f"seq {s} factors {V_SCALE_FACTORS[s]}")


def test_identity_and_permuted_tables_agree():
    print("[case] identity vs permuted", flush=True)
    for contiguous in (True, False):
        b = workloads.make_batch("llama8b_bf16", 121, "cpu", num_seqs=4, ctx_range=(1, 900),
                                 contiguous_tables=contiguous)
        g = _to(b, "cuda")
        out32, _ = _gpu_fp32_out(g)
        _check_out(out32, _oracle_decode(b), TOL_BF16, f"contiguous={contiguous}")


@pytest.mark.parametrize("cache", ["bf16", "fp32", "int8", "fp8"])
def test_pool_beyond_4gib(cache):
    """A pool whose K and V arrays are each larger than 4 GiB (8 KV heads,
    head_dim 128): the sequences' blocks sit mostly past the 4 GiB byte offset
    of their array, so the write and the split kernel address them with 64-bit
    offsets (the bf16 pool also with 32 query tokens per sequence, which the
    split kernel stages through LDS). Every sequence is written through the KV
    write on both sides; the oracle holds only the used blocks, renumbered
    0.., which gives the same result (attention does not depend on where a
    block sits in the pool).
    Written tiles are compared bytewise, outputs against the oracle."""
    print(f"[case] pool beyond 4 GiB, {cache} cache", flush=True)
    Hq, Hkv, D = 32, 8, 128
    t_dt, np_dt, elt = {"bf16": (torch.bfloat16, np.uint16, 2),
                        "fp32": (torch.float32, np.float32, 4),
                        "int8": (torch.int8, np.int8, 1),
                        "fp8": (torch.float8_e4m3fn, np.uint8, 1)}[cache]
    quant = cache in ("int8", "fp8")
    q_dt = torch.float32 if cache == "fp32" else torch.bfloat16
    block_bytes = Hkv * 16 * D * elt
    NB = (1 << 32) // block_bytes + 4096          # > 4 GiB per array
    lens = np.array([1, 200, 517, 1000, 2049], np.int32)
    need = [(int(L) + 15) // 16 for L in lens]
    rng = np.random.default_rng(41)
    # Mostly from the top of the pool, a few from the bottom.
    ids = np.concatenate([NB - 1 - rng.permutation(2048)[:sum(need) - 6],
                          rng.permutation(64)[:6]]).astype(np.int64)
    rng.shuffle(ids)
    mb = max(need)
    tables = np.zeros((len(lens), mb), np.int32)
    ctables = np.zeros_like(tables)
    slots, cslots, used = [], [], []
    k = 0
    for s, L in enumerate(lens):
        for i in range(need[s]):
            tables[s, i], ctables[s, i] = ids[k], k
            used.append(ids[k])
            k += 1
        t = np.arange(L)
        slots.append(tables[s, t // 16].astype(np.int64) * 16 + t % 16)
        cslots.append(ctables[s, t // 16].astype(np.int64) * 16 + t % 16)
    slots, cslots = np.concatenate(slots), np.concatenate(cslots)
    used = torch.from_numpy(np.array(used, np.int64))
    N = len(slots)
    kx = torch.from_numpy(rng.normal(size=(N, Hkv, D)).astype(np.float32)).to(q_dt)
    vx = torch.from_numpy(rng.normal(size=(N, Hkv, D)).astype(np.float32)).to(q_dt)
    q = torch.from_numpy(rng.normal(size=(len(lens), Hq, D)).astype(np.float32)).to(q_dt)
    scale = 1.0 / np.sqrt(D)

    # Oracle side: the used blocks only.
    nb = len(used)
    kc = np.zeros((nb, Hkv, 16, D), np_dt)
    vc = np.zeros_like(kc)
    ks = vs = None
    if quant:
        ks = np.zeros((nb, Hkv, 16), np.float32)
        vs = np.zeros_like(ks)
    oracle.kv_write(_np(kx), _np(vx), cslots, kc, vc, ks, vs)

    # Library side: the whole pool; the used blocks start at zero.
    gk = torch.empty((NB, Hkv, 16, D), dtype=t_dt, device="cuda")
    gv = torch.empty_like(gk)
    gks = gvs = None
    try:
        gk.view(torch.uint8)[used.cuda()] = 0
        gv.view(torch.uint8)[used.cuda()] = 0
        if quant:
            gks = torch.zeros((NB, Hkv, 16), dtype=torch.float32, device="cuda")
            gvs = torch.zeros_like(gks)
        pa().paged_kv_write(kx.cuda(), vx.cuda(), torch.from_numpy(slots).cuda(), gk, gv, gks,
                            gvs)
        torch.cuda.synchronize()
        ub = used.cuda()
        assert np.array_equal(_np(gk[ub]).view(np.uint8), kc.view(np.uint8))
        assert np.array_equal(_np(gv[ub]).view(np.uint8), vc.view(np.uint8))
        if quant:
            assert np.array_equal(_np(gks[ub]).view(np.uint32), ks.view(np.uint32))
            assert np.array_equal(_np(gvs[ub]).view(np.uint32), vs.view(np.uint32))
        ref = oracle.decode(_np(q), kc, vc, ctables, lens, scale, ks, vs)
        tol = TOL_F32 if cache == "fp32" else TOL_BF16
        gq, gt = q.cuda(), torch.from_numpy(tables).cuda()
        gl = torch.from_numpy(lens).cuda()
        for T in (64, None):
            parts = pa().paged_attn_decode_partial(gq, gk, gv, gt, gl, scale, gks, gvs,
                                                   max_context_len=int(lens.max()),
                                                   split_tokens=T)
            out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
            pa().paged_attn_reduce(parts, out)
            torch.cuda.synchronize()
            _check_out(out.cpu().double().numpy(), ref, tol, f"{cache}/T={T}")
        if cache == "bf16":
            # 32 query tokens per sequence (128 rows per KV head): the workgroup
            # stages each tile through LDS and addresses it past 4 GiB as well.
            q4 = torch.from_numpy(rng.normal(size=(len(lens), 32, Hq, D)).astype(np.float32))
            q4 = q4.to(q_dt)
            ref4 = oracle.decode(_np(q4), kc, vc, ctables, lens, scale)
            for T in (256, None):
                parts = pa().paged_attn_decode_partial(q4.cuda(), gk, gv, gt, gl, scale,
                                                       max_context_len=int(lens.max()),
                                                       split_tokens=T)
                out = torch.empty(q4.shape, dtype=torch.float32, device="cuda")
                pa().paged_attn_reduce(parts, out)
                torch.cuda.synchronize()
                _check_out(out.cpu().double().numpy(), ref4, tol, f"staged/T={T}")
    finally:
        del gk, gv, gks, gvs
        torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64)])
def test_sequence_indices_past_32767(dtype, D):
    """40,000 short sequences: the plan's first entry word holds the sequence
    in its high 16 bits, so the words of sequences from 32,768 on are negative
    as int32 and must be read as unsigned. Every sequence is listed, and the
    decode (new tokens written first) matches the oracle, MFMA and VALU
    engines, one and several splits per sequence."""
    print(f"[case] 40000 sequences {dtype} D={D}", flush=True)
    w = workloads.Workload("many_short_sequences", 40000, 8, 2, D, dtype, dtype, 1, 40)
    b = workloads.make_batch(w, 281, "cpu")
    g = _to(b, "cuda")
    _write_new_tokens(b, g)
    ref = _oracle_decode(b)
    plan = pa().paged_attn_plan(g.context_lens, g.block_tables.shape[1],
                                max_context_len=g.max_context_len, split_tokens=16)
    torch.cuda.synchronize()
    sched = plan.sched.cpu().numpy().astype(np.int64) & 0xffffffff
    n = int(sched[0])
    seqs = sched[8:8 + 2 * n:2] >> 16
    splits = sched[8:8 + 2 * n:2] & 0xffff
    lens = _np(b.context_lens).astype(np.int64)
    assert n == int(np.maximum(1, -(-lens // 16)).sum())
    assert np.array_equal(np.bincount(seqs, minlength=40000), np.maximum(1, -(-lens // 16)))
    assert splits.max() < 3
    for T in (16, None):
        out32, _ = _gpu_fp32_out(g, T)
        _check_out(out32, ref, _tol(b), f"40000 sequences T={T}")


# At T = 16 and 48 the longest sequence has 63 and 21 full splits (all
# threads list the entries together), at T = 64 and 512 15 and 1 (each
# sequence's thread lists its own).
@pytest.mark.parametrize("T", [16, 48, 64, 512])
def test_plan_lists_every_split_once(T):
    """The plan kernel's work list holds each (sequence, split) exactly once:
    full splits first, sequence by sequence in split order, then last splits
    ordered by decreasing tile count."""
    print(f"[case] plan T={T}", flush=True)
    lens = [0, 1, 15, 16, 17, 511, 512, 513, 1024, 31, 2, 700]
    b = workloads.make_batch("llama8b_bf16", 151, "cpu", num_seqs=len(lens),
                             ctx_range=(1024, 1024))
    b.context_lens = torch.tensor(lens, dtype=torch.int32)
    g = _to(b, "cuda")
    plan = pa().paged_attn_plan(g.context_lens, g.block_tables.shape[1],
                                max_context_len=g.max_context_len, split_tokens=T)
    torch.cuda.synchronize()
    sched = plan.sched.cpu().numpy()
    nsplit = [max(1, -(-L // T)) for L in lens]
    n = sum(nsplit)
    assert list(sched[:8]) == [n, T, len(lens), min(g.max_context_len, 16 * b.block_tables.shape[1]),
                               1, 0, 0, 0]
    entries = [((int(e) & 0xffffffff) >> 16, int(e) & 0xffff) for e in sched[8:8 + 2 * n:2]]
    assert list(sched[9:9 + 2 * n:2]) == [lens[s] for s, _ in entries]
    assert sorted(entries) == sorted((s, j) for s in range(len(lens)) for j in range(nsplit[s]))
    n_full = n - len(lens)
    assert all(j < nsplit[s] - 1 for s, j in entries[:n_full])
    assert entries[:n_full] == sorted(entries[:n_full])
    tiles = [max(1, -(-(lens[s] - j * T) // 16)) if lens[s] else 1 for s, j in entries[n_full:]]
    assert tiles == sorted(tiles, reverse=True)


def test_plan_is_shared_and_mismatch_is_ignored():
    """One plan serves several decode calls; a plan made for another split size
    writes nothing (the partials keep their previous contents)."""
    print("[case] plan reuse", flush=True)
    b = workloads.make_batch("llama8b_bf16", 161, "cpu", num_seqs=5, ctx_range=(1, 900))
    g = _to(b, "cuda")
    ref = _oracle_decode(b)
    plan = pa().paged_attn_plan(g.context_lens, g.block_tables.shape[1],
                                max_context_len=g.max_context_len, split_tokens=64)
    for _ in range(2):
        parts = pa().paged_attn_decode_partial(g.q, g.k_cache, g.v_cache, g.block_tables,
                                               g.context_lens, g.scale, plan=plan)
        out = torch.empty(g.q.shape, dtype=torch.float32, device="cuda")
        pa().paged_attn_reduce(parts, out)
        torch.cuda.synchronize()
        _check_out(out.cpu().double().numpy(), ref, TOL_BF16, "plan reuse")
    # Raw C call with split_tokens 32 against the 64-token plan: nothing is written.
    from paged_kv_cache_52_amd import _lib
    lib = _lib.load()
    S = pa().num_splits(g.max_context_len, 32)
    m = torch.full((5, g.q.shape[1], S), 7.0, device="cuda")
    l = torch.full_like(m, 7.0)
    acc = torch.full((5, g.q.shape[1], S, 128), 7.0, device="cuda")
    rc = lib.paged_attn_decode_partial(
        g.q.data_ptr(), 1, 5, 1, g.q.shape[1], 128, g.k_cache.data_ptr(), g.v_cache.data_ptr(),
        None, None, 1, g.k_cache.shape[0], g.k_cache.shape[1], g.block_tables.data_ptr(),
        g.block_tables.shape[1], g.context_lens.data_ptr(), None, g.max_context_len, 0, g.scale,
        32,
        S, m.data_ptr(), l.data_ptr(), acc.data_ptr(), plan.sched.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    assert bool((m == 7.0).all()) and bool((acc == 7.0).all())


@pytest.mark.parametrize("name", ["llama8b_bf16", "int8_kv", "fp8_kv"])
def test_prepare_equals_write_then_plan(name):
    """The fused write-and-plan launch gives the same pool bytes and the same
    plan as the two separate calls."""
    print(f"[case] prepare {name}", flush=True)
    b = workloads.make_batch(name, 171, "cpu", num_seqs=9, ctx_range=(1, 700))
    g1, g2 = _to(b, "cuda"), _to(b, "cuda")
    if b.fill_k is not None:
        for g in (g1, g2):
            pa().paged_kv_write(g.fill_k, g.fill_v, g.fill_slots, g.k_cache, g.v_cache,
                                g.k_scale, g.v_scale)
    Hq, mb = b.q.shape[1], b.block_tables.shape[1]
    pa().paged_kv_write(g1.new_k, g1.new_v, g1.slot_mapping, g1.k_cache, g1.v_cache, g1.k_scale,
                        g1.v_scale)
    p1 = pa().paged_attn_plan(g1.context_lens, mb, max_context_len=b.max_context_len,
                              split_tokens=64)
    p2 = pa().paged_decode_prepare(g2.new_k, g2.new_v, g2.slot_mapping, g2.k_cache, g2.v_cache,
                                   g2.context_lens, mb, g2.k_scale, g2.v_scale,
                                   max_context_len=b.max_context_len, split_tokens=64)
    torch.cuda.synchronize()
    for a, c in [(g1.k_cache, g2.k_cache), (g1.v_cache, g2.v_cache)]:
        assert torch.equal(a.view(torch.uint8), c.view(torch.uint8))
    if b.k_scale is not None:
        assert torch.equal(g1.k_scale, g2.k_scale) and torch.equal(g1.v_scale, g2.v_scale)
    n = int(p1.sched[0].item())
    s1, s2 = p1.sched[:8 + 2 * n].cpu(), p2.sched[:8 + 2 * n].cpu()
    assert torch.equal(s1[:8], s2[:8])
    # Entries within one tile-count bucket may come in any order.
    e1 = sorted(zip(s1[8::2].tolist(), s1[9::2].tolist()))
    e2 = sorted(zip(s2[8::2].tolist(), s2[9::2].tolist()))
    assert e1 == e2


def test_decode_is_deterministic():
    b = workloads.make_batch("llama8b_bf16", 131, "cpu", num_seqs=6, ctx_range=(1, 2000))
    g = _to(b, "cuda")
    a1, _ = _gpu_fp32_out(g)
    a2, _ = _gpu_fp32_out(g)
    assert np.array_equal(a1, a2)


def test_graph_capture_replays_match_eager():
    """The decode step enqueues only kernels on the caller's stream, so it can
    be captured; every replay must equal the eager result."""
    print("[case] graph capture", flush=True)
    b = workloads.make_batch("llama8b_bf16", 141, "cpu", num_seqs=8, ctx_range=(100, 2000))
    g = _to(b, "cuda")
    eager = pa().paged_attn_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                                   g.scale, max_context_len=g.max_context_len).clone()
    out = torch.empty_like(g.q)
    T = pa().default_split_tokens(8, g.q.shape[1], g.k_cache.shape[1], g.q.shape[2],
                                  g.k_cache.dtype, g.max_context_len)
    ws = torch.empty(pa().workspace_bytes(8, g.q.shape[1], g.q.shape[2],
                                          pa().num_splits(g.max_context_len, T)),
                     dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            pa().paged_attn_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                                   g.scale, out, max_context_len=g.max_context_len,
                                   workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


# ------------------------------------------------------------------ full size

def _sample_rows(B, Q, Hq, n, seed):
    rng = np.random.default_rng(seed)
    seqs = rng.integers(0, B, size=n).astype(np.int32)
    toks = rng.integers(0, Q, size=n).astype(np.int32)
    heads = rng.integers(0, Hq, size=n).astype(np.int32)
    seqs[0], toks[0], heads[0] = 0, 0, 0
    seqs[1], toks[1], heads[1] = B - 1, Q - 1, Hq - 1
    return seqs, toks, heads


def _cpu_copy(g):
    b = workloads.Batch(**{f: getattr(g, f) for f in g.__dataclass_fields__})
    for f in g.__dataclass_fields__:
        v = getattr(g, f)
        if isinstance(v, torch.Tensor):
            setattr(b, f, v.cpu())
    return b


# Full sizes, every row compared with the oracle; the two batches with
# 512-token prefill chunks (whose rows cost the oracle minutes) compare whole
# sequences plus 256 sampled rows.
FULL_ALL_ROWS = ["llama8b_bf16", "long_bf16", "int8_kv", "fp8_kv", "shared_prefix_bf16",
                 "mtp4_llama8b_bf16", "swa4k_bf16"]
FULL_SAMPLED = ["prefill512_bf16", "mixed_llama8b_bf16"]


def _full_rows(g, whole_seqs, n_sampled, seed):
    """(sequence, query token, head) rows: every row of the given sequences,
    plus n_sampled random rows; and their flat indices into out."""
    Hq = g.q.shape[-2]
    if g.query_start is None:
        B, Q = g.q.shape[0], g.query_tokens
        first = np.arange(B + 1, dtype=np.int64) * Q
    else:
        first = _np(g.query_start).astype(np.int64)
        B = len(first) - 1
    N = int(first[-1])
    rng = np.random.default_rng(seed)
    tok = [np.arange(first[s], first[s + 1]) for s in whole_seqs]
    tok = np.concatenate(tok + [rng.integers(0, N, size=n_sampled)])
    tok = np.repeat(tok, Hq)
    heads = np.tile(np.arange(Hq), len(tok) // Hq)
    heads[len(heads) - n_sampled * Hq:] = rng.integers(0, Hq, size=n_sampled * Hq)
    seqs = np.searchsorted(first, tok, side="right") - 1
    return ((seqs.astype(np.int32), (tok - first[seqs]).astype(np.int32),
             heads.astype(np.int32)), tok * Hq + heads)


@pytest.mark.parametrize("name", FULL_ALL_ROWS + FULL_SAMPLED)
def test_full_size_as_benchmarked(name):
    """Each workload at its full size and seed, run by bench.py's own Step
    object (the launches the benchmark times: fused write + plan with its
    default split and grouping, the split kernel, the reduce into q's dtype).
    The fused write is compared byte for byte with the oracle's, then the
    output row by row: bf16 (as benchmarked) and fp32 (the same partials
    reduced again). The one-call paged_attn_decode is checked on the same rows.
    The oracle reads only its own copy of the inputs and its own writes."""
    import bench
    print(f"[case] full-size {name} as benchmarked", flush=True)
    g = workloads.make_batch(name, 1, "cuda")
    b = _cpu_copy(g)
    if g.fill_k is not None:
        _fill_quantised(b, g)
    kc, vc = _np(b.k_cache).copy(), _np(b.v_cache).copy()
    ks = vs = None
    if b.k_scale is not None:
        ks, vs = _np(b.k_scale).copy(), _np(b.v_scale).copy()
    oracle.kv_write(_np(b.new_k), _np(b.new_v), _np(b.slot_mapping), kc, vc, ks, vs)
    b.k_cache, b.v_cache = _from_np(kc, b.k_cache.dtype), _from_np(vc, b.v_cache.dtype)
    if ks is not None:
        b.k_scale, b.v_scale = torch.from_numpy(ks), torch.from_numpy(vs)
    step = bench.Step(pa(), g)
    step()
    out32 = torch.empty(g.q.shape, dtype=torch.float32, device="cuda")
    step.reduce(out32)
    torch.cuda.synchronize()
    if name == "shared_prefix_bf16":
        assert step.M == 4 and (step.plan.sched[9:9 + 2 * int(step.plan.sched[0]):2] < 0).any()
    assert np.array_equal(_np(g.k_cache).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(_np(g.v_cache).view(np.uint8), vc.view(np.uint8))
    if ks is not None:
        assert np.array_equal(_np(g.k_scale).view(np.uint32), ks.view(np.uint32))
        assert np.array_equal(_np(g.v_scale).view(np.uint32), vs.view(np.uint32))
    one_call = pa().paged_attn_decode(g.q, g.k_cache, g.v_cache, g.block_tables,
                                      g.context_lens, g.scale, k_scale=g.k_scale,
                                      v_scale=g.v_scale, max_context_len=g.max_context_len,
                                      sliding_window=g.window, query_start=g.query_start)
    torch.cuda.synchronize()
    D = g.q.shape[-1]
    out32 = out32.cpu().double().numpy().reshape(-1, D)
    out_bf = step.out.cpu().reshape(-1, D)
    one_call = one_call.cpu().reshape(-1, D)
    assert np.isfinite(out32).all() and torch.isfinite(out_bf).all()
    if name in FULL_ALL_ROWS:
        ref = _oracle_decode(b).reshape(-1, D)
        sel = slice(None)
    else:
        # The shortest prefill chunk's sequence (and, mixed, the first decode).
        lens = _np(g.context_lens).astype(np.int64)
        if g.query_start is None:
            whole = [int(np.argmin(lens))]
        else:
            counts = np.diff(_np(g.query_start).astype(np.int64))
            chunk = np.flatnonzero(counts > 1)
            whole = [int(chunk[np.argmin(lens[chunk])]), 0]
        rows, flat = _full_rows(g, whole, 256, 7)
        ref = _oracle_decode(b, rows=rows)
        sel = torch.from_numpy(flat).long()
        out32 = out32[flat]
    _check_out(out32, ref, TOL_BF16, f"{name}/fp32-out")
    _check_bf16_out(out_bf[sel], ref, f"{name}/bf16-out as benchmarked")
    _check_bf16_out(one_call[sel], ref, f"{name}/bf16-out one call")


def test_long_contexts_with_thousands_of_splits():
    """The long-context batch at its full size (8 sequences up to 128k tokens)
    with 16-token splits: up to 8,192 splits per sequence, so the split index
    uses 13 of its 16 plan bits and the reduce merges thousands of partials per
    row. Sampled rows against the oracle."""
    print("[case] long contexts, 16-token splits", flush=True)
    g = workloads.make_batch("long_bf16", 3, "cuda")
    b = workloads.Batch(**{f: getattr(g, f) for f in g.__dataclass_fields__})
    for f in g.__dataclass_fields__:
        v = getattr(g, f)
        if isinstance(v, torch.Tensor):
            setattr(b, f, v.cpu())
    out32, parts = _gpu_fp32_out(g, 16)
    assert parts.max_splits >= 4096
    B, Hq = g.q.shape[0], g.q.shape[-2]
    seqs, toks, heads = _sample_rows(B, 1, Hq, 16, 9)
    ref = _oracle_decode(b, rows=(seqs, toks, heads))
    D = g.q.shape[-1]
    flat = seqs.astype(np.int64) * Hq + heads
    _check_out(out32.reshape(-1, D)[flat], ref, TOL_BF16, "long contexts T=16")


# ------------------------------------------------ several query tokens, windows

MTP_CASES = [
    # (workload, Q, window)
    ("llama8b_bf16", 4, 0),     # 16 rows per KV head: one full MFMA tile
    ("llama8b_bf16", 3, 0),     # 12 rows, 4 padding
    ("llama8b_bf16", 2, 0),
    ("llama8b_bf16", 8, 0),     # 32 rows: two row groups
    ("tiny_fp32", 4, 0),        # VALU engine: 16 rows as two groups of 8
    ("tiny_fp32", 3, 0),
    ("llama8b_bf16", 1, 37),
    ("llama8b_bf16", 4, 37),
    ("llama8b_bf16", 1, 1),
    ("llama8b_bf16", 4, 300),
    ("tiny_fp32", 1, 20),
    ("tiny_fp32", 4, 16),
    ("int8_kv", 4, 0),
    ("int8_kv", 1, 50),
    ("int8_kv", 4, 50),
    ("fp8_kv", 4, 0),
    ("fp8_kv", 1, 50),
    # prefill chunks: many row groups per KV head, handled four to a workgroup
    ("llama8b_bf16", 32, 0),    # 128 rows: 8 row groups, 2 workgroups per (split, KV head)
    ("llama8b_bf16", 100, 0),   # 400 rows: 25 row groups, the last set of four ragged
    ("llama8b_bf16", 257, 0),   # 1028 rows: a partial row group
    ("llama8b_bf16", 64, 100),
    ("tiny_fp32", 20, 0),       # VALU engine: 80 rows in groups of 8
    ("tiny_fp32", 9, 30),
    ("int8_kv", 40, 0),
    ("fp8_kv", 40, 0),
]


def _mtp_batch(name, Q, W, seed, **kw):
    small = name == "tiny_fp32"  # its pool is fixed at 64 blocks
    kw.setdefault("num_seqs", 4 if small else 6)
    kw.setdefault("ctx_range", (Q, 128 if small else max(700, 2 * Q)))
    return workloads.make_batch(name, seed, "cpu", query_tokens=Q, window=W, **kw)


@pytest.mark.parametrize("split_tokens", [16, 64, 512])
@pytest.mark.parametrize("name,Q,W", MTP_CASES)
def test_query_tokens_and_windows_match_oracle(name, Q, W, split_tokens):
    """Q query tokens per sequence (causal among them) and sliding windows,
    with NaN in every slot no query token attends and -1 table entries behind
    the window; the new tokens are written first (Q per sequence)."""
    print(f"[case] query rows {name} Q={Q} W={W} T={split_tokens}", flush=True)
    b = _mtp_batch(name, Q, W, 201, poison=True)
    g = _to(b, "cuda")
    if b.fill_k is not None:
        _fill_quantised(b, g)
    _write_new_tokens(b, g)
    ref = _oracle_decode(b)
    assert np.isfinite(ref).all()
    out32, _ = _gpu_fp32_out(g, split_tokens)
    _check_out(out32, ref, _tol(b), f"{name} Q={Q} W={W}")
    out = pa().paged_attn_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                                 g.scale, k_scale=g.k_scale, v_scale=g.v_scale,
                                 max_context_len=g.max_context_len, split_tokens=split_tokens,
                                 sliding_window=W)
    torch.cuda.synchronize()
    assert out.shape == g.q.shape
    if b.q.dtype == torch.bfloat16:
        _check_bf16_out(out, ref, f"{name} Q={Q} W={W}/bf16-out")
    else:
        _check_out(out.cpu().double().numpy(), ref, TOL_F32, f"{name} Q={Q} W={W}/out")


def test_query_tokens_before_the_sequence_start():
    """L < Q: query tokens at negative positions give zeros; L = 0 too."""
    print("[case] query rows L < Q", flush=True)
    b = workloads.make_batch("llama8b_bf16", 211, "cpu", lengths=[0, 1, 2, 3, 4, 5, 40],
                             query_tokens=4)
    g = _to(b, "cuda")
    ref = _oracle_decode(b)
    for T in (16, 512):
        out32, _ = _gpu_fp32_out(g, T)
        _check_out(out32, ref, TOL_BF16, f"L<Q T={T}")
        assert np.all(out32[0] == 0) and np.all(out32[1, :3] == 0) and np.all(out32[2, :2] == 0)


@pytest.mark.parametrize("Q,W", [(4, 0), (1, 37), (4, 37)])
def test_partials_with_query_ranges(Q, W):
    """Per-split partials with empty per-row splits (m = -inf, l = 0)."""
    print(f"[case] partials Q={Q} W={W}", flush=True)
    b = _mtp_batch("llama8b_bf16", Q, W, 221, ctx_range=(Q, 300))
    g = _to(b, "cuda")
    T = 16
    _, parts = _gpu_fp32_out(g, T)
    m, l, acc = oracle.decode_split(_np(b.q), _np(b.k_cache), _np(b.v_cache),
                                    _np(b.block_tables), _np(b.context_lens), b.scale, T,
                                    max_splits=parts.max_splits, window=W)
    rows = tuple(parts.m.shape[:3])  # (B, Q, Hq); the oracle's follow q's shape
    m, l = m.reshape(rows + m.shape[-1:]), l.reshape(rows + l.shape[-1:])
    acc = acc.reshape(rows + acc.shape[-2:])
    gm, gl, ga = (t.cpu().double().numpy() for t in (parts.m, parts.l, parts.acc))
    for s, L in enumerate(b.context_lens.tolist()):
        n = oracle.num_splits(L, T, Q, W)
        empty = l[s, :, :, :n] == 0
        assert np.all(gl[s, :, :, :n][empty] == 0) and np.all(gm[s, :, :, :n][empty] == -np.inf)
        full = ~empty
        np.testing.assert_allclose(gm[s, :, :, :n][full], m[s, :, :, :n][full], rtol=0, atol=1e-4)
        np.testing.assert_allclose((gl * np.exp(gm))[s, :, :, :n][full],
                                   (l * np.exp(m))[s, :, :, :n][full], rtol=1e-4)
        np.testing.assert_allclose((ga / np.where(gl > 0, gl, 1)[..., None])[s, :, :, :n][full],
                                   (acc / np.where(l > 0, l, 1)[..., None])[s, :, :, :n][full],
                                   rtol=0, atol=TOL_BF16)


def test_reduce_alone_with_query_rows():
    print("[case] reduce alone Q=3 W=40", flush=True)
    b = _mtp_batch("llama8b_bf16", 3, 40, 231, num_seqs=5, ctx_range=(3, 600))
    T = 16
    m, l, acc = oracle.decode_split(_np(b.q), _np(b.k_cache), _np(b.v_cache),
                                    _np(b.block_tables), _np(b.context_lens), b.scale, T,
                                    window=40)
    ref = oracle.merge(m, l, acc)
    parts = pa().Partials(m=torch.from_numpy(m).float().cuda(), l=torch.from_numpy(l).float().cuda(),
                          acc=torch.from_numpy(acc).float().cuda(),
                          context_lens=b.context_lens.cuda(), split_tokens=T, sliding_window=40)
    out = torch.empty(b.q.shape, dtype=torch.float32, device="cuda")
    pa().paged_attn_reduce(parts, out)
    torch.cuda.synchronize()
    _check_out(out.cpu().double().numpy(), ref, 1e-5, "reduce Q=3 W=40")


@pytest.mark.parametrize("Q,W,T", [(1, 100, 16), (4, 100, 64), (4, 0, 16), (2, 33, 512)])
def test_plan_with_query_ranges(Q, W, T):
    """The plan lists max(1, ceil((L - base) / T)) splits per sequence and
    records Q and W in its header."""
    print(f"[case] plan Q={Q} W={W} T={T}", flush=True)
    lens = [4, 5, 16, 17, 100, 101, 116, 117, 500, 1000, 1023, 37]
    b = workloads.make_batch("llama8b_bf16", 241, "cpu", lengths=lens, query_tokens=Q, window=W)
    g = _to(b, "cuda")
    plan = pa().paged_attn_plan(g.context_lens, g.block_tables.shape[1],
                                max_context_len=g.max_context_len, split_tokens=T,
                                num_query_tokens=Q, sliding_window=W)
    torch.cuda.synchronize()
    sched = plan.sched.cpu().numpy()
    nsplit = [oracle.num_splits(L, T, Q, W) for L in lens]
    n = sum(nsplit)
    assert list(sched[:8]) == [n, T, len(lens), g.max_context_len, Q, W, 0, 0]
    entries = [((int(e) & 0xffffffff) >> 16, int(e) & 0xffff) for e in sched[8:8 + 2 * n:2]]
    assert sorted(entries) == sorted((s, j) for s in range(len(lens)) for j in range(nsplit[s]))


@pytest.mark.parametrize("nbytes,blocks", [(1 << 20, 4), ((1 << 20) + 48, 4), (8192 * 7 + 16, 3),
                                           (48, 1), (64 << 20, 1024)])
def test_hbm_read_probe_reads_every_word_once(nbytes, blocks):
    """The probe's sink, XORed together, equals the XOR of every word of the
    buffer: each 16-byte word (whole chunks and the ragged tail) is read once."""
    print(f"[case] probe bytes={nbytes} blocks={blocks}", flush=True)
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda")
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    pa().hbm_read_probe(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


# ---------------------------------------------------------------------------
# Plans with group entries: full splits j of consecutive sequences that start
# on the same physical block (shared prefix blocks) become one work item.

@pytest.mark.parametrize("T,M", [(64, 4), (512, 3), (1024, 4), (2048, 4)])
def test_grouped_shared_prefix_with_poison(T, M):
    """Group entries of 16-row members (their shared tiles staged once per
    workgroup) with NaN in every slot no query token attends."""
    print(f"[case] grouped shared prefix poison T={T} M={M}", flush=True)
    b = workloads.make_batch("shared_prefix_bf16", 263, "cpu", groups=2, suffix_max=600,
                             poison=True)
    g = _to(b, "cuda")
    ref = _oracle_decode(b)
    assert np.isfinite(ref).all()
    plan = pa().paged_attn_plan(g.context_lens, g.block_tables.shape[1],
                                max_context_len=g.max_context_len, split_tokens=T,
                                block_tables=g.block_tables, group_members=M)
    parts = pa().paged_attn_decode_partial(g.q, g.k_cache, g.v_cache, g.block_tables,
                                           g.context_lens, g.scale,
                                           max_context_len=g.max_context_len, plan=plan)
    out = torch.empty(g.q.shape, dtype=torch.float32, device="cuda")
    pa().paged_attn_reduce(parts, out)
    torch.cuda.synchronize()
    sched = plan.sched.cpu().numpy()
    assert (sched[9:9 + 2 * int(sched[0]):2] < 0).any(), "the batch should form groups"
    _check_out(out.cpu().double().numpy(), ref, _tol(b), f"grouped poison T={T} M={M}")


def _share_prefixes(b, n_blocks=None):
    """Let every odd sequence share the leading blocks of the sequence before
    it (all but its last block, or n_blocks), as prefix sharing does."""
    t = b.block_tables.clone()
    lens = b.context_lens.tolist()
    for s in range(1, len(lens), 2):
        n = min(-(-lens[s] // 16), -(-lens[s - 1] // 16)) - 1
        if n_blocks is not None:
            n = min(n, n_blocks)
        if n > 0:
            t[s, :n] = t[s - 1, :n]
    b.block_tables = t
    return b


def _expected_group_entries(tables, lens, T, M):
    """Full-split entries of a plan with groups of up to M, in list order: a
    sequence joins the previous one for its full split j when both splits are
    full and start on the same physical block, within aligned runs of M."""
    nsp = [max(1, -(-L // T)) for L in lens]

    def joins(s, j):
        if s <= 0 or s >= len(lens) or j >= nsp[s] - 1 or j >= nsp[s - 1] - 1:
            return False
        return tables[s, j * T // 16] == tables[s - 1, j * T // 16]

    out = []
    for s in range(len(lens)):
        for j in range(nsp[s] - 1):
            pos = s % M
            if pos > 0 and joins(s, j):
                continue
            cnt = 1
            while pos + cnt < M and joins(s + cnt, j):
                cnt += 1
            out.append(((s << 16) | j, -cnt if cnt > 1 else lens[s]))
    return out


# Lengths reach 2600 tokens: at T = 160 the longest sequence has 16 full
# splits, at T = 144 it has 18 (the plan's one-round path takes at most 16).
@pytest.mark.parametrize("T,M", [(64, 2), (64, 4), (512, 4), (16, 3), (144, 4), (160, 4),
                                 (160, 3), (1024, 4)])
def test_grouped_plan(T, M):
    """Group entries cover every full split exactly once, only join
    sequences whose split starts on the same block, and keep the list order."""
    print(f"[case] grouped plan T={T} M={M}", flush=True)
    b = workloads.make_batch("shared_prefix_bf16", 251, "cpu", groups=3, suffix_max=600)
    lens = b.context_lens.clone()
    lens[9] = 10                         # no full split inside a group
    lens[13] = 2000                      # prefix only
    b.context_lens = lens
    t = b.block_tables.clone()
    half = b.block_tables.shape[1] // 2
    t[5, 4] = t[5, 4 + half]           # breaks sharing of the splits starting there
    t[6, 32] = t[6, 32 + half]
    b.block_tables = t
    g = _to(b, "cuda")
    mb = g.block_tables.shape[1]
    plan = pa().paged_attn_plan(g.context_lens, mb, max_context_len=g.max_context_len,
                                split_tokens=T, block_tables=g.block_tables, group_members=M)
    torch.cuda.synchronize()
    sched = plan.sched.cpu().numpy()
    lmax = min(g.max_context_len, 16 * mb)
    L = [min(int(x), lmax) for x in lens]
    full = _expected_group_entries(b.block_tables.numpy(), L, T, M)
    n = len(full) + len(L)
    assert list(sched[:8]) == [n, T, len(L), lmax, 1, 0, M, 0]
    got = list(zip(sched[8:8 + 2 * len(full):2].tolist(), sched[9:9 + 2 * len(full):2].tolist()))
    assert got == full
    assert any(w1 < 0 for _, w1 in got), "the batch should form groups"
    # Expanded, the list covers every (sequence, split) exactly once.
    pairs = []
    for w0, w1 in zip(sched[8:8 + 2 * n:2].tolist(), sched[9:9 + 2 * n:2].tolist()):
        s, j = (w0 & 0xffffffff) >> 16, w0 & 0xffff
        pairs += [(s + i, j) for i in range(-w1 if w1 < 0 else 1)]
    assert sorted(pairs) == sorted((s, j) for s in range(len(L))
                                   for j in range(max(1, -(-L[s] // T))))


@pytest.mark.parametrize("T,M", [(512, 4), (1024, 3), (64, 3)])
def test_grouped_plan_across_chunks(T, M):
    """A grouped plan of 320 sequences (40 prompts x 8 samples) spans two
    256-sequence chunks of the plan workgroup. Sequence 256 is given the
    prefix blocks of sequence 255 (another prompt's), so with runs of 3 a group
    straddles the chunk boundary. The entries match the independent listing."""
    print(f"[case] grouped plan across chunks T={T} M={M}", flush=True)
    b = workloads.make_batch("shared_prefix_bf16", 252, "cpu", groups=40, suffix_max=600)
    assert b.num_seqs == 320
    t = b.block_tables.clone()
    t[256, :125] = t[255, :125]  # the 2000-token prefix: 125 blocks
    b.block_tables = t
    g = _to(b, "cuda")
    mb = g.block_tables.shape[1]
    plan = pa().paged_attn_plan(g.context_lens, mb, max_context_len=g.max_context_len,
                                split_tokens=T, block_tables=g.block_tables, group_members=M)
    torch.cuda.synchronize()
    sched = plan.sched.cpu().numpy()
    lmax = min(g.max_context_len, 16 * mb)
    L = [min(int(x), lmax) for x in b.context_lens]
    full = _expected_group_entries(b.block_tables.numpy(), L, T, M)
    n = len(full) + len(L)
    assert list(sched[:8]) == [n, T, len(L), lmax, 1, 0, M, 0]
    got = list(zip(sched[8:8 + 2 * len(full):2].tolist(), sched[9:9 + 2 * len(full):2].tolist()))
    assert got == full
    if M == 3:
        assert any(w1 < 0 and (w0 >> 16) < 256 <= (w0 >> 16) - w1 - 1 for w0, w1 in got)


SCALE_CASES = [0.0, -0.0884, 3.0]


@pytest.mark.parametrize("scale", SCALE_CASES)
@pytest.mark.parametrize("kind", ["decode", "staged", "packed", "grouped"])
def test_softmax_scale_zero_negative_and_large(kind, scale):
    """The logit scale is any float: zero gives the mean of V over the tokens
    a row attends, a negative scale reverses the logits, a large one makes the
    weights peaked (and the running max move often). The LDS-staged walks
    (many query rows per KV head, packed prefill chunks, group entries) fold
    the scale's sign into q and take |scale| (a zero scale as the smallest
    normal float); the streaming decode keeps the scale as given. Every form
    is compared with the oracle at the same scale."""
    print(f"[case] scale {scale} {kind}", flush=True)
    if kind == "decode":
        b = _mtp_batch("llama8b_bf16", 1, 0, 281)
    elif kind == "staged":
        b = _mtp_batch("llama8b_bf16", 100, 0, 282)  # 400 rows per KV head
    elif kind == "packed":
        b = _packed_batch("llama8b_bf16", [300, 700, 90], [1, 40, 17], 0, 283)
    else:
        b = workloads.make_batch("shared_prefix_bf16", 284, "cpu", groups=2, suffix_max=600)
    b.scale = scale
    g = _to(b, "cuda")
    ref = _oracle_decode(b)
    assert np.isfinite(ref).all()
    if kind != "grouped":
        out, _ = _gpu_fp32_out(g, 64)
    else:
        plan = pa().paged_attn_plan(g.context_lens, g.block_tables.shape[1],
                                    max_context_len=g.max_context_len, split_tokens=1024,
                                    num_query_tokens=b.query_tokens,
                                    block_tables=g.block_tables, group_members=4)
        parts = pa().paged_attn_decode_partial(g.q, g.k_cache, g.v_cache, g.block_tables,
                                               g.context_lens, g.scale,
                                               max_context_len=g.max_context_len, plan=plan)
        o = torch.empty(g.q.shape, dtype=torch.float32, device="cuda")
        pa().paged_attn_reduce(parts, o)
        torch.cuda.synchronize()
        sched = plan.sched.cpu().numpy()
        assert (sched[9:9 + 2 * int(sched[0]):2] < 0).any(), "the batch should form groups"
        out = o.cpu().double().numpy()
    _check_out(out.reshape(ref.shape), ref, _tol(b), f"scale {scale} {kind}")


GROUPED_CASES = [
    ("shared_prefix_bf16", 64, 2),
    ("shared_prefix_bf16", 64, 4),
    ("shared_prefix_bf16", 512, 4),
    ("shared_prefix_bf16", 1024, 4),  # the benchmark's split and grouping
    ("shared_prefix_bf16", 2048, 4),  # 128 tiles: the staged walk takes two chunks of 64
    ("llama8b_bf16", 64, 4),          # shared blocks built by the test
    ("mtp4_llama8b_bf16", 64, 4),     # Q = 4: 16 rows per KV head
    ("int8_kv", 64, 4),
    ("fp8_kv", 16, 3),
    ("tiny_fp32", 16, 4),             # VALU engine
]


@pytest.mark.parametrize("name,T,M", GROUPED_CASES)
def test_grouped_decode_matches_oracle(name, T, M):
    """Decode through a plan with group entries: each member still reads its
    own table, so results match the oracle whatever the grouping."""
    print(f"[case] grouped decode {name} T={T} M={M}", flush=True)
    if name == "shared_prefix_bf16":
        b = workloads.make_batch(name, 261, "cpu", groups=2, suffix_max=600)
    else:
        b = _share_prefixes(_mtp_batch(name, workloads.WORKLOADS[name].query_tokens, 0, 262))
    g = _to(b, "cuda")
    if b.fill_k is not None:
        _fill_quantised(b, g)
    ref = _oracle_decode(b)
    plan = pa().paged_attn_plan(g.context_lens, g.block_tables.shape[1],
                                max_context_len=g.max_context_len, split_tokens=T,
                                num_query_tokens=b.query_tokens, block_tables=g.block_tables,
                                group_members=M)
    parts = pa().paged_attn_decode_partial(g.q, g.k_cache, g.v_cache, g.block_tables,
                                           g.context_lens, g.scale, g.k_scale, g.v_scale,
                                           max_context_len=g.max_context_len, plan=plan)
    out = torch.empty(g.q.shape, dtype=torch.float32, device="cuda")
    pa().paged_attn_reduce(parts, out)
    torch.cuda.synchronize()
    sched = plan.sched.cpu().numpy()
    n = int(sched[0])
    assert (sched[9:9 + 2 * n:2] < 0).any(), "the batch should form groups"
    _check_out(out.cpu().double().numpy(), ref, _tol(b), f"grouped {name} T={T} M={M}")


def test_grouped_prepare_equals_write_then_plan():
    print("[case] grouped prepare", flush=True)
    b = workloads.make_batch("shared_prefix_bf16", 271, "cpu", groups=2, suffix_max=600)
    g1, g2 = _to(b, "cuda"), _to(b, "cuda")
    mb = b.block_tables.shape[1]
    pa().paged_kv_write(g1.new_k, g1.new_v, g1.slot_mapping, g1.k_cache, g1.v_cache)
    p1 = pa().paged_attn_plan(g1.context_lens, mb, max_context_len=b.max_context_len,
                              split_tokens=64, block_tables=g1.block_tables, group_members=4)
    p2 = pa().paged_decode_prepare(g2.new_k, g2.new_v, g2.slot_mapping, g2.k_cache, g2.v_cache,
                                   g2.context_lens, mb, max_context_len=b.max_context_len,
                                   split_tokens=64, block_tables=g2.block_tables,
                                   group_members=4)
    torch.cuda.synchronize()
    assert torch.equal(g1.k_cache.view(torch.uint8), g2.k_cache.view(torch.uint8))
    assert torch.equal(g1.v_cache.view(torch.uint8), g2.v_cache.view(torch.uint8))
    n = int(p1.sched[0].item())
    s1, s2 = p1.sched[:8 + 2 * n].cpu(), p2.sched[:8 + 2 * n].cpu()
    assert torch.equal(s1[:8], s2[:8])
    n_full = n - b.num_seqs
    assert torch.equal(s1[8:8 + 2 * n_full], s2[8:8 + 2 * n_full])  # full splits: list order
    e1 = sorted(zip(s1[8 + 2 * n_full::2].tolist(), s1[9 + 2 * n_full::2].tolist()))
    e2 = sorted(zip(s2[8 + 2 * n_full::2].tolist(), s2[9 + 2 * n_full::2].tolist()))
    assert e1 == e2


def test_grouped_plan_needs_one_row_group():
    """A plan with group entries is refused where a KV head's rows span
    several row groups (Q * g > 16 on the MFMA engine)."""
    b = workloads.make_batch("llama8b_bf16", 281, "cpu", num_seqs=4, ctx_range=(100, 300),
                             query_tokens=8)
    g = _to(b, "cuda")
    plan = pa().paged_attn_plan(g.context_lens, g.block_tables.shape[1],
                                max_context_len=g.max_context_len, split_tokens=64,
                                num_query_tokens=8, block_tables=g.block_tables, group_members=2)
    with pytest.raises(pa().PagedAttnError):
        pa().paged_attn_decode_partial(g.q, g.k_cache, g.v_cache, g.block_tables,
                                       g.context_lens, g.scale,
                                       max_context_len=g.max_context_len, plan=plan)


# ---------------------------------------------------------------------------
# Packed queries: every sequence has its own query count (decodes mixed with
# prefill chunks in one call), q / out / partials packed as [N][Hq].

PACKED_CASES = [
    # (workload, lengths, query counts, window)
    ("llama8b_bf16", [40, 1, 100, 17, 70, 5, 33], [3, 1, 0, 17, 1, 8, 33], 0),
    ("llama8b_bf16", [40, 1, 100, 17, 70, 5, 33], [3, 1, 0, 17, 1, 8, 33], 20),
    # decodes beside prefill chunks (1028 rows: 17 row blocks, the last ragged)
    ("llama8b_bf16", [300, 700, 650, 90, 520, 611], [1, 1, 100, 1, 257, 1], 0),
    ("llama8b_bf16", [300, 700, 650, 90, 520, 611], [1, 1, 100, 1, 257, 1], 64),
    ("tiny_fp32", [100, 3, 128, 60], [1, 9, 20, 0], 0),     # VALU engine, 2 passes per block
    ("tiny_fp32", [100, 3, 128, 60], [1, 9, 20, 4], 16),
    ("int8_kv", [300, 700, 650, 90], [1, 40, 1, 17], 0),
    ("fp8_kv", [300, 700, 650, 90], [1, 40, 1, 17], 50),
    ("llama8b_bf16", [500, 400], [0, 0], 0),                 # no query tokens at all
]


def _packed_batch(name, lens, counts, W, seed, **kw):
    return workloads.make_batch(name, seed, "cpu", lengths=lens, query_counts=counts, window=W,
                                **kw)


@pytest.mark.parametrize("split_tokens", [16, 64, 512])
@pytest.mark.parametrize("name,lens,counts,W", PACKED_CASES)
def test_packed_queries_match_oracle(name, lens, counts, W, split_tokens):
    """Per-sequence query counts in one call against the oracle, with the new
    tokens written first, NaN poison in every slot no query token reaches and
    the whole decode through paged_attn_decode with a bf16 output."""
    print(f"[case] packed {name} counts={counts} W={W} T={split_tokens}", flush=True)
    b = _packed_batch(name, lens, counts, W, 301, poison=True)
    g = _to(b, "cuda")
    if b.fill_k is not None:
        _fill_quantised(b, g)
    if b.new_k.shape[0]:
        _write_new_tokens(b, g)
    ref = _oracle_decode(b)
    assert np.isfinite(ref).all()
    out32, parts = _gpu_fp32_out(g, split_tokens)
    assert parts.m.shape[:2] == tuple(g.q.shape[:2])
    if ref.size:
        _check_out(out32, ref, _tol(b), f"packed {name} W={W}")
    out = pa().paged_attn_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                                 g.scale, k_scale=g.k_scale, v_scale=g.v_scale,
                                 max_context_len=g.max_context_len, split_tokens=split_tokens,
                                 sliding_window=W, query_start=g.query_start)
    torch.cuda.synchronize()
    assert out.shape == g.q.shape
    if not ref.size:
        return
    if b.q.dtype == torch.bfloat16:
        _check_bf16_out(out, ref, f"packed {name}/bf16-out")
    else:
        _check_out(out.cpu().double().numpy(), ref, TOL_F32, f"packed {name}/out")


def test_packed_partials_match_oracle_splits():
    """Per-split partials of packed rows, empty splits included."""
    print("[case] packed partials", flush=True)
    b = _packed_batch("llama8b_bf16", [40, 1, 100, 17, 70, 5, 33], [3, 1, 0, 17, 1, 8, 33], 20,
                      303)
    g = _to(b, "cuda")
    T = 16
    _, parts = _gpu_fp32_out(g, T)
    m, l, acc = oracle.decode_split(_np(b.q), _np(b.k_cache), _np(b.v_cache),
                                    _np(b.block_tables), _np(b.context_lens), b.scale, T,
                                    max_splits=parts.max_splits, window=20,
                                    query_start=_np(b.query_start))
    gm, gl, ga = (t.cpu().double().numpy() for t in (parts.m, parts.l, parts.acc))
    qs = _np(b.query_start)
    for s, (L, Q) in enumerate(zip(b.context_lens.tolist(), np.diff(qs))):
        if Q == 0:
            continue
        S = oracle.num_splits(L, T, int(Q), 20)
        r = slice(qs[s], qs[s + 1])
        live = l[r, :, :S] > 0
        assert np.array_equal(gl[r, :, :S] > 0, live)
        np.testing.assert_allclose(gm[r, :, :S][live], m[r, :, :S][live], atol=1e-4)
        np.testing.assert_allclose((gl * np.exp(gm))[r, :, :S][live],
                                   (l * np.exp(m))[r, :, :S][live], rtol=1e-4)
        ratio_g = ga[r, :, :S][live] / gl[r, :, :S][live][:, None]
        ratio_o = acc[r, :, :S][live] / l[r, :, :S][live][:, None]
        assert np.abs(ratio_g - ratio_o).max() <= TOL_BF16


@pytest.mark.parametrize("T,W", [(16, 0), (64, 30), (512, 0)])
def test_packed_plan_lists_every_row_block_once(T, W):
    """The packed plan lists, per sequence with query tokens, every (split,
    block of 64 query rows) once: full splits sequence by sequence with the
    row blocks of a split adjacent, then last splits by decreasing tile
    count; the header records N and g."""
    print(f"[case] packed plan T={T} W={W}", flush=True)
    lens = [40, 1, 100, 17, 700, 5, 33, 0, 260]
    counts = [3, 1, 0, 17, 40, 8, 33, 2, 1]
    b = _packed_batch("llama8b_bf16", lens, counts, W, 305)
    g = _to(b, "cuda")
    N, Hq, Hkv = int(sum(counts)), b.q.shape[1], b.k_cache.shape[1]
    grp = Hq // Hkv
    mb = g.block_tables.shape[1]
    plan = pa().paged_attn_plan(g.context_lens, mb, max_context_len=g.max_context_len,
                                split_tokens=T, num_query_tokens=N, sliding_window=W,
                                query_start=g.query_start, q_heads_per_kv=grp)
    torch.cuda.synchronize()
    sched = plan.sched.cpu().numpy()
    nsp = [oracle.num_splits(L, T, Q, W) for L, Q in zip(lens, counts)]
    per = [-(-Q * grp // 64) for Q in counts]
    full = [((s << 16) | j, rb) for s in range(len(lens)) for j in range(nsp[s] - 1)
            for rb in range(per[s])]
    last = sorted(((s << 16) | (nsp[s] - 1), rb) for s in range(len(lens)) for rb in range(per[s]))
    n = len(full) + len(last)
    lmax = min(g.max_context_len, 16 * mb)
    assert list(sched[:8]) == [n, T, len(lens), lmax, N, W, 0, grp]
    got = list(zip(sched[8:8 + 2 * n:2].tolist(), sched[9:9 + 2 * n:2].tolist()))
    assert got[:len(full)] == full
    assert sorted(got[len(full):]) == last

    def tiles(w0):
        s = (w0 & 0xffffffff) >> 16
        base = oracle.split_base(lens[s], counts[s], W)
        rest = lens[s] - base - (nsp[s] - 1) * T
        return max(1, -(-rest // 16)) if lens[s] - base > 0 else 1
    t = [tiles(w0) for w0, _ in got[len(full):]]
    assert t == sorted(t, reverse=True)


def test_packed_equal_counts_match_the_batched_layout():
    """Q_s = 4 for every sequence: the packed call gives the [B][Q][Hq][D]
    call's result."""
    print("[case] packed vs batched", flush=True)
    b = workloads.make_batch("mtp4_llama8b_bf16", 307, "cpu", num_seqs=6, ctx_range=(4, 900))
    g = _to(b, "cuda")
    ref, _ = _gpu_fp32_out(g, 64)
    qs = torch.arange(0, 4 * 6 + 1, 4, dtype=torch.int32, device="cuda")
    flat = g.q.reshape(-1, *g.q.shape[2:])
    parts = pa().paged_attn_decode_partial(flat, g.k_cache, g.v_cache, g.block_tables,
                                           g.context_lens, g.scale,
                                           max_context_len=g.max_context_len, split_tokens=64,
                                           query_start=qs)
    out = torch.empty(flat.shape, dtype=torch.float32, device="cuda")
    pa().paged_attn_reduce(parts, out)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.cpu().double().numpy().reshape(ref.shape), ref, rtol=0,
                               atol=1e-6)


def test_packed_prepare_equals_write_then_plan():
    print("[case] packed prepare", flush=True)
    b = _packed_batch("llama8b_bf16", [300, 700, 650, 90], [1, 40, 1, 17], 0, 309)
    g1, g2 = _to(b, "cuda"), _to(b, "cuda")
    mb, Hq = b.block_tables.shape[1], b.q.shape[1]
    N = b.q.shape[0]
    pa().paged_kv_write(g1.new_k, g1.new_v, g1.slot_mapping, g1.k_cache, g1.v_cache)
    p1 = pa().paged_attn_plan(g1.context_lens, mb, max_context_len=b.max_context_len,
                              split_tokens=64, num_query_tokens=N, query_start=g1.query_start,
                              q_heads_per_kv=Hq // b.k_cache.shape[1])
    p2 = pa().paged_decode_prepare(g2.new_k, g2.new_v, g2.slot_mapping, g2.k_cache, g2.v_cache,
                                   g2.context_lens, mb, max_context_len=b.max_context_len,
                                   split_tokens=64, num_query_tokens=N, num_q_heads=Hq,
                                   query_start=g2.query_start)
    torch.cuda.synchronize()
    assert torch.equal(g1.k_cache.view(torch.uint8), g2.k_cache.view(torch.uint8))
    n = int(p1.sched[0].item())
    s1, s2 = p1.sched[:8 + 2 * n].cpu(), p2.sched[:8 + 2 * n].cpu()
    assert torch.equal(s1[:8], s2[:8])
    e1 = sorted(zip(s1[8::2].tolist(), s1[9::2].tolist()))
    e2 = sorted(zip(s2[8::2].tolist(), s2[9::2].tolist()))
    assert e1 == e2


def test_packed_batch_without_query_tokens():
    """N = 0: nothing to compute, nothing enqueued, an empty output."""
    b = _packed_batch("llama8b_bf16", [10, 20], [0, 0], 0, 311)
    g = _to(b, "cuda")
    out = pa().paged_attn_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens,
                                 g.scale, max_context_len=g.max_context_len,
                                 query_start=g.query_start)
    torch.cuda.synchronize()
    assert out.shape == (0, b.q.shape[1], b.q.shape[2])

