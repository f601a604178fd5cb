"""Benchmark of the paged-KV decode hot path on one MI355X.

One step = one decode step of one attention layer over a synthetic batch:
write the new token of every sequence into the pool and plan the splits
(paged_decode_prepare: paged_kv_write + paged_attn_plan in one launch), the
split-K decode kernel, and the reduce kernel. Inputs are resident in HBM
before the timed region starts.

Default workload: 8B-shaped bf16 decode batch (64 sequences, 32 q / 8 KV heads,
head_dim 128, block 16, context lengths uniform in [512, 4096], random
non-contiguous block tables over a pool of 1.1x the tokens).

Prints ONE JSON line. `value` is tokens/s for the whole step (query tokens /
t_step: one new token per sequence, Q per sequence for multi-token decode and
prefill chunks, the packed total N for a batch with per-sequence counts).
The split kernel's roofline uses its own duration: HIP events on the launch
stream around `steps` back-to-back launches of it after the timed region.
Per-kernel p10/p50/p90 come from a pass with events between the kernels of
each step. The line also carries the practical HBM read ceiling measured by
the library's read probe on the same device.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("decode attention tokens/s and achieved KV-read GB/s (% of HBM peak), 1 MI355X")
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of MI355X
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b_bf16")
    ap.add_argument("--split-tokens", type=int, default=0, help="0: library default")
    ap.add_argument("--group-members", type=int, default=0,
                    help="plan groups of sequences sharing blocks (1: off; 0: 4 for "
                         "shared-prefix workloads, else 1)")
    ap.add_argument("--contiguous-tables", action="store_true",
                    help="blocks in logical order (contiguous-slice layout)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--ctx-range", type=int, nargs=2, default=None, metavar=("LO", "HI"),
                    help="override the workload's context-length range (inclusive)")
    ap.add_argument("--probe-mib", type=int, default=1024,
                    help="measure the practical HBM read ceiling with the library's read probe "
                         "over a buffer of this many MiB (0: skip)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB "
                         "(reference kernel for scaling HBM byte counters)")
    return ap.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_52_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "pagedattn.h"), "rb").read())
    return h.hexdigest()[:16]


def query_counts(b):
    """Query tokens of every sequence (per-sequence counts with packed queries)."""
    import numpy as np
    if b.query_start is not None:
        return np.diff(b.query_start.to("cpu").numpy().astype(np.int64))
    return np.full(b.num_seqs, b.query_tokens, dtype=np.int64)


def algorithmic_flops(b):
    """Useful flops of the split kernel: per (query token, query head) and
    attended token, q.k and p.v are 2 * head_dim multiply-adds each."""
    import numpy as np
    L = b.context_lens.to("cpu").numpy().astype(np.int64)
    Qs, W = query_counts(b), b.window
    seq = np.repeat(np.arange(len(L)), Qs)
    first = np.concatenate([[0], np.cumsum(Qs)])[:-1]
    pos = L[seq] - Qs[seq] + (np.arange(int(Qs.sum())) - first[seq])   # query positions
    lo = np.maximum(pos - W + 1, 0) if W > 0 else np.zeros_like(pos)
    attended = np.clip(pos + 1 - lo, 0, None)
    w = b.workload
    return int(attended.sum()) * w.num_q_heads * 4 * w.head_dim


def algorithmic_bytes(b):
    """Bytes the split kernel must read by definition: the K and V rows (plus
    INT8 scales) of every token some query token attends (with a sliding
    window only the tokens it reaches; nothing of a sequence without query
    tokens), q, and the block-table entries used."""
    import numpy as np
    import workloads
    L = b.context_lens.to("cpu").numpy().astype(np.int64)
    Qs = query_counts(b)
    lo = workloads.reach_start(L, Qs, b.window)
    live = Qs > 0
    w = b.workload
    per_token = workloads.kv_bytes_per_token(w.num_kv_heads, w.head_dim, w.cache_dtype)
    kv = int((L - lo)[live].sum()) * per_token
    q = b.q.numel() * b.q.element_size()
    tables = int(((L + 15) // 16 - lo // 16)[live].sum()) * 4 + L.size * 4
    if b.query_start is not None:
        tables += (L.size + 1) * 4
    return kv, kv + q + tables


def cpu_baseline(b, seconds):
    """Time the oracle on a bounded sample of the same batch: whole sequences
    (all heads) in order until about `seconds` of CPU time have passed."""
    import numpy as np
    import torch
    import oracle

    def host(t):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy()
        return t.numpy()

    q, kc, vc = host(b.q), host(b.k_cache), host(b.v_cache)
    ks = None if b.k_scale is None else host(b.k_scale)
    vs = None if b.v_scale is None else host(b.v_scale)
    bt, cl = host(b.block_tables), host(b.context_lens)
    qs = None if b.query_start is None else host(b.query_start)
    B, Hq = b.num_seqs, q.shape[-2]
    Qs = query_counts(b)
    done, tokens, queries, t0 = 0, 0, 0, time.perf_counter()
    elapsed = 0.0
    # Whole sequences in batch order, wrapping around, until the time budget.
    while elapsed < seconds:
        s = done % B
        Q = int(Qs[s])
        tok = np.repeat(np.arange(Q, dtype=np.int32), Hq)
        h = np.tile(np.arange(Hq, dtype=np.int32), Q)
        oracle.decode(q, kc, vc, bt, cl, b.scale, ks, vs,
                      rows=(np.full(Q * Hq, s, np.int32), tok, h), window=b.window,
                      query_start=qs)
        tokens += int(cl[s])
        queries += Q
        done += 1
        elapsed = time.perf_counter() - t0
    return {
        "value": queries / elapsed, "unit": "tokens/s", "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{done} sequences ({done / B:.2f} passes over the {B}-sequence batch, "
                  f"{queries} query tokens x {Hq} q heads, {tokens} context tokens), fp64 "
                  f"block-table walk, {elapsed:.1f} s",
    }


def load_counters(workload):
    """HBM bytes per launch from committed rocprofv3 counter runs on this
    workload, if they were taken on the current kernel sources."""
    try:
        with open(os.path.join(PROFILES, f"decode_{workload}_counters.json")) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return c


def pct(sorted_vals, q):
    """Nearest-rank percentile of an ascending list."""
    i = min(len(sorted_vals) - 1, max(0, math.ceil(q * len(sorted_vals)) - 1))
    return sorted_vals[i]


def hbm_probe(pa, torch, dev, stream, mib, reps=10):
    """Practical HBM read ceiling: the library's read probe over a `mib` MiB
    buffer, `reps` back-to-back launches after one warm-up, timed like the
    split kernel (GB/s)."""
    buf = torch.ones((mib << 20) // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(2048 * 256, dtype=torch.int32, device=dev)
    pa.hbm_read_probe(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        pa.hbm_read_probe(buf, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf, sink
    return (mib << 20) / (ms * 1e-3) / 1e9


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path runs on a single MI355X and "
              "this build has no multi-GPU leg (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_52_amd as pa
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    b = workloads.make_batch(args.workload, args.seed, dev,
                             contiguous_tables=args.contiguous_tables,
                             ctx_range=tuple(args.ctx_range) if args.ctx_range else None)
    w = b.workload
    if b.fill_k is not None:  # quantised pools are filled through the KV write
        pa.paged_kv_write(b.fill_k, b.fill_v, b.fill_slots, b.k_cache, b.v_cache, b.k_scale,
                          b.v_scale)
        b.fill_k = b.fill_v = None
    B, Hq, D = b.num_seqs, b.q.shape[-2], b.q.shape[-1]
    W = b.window
    packed = b.query_start is not None
    # Query tokens: per sequence, or the packed total N (per-sequence counts).
    Q = b.q.shape[0] if packed else b.query_tokens
    n_query = b.q.shape[0] if packed else B * Q
    Qb = min(Q, pa.MAX_QUERY_TOKENS) if packed else Q          # per-sequence bound
    Qd = max(1, min(pa.MAX_QUERY_TOKENS, -(-Q // B))) if packed else Q  # default-T count
    mb = b.block_tables.shape[1]
    T = args.split_tokens or pa.default_split_tokens(B, Hq, w.num_kv_heads, w.head_dim,
                                                       b.k_cache.dtype, b.max_context_len, Qd, W)
    S = pa.max_splits(min(b.max_context_len, mb * 16), T, Qb, W)
    out = torch.empty_like(b.q)
    lead = (n_query, Hq) if packed else (B, Q, Hq)
    parts = pa.Partials(m=torch.empty(lead + (S,), dtype=torch.float32, device=dev),
                        l=torch.empty(lead + (S,), dtype=torch.float32, device=dev),
                        acc=torch.empty(lead + (S, D), dtype=torch.float32, device=dev),
                        context_lens=b.context_lens, split_tokens=T, sliding_window=W,
                        query_start=b.query_start)
    sched = torch.empty(pa.sched_bytes(B, S, Q if packed else None, Hq // w.num_kv_heads) // 4,
                        dtype=torch.int32, device=dev)
    M = args.group_members or (4 if w.groups and W == 0 and not packed else 1)
    stream = torch.cuda.current_stream(dev)
    plan = [None]

    def prepare():
        # KV write of the step's new tokens and the split plan, one launch.
        plan[0] = pa.paged_decode_prepare(b.new_k, b.new_v, b.slot_mapping, b.k_cache,
                                          b.v_cache, b.context_lens, mb, b.k_scale, b.v_scale,
                                          max_context_len=b.max_context_len, split_tokens=T,
                                          num_query_tokens=Q, sliding_window=W,
                                          num_q_heads=Hq, query_start=b.query_start,
                                          block_tables=b.block_tables, group_members=M,
                                          sched=sched)

    def decode():
        pa.paged_attn_decode_partial(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                                     b.scale, b.k_scale, b.v_scale,
                                     max_context_len=b.max_context_len, split_tokens=T,
                                     sliding_window=W, plan=plan[0], query_start=b.query_start,
                                     partials=parts)

    def reduce():
        pa.paged_attn_reduce(parts, out)

    def step():
        prepare(); decode(); reduce()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` whole steps.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps

    # Per-kernel durations: identical launches with events between them.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evs:
        e[0].record(stream); prepare()
        e[1].record(stream); decode()
        e[2].record(stream); reduce()
        e[3].record(stream)
    torch.cuda.synchronize()
    per = {k: sorted(e[i].elapsed_time(e[i + 1]) for e in evs)
           for i, k in enumerate(("write_and_plan", "decode_split", "reduce"))}
    t_prep, t_dec, t_red = (sum(per[k]) / args.steps
                            for k in ("write_and_plan", "decode_split", "reduce"))

    # The split kernel's own duration: `steps` back-to-back launches on the
    # same stream (each waits for the previous), no events or other kernels
    # in between; this is what a kernel trace reports as its duration.
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for _ in range(args.steps):
        decode()
    d1.record(stream)
    torch.cuda.synchronize()
    t_dec_b2b = d0.elapsed_time(d1) / args.steps

    kv_bytes, alg_bytes = algorithmic_bytes(b)
    alg_flops = algorithmic_flops(b)
    dec_gbps = alg_bytes / (t_dec_b2b * 1e-3) / 1e9
    dec_tflops = alg_flops / (t_dec_b2b * 1e-3) / 1e12
    # The kernel's bound: matrix cores once its arithmetic intensity passes
    # the ridge point of the two peaks (dense bf16 MFMA / HBM).
    mfma_bound = alg_flops / alg_bytes > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    kv_gbps_step = kv_bytes / (ms_step * 1e-3) / 1e9
    counters = load_counters(w.name)
    traffic = None
    if counters is not None:
        traffic = counters["fetch_bytes_per_launch"] + counters["write_bytes_per_launch"]
    probe_gbps = hbm_probe(pa, torch, dev, stream, args.probe_mib) if args.probe_mib else None

    line = {
        "metric": METRIC,
        "value": n_query / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp32": "f32", "bf16": "bf16"}[w.dtype] +
                 {"int8": "+i8kv", "fp8": "+fp8kv"}.get(w.cache_dtype, ""),
        "data": "synthetic",
        "config": {
            "workload": w.name, "num_seqs": B, "q_heads": Hq, "kv_heads": w.num_kv_heads,
            "head_dim": D, "block_size": 16, "cache_dtype": w.cache_dtype,
            "context_tokens": int(b.context_lens.sum()), "max_context_len": b.max_context_len,
            "split_tokens": T, "max_splits": S, "pool_blocks": int(b.k_cache.shape[0]),
            "query_tokens": (f"packed: {n_query} over {B} sequences" if packed else Q),
            "sliding_window": W, "group_members": M,
            "tables": "contiguous" if args.contiguous_tables else "permuted",
            "context_range": list(args.ctx_range) if args.ctx_range else
            [b.workload.ctx_lo, b.workload.ctx_hi],
            "seed": args.seed,
        },
        "kv_read_gbps": kv_gbps_step,
        "kv_read_frac_of_peak": kv_gbps_step / HBM_PEAK_GBPS,
        "decode_reduce_tokens_per_s": n_query / ((t_dec + t_red) * 1e-3),
        "kernel_ms": {"write_and_plan": t_prep, "decode_split": t_dec, "reduce": t_red,
                      "decode_split_back_to_back": t_dec_b2b},
        "kernel_us_p10_p50_p90": {k: [round(1e3 * pct(v, q), 2) for q in (0.1, 0.5, 0.9)]
                                  for k, v in per.items()},
        "roofline": ({
            "kernel": "decode_split_kernel", "bound": "mfma", "achieved": dec_tflops,
            "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": dec_tflops / MFMA_PEAK_TFLOPS,
            "traffic": traffic, "algorithmic_flops_per_launch": alg_flops,
            "algorithmic_bytes_per_launch": alg_bytes, "kv_read_gbps": dec_gbps,
            "duration_us": 1e3 * t_dec_b2b,
        } if mfma_bound else {
            "kernel": "decode_split_kernel", "bound": "hbm", "achieved": dec_gbps,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": dec_gbps / HBM_PEAK_GBPS,
            "traffic": traffic, "algorithmic_bytes_per_launch": alg_bytes,
            "algorithmic_flops_per_launch": alg_flops, "duration_us": 1e3 * t_dec_b2b,
            "read_probe_gbps": probe_gbps,
            "frac_of_read_probe": dec_gbps / probe_gbps if probe_gbps else None,
        }),
        "wall_s_timed": wall,
    }
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_probe_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(b, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
