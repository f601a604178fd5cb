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
Its bytes are the unique K/V bytes the launch must read (a block shared by
several sequences counts once) plus q, out and the table entries used; the
logical bytes (every sequence's tokens counted in full) are a side figure.
Per-kernel p10/p50/p90 come from a pass with events between the kernels of
each step. The line also carries the practical HBM read ceiling measured by
the library's read probe on the same device.
"""
import argparse
import glob
import hashlib
import re
import json
import math
import os
import shutil
import subprocess
import sys
import tempfile
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
    ap.add_argument("--cpu-baseline-child", default=None, help=argparse.SUPPRESS)
    return ap.parse_args()


def _code_only(text):
    """C/C++ source without its comments and blank space."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    """Hash of the library's sources (code only: comments and blank space do
    not count), which keys the stored counters to the code they were taken
    from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_52_amd", "csrc")
    paths = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc)) if f.endswith((".hip", ".h"))]
    for path in paths + [os.path.join(ROOT, "include", "pagedattn.h")]:
        h.update(_code_only(open(path, encoding="utf-8").read()).encode())
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
    """Bytes one decode step must move by definition: the K and V rows (plus
    INT8 / FP8 scales) of every token some query token attends (with a
    sliding window only the tokens it reaches; nothing of a sequence without
    query tokens), q, out, the block-table entries used and the lengths.
    Returns (unique, logical): unique counts each pool slot once however many
    sequences attend it (shared prefix blocks), logical counts every
    sequence's tokens in full. The two differ only when tables share blocks."""
    import numpy as np
    import workloads
    L = b.context_lens.to("cpu").numpy().astype(np.int64)
    Qs = query_counts(b)
    lo = workloads.reach_start(L, Qs, b.window)
    live = Qs > 0
    w = b.workload
    per_token = workloads.kv_bytes_per_token(w.num_kv_heads, w.head_dim, w.cache_dtype)
    kv_logical = int((L - lo)[live].sum()) * per_token
    tables = b.block_tables.to("cpu").numpy()[live]
    slots = workloads.attended_slots(tables, L[live], lo[live])
    kv_unique = int(np.unique(slots).size) * per_token
    qo = 2 * b.q.numel() * b.q.element_size()  # out has q's shape and dtype
    meta = int(((L + 15) // 16 - lo // 16)[live].sum()) * 4 + L.size * 4
    if b.query_start is not None:
        meta += (L.size + 1) * 4
    return kv_unique + qo + meta, kv_logical + qo + meta, kv_unique, kv_logical


def fragmentation(b):
    """Internal fragmentation of the batch's K/V memory [LLM Primer ch. 8,
    8.1]: the fraction of reserved token slots that hold no token. `paged`:
    the distinct 16-token blocks the tables reference for the tokens they
    hold (shared blocks once) against those tokens; `max_length_slots`: every
    sequence reserving a contiguous slot of the batch's longest context, with
    its whole context stored privately."""
    import numpy as np
    import workloads
    L = b.context_lens.to("cpu").numpy().astype(np.int64)
    lo = workloads.reach_start(L, query_counts(b), b.window) // 16 * 16
    tables = b.block_tables.to("cpu").numpy()
    slots = np.unique(workloads.attended_slots(tables, L, lo))
    blocks = np.unique(slots // 16)
    paged = 1.0 - slots.size / (16.0 * max(blocks.size, 1))
    maxlen = 1.0 - float(L.sum()) / max(1, L.size * int(L.max(initial=0)))
    return {"paged": paged, "max_length_slots": maxlen,
            "paged_figure_of_the_primer": 0.04}


def host_description():
    """CPU model, NUMA nodes and usable cores of the machine the CPU baseline
    runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    nodes = len(glob.glob("/sys/devices/system/node/node[0-9]*")) or 1
    return {"cpu_model": model, "numa_nodes": nodes, "usable_cpus": len(os.sched_getaffinity(0))}


# Binding of the CPU baseline's OpenMP threads: one per core, close together.
CPU_BASELINE_ENV = {"OMP_PROC_BIND": "close", "OMP_PLACES": "cores"}


def cpu_baseline(b, seconds):
    """Time the oracle on a bounded sample of the same batch: whole sequences
    (all heads) in order until about `seconds` of CPU time have passed. It
    runs in a child process started with CPU_BASELINE_ENV (OpenMP binds the
    thread that starts its runtime, so the binding stays out of this GPU
    process), on the batch's host copies handed over as .npy files."""
    import numpy as np
    import torch

    def host(t):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy()
        return t.numpy()

    arrays = {"q": b.q, "k_cache": b.k_cache, "v_cache": b.v_cache, "k_scale": b.k_scale,
              "v_scale": b.v_scale, "block_tables": b.block_tables,
              "context_lens": b.context_lens, "query_start": b.query_start}
    arrays = {k: host(v) for k, v in arrays.items() if v is not None}
    need = sum(a.nbytes for a in arrays.values())
    shm = "/dev/shm" if os.path.isdir("/dev/shm") and \
        shutil.disk_usage("/dev/shm").free > 2 * need else None
    d = tempfile.mkdtemp(prefix="pa_cpu_baseline_", dir=shm)
    try:
        for k, a in arrays.items():
            np.save(os.path.join(d, k + ".npy"), a)
        del arrays
        with open(os.path.join(d, "meta.json"), "w") as f:
            json.dump({"scale": b.scale, "window": b.window, "query_tokens": b.query_tokens,
                       "seconds": seconds}, f)
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", d],
                           env=dict(os.environ, **CPU_BASELINE_ENV), capture_output=True,
                           text=True, timeout=600 + 2 * seconds)
        if r.returncode != 0:
            raise RuntimeError(f"CPU baseline failed ({r.returncode}): {r.stderr[-2000:]}")
        return json.loads(r.stdout.strip().splitlines()[-1])
    finally:
        shutil.rmtree(d, ignore_errors=True)


def cpu_baseline_child(d):
    """The CPU baseline's own process: the oracle over whole sequences of the
    batch in `d`. On a machine with several NUMA nodes a pool over 1 GiB is
    first spread over all of them."""
    import numpy as np
    hw = host_description()  # before OpenMP starts and binds this thread
    import oracle
    with open(os.path.join(d, "meta.json")) as f:
        meta = json.load(f)
    arr = {os.path.basename(p)[:-4]: np.load(p) for p in glob.glob(os.path.join(d, "*.npy"))}
    q, kc, vc = arr["q"], arr["k_cache"], arr["v_cache"]
    ks, vs, qs = arr.get("k_scale"), arr.get("v_scale"), arr.get("query_start")
    bt, cl = arr["block_tables"], arr["context_lens"]
    pool = kc.nbytes + vc.nbytes
    policy = "first touch (one NUMA node)" if hw["numa_nodes"] == 1 else \
        f"first touch (pool {pool / 2**30:.2f} GiB, not over 1 GiB)"
    if hw["numa_nodes"] > 1 and pool > 2**30:
        errs = [oracle.interleave(a, hw["numa_nodes"]) for a in (kc, vc)]
        policy = (f"interleaved over {hw['numa_nodes']} nodes" if not any(errs) else
                  f"interleave failed (errno {max(errs)}), first touch")
    B, Hq = len(cl), q.shape[-2]
    Qs = np.diff(qs.astype(np.int64)) if qs is not None else \
        np.full(B, meta["query_tokens"], dtype=np.int64)
    done, tokens, queries, t0 = 0, 0, 0, time.perf_counter()
    elapsed = 0.0
    # Whole sequences in batch order, wrapping around, until the time budget.
    while elapsed < meta["seconds"]:
        s = done % B
        Q = int(Qs[s])
        tok = np.repeat(np.arange(Q, dtype=np.int32), Hq)
        h = np.tile(np.arange(Hq, dtype=np.int32), Q)
        oracle.decode(q, kc, vc, bt, cl, meta["scale"], ks, vs,
                      rows=(np.full(Q * Hq, s, np.int32), tok, h), window=meta["window"],
                      query_start=qs)
        tokens += int(cl[s])
        queries += Q
        done += 1
        elapsed = time.perf_counter() - t0
    print(json.dumps({
        "value": queries / elapsed, "unit": "tokens/s", "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{done} sequences ({done / B:.2f} passes over the {B}-sequence batch, "
                  f"{queries} query tokens x {Hq} q heads, {tokens} context tokens), fp64 "
                  f"block-table walk, {elapsed:.1f} s",
        "host": dict(hw, omp_threads=oracle.num_threads(), omp_proc_bind=oracle.proc_bind(),
                     omp_places=os.environ.get("OMP_PLACES", ""), numa_policy=policy),
    }), flush=True)


def run_tag(args):
    """Suffix naming a run's departures from the workload's defaults (it
    selects the committed counter file that belongs to the run)."""
    tag = ""
    if args.split_tokens:
        tag += f"_T{args.split_tokens}"
    if args.group_members:
        tag += f"_M{args.group_members}"
    if args.contiguous_tables:
        tag += "_contiguous"
    if args.seed != 1:
        tag += f"_seed{args.seed}"
    if args.ctx_range:
        tag += f"_ctx{args.ctx_range[0]}-{args.ctx_range[1]}"
    return tag


def load_counters(workload, tag, launch):
    """HBM bytes per launch from committed rocprofv3 counter runs of this
    workload and launch configuration, if they were taken on the current
    kernel sources."""
    try:
        with open(os.path.join(PROFILES, f"decode_{workload}{tag}_counters.json")) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash() or c.get("launch") != launch:
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


class Step:
    """One decode step of one attention layer, exactly as the benchmark times
    it: paged_decode_prepare (the step's new tokens written into the pool and
    the split plan made, one launch), paged_attn_decode_partial (the split
    kernel, through that plan) and paged_attn_reduce into `out` (q's dtype).
    split_tokens 0 takes the library default; group_members 0 takes 4 (group
    entries over shared blocks) for shared-prefix batches without a window or
    packed queries, else 1. The parity tests run this same object."""

    def __init__(self, pa, b, split_tokens=0, group_members=0):
        import torch
        w = b.workload
        dev = b.q.device
        self.pa, self.b = pa, b
        B, Hq, D = b.num_seqs, b.q.shape[-2], b.q.shape[-1]
        W = b.window
        self.packed = packed = b.query_start is not None
        # Query tokens: per sequence, or the packed total N (per-sequence counts).
        Q = b.q.shape[0] if packed else b.query_tokens
        self.num_query_tokens = Q
        self.n_query = b.q.shape[0] if packed else B * Q
        Qb = min(Q, pa.MAX_QUERY_TOKENS) if packed else Q          # per-sequence bound
        Qd = max(1, min(pa.MAX_QUERY_TOKENS, -(-Q // B))) if packed else Q  # default-T count
        self.mb = mb = b.block_tables.shape[1]
        self.T = T = split_tokens or pa.default_split_tokens(
            B, Hq, w.num_kv_heads, w.head_dim, b.k_cache.dtype, b.max_context_len, Qd, W)
        self.S = S = pa.max_splits(min(b.max_context_len, mb * 16), T, Qb, W)
        self.out = torch.empty_like(b.q)
        lead = (self.n_query, Hq) if packed else (B, Q, Hq)
        self.parts = pa.Partials(
            m=torch.empty(lead + (S,), dtype=torch.float32, device=dev),
            l=torch.empty(lead + (S,), dtype=torch.float32, device=dev),
            acc=torch.empty(lead + (S, D), dtype=torch.float32, device=dev),
            context_lens=b.context_lens, split_tokens=T, sliding_window=W,
            query_start=b.query_start)
        self.sched = torch.empty(pa.sched_bytes(B, S, Q if packed else None,
                                                Hq // w.num_kv_heads) // 4,
                                 dtype=torch.int32, device=dev)
        self.M = group_members or (4 if w.groups and W == 0 and not packed else 1)
        self.plan = None

    def prepare(self):
        b = self.b
        self.plan = self.pa.paged_decode_prepare(
            b.new_k, b.new_v, b.slot_mapping, b.k_cache, b.v_cache, b.context_lens, self.mb,
            b.k_scale, b.v_scale, max_context_len=b.max_context_len, split_tokens=self.T,
            num_query_tokens=self.num_query_tokens, sliding_window=b.window,
            num_q_heads=b.q.shape[-2], query_start=b.query_start, block_tables=b.block_tables,
            group_members=self.M, sched=self.sched)

    def decode(self):
        b = self.b
        self.pa.paged_attn_decode_partial(
            b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, b.scale, b.k_scale,
            b.v_scale, max_context_len=b.max_context_len, split_tokens=self.T,
            sliding_window=b.window, plan=self.plan, query_start=b.query_start,
            partials=self.parts)

    def reduce(self, out=None):
        self.pa.paged_attn_reduce(self.parts, self.out if out is None else out)

    def write(self):
        b = self.b
        self.pa.paged_kv_write(b.new_k, b.new_v, b.slot_mapping, b.k_cache, b.v_cache, b.k_scale,
                               b.v_scale)

    def __call__(self):
        self.prepare()
        self.decode()
        self.reduce()

    def layer(self):
        """One more attention layer of the same decode step: the plan of the
        step's prepare() serves every layer, so a layer writes its new K/V
        rows and runs the split kernel and the reduce."""
        self.write()
        self.decode()
        self.reduce()


def main():
    args = parse()
    if args.cpu_baseline_child:
        cpu_baseline_child(args.cpu_baseline_child)
        return
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
    st = Step(pa, b, args.split_tokens, args.group_members)
    B, Hq, D = b.num_seqs, b.q.shape[-2], b.q.shape[-1]
    W, T, S, M = b.window, st.T, st.S, st.M
    packed, n_query = st.packed, st.n_query
    stream = torch.cuda.current_stream(dev)

    for _ in range(args.warmup):
        st()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` whole steps.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        st()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps

    # Per-kernel durations: identical launches with events between them.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evs:
        e[0].record(stream); st.prepare()
        e[1].record(stream); st.decode()
        e[2].record(stream); st.reduce()
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
        st.decode()
    d1.record(stream)
    torch.cuda.synchronize()
    t_dec_b2b = d0.elapsed_time(d1) / args.steps

    # Later layers of a step: the plan is made once per step and reused, so a
    # layer is the KV write (alone), the split kernel and the reduce.
    st.prepare()
    l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    l0.record(stream)
    for _ in range(args.steps):
        st.layer()
    l1.record(stream)
    torch.cuda.synchronize()
    ms_layer = l0.elapsed_time(l1) / args.steps

    alg_bytes, logical_bytes, kv_unique, kv_logical = algorithmic_bytes(b)
    alg_flops = algorithmic_flops(b)
    dec_gbps = alg_bytes / (t_dec_b2b * 1e-3) / 1e9
    dec_tflops = alg_flops / (t_dec_b2b * 1e-3) / 1e12
    # The kernel's bound: matrix cores once its arithmetic intensity passes
    # the ridge point of the two peaks (dense bf16 MFMA / HBM).
    mfma_bound = alg_flops / alg_bytes > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    kv_gbps_step = kv_unique / (ms_step * 1e-3) / 1e9
    launch = {"split_tokens": T, "group_members": M,
              "tables": "contiguous" if args.contiguous_tables else "permuted"}
    counters = load_counters(w.name, run_tag(args), launch)
    traffic = None
    if counters is not None:
        traffic = counters["fetch_bytes_per_launch"] + counters["write_bytes_per_launch"]
    probe_gbps = hbm_probe(pa, torch, dev, stream, args.probe_mib) if args.probe_mib else None
    shared = kv_unique != kv_logical

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
            "query_tokens": (f"packed: {n_query} over {B} sequences" if packed else
                             st.num_query_tokens),
            "sliding_window": W, "group_members": M,
            "tables": "contiguous" if args.contiguous_tables else "permuted",
            "context_range": list(args.ctx_range) if args.ctx_range else
            [b.workload.ctx_lo, b.workload.ctx_hi],
            "seed": args.seed,
        },
        "kv_read_gbps": kv_gbps_step,
        "kv_read_frac_of_peak": kv_gbps_step / HBM_PEAK_GBPS,
        "decode_reduce_tokens_per_s": n_query / ((t_dec + t_red) * 1e-3),
        "layer_step_plan_reused": {
            "ms": ms_layer, "tokens_per_s": n_query / (ms_layer * 1e-3),
            "kv_read_gbps": kv_unique / (ms_layer * 1e-3) / 1e9,
            "kv_read_frac_of_peak": kv_unique / (ms_layer * 1e-3) / 1e9 / HBM_PEAK_GBPS},
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
        "fragmentation": fragmentation(b),
        "wall_s_timed": wall,
    }
    if shared:
        # Blocks shared by several sequences: the roofline counts them once;
        # the logical figure counts every sequence's tokens in full (it can
        # pass the HBM peak, since a shared block is read once for several).
        line["roofline"]["bytes_basis"] = "unique"
        line["roofline"]["algorithmic_bytes_logical"] = logical_bytes
        line["roofline"]["logical_gbps"] = logical_bytes / (t_dec_b2b * 1e-3) / 1e9
        line["kv_read_gbps_logical"] = kv_logical / (ms_step * 1e-3) / 1e9
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
