"""Benchmark of the sparse MLA decode hot path on one MI355X.

One step = one mla_sparse_decode call over one batch of synthetic input already resident in HBM
(the decode kernel, plus the log-sum-exp merge kernel when the schedule splits rows); the tile
scheduler metadata is computed once before the loop, as the method prescribes, and timed separately.
Successive steps cycle through independent index sets over the same paged pool, enough of them that
the records one cycle selects exceed 512 MiB: by the time a set comes round again, its records have
been pushed out of L2 and the 256 MiB Infinity Cache by the other sets' traffic, so the timed steps
read their records from HBM. The long workload selects every token of its 553 MB pool in order, a
stream larger than the Infinity Cache, and uses one set.

Prints one JSON line: TFLOP/s over valid selected tokens (2 * h_q * (512 + 512) flops per valid
token and row), KV GB/s, the roofline block for the decode kernel, and the CPU oracle baseline.

Right after an idle period the GPU's power management holds the decode kernel about 20% below its
sustained rate for roughly the first 100 launches (~15 ms). Before the --warmup steps, every mode
therefore runs untimed steps of the same call for --prewarm-s seconds of wall time (0.3 s by
default; the JSON line reports the time and step count as prewarm_s and prewarm_steps), so that
even a short timed run measures a decode loop's steady state rather than that transient. The timed
region is unchanged: exactly --steps calls, bracketed by HIP events on the launch stream. With
--graph those calls are captured once as a HIP graph and the timed region replays it, so that steps
shorter than the host's launch time (the mid and mixed workloads, or any run under a kernel tracer)
measure the GPU rather than the launch rate.

  python bench.py [--gpus 1] [--steps 2000] [--warmup 300] [--prewarm-s 0.3] [--config 2]
                  [--batch N] [--parts N] [--graph] [--no-cpu-baseline]
"""
import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "sparse MLA decode TFLOP/s + KV GB/s, fp8 528B/tok, B=128 H=128 topk=2048"
CSRC = os.path.join(ROOT, "sparse_mla_decode_get_amd", "csrc")
# decode kernel sources (and the headers they include) for head counts above 64 and up to 64 (the
# single-stream and the two-half kernel, either of which the schedule may select)
DECODE_SRCS = {True: ["mla_decode_wide.hip", "mla_device.h", "mla_internal.h"],
               False: ["mla_decode_h64.hip", "mla_decode.hip", "mla_device.h", "mla_internal.h"]}


def kernel_source_hash(wide: bool) -> str:
    """Hash of the decode kernel's sources (stored counter traffic is valid only for them)."""
    h = hashlib.sha256()
    for f in DECODE_SRCS[wide]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(config: int, wide: bool):
    """HBM bytes per launch measured with rocprofv3 --pmc for this decode kernel source, if the
    committed counter summary was taken on the current kernel; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"mla_decode_config{config}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_hash(wide):
        return None
    return float(m_b.group(1))


def cpu_baseline(w, seconds: float):
    """Time the float64 oracle (as it stands) on whole rows of the same workload until `seconds`."""
    from oracle import oracle_decode_rows
    spec = w["spec"]
    rows = spec.rows
    order = np.random.default_rng(0).permutation(rows)
    done, flops, kv = 0, 0.0, 0.0
    idx = w["indices"].reshape(rows, -1)
    xidx = None if w["extra_indices"] is None else w["extra_indices"].reshape(rows, -1)
    t0 = time.perf_counter()
    while done < rows and time.perf_counter() - t0 < seconds:
        r = int(order[done])
        oracle_decode_rows(w["q_bits"], w["k_cache"], w["indices"], w["softmax_scale"], [r],
                           w["extra_k_cache"], w["extra_indices"])
        nv = int((idx[r] >= 0).sum())
        nx = 0 if xidx is None else int((xidx[r] >= 0).sum())
        flops += 2.0 * spec.h_q * 1024 * (nv + nx)
        kv += 528.0 * nv + 288.0 * nx
        done += 1
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas = max(i.get("num_threads", 1) for i in info) if info else 1
    except Exception:
        blas = None
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "blas_threads": blas,
            "kind": "oracle",
            "sample": f"{done} of {rows} query rows of the same workload (all {spec.h_q} heads each), "
                      f"{dt:.1f} s wall, float64 NumPy oracle on the host; KV {kv / dt / 1e9:.3f} GB/s"}


def prewarm(step, seconds: float):
    """Untimed calls of `step` until `seconds` of wall time have passed (synchronizing every 32
    calls), to bring the GPU's clocks out of their idle state. Returns (elapsed seconds, calls)."""
    import torch
    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(32):
            step(k)
            k += 1
        torch.cuda.synchronize()
    return time.perf_counter() - t0, k


def bench_quantize(args):
    """The cache writer: one step quantizes `--tokens` bf16 latents (N(0,1) per 32-value block times
    2^u, u ~ U(-4, 4)) into records scattered to random distinct token slots of a pool twice that
    size. HBM-bound: each token reads 1024 B of bf16 and 4 B of slot and writes one record."""
    import torch

    import sparse_mla_decode_get_amd as mla
    mla.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    n, rec = args.tokens, args.record
    rng = np.random.default_rng(77)
    sets = []
    for k in range(2):                     # two input sets alternate, each larger than the MALL
        x = torch.randn((n, 512), dtype=torch.float32, generator=torch.Generator().manual_seed(k))
        x = (x.view(n, 16, 32) * torch.exp2(torch.empty((n, 16, 1)).uniform_(-4, 4))).view(n, 512)
        slots = torch.from_numpy(rng.permutation(2 * n)[:n].astype(np.int32))
        sets.append((x.to(torch.bfloat16).to(dev), slots.to(dev)))
    cache = torch.zeros((2 * n, rec), dtype=torch.uint8, device=dev)

    def step(k):
        x, slots = sets[k % 2]
        mla.quantize_records(x, rec, cache=cache, slots=slots)

    pw_s, pw_n = prewarm(step, args.prewarm_s)
    for k in range(args.warmup):
        step(k)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for k in range(args.steps):
        step(k)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    alg = n * (1024.0 + 4.0 + rec)
    gbs = alg / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": f"cache writer GB/s, bf16 -> {rec} B records", "value": gbs, "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "prewarm_s": pw_s, "prewarm_steps": pw_n,
        "config": {"workload": f"quantize {n} bf16 latents into {rec} B records at random slots of a "
                               f"{2 * n}-token pool", "tokens": n, "record_bytes": rec},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        "cpu_baseline": None}))


def bench_prefill(args):
    """Sparse prefill: --seq-q query rows of one sequence (128 heads) over a 65536-token fp8 cache,
    2048 distinct selected tokens per row with the last 0-10% ignored, values spread over 2^+-4 per
    32-block (the headline decode's per-row recipe). Two index sets alternate between steps; the
    selected records (~1 GB per set at 4096 rows, read with heavy reuse) come through L2/MALL."""
    import torch

    import sparse_mla_decode_get_amd as mla
    from workloads import Spec, add_index_set, make_workload
    mla.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    s_q, h, topk = args.seq_q, 128, 2048
    spec = Spec("prefill", 1, s_q, h, topk, 65536, values="spread", neg="tail10")
    w = make_workload(spec, seed=3000)
    sets = [w["indices"], add_index_set(w, 3001)]
    q = torch.from_numpy(w["q_bits"].view(np.int16)).view(torch.bfloat16).to(dev).reshape(s_q, h, 512)
    k_cache = torch.from_numpy(w["k_cache"]).to(dev)
    idx = [torch.from_numpy(x.reshape(s_q, topk)).to(dev) for x in sets]
    out = torch.empty((s_q, h, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((s_q, h), dtype=torch.float32, device=dev)

    def step(k):
        mla.sparse_prefill(q, k_cache, idx[k % 2], w["softmax_scale"], out=out, lse=lse)

    pw_s, pw_n = prewarm(step, args.prewarm_s)
    for k in range(args.warmup):
        step(k)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for k in range(args.steps):
        step(k)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nv = np.mean([(sets[k % 2] >= 0).sum() for k in range(args.steps)])
    flops = 2.0 * h * 1024 * nv
    tflops = flops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "sparse MLA prefill TFLOP/s, fp8 528B/tok, H=128 topk=2048", "value": tflops,
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic", "prewarm_s": pw_s, "prewarm_steps": pw_n,
        "config": {"workload": f"sparse prefill: {s_q} query rows, h_q {h}, topk {topk} over a "
                               "65536-token cache, 528 B fp8 records", "seq_len_q": s_q, "h_q": h,
                   "topk": topk},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / BF16_MFMA_PEAK_TFLOPS, "traffic": None},
        "valid_tokens_per_step": float(nv), "cpu_baseline": None}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--prewarm-s", type=float, default=0.3,
                    help="untimed steps for this many seconds before the warm-up steps")
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--batch", type=int, default=0,
                    help="run the --config workload's per-row recipe at this batch instead (0: the "
                         "config's own); fewer rows leave CUs idle, for occupancy and clock studies")
    ap.add_argument("--parts", type=int, default=0,
                    help="decode parts of the schedule (0: the library's default for the shape)")
    ap.add_argument("--sets", type=int, default=0,
                    help="independent index sets cycled over steps (0: enough that one cycle "
                         "selects more than 512 MiB of records, at least 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed steps as one HIP graph and replay it (decode and fused)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one 1 GiB device copy first (calibrates HBM byte counters)")
    ap.add_argument("--op", choices=["decode", "quantize", "prefill", "fused"], default="decode",
                    help="decode (the hot path, default), quantize (the cache writer), prefill "
                         "(sparse prefill, --seq-q query rows of one sequence) or fused (the fused "
                         "norm-RoPE-attention-RoPE-fp8 decode on the --config workload)")
    ap.add_argument("--seq-q", type=int, default=4096, help="--op prefill: query rows")
    ap.add_argument("--tokens", type=int, default=1 << 20, help="--op quantize: tokens per step")
    ap.add_argument("--record", type=int, default=528, help="--op quantize: 528 (fp8) or 288 (fp4)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(rows shard across GPUs with no exchange; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    if args.op == "quantize":
        bench_quantize(args)
        return
    if args.op == "prefill":
        bench_prefill(args)
        return

    import torch

    import sparse_mla_decode_get_amd as mla
    from workloads import CONFIGS, add_extra_index_set, add_index_set, make_workload

    mla.load_library()          # fails loudly when the HIP library is missing
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    t_gen = time.perf_counter()
    if args.batch > 0:
        w = make_workload(dataclasses.replace(CONFIGS[args.config], batch=args.batch),
                          seed=1000 + args.config)
    else:
        w = make_workload(args.config)
    spec = w["spec"]
    set_kv = 528.0 * (w["indices"] >= 0).sum() + (
        0.0 if w["extra_indices"] is None else 288.0 * (w["extra_indices"] >= 0).sum())
    n_sets = args.sets or max(4, int(np.ceil(512 * 2**20 / set_kv)) + 1)
    if spec.order != "random":
        n_sets = 1
    sets = [w["indices"]] + [add_index_set(w, 5000 + k) for k in range(n_sets - 1)]
    xsets = None
    if w["extra_indices"] is not None:
        xsets = [w["extra_indices"]] + [add_extra_index_set(w, 7000 + k) for k in range(n_sets - 1)]
    t_gen = time.perf_counter() - t_gen

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    q = torch.from_numpy(w["q_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
    k_cache = torch.from_numpy(w["k_cache"]).to(dev)
    idx_sets = [torch.from_numpy(s).to(dev) for s in sets]
    xc = None
    xidx_sets = [None] * len(sets)
    if w["extra_k_cache"] is not None:
        xc = torch.from_numpy(w["extra_k_cache"]).to(dev)
        xidx_sets = [torch.from_numpy(s).to(dev) for s in xsets]
    b, s, h = spec.batch, spec.seq_len_q, spec.h_q
    out = torch.empty((b, s, h, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b, s, h), dtype=torch.float32, device=dev)

    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    md = mla.get_metadata(b, s, h, spec.topk, spec.extra_topk,
                          **({"num_parts": args.parts} if args.parts > 0 else {}))
    e1.record(stream)
    torch.cuda.synchronize()
    metadata_ms = e0.elapsed_time(e1)

    if args.op == "fused":
        # the fused decode reads the raw query: an RMSNorm weight near 1 and rotary angles of
        # random positions (base 10000 over the 32 pairs), as a model's decode step would pass
        rng = np.random.default_rng(9)
        qn_w = torch.from_numpy((1 + 0.1 * rng.standard_normal(512)).astype(np.float32)).to(
            torch.bfloat16).to(dev)
        ang = rng.integers(0, 65536, b * s)[:, None] * 10000.0 ** (-np.arange(32) / 32.0)
        r_cos = torch.from_numpy(np.cos(ang).astype(np.float32).reshape(b, s, 32)).to(dev)
        r_sin = torch.from_numpy(np.sin(ang).astype(np.float32).reshape(b, s, 32)).to(dev)
        out = torch.empty((b, s, h, 528), dtype=torch.uint8, device=dev)

    def step(k):
        j = k % len(idx_sets)
        if args.op == "fused":
            mla.sparse_decode_fused(q, qn_w, 1e-6, r_cos, r_sin, k_cache, idx_sets[j],
                                    w["softmax_scale"], md, xc, xidx_sets[j], out=out, lse=lse)
        else:
            mla.sparse_decode(q, k_cache, idx_sets[j], w["softmax_scale"], md, xc, xidx_sets[j],
                              out=out, lse=lse)

    pw_s, pw_n = prewarm(step, args.prewarm_s)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        # the timed steps captured once as one HIP graph: the same --steps calls, replayed with no
        # host launch work between them (short steps otherwise measure the host's launch rate)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(args.steps):
                step(k)
        graph.replay()                      # untimed first replay
        torch.cuda.synchronize()

    # HIP events on the launch stream bracket the timed region only: an event recorded between
    # two launches costs the GPU several microseconds, so per-step events would time themselves
    # along with short steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for k in range(args.steps):
            step(k)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e0.elapsed_time(e1)
    per_launch_ms = total_ms / args.steps      # one decode call (decode kernel, plus the merge)
    ms_per_step = total_ms / args.steps

    # algorithmic work per step (valid tokens only), averaged over the index sets the steps used
    nv = np.mean([[(sets[k % len(sets)] >= 0).sum()] for k in range(args.steps)])
    nx = 0 if xsets is None else np.mean([[(xsets[k % len(xsets)] >= 0).sum()]
                                          for k in range(args.steps)])
    flops = 2.0 * h * 1024 * (nv + nx)
    kv_bytes = 528.0 * nv + 288.0 * nx
    rows = b * s
    alg_bytes = kv_bytes + 4.0 * rows * (spec.topk + spec.extra_topk) + 2 * rows * h * 512 * 2 \
        + rows * h * 4
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    kv_gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    intensity = flops / alg_bytes
    ridge = BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity >= ridge:
        roof = {"bound": "mfma", "achieved": flops / (per_launch_ms * 1e-3) / 1e12,
                "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": alg_bytes / (per_launch_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(args.config, h > 64)

    # measured HBM bandwidth of a plain 1 GiB device-to-device copy (read + write bytes over time),
    # reported beside the 8 TB/s spec; taken after the timed region
    copy_gbs = None
    if not args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        c0.record()
        for _ in range(reps):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        copy_gbs = 2.0 * src.numel() * reps / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    line = {
        "metric": METRIC if args.op == "decode" else
        "fused norm-RoPE-sparse MLA-RoPE-fp8 decode TFLOP/s, fp8 528B/tok, B=128 H=128 topk=2048",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_s": pw_s,
        "prewarm_steps": pw_n,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{spec.name} {'fused ' if args.op == 'fused' else ''}sparse MLA decode: batch {b}, seq_len_q {s}, h_q {h}, "
                               f"topk {spec.topk}" + (f" + extra {spec.extra_topk} fp4" if spec.extra_topk else "")
                               + f", {spec.tokens_per_seq} tokens per sequence in 64-token blocks, "
                               f"528 B fp8 records",
                   "batch": b, "seq_len_q": s, "h_q": h, "topk": spec.topk,
                   "extra_topk": spec.extra_topk, "index_sets": len(sets),
                   "num_parts": md.num_parts},
        "kv_gbps": kv_gbs,
        "alg_gbps": alg_bytes / (ms_per_step * 1e-3) / 1e9,
        "valid_tokens_per_step": float(nv + nx),
        "hbm_frac": alg_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "hbm_copy_gbps_measured": copy_gbs,
        "index_set_mib_per_cycle": len(sets) * set_kv / 2**20,
        "metadata_ms": metadata_ms,
        "per_launch_ms": per_launch_ms,
        "graph": bool(args.graph),
        "wall_s_timed": wall,
        "gen_s": t_gen,
        "kernel_source_sha256_16": kernel_source_hash(h > 64),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
