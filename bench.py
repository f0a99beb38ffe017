#!/usr/bin/env python3
"""Benchmark: paged decode attention on one MI355X.

A step is one pass of the whole hot path over the 40-layer GQA workload
(40 sequences of 8192 tokens, 32 query / 8 KV heads, d 128, fp16 KV in
16-token blocks, one block table shared by all layers): for each of the 40
layers, append the new token's K/V rows through the slot mapping, then run
paged decode (one launch: the batch's tiles split evenly over the device's
worker waves, split segments merged by log-sum-exp inside it). Every layer
has its own 1.25 GiB of cache, so nothing is served from a cache level across
layers; all inputs are resident in HBM before timing starts.

Printed (one JSON line, last): value = algorithmic KV bytes read per second
(GB/s, 1e9), decode sequences per second, and the roofline of the dominant
kernel (the decode kernel, one launch per layer) timed with HIP events on the
stream it runs on, plus the CPU oracle timed on a bounded sample of the same
workload on this host's cores.

Other workloads (--workload gqa40_tp8|qwen|prefix|prefix_shared|fp8|tiny)
print the same fields; they are for profiling, not the headline line.
gqa40_tp8 is the same 40-layer step at one GPU's share under 8-way KV-head
parallelism (4 query / 1 KV head). The others time the decode call alone.
prefix_shared is the prefix workload through the shared-prefix decode (each
shared block read once per KV head): its value and roofline count the unique
KV bytes (the shared prefix once, every suffix), and it also reports the
logical bytes plain decode would read. --cold adds launches timed after a
1 GiB write that evicts the caches (a small layer such as qwen's otherwise
stays in the 256 MB MALL between iterations).

--workload prefill times one chunked-prefill step (four 2048-token chunks at
contexts 2048..8192, fp16, the 32/8-head d-128 shape) in TFLOP/s against the
matrix-core peak; --workload prefill_small times eight 16-token chunks over
8192-token contexts (keys split over workgroups through the workspace; HBM
bound) and also reports the unsplit launch. Both warm up for at least
PREFILL_MIN_WARMUP_S before timing, since a launch is too short for the clock
to settle within a few warm-up steps.
"""
import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "fp8": 2500.0, "f32": 157.3}
# (fp8 KV is widened to the 16-bit query type before the matrix cores: its
# products run at the 16-bit rate; float32 caches use the float32 MFMA)

# Chunked-prefill step: one 2048-token chunk (the pages' deployment token
# budget) for each of four sequences at different stages of their prompts,
# in the 40-layer GQA head shape.
PREFILL_CONTEXTS = [2048, 4096, 6144, 8192]
PREFILL_CHUNK = 2048
# Few-row prefill: 16-token chunks (a chunked prefill's tail, or a few draft
# tokens checked at once) of eight sequences at 8192-token contexts. Each KV
# head has one 128-row tile per sequence, so the keys are split over
# workgroups (the prefill workspace); the step reads each sequence's KV once
# and is bound by HBM.
PREFILL_SMALL_CONTEXTS = [8192] * 8
PREFILL_SMALL_CHUNK = 16
PREFILL_MIN_WARMUP_S = 0.25  # untimed warm-up of the prefill workloads, at least


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa40",
                    choices=["gqa40", "gqa40_tp8", "qwen", "prefix", "prefix_shared", "fp8", "tiny",
                             "prefill", "prefill_small"])
    ap.add_argument("--workers", type=int, default=0, help="worker waves (0 = fill the device)")
    ap.add_argument("--partition-size", type=int, default=0,
                    help="decode split: 0 = balanced split, else tokens per fixed partition")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed (reported as "
                         "a 'graph' object; value and roofline stay the eager, event-timed run)")
    ap.add_argument("--cold", action="store_true",
                    help="also time decode launches that each follow a 1 GiB device write, "
                         "which evicts the L2 caches and the 256 MB MALL (the timed launch then "
                         "reads its KV from HBM)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (for counter scaling)")
    return ap.parse_args()


def kernel_hash() -> str:
    """Hash of the decode kernel sources: counter figures are valid only for
    the build they were taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in ("paged_decode.hip", "pkv_tile.h", "pkv_device.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_101_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM traffic per decode launch from the committed counter summary, or
    None if it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as fh:
        for line in fh:
            if line.startswith("{"):
                rec = json.loads(line)
    if rec is None or rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("traffic_bytes_per_launch", {}).get("total")


def copy_calibration(mib: int):
    import torch
    n = mib * 2**20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def build_layers(workload: str, device):
    from paged_kv_cache_101_amd import workloads as W
    if workload == "gqa40":
        layers = [W.gqa40_layer(device=device, layer=l, append_last=True) for l in range(40)]
    elif workload == "gqa40_tp8":
        layers = [W.gqa40_tp8_layer(device=device, layer=l, append_last=True) for l in range(40)]
    elif workload == "qwen":
        layers = [W.qwen_layer(device=device)]
    elif workload in ("prefix", "prefix_shared"):
        layers = [W.prefix_shared(device=device)]
    elif workload == "fp8":
        layers = [W.fp8_long(device=device)]
    else:
        layers = [W.tiny(device=device)]
    return layers


def describe(workload: str, layers, workers: int) -> dict:
    b = layers[0]
    return {
        "workload": {
            "gqa40": "40-layer GQA decode step: 40 layers x 40 seqs x 8192 ctx",
            "gqa40_tp8": "40-layer GQA decode step, one GPU's share under 8-way head "
                         "parallelism: 40 layers x 40 seqs x 8192 ctx, 4 query / 1 KV head",
            "qwen": "Qwen2.5-1.5B-shaped layer decode: 64 seqs, ctx U[128,4096]",
            "prefix": "prefix sharing decode: 256 seqs, 2048 shared + U[64,512] ctx",
            "prefix_shared": "prefix sharing decode, shared-prefix path: 256 seqs, "
                             "2048 shared + U[64,512] ctx",
            "fp8": "long-context fp8 decode: 16 seqs x 32768 ctx",
            "tiny": "tiny MQA decode: 4 seqs, ctx {1,15,16,33}",
        }[workload],
        "layers": len(layers), "num_seqs": b.num_seqs, "q_heads": b.num_q_heads,
        "kv_heads": b.num_kv_heads, "head_dim": b.head_dim, "kv_dtype": b.kv_dtype,
        "block_size": 16, "workers": workers or "device default",
    }


def cpu_baseline(layer, target_s: float):
    """The oracle (as it stands) on a bounded sample: the first k sequences of
    one layer, all their heads; k grows until about target_s of CPU work."""
    import numpy as np
    import oracle
    from paged_kv_cache_101_amd import workloads as W

    h = dict(q=W.to_numpy(layer.q), k=W.to_numpy(layer.k_cache), v=W.to_numpy(layer.v_cache),
             bt=layer.block_tables.cpu().numpy(), ctx=layer.context_lens.cpu().numpy())
    bpt = 2 * layer.num_kv_heads * layer.head_dim * W.STORAGE[layer.kv_dtype][1]

    def run(k):
        t0 = time.perf_counter()
        oracle.paged_decode(np.ascontiguousarray(h["q"][:k]), h["k"], h["v"],
                            np.ascontiguousarray(h["bt"][:k]), np.ascontiguousarray(h["ctx"][:k]),
                            layer.scale, layer.k_scale, layer.v_scale)
        return time.perf_counter() - t0

    k, el = 1, run(1)
    S = layer.num_seqs
    if el < target_s:
        k = max(1, min(S, int(target_s / max(el, 1e-3))))
        if k > 1:
            el = run(k)
    # a whole layer that still takes well under the target is timed over
    # several passes (at most 10), and the mean pass is reported
    passes = 1
    if k == S and el < target_s / 2:
        passes = min(10, max(2, int(target_s / max(el, 1e-3))))
        el = sum(run(k) for _ in range(passes)) / passes
    tokens = int(h["ctx"][:k].clip(min=0).sum())
    return {
        "value": round(tokens * bpt / el / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"layer 0, sequences 0..{k - 1} of {S} (all {layer.num_q_heads} query heads), "
                  f"{tokens} tokens, {tokens * bpt} KV bytes, {el:.2f} s per pass, "
                  f"mean of {passes} pass{'es' if passes > 1 else ''}",
        "seqs_per_s": round(k / el, 4),
    }


def prefill_flops(contexts, chunk, num_q_heads, head_dim) -> int:
    """4 * d * H_q flops per (query token, visible key): QK and P.V, a
    multiply and an add each."""
    total = 0
    for n in contexts:
        base = n - chunk
        total += sum(base + i + 1 for i in range(chunk))
    return 4 * head_dim * num_q_heads * total


def bench_prefill(args):
    import numpy as np
    import torch
    from paged_kv_cache_101_amd import binding as B
    from paged_kv_cache_101_amd import workloads as W

    dev = torch.device("cuda:0")
    Hq, H, d, dt = 32, 8, 128, "f16"
    small = args.workload == "prefill_small"
    contexts = PREFILL_SMALL_CONTEXTS if small else PREFILL_CONTEXTS
    chunk = PREFILL_SMALL_CHUNK if small else PREFILL_CHUNK
    b = W.make_batch("prefill-small" if small else "prefill-step", 8 if small else 6, contexts, Hq, H,
                     d, dt, dt, device=dev)
    desc = B.desc_for(b.k_cache, dt)
    kc, vc = B.fill_cache(b.k_cache, b.v_cache, desc)
    S = len(contexts)
    T = S * chunk
    g = torch.Generator(device=dev)
    g.manual_seed(66)
    q = torch.randn((T, Hq, d), generator=g, device=dev).to(torch.float16)
    qs = torch.arange(0, T + 1, chunk, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws = B.prefill_workspace(d, dev)
    stream = torch.cuda.current_stream()

    def timed(workspace):
        def step():
            B.pkv_paged_attention_prefill(q, kc, vc, desc, b.block_tables, b.context_lens, qs,
                                          b.scale, out, workspace=workspace)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        # A launch lasts well under a millisecond, too short for the GPU's
        # clock to settle within a few warm-up steps: keep warming up (untimed)
        # for at least PREFILL_MIN_WARMUP_S.
        t_end = time.perf_counter() + PREFILL_MIN_WARMUP_S
        while time.perf_counter() < t_end:
            for _ in range(20):
                step()
            torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in evs:
            e0.record(stream)
            step()
            e1.record(stream)
        torch.cuda.synchronize()
        return statistics.fmean(a.elapsed_time(c) for a, c in evs)

    avg = timed(ws)
    flops = prefill_flops(contexts, chunk, Hq, d)
    tflops = flops / (avg * 1e-3) / 1e12
    kv_bytes = sum(contexts) * H * 2 * d * 2  # each sequence's K and V, read once per KV head
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # sample: the first k rows of the last chunk (the longest contexts)
        kh, vh = W.to_numpy(b.k_cache), W.to_numpy(b.v_cache)
        bt, cl = b.block_tables.cpu().numpy(), b.context_lens.cpu().numpy()
        qh = W.to_numpy(q)
        k = 1
        while True:
            rows = np.arange(T - chunk, T - chunk + k)
            pos = cl[-1] - chunk + (rows - (T - chunk))
            t0 = time.perf_counter()
            oracle.paged_prefill(np.ascontiguousarray(qh[rows]), kh, vh,
                                 np.ascontiguousarray(bt[[S - 1] * k]), (pos + 1).astype(np.int32),
                                 np.arange(k + 1, dtype=np.int32), b.scale)
            el = time.perf_counter() - t0
            if el > args.cpu_seconds / 4 or k >= chunk:
                break
            k = min(chunk, k * 4)
        sample_flops = 4 * d * Hq * int((pos + 1).sum())
        cpu = {"value": round(sample_flops / el / 1e12, 6), "unit": "TFLOP/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"rows {int(rows[0])}..{int(rows[-1])} of the last chunk (context "
                         f"{int(cl[-1])}), all {Hq} query heads, {el:.2f} s"}
    line = {
        "metric": "paged chunked-prefill attention: TFLOP/s (% of MFMA peak)",
        "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(avg, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dt, "data": "synthetic",
        "config": {"workload": f"chunked prefill: {S} sequences x {chunk}-token chunks "
                               f"at contexts {contexts}", "q_heads": Hq, "kv_heads": H,
                   "head_dim": d, "kv_dtype": dt, "block_size": 16},
        "flops_per_step": flops, "kv_bytes_per_step": kv_bytes,
        "cpu_baseline": cpu,
    }
    if flops / kv_bytes < MFMA_PEAK_TFLOPS[dt] * 1e12 / (HBM_PEAK_GBS * 1e9):
        # below the ridge (few query rows per key): bound by reading the KV once
        gbs = kv_bytes / (avg * 1e-3) / 1e9
        line["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                            "kernel": "paged_prefill_kernel (split keys) + chunk_merge_kernel",
                            "launch_avg_us": round(avg * 1e3, 2)}
        line["unsplit_avg_us"] = round(timed(None) * 1e3, 2)  # the same call without a workspace
    else:
        line["roofline"] = {"bound": "mfma", "achieved": round(tflops, 1),
                            "peak": MFMA_PEAK_TFLOPS[dt], "unit": "TFLOP/s",
                            "frac": round(tflops / MFMA_PEAK_TFLOPS[dt], 4), "traffic": None,
                            "kernel": "paged_prefill_kernel (one launch per call)",
                            "launch_avg_us": round(avg * 1e3, 2)}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "paged decode shards over sequences or KV heads with no exchange, and this build "
              "measures the single-GPU share.", file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_cache_101_amd import binding as B
    from paged_kv_cache_101_amd import workloads as W

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.workload in ("prefill", "prefill_small"):
        B.lib()
        bench_prefill(args)
        return
    B.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    layers = build_layers(args.workload, dev)
    descs = [B.desc_for(b.k_cache, b.kv_dtype, b.k_scale, b.v_scale) for b in layers]
    # The library's caches, filled from each layer's token rows with
    # pkv_kv_append (the row-order copies are dropped after, except layer 0's,
    # which the CPU baseline reads).
    caches = []
    for i, b in enumerate(layers):
        caches.append(B.fill_cache(b.k_cache, b.v_cache, descs[i]))
        if i > 0:
            b.k_cache = b.v_cache = None
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    outs = [torch.empty_like(b.q) for b in layers]
    b0 = layers[0]
    shared = args.workload == "prefix_shared"
    if shared:
        ng = int(b0.group_prefix.numel())
        ws = B.shared_prefix_workspace(b0.num_seqs, b0.num_q_heads, b0.num_kv_heads, b0.head_dim,
                                       ng, args.workers, dev)
    else:
        ws = B.decode_workspace(b0.num_seqs, b0.num_q_heads, b0.num_kv_heads, b0.head_dim,
                                args.workers, dev, b0.max_blocks_per_seq, args.partition_size)
    do_append = args.workload in ("gqa40", "gqa40_tp8")
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def decode(i):
        b = layers[i]
        if shared:
            B.pkv_paged_attention_decode_shared_prefix(
                b.q, *caches[i], descs[i], b.block_tables, b.context_lens, b.group_starts,
                b.group_prefix, b.scale, outs[i], num_workers=args.workers, workspace=ws)
        else:
            B.pkv_paged_attention_decode(b.q, *caches[i], descs[i], b.block_tables,
                                         b.context_lens, b.scale, outs[i],
                                         num_workers=args.workers, workspace=ws,
                                         partition_size=args.partition_size)

    def step(evs=None):
        for i, b in enumerate(layers):
            if do_append:
                B.pkv_kv_append(b.new_k, b.new_v, b.slot_mapping, *caches[i], descs[i])
            if evs is not None:
                evs[i][0].record(stream)
            decode(i)
            if evs is not None:
                evs[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in layers] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        step(evs[s])
    t_end.record(stream)
    torch.cuda.synchronize()

    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    decode_ms = [a.elapsed_time(b) for st in evs for (a, b) in st]
    decode_avg_ms = statistics.fmean(decode_ms)
    kv_bytes_step = sum(b.kv_bytes() for b in layers)
    kv_bytes_launch = b0.kv_bytes()
    logical_launch = kv_bytes_launch
    if shared:
        # bytes a call must read: every physical row some sequence attends to, once
        used = W.used_rows_per_block(b0.block_tables.cpu().numpy(), b0.context_lens.cpu().numpy(),
                                     b0.num_blocks)
        kv_bytes_launch = int(used.sum()) * 2 * b0.num_kv_heads * b0.head_dim * \
            W.STORAGE[b0.kv_dtype][1]
        kv_bytes_step = kv_bytes_launch * len(layers)
    seqs = b0.num_seqs
    value = kv_bytes_step / (ms_step * 1e-3) / 1e9
    achieved = kv_bytes_launch / (decode_avg_ms * 1e-3) / 1e9
    traffic = load_traffic(args.workload)
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
        "kernel": ("paged_decode_kernel suffix pass + paged_prefill_kernel prefix mode (two launches per "
                   "pkv_paged_attention_decode_shared_prefix call)" if shared else
                   "paged_decode_kernel (one launch per pkv_paged_attention_decode call)"),
        "algorithmic_bytes_per_launch": kv_bytes_launch,
        "launch_avg_us": round(decode_avg_ms * 1e3, 2),
        "launch_p10_us": round(sorted(decode_ms)[len(decode_ms) // 10] * 1e3, 2),
        "launch_p90_us": round(sorted(decode_ms)[(9 * len(decode_ms)) // 10] * 1e3, 2),
    }
    graph = None
    if args.graph:
        # the whole step (every append and decode launch) captured once and
        # replayed: the launches are the same, only the host submission and
        # the dispatch gaps between dependent kernels change
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.steps
        graph = {"ms_per_step": round(gms, 4), "value": round(kv_bytes_step / (gms * 1e-3) / 1e9, 1),
                 "unit": "GB/s", "steps": args.steps}
        del g
    cold = None
    if args.cold:
        # a 1 GiB write before every decode launch, outside its events
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold_ms = []
        for s in range(args.steps):
            for i in range(len(layers)):
                scratch.fill_(s & 0xFF)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                decode(i)
                e1.record(stream)
                cold_ms.append((e0, e1))
        torch.cuda.synchronize()
        cms = sorted(a.elapsed_time(b) for a, b in cold_ms)
        cavg = statistics.fmean(cms)
        del scratch
        cold = {"launch_avg_us": round(cavg * 1e3, 2),
                "launch_p10_us": round(cms[len(cms) // 10] * 1e3, 2),
                "launch_p90_us": round(cms[(9 * len(cms)) // 10] * 1e3, 2),
                "achieved_gbps": round(kv_bytes_launch / (cavg * 1e-3) / 1e9, 1),
                "frac": round(kv_bytes_launch / (cavg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(b0, args.cpu_seconds)
    line = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) + decode seqs/sec",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": b0.kv_dtype, "data": "synthetic",
        "config": describe(args.workload, layers, args.workers),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_seqs_per_s": round(seqs / (ms_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes_step,
        "roofline": roofline, "cpu_baseline": cpu,
    }
    if cold is not None:
        line["cold"] = cold
    if graph is not None:
        line["graph"] = graph
    if shared:
        line["logical_kv_bytes_per_launch"] = logical_launch
        line["logical_kv_gbps"] = round(logical_launch / (decode_avg_ms * 1e-3) / 1e9, 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
