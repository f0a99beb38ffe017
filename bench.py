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

Beside the peak, the line reports `achievable_read`: the bandwidth of a plain
streaming read (pkv_stream_read, 16-byte nontemporal loads) over as many bytes
as one decode launch reads, and roofline.frac_of_achievable. The default
gqa40 line also carries `workloads`: the Qwen2.5-1.5B-shaped layer (append +
decode, warm and after a cache-evicting write) and the long-context fp8 batch
(quantising append + decode, balanced split and 512-token partitions), each
timed after the headline's timed region (--no-summaries skips them).
Every workload with new token rows appends them before decode in its step;
the append calls are timed by their own events in extra steps outside the
timed region.

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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa40",
                    choices=["gqa40", "gqa40_tp8", "qwen", "prefix", "prefix_shared", "fp8", "tiny",
                             "prefill", "prefill_small"])
    ap.add_argument("--workers", type=int, default=0, help="worker waves (0 = fill the device)")
    ap.add_argument("--partition-size", type=int, default=0,
                    help="decode split: 0 = balanced split, else tokens per fixed partition")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-summaries", action="store_true",
                    help="skip the Qwen-shaped and fp8 summaries of the default gqa40 line")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed (reported as "
                         "a 'graph' object; value and roofline stay the eager, event-timed run)")
    ap.add_argument("--cold", action="store_true",
                    help="also time decode launches that each follow a 1 GiB device write, "
                         "which evicts the L2 caches and the 256 MB MALL (the timed launch then "
                         "reads its KV from HBM)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (for counter scaling)")
    return ap.parse_args()


PREFILL_WORKLOADS = ("prefill", "prefill_small")


def kernel_hash(workload: str = None, root: str = None) -> str:
    """Hash of the sources of the attention kernels a workload launches (a
    decode workload: the decode kernel and its merge, and for the
    shared-prefix call also the prefix pass and its merge from
    paged_prefill.hip; a prefill workload: paged_prefill.hip with what it
    includes, and the split's chunk target), with comments and white space
    removed: counter figures are valid only for the code they were taken on,
    and a comment does not change it. workload None: every attention source
    of the decode workloads."""
    import hashlib
    import re
    h = hashlib.sha256()
    files = ["paged_decode.hip", "decode_wave.h", "pkv_tile.h", "pkv_device.h"]
    if workload in (None, "prefix_shared"):
        files.insert(1, "paged_prefill.hip")
    if workload in PREFILL_WORKLOADS:
        files = ["paged_prefill.hip", "decode_wave.h", "pkv_tile.h", "pkv_device.h", "pkv_internal.h"]
    for f in files:
        with open(os.path.join(root or ROOT, "paged_kv_cache_101_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counter_file(workload: str) -> str:
    """The committed counter summary of a workload (decode workloads: the
    workload's name, with the partition size for fixed partitions)."""
    if workload == "prefill":
        return "prefill_step_counters.txt"
    if workload == "prefill_small":
        return "prefill_small_counters.txt"
    return f"decode_{workload}_counters.txt"


def load_traffic(workload: str):
    """HBM traffic per call from the committed counter summary, or None if it
    was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", counter_file(workload))
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as fh:
        for line in fh:
            if line.startswith("{"):
                rec = json.loads(line)
    if rec is None or rec.get("kernel_hash") != kernel_hash(workload.split(":")[0]):
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
        layers = [W.fp8_long(device=device, append_last=True)]
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
        # grow the sample until one run takes about cpu_seconds: each next
        # size from the rate just measured (at most 8x at a time)
        k = 1
        while True:
            rows = np.arange(T - chunk, T - chunk + k)
            pos = cl[-1] - chunk + (rows - (T - chunk))
            t0 = time.perf_counter()
            oracle.paged_prefill(np.ascontiguousarray(qh[rows]), kh, vh,
                                 np.ascontiguousarray(bt[[S - 1] * k]), (pos + 1).astype(np.int32),
                                 np.arange(k + 1, dtype=np.int32), b.scale)
            el = time.perf_counter() - t0
            if el >= 0.7 * args.cpu_seconds or k >= chunk:
                break
            k = min(chunk, max(k + 1, min(8 * k, int(k * args.cpu_seconds / max(el, 1e-3)))))
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
                            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                            "traffic": load_traffic(args.workload),
                            "kernel": "paged_prefill_kernel (split keys) + chunk_merge_kernel",
                            "algorithmic_bytes_per_launch": kv_bytes,
                            "launch_avg_us": round(avg * 1e3, 2)}
        line["unsplit_avg_us"] = round(timed(None) * 1e3, 2)  # the same call without a workspace
    else:
        line["roofline"] = {"bound": "mfma", "achieved": round(tflops, 1),
                            "peak": MFMA_PEAK_TFLOPS[dt], "unit": "TFLOP/s",
                            "frac": round(tflops / MFMA_PEAK_TFLOPS[dt], 4),
                            "traffic": load_traffic(args.workload),
                            "kernel": "paged_prefill_kernel (one launch per call)",
                            "algorithmic_bytes_per_launch": kv_bytes,
                            "launch_avg_us": round(avg * 1e3, 2)}
    print(json.dumps(line), flush=True)


def cpu_model() -> str:
    """The host CPU's model name, as lscpu reports it (else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.strip().lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def achievable_read_bandwidth(nbytes: int, steps: int, dev) -> dict:
    """The read bandwidth a plain streaming kernel gets on this device
    (pkv_stream_read over a buffer of nbytes, the decode launch's KV bytes),
    timed with HIP events on the launch stream."""
    import torch
    from paged_kv_cache_101_amd import binding as B
    nbytes = max(16, nbytes // 16 * 16)
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        B.pkv_stream_read(buf, sink)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        B.pkv_stream_read(buf, sink)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = statistics.fmean(a.elapsed_time(b) for a, b in evs)
    del buf
    return {"gbps": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes,
            "launch_avg_us": round(ms * 1e3, 2),
            "kernel": "stream_read_kernel (pkv_stream_read: 16-byte nontemporal loads, "
                      "one workgroup of 256 threads per CU, 8 loads in flight per thread)"}


class DecodeRun:
    """The layers of one decode workload, their library caches and the
    calls of one step: optionally the append of each layer's new token rows
    (a quantising append for fp8 caches), then the decode call."""

    def __init__(self, workload: str, dev, workers: int, partition_size: int, append: bool):
        import torch
        from paged_kv_cache_101_amd import binding as B
        from paged_kv_cache_101_amd import workloads as W
        self.B, self.W, self.torch = B, W, torch
        self.workload, self.workers, self.partition_size = workload, workers, partition_size
        self.layers = build_layers(workload, dev)
        self.descs = [B.desc_for(b.k_cache, b.kv_dtype, b.k_scale, b.v_scale) for b in self.layers]
        # The library's caches, filled from each layer's token rows with
        # pkv_kv_append (the row-order copies are dropped after, except layer
        # 0's, which the CPU baseline reads).
        self.caches = []
        for i, b in enumerate(self.layers):
            self.caches.append(B.fill_cache(b.k_cache, b.v_cache, self.descs[i]))
            if i > 0:
                b.k_cache = b.v_cache = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        self.outs = [torch.empty_like(b.q) for b in self.layers]
        b0 = self.layers[0]
        self.shared = workload == "prefix_shared"
        if self.shared:
            ng = int(b0.group_prefix.numel())
            self.ws = B.shared_prefix_workspace(b0.num_seqs, b0.num_q_heads, b0.num_kv_heads,
                                                b0.head_dim, ng, workers, dev)
        else:
            self.ws = B.decode_workspace(b0.num_seqs, b0.num_q_heads, b0.num_kv_heads,
                                         b0.head_dim, workers, dev, b0.max_blocks_per_seq,
                                         partition_size)
        self.append = append and b0.slot_mapping is not None
        self.stream = torch.cuda.current_stream()
        torch.cuda.synchronize()

    def decode(self, i):
        b, B = self.layers[i], self.B
        if self.shared:
            B.pkv_paged_attention_decode_shared_prefix(
                b.q, *self.caches[i], self.descs[i], b.block_tables, b.context_lens,
                b.group_starts, b.group_prefix, b.scale, self.outs[i], num_workers=self.workers,
                workspace=self.ws)
        else:
            B.pkv_paged_attention_decode(b.q, *self.caches[i], self.descs[i], b.block_tables,
                                         b.context_lens, b.scale, self.outs[i],
                                         num_workers=self.workers, workspace=self.ws,
                                         partition_size=self.partition_size)

    def append_rows(self, i):
        b = self.layers[i]
        k, v = (b.new_k, b.new_v) if b.new_k_rows is None else (b.new_k_rows, b.new_v_rows)
        self.B.pkv_kv_append(k, v, b.slot_mapping, *self.caches[i], self.descs[i])

    def step(self, evs=None, aevs=None):
        """One step; evs / aevs: per-layer (start, end) event pairs recorded
        around each decode / append call."""
        for i in range(len(self.layers)):
            if self.append:
                if aevs is not None:
                    aevs[i][0].record(self.stream)
                self.append_rows(i)
                if aevs is not None:
                    aevs[i][1].record(self.stream)
            if evs is not None:
                evs[i][0].record(self.stream)
            self.decode(i)
            if evs is not None:
                evs[i][1].record(self.stream)

    def kv_bytes_per_launch(self) -> int:
        """Algorithmic KV bytes of one decode call (unique bytes for the
        shared-prefix path: every physical row some sequence reads, once)."""
        b0, W = self.layers[0], self.W
        if self.shared:
            used = W.used_rows_per_block(b0.block_tables.cpu().numpy(),
                                         b0.context_lens.cpu().numpy(), b0.num_blocks)
            return int(used.sum()) * 2 * b0.num_kv_heads * b0.head_dim * W.STORAGE[b0.kv_dtype][1]
        return b0.kv_bytes()

    def _events(self):
        torch = self.torch
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in self.layers]

    def timed(self, steps: int, warmup: int) -> dict:
        """Warm-up steps, then `steps` timed ones: the whole region between
        two events, and every decode call by its own events. The append calls
        are then timed alone by their own events in `steps` more steps
        (outside the timed region, whose events would otherwise add gaps)."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [self._events() for _ in range(steps)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(self.stream)
        for s in range(steps):
            self.step(evs[s])
        t1.record(self.stream)
        torch.cuda.synchronize()
        dec = sorted(a.elapsed_time(b) for st in evs for (a, b) in st)
        r = {"ms_per_step": t0.elapsed_time(t1) / steps, "decode_ms": dec,
             "decode_avg_ms": statistics.fmean(dec)}
        if self.append:
            aevs = [self._events() for _ in range(steps)]
            for s in range(steps):
                self.step(None, aevs[s])
            torch.cuda.synchronize()
            r["append_avg_ms"] = statistics.fmean(a.elapsed_time(b) for st in aevs
                                                  for (a, b) in st)
        return r

    def cold(self, steps: int) -> dict:
        """Decode calls each timed after a 1 GiB device write that evicts the
        L2 caches and the 256 MB MALL (the call then reads its KV from HBM)."""
        torch = self.torch
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=self.outs[0].device)
        pairs = []
        for s in range(steps):
            for i in range(len(self.layers)):
                scratch.fill_(s & 0xFF)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(self.stream)
                self.decode(i)
                e1.record(self.stream)
                pairs.append((e0, e1))
        torch.cuda.synchronize()
        cms = sorted(a.elapsed_time(b) for a, b in pairs)
        del scratch
        cavg = statistics.fmean(cms)
        nb = self.kv_bytes_per_launch()
        return {"launch_avg_us": round(cavg * 1e3, 2),
                "launch_median_us": round(statistics.median(cms) * 1e3, 2),
                "launch_p10_us": round(cms[len(cms) // 10] * 1e3, 2),
                "launch_p90_us": round(cms[(9 * len(cms)) // 10] * 1e3, 2),
                "achieved_gbps": round(nb / (cavg * 1e-3) / 1e9, 1),
                "frac": round(nb / (cavg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    def free(self):
        self.layers = self.caches = self.outs = self.ws = None
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def summary(workload: str, dev, steps: int, warmup: int, partition_sizes=(0,),
            cold: bool = False) -> dict:
    """A compact record of another workload's step (append + decode), for
    the headline line: per partition size, the decode call's average time
    and roofline fraction, the append's time, and the step's."""
    res = {}
    run = None
    for P in partition_sizes:
        run = DecodeRun(workload, dev, 0, P, append=True)
        t = run.timed(steps, warmup)
        nb = run.kv_bytes_per_launch()
        b0 = run.layers[0]
        rec = {"decode_avg_us": round(t["decode_avg_ms"] * 1e3, 2),
               "decode_median_us": round(statistics.median(t["decode_ms"]) * 1e3, 2),
               "decode_p10_us": round(t["decode_ms"][len(t["decode_ms"]) // 10] * 1e3, 2),
               "decode_p90_us": round(t["decode_ms"][(9 * len(t["decode_ms"])) // 10] * 1e3, 2),
               "achieved_gbps": round(nb / (t["decode_avg_ms"] * 1e-3) / 1e9, 1),
               "frac": round(nb / (t["decode_avg_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "step_us": round(t["ms_per_step"] * 1e3, 2),
               "decode_seqs_per_s": round(b0.num_seqs / (t["ms_per_step"] * 1e-3), 1),
               "kv_bytes_per_launch": nb,
               "traffic": load_traffic(workload if P == 0 else f"{workload}_p{P}")}
        if "append_avg_ms" in t:
            rec["append_avg_us"] = round(t["append_avg_ms"] * 1e3, 2)
        if cold:
            rec["cold"] = run.cold(max(5, steps // 2))
        res["balanced" if P == 0 else f"partition_{P}"] = rec
        run.free()
    return res


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

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.workload in ("prefill", "prefill_small"):
        B.lib()
        bench_prefill(args)
        return
    B.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    # every workload's step appends its new token rows (where it has them:
    # the 40-layer steps, the Qwen-shaped layer, the fp8 batch) before decode
    run = DecodeRun(args.workload, dev, args.workers, args.partition_size, append=True)
    t = run.timed(args.steps, args.warmup)
    layers, b0 = run.layers, run.layers[0]
    shared = run.shared

    ms_step = t["ms_per_step"]
    decode_ms = t["decode_ms"]
    decode_avg_ms = t["decode_avg_ms"]
    kv_bytes_launch = run.kv_bytes_per_launch()
    logical_launch = b0.kv_bytes()
    kv_bytes_step = kv_bytes_launch * len(layers)
    seqs = b0.num_seqs
    value = kv_bytes_step / (ms_step * 1e-3) / 1e9
    achieved = kv_bytes_launch / (decode_avg_ms * 1e-3) / 1e9
    traffic = load_traffic(args.workload if args.partition_size == 0 else
                           f"{args.workload}_p{args.partition_size}")
    kernel = ("paged_prefill_kernel (suffix-pass and prefix-pass workgroups in one launch) + "
              "chunk_merge_kernel (pkv_paged_attention_decode_shared_prefix)" if shared else
              "paged_decode_kernel + partition_merge_kernel (pkv_paged_attention_decode, fixed "
              f"{args.partition_size}-token partitions)" if args.partition_size else
              "paged_decode_kernel (one launch per pkv_paged_attention_decode call)")
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
        "algorithmic_bytes_per_launch": kv_bytes_launch,
        "launch_avg_us": round(decode_avg_ms * 1e3, 2),
        "launch_median_us": round(statistics.median(decode_ms) * 1e3, 2),
        "launch_p10_us": round(decode_ms[len(decode_ms) // 10] * 1e3, 2),
        "launch_p90_us": round(decode_ms[(9 * len(decode_ms)) // 10] * 1e3, 2),
    }
    graph = None
    if args.graph:
        # the whole step (every append and decode launch) captured once and
        # replayed: the launches are the same, only the host submission and
        # the dispatch gaps between dependent kernels change
        stream = run.stream
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            run.step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run.step()
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
    cold = run.cold(args.steps) if args.cold else None
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(b0, args.cpu_seconds)
        cpu["cpu_model"] = cpu_model()
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
    if args.partition_size:
        line["config"]["partition_size"] = args.partition_size
    if "append_avg_ms" in t:
        line["append_avg_us"] = round(t["append_avg_ms"] * 1e3, 2)
    if cold is not None:
        line["cold"] = cold
    if graph is not None:
        line["graph"] = graph
    if shared:
        line["logical_kv_bytes_per_launch"] = logical_launch
        line["logical_kv_gbps"] = round(logical_launch / (decode_avg_ms * 1e-3) / 1e9, 1)
    run.free()
    # the read bandwidth a plain streaming kernel gets here, over as many
    # bytes as one decode launch reads
    ach = achievable_read_bandwidth(kv_bytes_launch, max(10, args.steps), dev)
    line["achievable_read"] = ach
    line["roofline"]["frac_of_achievable"] = round(achieved / ach["gbps"], 4)
    if args.workload == "gqa40" and not args.no_summaries:
        # the other single-GPU configurations, each one step of append +
        # decode, outside the headline's timed region
        line["workloads"] = {
            "qwen2.5_1.5b_layer": summary("qwen", dev, 20, 3, cold=True),
            "fp8_long_32k": summary("fp8", dev, 10, 3, partition_sizes=(0, 512)),
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
