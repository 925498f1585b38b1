"""Benchmark: decode-step weight-read bandwidth of the skinny W4A8/W6A8 linears.

One step is one launch of the fused decode-step walk (per layer: RMSNorm+quant
-> q/k/v, quant -> o, quant -> gate/up, quant -> down; with --dataflow swiglu
the norms carry weights and down reads silu(gate) * up) over a synthetic
27B-shaped (default) or 9B-shaped weight set, every weight matrix read once.
Weights, buffers and the workspace are resident in HBM before the timed
region.  Prints one JSON line: the walk at --m (default 1) as the headline,
the other row counts (--extra-m, default 2 3 4) as fields, the HBM
stream-read ceiling measured in the same process, the single 4096 x 4096
W4A8 linear at M = 1 over 128 rotated copies (alone and with its
quantisation), and the CPU oracle on all host cores and on one.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--set 27b|9b] [--bits 4|6]
                  [--m 1] [--extra-m 2 3 4] [--dataflow plain|swiglu] [--no-cpu]
                  [--no-linear] [--no-ceiling]

--workload linear prints the single-linear measurement as the headline instead;
--workload attention times the split-prefix decode attention of one
27B-shaped attention layer (32 query heads, 4 key/value heads of 256) over a
--ctx-token bf16 KV cache and reports the cache-read rate; successive calls
read distinct caches, about 1 GiB in all, so that none is served from the
last-level cache.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "weight-read GB/s (% of HBM peak) and equiv. tokens/s per decode step, M=1 and M=3"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def build_set(mbq, set_name, bits, n_layers, dataflow="plain"):
    """Pack every matrix of the weight set on the GPU; returns (ops, widths, dev_ops)."""
    import torch
    shapes_fn, _ = synth.WEIGHT_SETS[set_name]
    ops, widths = synth.layer_program(shapes_fn, n_layers, dataflow=dataflow)
    dev_ops = []
    norms = {}   # one device copy per norm: the ops behind one norm share its weights
    t0 = time.time()
    for o in ops:
        canon, S = synth.weights(bits, o["N"], o["K"], seed=1 + o["matrix"])
        packed = mbq.pack_weights(bits, to_dev(canon), to_dev(S), o["N"], o["K"])
        d = dict(bits=bits, prologue=o["prologue"], N=o["N"], K=o["K"], packed=packed,
                 in_buf=o["in_buf"], out_buf=o["out_buf"])
        if "norm_seed" in o:
            if o["norm_seed"] not in norms:
                norms[o["norm_seed"]] = to_dev(synth.norm_weights(o["K"], o["norm_seed"]))
            d["norm_w"] = norms[o["norm_seed"]]
        if "in_buf2" in o:
            d["in_buf2"] = o["in_buf2"]
        dev_ops.append(d)
        if o["matrix"] % 28 == 27:
            log(f"packed {o['matrix'] + 1}/{len(ops)} matrices ({time.time() - t0:.0f} s)")
    torch.cuda.synchronize()
    return ops, widths, dev_ops


def time_sequence_graph(mbq, dev_ops, widths, M, reps):
    """Milliseconds per step of the one-launch-per-op walk captured once in a HIP
    graph and replayed (event-timed): the per-op launches without host gaps."""
    import torch
    bufs = [torch.zeros((M, w), dtype=torch.bfloat16, device="cuda") for w in widths]
    bufs[0].copy_(to_dev(synth.activations(M, widths[0])))
    seq = mbq.LayerSequence(dev_ops, bufs, M, fused=False)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq.run()                       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        seq.run()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        g.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    for b in bufs:
        assert torch.isfinite(b.float()).all(), "non-finite output in the captured unfused walk"
    return float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))


def time_sequence(mbq, dev_ops, widths, M, steps, warmup, fused=True):
    import torch
    bufs = [torch.zeros((M, w), dtype=torch.bfloat16, device="cuda") for w in widths]
    bufs[0].copy_(to_dev(synth.activations(M, widths[0])))
    seq = mbq.LayerSequence(dev_ops, bufs, M, fused=fused)
    for _ in range(warmup):
        seq.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        seq.run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if fused:
        seq.check()      # raises if a bounded wait inside the walk gave up
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])  # ms
    for b in bufs:
        assert torch.isfinite(b.float()).all(), "non-finite output in the timed walk"
    return dict(ms_per_step=wall * 1e3 / steps, event_ms_median=float(np.median(per)),
                event_ms_best=float(per.min()), event_ms_mean=float(per.mean()))


# Counter records of each workload's dominant kernel, valid while the sources
# they were taken from are unchanged: (file, kernel sources).
KERNEL_SOURCES = ["seq_walk.h", "seq_plain.hip", "seq_full.hip", "seqplan.hip", "mbq_seq.h", "mbq_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "seq_kernel_traffic.json")
ATTN_TRAFFIC = (os.path.join(ROOT, "profiles", "decode_attention_traffic.json"),
                ["attn.hip", "mbq_internal.h", "mbq_kernels.h"])
LINEAR_TRAFFIC = (os.path.join(ROOT, "profiles", "linear_traffic.json"),
                  ["linear.hip", "quant_rows.h", "mbq_internal.h", "mbq_kernels.h"])


def kernel_sources_sha256(sources=KERNEL_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "memory_bound_quantised_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(key, record=(TRAFFIC_FILE, KERNEL_SOURCES)):
    """HBM bytes per launch from the committed counter runs (FETCH_SIZE + WRITE_SIZE, each
    scaled by what the counter reads for a copy kernel of known size), or None when there
    is none for this workload or the kernel sources changed since it was taken."""
    path, sources = record
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    e = rec.get("workloads", {}).get(key)
    if not e or rec.get("kernel_sources_sha256") != kernel_sources_sha256(sources):
        return None
    return e["fetch_bytes_per_launch"] + e["write_bytes_per_launch"]


ATTN_SHAPE = dict(n_q=32, n_kv=4, D=256)

# The only performance figures the source pages give for this path: whole-model
# decode rates on NVIDIA consumer GPUs, before and after the kernel work
# ("Doubling LLM token rates in ComfyUI", introduction).  They include
# attention, speculative decoding and everything else on other hardware, so
# they are context for tokens_per_s, not a baseline for this metric.
PAGES_CONTEXT = {
    "source": "Doubling LLM token rates in ComfyUI, introduction (whole-model decode, other GPUs)",
    "9b_tokens_per_s_rtx5090_before_after": [106, 219],
    "9b_tokens_per_s_rtx5080_before_after": [91, 129],
    "27b_tokens_per_s_rtx5090_before_after": [55, 122],
    "27b_w4a8_tokens_per_s_rtx5090_with_mtp": 137,
}


# Distinct KV caches the attention calls rotate over: at least four, and at
# least this many bytes in all (four times the GPU's 256 MiB last-level
# "Infinity" cache), so that no call finds its cache there -- a decode step
# reads each layer's cache once.
ATTN_ROTATE_BYTES = 1 << 30


def run_attention(args):
    """One JSON line for the decode attention: KV-cache bytes per launch over the
    event-timed launch, for M = args.m (and args.extra_m as extra fields).
    Successive calls read distinct caches (ATTN_ROTATE_BYTES in all)."""
    import torch
    import memory_bound_quantised_amd as mbq
    n_q, n_kv, D, P = ATTN_SHAPE["n_q"], ATTN_SHAPE["n_kv"], ATTN_SHAPE["D"], args.ctx
    Ms = [args.m] + [m for m in args.extra_m if m != args.m]
    L = P + max(Ms)
    layer_bytes = 2 * n_kv * L * D * 2
    copies = max(4, -(-ATTN_ROTATE_BYTES // layer_bytes))
    g = torch.Generator(device="cuda").manual_seed(1234)
    k = torch.randn((copies, n_kv, L, D), device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn((copies, n_kv, L, D), device="cuda", generator=g).to(torch.bfloat16)
    res = {}
    for M in Ms:
        q = torch.randn((M, n_q, D), device="cuda", generator=g).to(torch.bfloat16)
        ws = torch.zeros(mbq.attention_workspace_bytes(M, n_q, n_kv, D, P), dtype=torch.uint8, device="cuda")
        out = torch.empty((M, n_q, D), dtype=torch.bfloat16, device="cuda")
        for i in range(max(args.warmup, copies)):
            mbq.decode_attention(q, k[i % copies], v[i % copies], P, out=out, ws=ws)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        t0 = time.perf_counter()
        ev[0].record(stream)
        for i in range(args.steps):
            mbq.decode_attention(q, k[i % copies], v[i % copies], P, out=out, ws=ws)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
        assert torch.isfinite(out.float()).all()
        kv_bytes = 2 * (P + M) * n_kv * D * 2
        res[M] = dict(ms=float(np.median(per)), wall_ms=wall * 1e3 / args.steps, kv_bytes=kv_bytes)
        log(f"attention M={M}: {res[M]}")
    r = res[args.m]
    gbs = r["kv_bytes"] / (r["ms"] / 1e3) / 1e9
    out = {
        "metric": "decode-attention KV-cache read GB/s (% of HBM peak), 27B-shaped layer",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(r["wall_ms"], 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"split-prefix decode attention, 32 query / 4 key-value heads of 256, "
                               f"{P}-token bf16 cache, M={args.m}, {copies} rotated caches", "ctx": P, "M": args.m,
                   "combine": args.attn_combine, "rotated_caches": copies, **ATTN_SHAPE},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": ("decode_attention_kernel, then attn_merge_kernel when the prefix has "
                                                 "several splits (timed together per call)")
                     if args.attn_combine == "kernel" else
                     "decode_attention_kernel, combining its splits in the same cooperative launch",
                     "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"27b/ctx{P}/m{args.m}/{args.attn_combine}", ATTN_TRAFFIC),
                     "traffic_kernel": "decode_attention_kernel (the split kernel alone)",
                     "bytes_per_launch": r["kv_bytes"], "launch_ms": round(r["ms"], 4)},
    }
    for M, rm in res.items():
        if M != args.m:
            out[f"m{M}"] = {"GB/s": round(rm["kv_bytes"] / (rm["ms"] / 1e3) / 1e9, 2), "launch_ms": round(rm["ms"], 4)}
    if not args.no_cpu:
        import oracle
        rng = np.random.default_rng(5)
        heads_kv = 1   # a bounded sample: one key/value head group (8 query heads) at M=1
        qh = synth.f32_to_bf16_bits(rng.standard_normal((1, n_q // n_kv * heads_kv, D), dtype=np.float32))
        kh = synth.f32_to_bf16_bits(rng.standard_normal((heads_kv, P + 1, D), dtype=np.float32))
        vh = synth.f32_to_bf16_bits(rng.standard_normal((heads_kv, P + 1, D), dtype=np.float32))
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 10.0 or reps == 0:
            oracle.decode_attention(qh, kh, vh, P)
            reps += 1
        dt = time.perf_counter() - t0
        b = reps * 2 * (P + 1) * heads_kv * D * 2
        out["cpu_baseline"] = dict(value=round(b / dt / 1e9, 4), unit="GB/s", cores=oracle.num_threads(), kind="oracle",
                                   sample=f"{reps} oracle calls of one key/value head group (8 query heads, M=1) over the "
                                          f"{P}-token cache, {dt:.1f} s; KV bytes read per second")
    print(json.dumps(out), flush=True)


CEILING_BYTES = 4 << 30


def measure_ceiling(mbq, reps=10):
    """HBM stream-read ceiling: one pass of mbq_stream_read over 4 GiB, best and
    median of `reps` event-timed passes after 3 warm-up passes."""
    import torch
    buf = torch.ones(CEILING_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        mbq.stream_read(buf, sink)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        mbq.stream_read(buf, sink)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]) / 1e3
    del buf
    torch.cuda.empty_cache()
    return {"GB/s_best": round(CEILING_BYTES / per.min() / 1e9, 1),
            "GB/s_median": round(CEILING_BYTES / float(np.median(per)) / 1e9, 1),
            "bytes": CEILING_BYTES, "kernel": "stream_read_kernel (mbq_stream_read): dwordx4 nt loads, "
                                             "8 waves per CU, one pass over 4 GiB"}


def _graph_time(fn, n_calls, reps):
    """Per-call milliseconds of fn(i) for i in range(n_calls), captured once in a
    HIP graph and replayed `reps` times (event-timed), so that back-to-back
    launches run without host gaps.  Falls back to eager launches if capture fails."""
    import torch
    torch.cuda.synchronize()
    mode = "graph"
    try:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(n_calls):       # warm-up outside the capture
                fn(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(n_calls):
                fn(i)
        run = g.replay
    except Exception as e:   # pragma: no cover - depends on the runtime
        log(f"graph capture failed ({e}); timing eager launches")
        mode = "eager"

        def run():
            for i in range(n_calls):
                fn(i)
    run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for r in range(reps):
        run()
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]) / n_calls
    return float(np.median(per)), float(per.min()), mode


def run_linear_config(mbq, copies=128, reps=8):
    """The single 4096 x 4096 W4A8 linear at M = 1 (activations N(0,1) bf16, int4
    codes uniform, fp16 group-128 scales U(0.005, 0.02)) over `copies` distinct
    packed matrices used in turn (8.65 MB each, together over 1 GB, so no copy is
    still cached when it comes round again): the linear alone, the per-row
    quantisation followed by the linear, and the linear with the quantisation
    inside it (mbq_linear_prologue)."""
    import torch
    N = K = 4096
    bits = 4
    packed = []
    for i in range(copies):
        canon, S = synth.weights(bits, N, K, seed=10_000 + i)
        packed.append(mbq.pack_weights(bits, to_dev(canon), to_dev(S), N, K))
    x = to_dev(synth.activations(1, K))
    q, s = mbq.quantize_act(x)
    ws = torch.zeros(mbq.linear_workspace_bytes(bits, 1, N, K), dtype=torch.uint8, device="cuda")
    y = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
    qb = torch.empty_like(q)
    sb = torch.empty_like(s)
    L = mbq.lib()
    st = lambda: mbq._stream()

    def lin(i):
        mbq._check("mbq_w4a8_linear", L.mbq_w4a8_linear(1, N, K, q.data_ptr(), s.data_ptr(),
                                                        packed[i].data_ptr(), y.data_ptr(), ws.data_ptr(),
                                                        ws.numel(), st()))

    def quant_lin(i):
        mbq._check("mbq_quantize_act", L.mbq_quantize_act(1, K, x.data_ptr(), qb.data_ptr(), sb.data_ptr(), st()))
        mbq._check("mbq_w4a8_linear", L.mbq_w4a8_linear(1, N, K, qb.data_ptr(), sb.data_ptr(),
                                                        packed[i].data_ptr(), y.data_ptr(), ws.data_ptr(),
                                                        ws.numel(), st()))
    fws = torch.zeros(mbq.linear_prologue_workspace_bytes(bits, 1, N, K), dtype=torch.uint8, device="cuda")

    def fused(i):   # the quantisation inside the linear: one call
        mbq._check("mbq_linear_prologue", L.mbq_linear_prologue(bits, mbq.PRO_QUANT, 1, N, K, x.data_ptr(), None, None,
                                                                packed[i].data_ptr(), y.data_ptr(), fws.data_ptr(),
                                                                fws.numel(), st()))
    wb = synth.weight_bytes(bits, [("w", K, N)])
    lin_ms, lin_best, mode = _graph_time(lin, copies, reps)
    ql_ms, ql_best, _ = _graph_time(quant_lin, copies, reps)
    fu_ms, fu_best, _ = _graph_time(fused, copies, reps)
    assert torch.isfinite(y.float()).all()
    del packed
    torch.cuda.empty_cache()
    return {"workload": "single 4096x4096 W4A8 linear, M=1, 128 rotated copies", "weight_bytes_per_call": wb,
            "timing": f"{mode} of {copies} back-to-back calls, median of {reps} replays",
            "linear_us": round(lin_ms * 1e3, 3), "linear_GB/s": round(wb / (lin_ms / 1e3) / 1e9, 1),
            "linear_pct_hbm_peak": round(100 * wb / (lin_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 2),
            "linear_us_best": round(lin_best * 1e3, 3),
            "quant_plus_linear_us": round(ql_ms * 1e3, 3),
            "quant_plus_linear_GB/s": round(wb / (ql_ms / 1e3) / 1e9, 1),
            "quant_inside_linear_us": round(fu_ms * 1e3, 3),
            "quant_inside_linear_GB/s": round(wb / (fu_ms / 1e3) / 1e9, 1)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(set_name, bits, n_layers, dataflow="plain", budget_s=10.0, sample_layers=8):
    """The oracle on the host cores: the M=1 walk of the first `sample_layers`
    layers of the set, layer after layer (starting over after the last of
    them), until about budget_s seconds of oracle time have been spent; once on
    every host core and once on one thread."""
    import oracle
    shapes_fn, _ = synth.WEIGHT_SETS[set_name]
    L = min(n_layers, sample_layers)
    ops, widths = synth.layer_program(shapes_fn, L, dataflow=dataflow)
    for o in ops:
        if "norm_seed" in o:
            o["norm_w"] = synth.norm_weights(o["K"], o["norm_seed"])
    per_layer = len(shapes_fn())
    mats = {}
    step_bytes = synth.weight_bytes(bits, [(o["name"], o["K"], o["N"]) for o in ops]) * n_layers // L

    def timed(threads):
        oracle.set_threads(threads)
        used = oracle.num_threads()
        M = 1
        bufs = {i: np.zeros((M, w), np.uint16) for i, w in enumerate(widths)}
        bufs[0] = synth.activations(M, widths[0])
        spent, done_bytes, layers = 0.0, 0, 0
        while spent < budget_s:
            layer = layers % L
            lops = ops[layer * per_layer:(layer + 1) * per_layer]
            for o in lops:
                if o["matrix"] not in mats:
                    mats[o["matrix"]] = synth.weights(bits, o["N"], o["K"], seed=1 + o["matrix"])
            t0 = time.perf_counter()
            oracle.layer_sequence(bits, lops, bufs, lambda i: mats[i])
            spent += time.perf_counter() - t0
            done_bytes += synth.weight_bytes(bits, [(o["name"], o["K"], o["N"]) for o in lops])
            layers += 1
        return used, done_bytes / spent / 1e9, layers, done_bytes, spent

    all_threads = os.cpu_count() or 1
    used, gbs, layers, done, spent = timed(all_threads)
    used1, gbs1, layers1, done1, spent1 = timed(1)
    oracle.set_threads(all_threads)
    return dict(value=round(gbs, 4), unit="GB/s", cores=used, kind="oracle",
                sample=f"{layers} layer walks (cycling over the first {L} layers of the {n_layers}-layer set) at M=1, "
                       f"{done / 1e9:.3f} GB of weights in {spent:.1f} s of oracle time on {used} threads, "
                       f"scaled to GB/s; equivalent {gbs * 1e9 / step_bytes:.4f} steps/s",
                cpu_model=cpu_model(),
                one_thread={"value": round(gbs1, 4), "unit": "GB/s", "cores": used1,
                            "sample": f"{layers1} layer walks, {done1 / 1e9:.3f} GB in {spent1:.1f} s"})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--set", default="27b", choices=sorted(synth.WEIGHT_SETS))
    ap.add_argument("--bits", type=int, default=4, choices=[4, 6])
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--m", type=int, default=1)
    ap.add_argument("--extra-m", type=int, nargs="*", default=[2, 3, 4])
    ap.add_argument("--workload", default="walk", choices=["walk", "linear", "attention"],
                    help="linear: the single 4096x4096 W4A8 linear as the headline; attention: the "
                         "split-prefix decode attention of one 27B-shaped layer instead of the walk")
    ap.add_argument("--no-linear", action="store_true", help="skip the single-linear measurement")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the stream-read ceiling")
    ap.add_argument("--ctx", type=int, default=32768, help="attention: cached prefix length")
    ap.add_argument("--attn-combine", default="kernel", choices=["kernel", "inline"],
                    help="attention: combine the splits in a second kernel (default) or at the end of a "
                         "cooperative split launch (sets MBQ_ATTN_COMBINE)")
    ap.add_argument("--dataflow", default="plain", choices=["plain", "swiglu"],
                    help="swiglu: weighted RMSNorms before q/k/v and gate/up, silu(gate) * up before down")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--unfused", action="store_true", help="also time the one-launch-per-op walk")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device three times (a plain copy kernel of known "
                         "size, to calibrate hardware byte counters against)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the skinny linear would shard by output rows with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch
    import memory_bound_quantised_amd as mbq
    mbq.lib()   # fails loudly if the HIP library is not built
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.calib_copy > 0:
        src = torch.ones(args.calib_copy << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calib_copy} MiB x 3")
        del src, dst

    if args.workload == "attention":
        if args.attn_combine == "inline":
            os.environ["MBQ_ATTN_COMBINE"] = "inline"
        else:
            os.environ.pop("MBQ_ATTN_COMBINE", None)
        run_attention(args)
        return

    ceiling = None
    if not args.no_ceiling:
        log("measuring the HBM stream-read ceiling (4 GiB)")
        ceiling = measure_ceiling(mbq)
        log(f"ceiling: {ceiling}")

    if args.workload == "linear":
        r = run_linear_config(mbq)
        gbs = r["linear_GB/s"]
        out = {"metric": "single-linear weight-read GB/s (% of HBM peak), 4096x4096 W4A8, M=1", "value": gbs,
               "unit": "GB/s", "n_gpus": 1, "steps": 8, "warmup": 1, "ms_per_step": r["linear_us"] / 1e3,
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
               "data": "synthetic", "config": {"workload": r["workload"]}, "linear": r,
               "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
               "roofline": {"bound": "hbm", "kernel": "linear_rs_kernel (row-set form: four workgroups per "
                                                     "64-row block, one launch per call)",
                            "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(gbs / HBM_PEAK_GBS, 4),
                            "traffic": measured_traffic("4096x4096/w4/m1", LINEAR_TRAFFIC),
                            "bytes_per_launch": r["weight_bytes_per_call"], "launch_us": r["linear_us"]}}
        if ceiling:
            out["ceiling"] = ceiling
            out["pct_of_ceiling"] = round(100 * gbs / ceiling["GB/s_best"], 2)
        print(json.dumps(out), flush=True)
        return

    n_layers = args.layers or synth.WEIGHT_SETS[args.set][1]
    shapes = synth.weight_set(args.set, n_layers)
    wbytes = synth.weight_bytes(args.bits, shapes)
    log(f"set {args.set} W{args.bits}A8, {n_layers} layers, {len(shapes)} matrices, "
        f"{wbytes / 1e9:.3f} GB of weights + scales")
    ops, widths, dev_ops = build_set(mbq, args.set, args.bits, n_layers, args.dataflow)

    results = {}
    for M in [args.m] + [m for m in args.extra_m if m != args.m]:
        log(f"timing M={M}: {args.warmup} warmup + {args.steps} steps")
        results[M] = time_sequence(mbq, dev_ops, widths, M, args.steps, args.warmup)
        log(f"M={M}: {results[M]}")

    unfused = None
    if args.unfused:
        log(f"timing the unfused walk at M={args.m}")
        unfused = time_sequence(mbq, dev_ops, widths, args.m, max(3, args.steps // 4), 1, fused=False)
        try:
            unfused["graph_ms"] = time_sequence_graph(mbq, dev_ops, widths, args.m, max(3, args.steps // 4))
        except Exception as e:   # pragma: no cover - depends on the runtime
            log(f"capturing the unfused walk failed: {e}")
    main_r = results[args.m]
    t_s = main_r["event_ms_median"] / 1e3
    gbs = wbytes / t_s / 1e9
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{args.set}-shaped decode step, {n_layers} layers x 7 W{args.bits}A8 "
                               f"linears, M={args.m}" + (", SwiGLU dataflow" if args.dataflow == "swiglu" else ""),
                   "weight_bytes": wbytes, "layers": n_layers, "bits": args.bits, "M": args.m,
                   "dataflow": args.dataflow},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(1.0 / t_s, 2),
        "event_ms": {k: round(v, 4) for k, v in main_r.items()},
    }
    for M, r in results.items():
        if M == args.m:
            continue
        tm = r["event_ms_median"] / 1e3
        out[f"m{M}"] = {"GB/s": round(wbytes / tm / 1e9, 2), "ms_per_step": round(r["ms_per_step"], 4),
                        "event_ms_median": round(r["event_ms_median"], 4),
                        "steps_per_s": round(1 / tm, 2), "rows_per_s_upper_bound": round(M / tm, 2),
                        "marginal_cost_vs_m%d" % args.m: round(tm / t_s - 1, 4)}
    if unfused is not None:
        out["unfused_walk"] = {"event_ms_median": round(unfused["event_ms_median"], 4),
                               "GB/s": round(wbytes / (unfused["event_ms_median"] / 1e3) / 1e9, 2)}
        if "graph_ms" in unfused:
            out["unfused_walk"]["graph_ms"] = round(unfused["graph_ms"], 4)
            out["unfused_walk"]["graph_GB/s"] = round(wbytes / (unfused["graph_ms"] / 1e3) / 1e9, 2)
    # One step is one launch of the persistent walk kernel, timed with HIP events
    # recorded on the stream it is launched on.
    out["roofline"] = {"bound": "hbm", "kernel": "seq_kernel (fused decode-step walk, 1 launch per step)",
                       "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gbs / HBM_PEAK_GBS, 4),
                       "traffic": measured_traffic(f"{args.set}/w{args.bits}/m{args.m}/l{n_layers}"
                                                   + ("/swiglu" if args.dataflow == "swiglu" else "")),
                       "bytes_per_launch": wbytes, "launch_ms": round(main_r["event_ms_median"], 4)}
    if ceiling:
        out["ceiling"] = ceiling
        out["pct_of_ceiling"] = round(100 * gbs / ceiling["GB/s_best"], 2)
    if not args.no_linear:
        log("timing the single 4096x4096 W4A8 linear over 128 rotated copies")
        out["linear_4096"] = run_linear_config(mbq)
        log(f"linear: {out['linear_4096']}")
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample (all host cores, then one thread)")
        out["cpu_baseline"] = cpu_baseline(args.set, args.bits, n_layers, args.dataflow)
    out["pages_context"] = PAGES_CONTEXT
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
