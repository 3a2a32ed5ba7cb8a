"""Decode benchmark: one step = the whole int4 weight-streaming decode path.

Default workload (the headline metric): the 27B-shaped int4 decoder stack
(64 layers, D 5120, 64 query / 8 KV heads, head_dim 128, d_ff 17408, groups of
128) plus the 152064 x 5120 int4 LM head swept in chunks of 8192 rows, batch 1,
8192 cached tokens at the first timed step (the position advances by one per
step).  Inputs are synthetic (seeded, generated on the GPU, resident in HBM
before timing).  At batch 1 the stack runs as one launch of the streaming
kernel (k_stream_decode); other batches run one launch per phase (1..8) or the
matrix-core GEMM path (9..32).

Prints one JSON line: `value` (tok/s) from K timed steps with no
instrumentation; `kernels`, every kernel of the step timed by HIP events on
its own stream over a few more steps, with its algorithmic bytes, GB/s, share
of the step and fraction of 8 TB/s; `roofline`, the kernel with the largest
share of the step, timed over K more steps; `step_roofline`, the whole step
against 8 TB/s and against the measured streaming-read rate of the read probe;
bytes per token and FLOP per byte of the step; the CPU oracle's rate on a
bounded sample.

--layers N runs the first N layers of a stack at its full shape (for a batch
whose whole stack does not fit in HBM, e.g. the 70B shape at batch 32) and
adds the per-step figures scaled to the full depth, labelled as extrapolated.

--prefill N measures prefill instead (one JSON line of its own): one step is
i4d_prefill of one N-token prompt through the stack (int4 MFMA GEMMs over the
prompt, causal prompt attention); `value` is prompt tokens/s, `roofline` the
gate/up GEMM against the 2.5 PFLOP/s dense fp16 matrix-core peak.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--prefill N]
                       [--batch B] [--layers N] [--exec-mode M] [--breakdown-steps N]
                       [--calibrate-copy-mib MIB] [--no-cpu-baseline] [--no-read-probe]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from int4_weight_streaming_decode_amd import roofline  # noqa: E402

METRIC = "decode tokens/s at batch 1 and achieved HBM GB/s (% of peak), 27B-shaped int4"

WORKLOADS = {
    # name: (shape, weight dtype, LM head)
    "27b_lm": ("27b_lm", "int4", True),
    "27b": ("27b", "int4", False),
    "27b_bf16": ("27b", "bf16", False),
    "7b": ("7b", "int4", False),
    "70b": ("70b", "int4", False),
}


# library kernel behind each timed phase (batch 1: the streaming kernel;
# batches of 2..8: matrix-vector kernels; 9..32: the matrix-core GEMM kernels)
KERNEL_NAMES = {"qkv": "k_gemv_qkv", "attention": "k_attention<128, false>", "wo": "k_gemv_rows (Wo)",
                "gate_up": "k_gemv_swiglu", "down": "k_gemv_rows (W_down)", "lm_head": "k_lm_head",
                "stream": "k_stream_decode"}
KERNEL_NAMES_BATCHED = {"qkv": "k_mfma_qkv", "attention": "k_attention<128, false>", "wo": "k_mfma_rows (Wo)",
                        "gate_up": "k_mfma_swiglu", "down": "k_mfma_rows (W_down)", "lm_head": "k_mfma_lm"}


# HBM traffic of the roofline kernel as hardware counters saw it, recorded in
# this profile by two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) scaled by
# a plain copy of known size, with a hash of the kernel sources it was taken
# on.  Reported only while the sources still hash the same.
TRAFFIC_RECORDS = [os.path.join(ROOT, "profiles", f) for f in ("k_stream_decode_27b_lm_b1_hbm_traffic.md",
                                                                 "phase_launches_gate_up_27b_int4_hbm_traffic.md")]


def sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "int4_weight_streaming_decode_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(kernel: str, workload: str):
    """Bytes per launch from a traffic record of this kernel on this workload,
    or None if absent or taken on other sources."""
    import re
    for path in TRAFFIC_RECORDS:
        if not os.path.exists(path):
            continue
        for line in open(path):
            m = re.match(r"traffic-record: kernel=(\S+) workload=(\S+) bytes_per_launch=(\d+) sources_sha256=([0-9a-f]{64})",
                         line.strip())
            if m and m.group(1) == kernel and m.group(2) == workload and m.group(4) == sources_sha256():
                return int(m.group(3))
    return None


def describe(shape, dtype, lm, batch):
    s = (f"{shape.name}-shaped {dtype} decoder stack: {shape.n_layers} layers, D={shape.d_model}, "
         f"{shape.n_q_heads}/{shape.n_kv_heads} heads, head_dim {shape.head_dim}, d_ff {shape.d_ff}, "
         f"group {shape.group}; KV {shape.kv_len} cached tokens; batch {batch}")
    if lm:
        s += f"; int4 LM head {shape.vocab} x {shape.d_model} with greedy argmax (chunk_rows {shape.lm_chunk} requested)"
    return s


def cpu_baseline(shape, dtype, lm):
    """The CPU oracle as it stands, on a bounded sample of the same workload,
    scaled to one full step."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    cap = ((shape.kv_len + 1 + 15) // 16) * 16
    layer = synth.make_layer(shape, 17, 0, dtype)
    kc, vc = synth.make_kv(shape, 17, 0, 1, [shape.kv_len], cap)
    x = synth.make_x(shape, 17, 1).astype(np.float64)
    t0 = time.perf_counter()
    oracle.decode_layer(shape, layer, x, kc, vc, [shape.kv_len])
    t_layer = time.perf_counter() - t0
    step = shape.n_layers * t_layer
    sample = f"1 of {shape.n_layers} layers at KV {shape.kv_len} ({t_layer:.2f} s)"
    if lm:
        w = synth.make_lm_head(shape.lm_chunk, shape.d_model, shape.group, 18)
        h = synth.make_hidden(shape.d_model, 19, 1).astype(np.float64)
        t0 = time.perf_counter()
        oracle.lm_head_chunked_argmax(w, h, shape.lm_chunk)
        t_chunk = time.perf_counter() - t0
        step += t_chunk * shape.vocab / shape.lm_chunk
        sample += f" + 1 LM-head chunk of {shape.lm_chunk} rows ({t_chunk:.2f} s), scaled to the full step"
    return {"value": 1.0 / step, "unit": "tokens/s", "cores": int(threads), "kind": "oracle", "sample": sample,
            "host_cpus": len(os.sched_getaffinity(0))}


PREFILL_KERNELS = {"qkv": "k_pf_qkv", "attention": "k_pf_attn<128>", "wo": "k_pf_rows (Wo)",
                   "gate_up": "k_pf_swiglu", "down": "k_pf_rows (W_down)"}
MFMA_F16_PEAK_TFLOPS = 2500.0        # dense fp16 matrix-core peak of the chip


def prefill_cpu_baseline(shape, n_sample=2):
    """The CPU oracle's prefill (token after token) of a short prompt through
    one layer of the workload's shape, scaled to the whole stack."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    cap = ((n_sample + 15) // 16) * 16
    layer = synth.make_layer(shape, 17, 0, "int4")
    kc, vc = synth.make_kv(shape, 17, 0, 1, [0], cap)
    x = np.stack([synth.make_x(shape, 17, 1, step=t)[0] for t in range(n_sample)]).astype(np.float64)
    t0 = time.perf_counter()
    oracle.prefill(shape, [layer], x, [(kc, vc)], 0)
    t = time.perf_counter() - t0
    return {"value": n_sample / (t * shape.n_layers), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_sample} prompt tokens through 1 of {shape.n_layers} layers ({t:.2f} s), scaled to the stack",
            "host_cpus": len(os.sched_getaffinity(0))}


def prefill_main(args):
    """One step = i4d_prefill of one prompt of args.prefill tokens (positions
    0 .. n-1) through the whole int4 stack; the same prompt every step (each
    step rewrites the same cache slots)."""
    import torch

    from int4_weight_streaming_decode_amd import binding as B
    from synth import gpu as G

    shape_name, wdtype, _ = WORKLOADS[args.workload]
    if wdtype != "int4":
        sys.exit("prefill runs on int4 weights")
    shape = synth.SHAPES[shape_name]
    full_layers = shape.n_layers
    if 0 < args.layers < full_layers:
        shape = shape.with_(n_layers=args.layers)
    n = args.prefill
    torch.cuda.set_device(0)
    cap = ((n + 15) // 16 + 1) * 16
    t_gen = time.perf_counter()
    keep, layers, kvs = [], [], []
    for l in range(shape.n_layers):
        p = G.make_layer_gpu(shape, 1, l, "int4")
        mats = {k: B.make_mat(p[k]["codes"], p[k]["scales"], p[k]["n"], p[k]["k"], p[k]["group"], B.WEIGHT_INT4)
                for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")}
        layers.append(B.make_layer(p["attn_norm"], p["ffn_norm"], mats))
        k, v = G.make_kv_gpu(shape, 1, l, 1, cap)
        kvs.append(B.make_kv(k, v, cap))
        keep.append((p, k, v))
        if (l + 1) % 8 == 0 or l + 1 == shape.n_layers:
            print(f"[bench] inputs: layer {l + 1}/{shape.n_layers} on the device", file=sys.stderr, flush=True)
    layers = (B.I4dLayer * len(layers))(*layers)
    kvs = (B.I4dKv * len(kvs))(*kvs)
    x = G.make_x_gpu(shape, 3, n)
    out = torch.empty_like(x)
    cfg = B.make_config(shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.d_ff,
                        shape.rms_eps, shape.rope_base, 0)
    ws = torch.zeros(B.prefill_workspace_size(cfg, n), dtype=torch.uint8, device="cuda")
    B.workspace_init(ws)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    def step():
        B.prefill(cfg, layers, n, x, out, kvs, 0, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    fl = roofline.prefill_flops(shape, n, 0)
    breakdown = {}
    nb = max(1, args.breakdown_steps)
    for kind in ("qkv", "attention", "wo", "gate_up", "down"):
        B.launch_timing_start(kind, 65536)
        for _ in range(nb):
            step()
        torch.cuda.synchronize()
        ms, launches = B.launch_timing_stop()
        avg_ms = ms / max(launches, 1)
        f = fl["per_layer"][kind]
        breakdown[kind] = {"kernel": PREFILL_KERNELS[kind], "launches_per_step": launches / nb, "avg_us": avg_ms * 1e3,
                           "flop_per_launch": f, "tflops": f / (avg_ms * 1e-3) / 1e12 if launches else None,
                           "share_of_step": (ms / nb) / ms_per_step}
    status = B.read_device_status(ws)
    rk = "gate_up"
    rk_e = breakdown[rk]
    tflops = fl["total"] / (ms_per_step * 1e-3) / 1e12
    result = {
        "metric": f"prefill tokens/s of one {n}-token prompt, {shape.name}-shaped int4 stack",
        "value": n * 1000.0 / ms_per_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights, f16 x f16 -> f32 MFMA GEMM (k/v rows: f16 + f16 remainder); bf16 MFMA attention",
        "data": "synthetic",
        "config": {"workload": f"{shape.name}-prefill{n}: {shape.n_layers} layers, D={shape.d_model}, "
                               f"{shape.n_q_heads}/{shape.n_kv_heads} heads, head_dim {shape.head_dim}, d_ff {shape.d_ff}, "
                               f"group {shape.group}; one prompt of {n} tokens at positions 0..{n - 1}",
                   "prompt_tokens": n, "layers": shape.n_layers, "weights": "int4"},
        "roofline": {"bound": "mfma", "kernel": rk_e["kernel"], "achieved": rk_e["tflops"], "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": (rk_e["tflops"] or 0.0) / MFMA_F16_PEAK_TFLOPS, "traffic": None,
                     "avg_launch_us": rk_e["avg_us"], "flop_per_launch": rk_e["flop_per_launch"]},
        "step_roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": tflops / MFMA_F16_PEAK_TFLOPS},
        "flop_per_step": fl["total"],
        "kernels": breakdown,
        "device_status": status,
        "input_generation_s": round(t_gen, 1),
    }
    if shape.n_layers < full_layers:
        full_ms = ms_per_step * full_layers / shape.n_layers
        result["extrapolated"] = {"layers": full_layers, "ms_per_step": full_ms, "tokens_per_s": n * 1000.0 / full_ms,
                                  "how": f"the first {shape.n_layers} layers timed, scaled by {full_layers}/{shape.n_layers}"}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = prefill_cpu_baseline(shape)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="27b_lm", choices=sorted(WORKLOADS))
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--kv-len", type=int, default=0,
                    help="cached tokens at the first timed step (0: the workload's own, e.g. 8192 for 27B; "
                         "131072 for a 128k-context decode)")
    ap.add_argument("--layers", type=int, default=0,
                    help="run only the first N layers of the stack (0: all); figures for the full depth are then "
                         "reported as extrapolated")
    ap.add_argument("--exec-mode", type=int, default=0, help="0 auto, 1 one launch per phase, 2 streaming kernel")
    ap.add_argument("--graph", action="store_true",
                    help="capture one whole step (stack, LM head, position advance) in a HIP graph and replay it in "
                         "the timed region; the attention split is then planned for the cache capacity")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="> 0: the LM head draws the token at this temperature (Gumbel-max) instead of the greedy argmax")
    ap.add_argument("--page-size", type=int, default=0,
                    help="> 0: paged KV caches (pages of this many positions, shuffled over a pool) instead of contiguous ones")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before the steps, run 3 plain device-to-device copies of this many MiB (a kernel of known "
                         "traffic for scaling hardware byte counters); 0: none")
    ap.add_argument("--breakdown-steps", type=int, default=10,
                    help="steps per extra pass that times one kernel of the step (0: no per-kernel figures)")
    ap.add_argument("--prefill", type=int, default=0,
                    help="measure prefill instead: one prompt of this many tokens through the stack per step")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU layout is a design note, "
              "not a measured path", file=sys.stderr)
        sys.exit(2)
    if args.prefill > 0:
        prefill_main(args)
        return

    import torch

    from int4_weight_streaming_decode_amd import binding as B
    from synth import gpu as G

    shape_name, wdtype, lm = WORKLOADS[args.workload]
    shape = synth.SHAPES[shape_name]
    full_layers = shape.n_layers
    if 0 < args.layers < full_layers:
        shape = shape.with_(n_layers=args.layers)
    if args.kv_len > 0:
        shape = shape.with_(kv_len=args.kv_len)
    batch = args.batch
    torch.cuda.set_device(0)
    torch.manual_seed(0)

    n_kinds = 7
    n_total = args.warmup + 1 + 2 * args.steps + n_kinds * args.breakdown_steps
    cap = ((shape.kv_len + n_total + 1 + 15) // 16) * 16
    if args.page_size > 0:
        if args.page_size % 16:
            sys.exit("--page-size must be a multiple of 16")
        cap = (cap + args.page_size - 1) // args.page_size * args.page_size
    pgen = torch.Generator(device="cpu").manual_seed(5)
    t_gen = time.perf_counter()
    keep = []
    layers, kvs = [], []
    for l in range(shape.n_layers):
        p = G.make_layer_gpu(shape, 1, l, wdtype)
        mats = {}
        for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
            m = p[n]
            if wdtype == "int4":
                mats[n] = B.make_mat(m["codes"], m["scales"], m["n"], m["k"], m["group"], B.WEIGHT_INT4)
            else:
                mats[n] = B.make_mat(m["bf16"], None, m["n"], m["k"], 0, B.WEIGHT_BF16)
        layers.append(B.make_layer(p["attn_norm"], p["ffn_norm"], mats))
        if args.page_size > 0:
            # a pool of batch * cap / P pages, each sequence's pages in shuffled order
            n_pages = batch * (cap // args.page_size)
            k, v = G.make_kv_gpu(shape, 1, l, n_pages, args.page_size)
            table = torch.randperm(n_pages, generator=pgen).to(torch.int32).reshape(batch, -1).cuda()
            kvs.append(B.make_kv(k, v, cap, table, args.page_size, n_pages))
            keep.append((p, k, v, table))
        else:
            k, v = G.make_kv_gpu(shape, 1, l, batch, cap)
            kvs.append(B.make_kv(k, v, cap))
            keep.append((p, k, v))
        if (l + 1) % 8 == 0 or l + 1 == shape.n_layers:
            print(f"[bench] inputs: layer {l + 1}/{shape.n_layers} on the device", file=sys.stderr, flush=True)
    lm_mat = None
    if lm:
        W = G.make_lm_head_gpu(shape.vocab, shape.d_model, shape.group, 2)
        keep.append(W)
        lm_mat = B.make_mat(W["codes"], W["scales"], W["n"], W["k"], W["group"], B.WEIGHT_INT4)
    layers = (B.I4dLayer * len(layers))(*layers)      # host arrays built once
    kvs = (B.I4dKv * len(kvs))(*kvs)
    x = G.make_x_gpu(shape, 3, batch)
    out = torch.empty_like(x)
    tok = torch.empty(batch, dtype=torch.int32, device="cuda")
    mx = torch.empty(batch, dtype=torch.float32, device="cuda")
    pos = torch.full((batch,), shape.kv_len, dtype=torch.int32, device="cuda")
    cfg = B.make_config(shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.d_ff,
                        shape.rms_eps, shape.rope_base, args.exec_mode)
    ws = torch.zeros(B.workspace_size(cfg, shape.n_layers, batch, cap - 1, shape.vocab), dtype=torch.uint8, device="cuda")
    B.workspace_init(ws)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    def lm_head(h):
        if args.temperature > 0:
            B.lm_head_sample(lm_mat, batch, h, shape.lm_chunk, args.temperature, 0x5EED, pos, tok, mx, ws)
        else:
            B.lm_head_chunked(lm_mat, batch, h, shape.lm_chunk, tok, mx, ws)

    done = 0

    def step():
        nonlocal done
        B.decode_stack(cfg, layers, batch, x, out, kvs, pos, shape.kv_len + done, ws)
        if lm:
            lm_head(out)
        pos.add_(1)
        done += 1

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    # which path runs the stack: one streaming launch, or one launch per phase
    B.launch_timing_start("stream", 4)
    step()
    torch.cuda.synchronize()
    streaming = B.launch_timing_stop()[1] > 0
    if streaming:
        kinds = ["stream"]
        names = KERNEL_NAMES
    else:
        kinds = ["qkv", "attention", "wo", "gate_up", "down"]
        names = KERNEL_NAMES_BATCHED if batch > 8 else KERNEL_NAMES
    if lm:
        kinds.append("lm_head")
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            B.decode_stack(cfg, layers, batch, x, out, kvs, pos, cap - 1, ws)
            if lm:
                lm_head(out)
            pos.add_(1)
        torch.cuda.current_stream().wait_stream(gs)
        torch.cuda.synchronize()

    # ---- the timed region: K steps, nothing instrumented
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    keys0 = shape.kv_len + done + 1
    t0.record()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
            done += 1
        else:
            step()
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    keys_avg = keys0 + (args.steps - 1) / 2.0

    # ---- every kernel of the step, each timed by events on its own stream
    def kernel_entry(kind, ms, launches, keys, steps):
        nbytes = roofline.phase_bytes(shape, kind, batch, keys, wdtype)
        avg_ms = ms / max(launches, 1)
        e = {"kernel": names[kind], "launches_per_step": launches / max(steps, 1), "avg_us": avg_ms * 1e3,
             "bytes_per_launch": nbytes}
        if launches:
            e["gbps"] = nbytes / (avg_ms * 1e-3) / 1e9
            e["frac_of_8tbps"] = e["gbps"] / 8000.0
            e["share_of_step"] = (ms / steps) / ms_per_step
        return e

    breakdown = {}
    if args.breakdown_steps > 0 and graph is None:
        for kind in kinds:
            k0 = shape.kv_len + done + 1
            B.launch_timing_start(kind, 65536)
            for _ in range(args.breakdown_steps):
                step()
            torch.cuda.synchronize()
            ms, n = B.launch_timing_stop()
            breakdown[kind] = kernel_entry(kind, ms, n, k0 + (args.breakdown_steps - 1) / 2.0, args.breakdown_steps)
    # ---- the roofline kernel: the largest share of the step, timed over K more steps
    rk = max(breakdown, key=lambda k: breakdown[k].get("share_of_step", 0.0)) if breakdown else kinds[0]
    rk_entry = None
    if graph is None:
        k0 = shape.kv_len + done + 1
        B.launch_timing_start(rk, 65536)
        t0.record()
        for _ in range(args.steps):
            step()
        t1.record()
        torch.cuda.synchronize()
        rk_ms, rk_launches = B.launch_timing_stop()
        rk_region_ms = t0.elapsed_time(t1) / args.steps
        rk_entry = kernel_entry(rk, rk_ms, rk_launches, k0 + (args.steps - 1) / 2.0, args.steps)
    status = B.read_device_status(ws)

    # ---- the measured streaming-read rate (plain 16-byte loads over 4 GiB)
    probe = None
    if not args.no_read_probe:
        buf = torch.ones((1 << 32) // 4, dtype=torch.int32, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        B.read_probe(buf, sink)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(5):
            B.read_probe(buf, sink)
        t1.record()
        torch.cuda.synchronize()
        probe = {"gbps": 5 * buf.numel() * 4 / (t0.elapsed_time(t1) * 1e-3) / 1e9, "bytes": buf.numel() * 4,
                 "how": "k_read_probe: one 512-thread workgroup per compute unit, 4 nontemporal 16-byte loads in "
                        "flight per lane, 5 sweeps of 4 GiB"}
        del buf

    stack_bytes = roofline.step_bytes(shape, batch, keys_avg, wdtype)
    lm_bytes = roofline.lm_head_bytes(shape.vocab, shape.d_model, shape.group) if lm else 0
    step_bytes = stack_bytes + lm_bytes
    step_flops = roofline.step_flops(shape, batch, keys_avg, lm_head=lm)
    hbm_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9

    workload_id = f"{args.workload}-b{batch}"
    result = {
        "metric": METRIC,
        "value": batch * 1000.0 / ms_per_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 weights, f32 FMA" if wdtype != "int4" else
                  "int4 weights, f16 x f16 -> f32 MFMA GEMM; bf16 MFMA attention" if batch > 8 else
                  "int4 weights x int4 digits of 16/24-bit activations -> i32 dot; bf16 MFMA attention" if streaming else
                  "int4 weights, f16 x f16 -> f32 dot; bf16 MFMA attention"),
        "data": "synthetic",
        "config": {"workload": describe(shape, wdtype, lm, batch), "batch": batch, "kv_len": shape.kv_len,
                   "layers": shape.n_layers, "weights": wdtype, "lm_head": lm, "exec_mode": args.exec_mode,
                   "stack_path": "streaming kernel" if streaming else ("matrix-core GEMM" if batch > 8 else
                                                                        "one launch per phase"),
                   "graph": bool(args.graph), "temperature": args.temperature, "page_size": args.page_size},
        "hbm_gbps": hbm_gbps,
        "hbm_frac_of_8tbps": hbm_gbps / 8000.0,
        "algorithmic_bytes_per_step": step_bytes,
        "bytes_per_token": step_bytes / batch,
        "flop_per_token": step_flops / batch,
        "flop_per_byte": step_flops / step_bytes,
        "step_roofline": {"bound": "hbm", "achieved": hbm_gbps, "peak": 8000.0, "unit": "GB/s",
                          "frac": hbm_gbps / 8000.0,
                          "frac_of_read_probe": hbm_gbps / probe["gbps"] if probe else None},
        "read_probe": probe,
        "kernels": breakdown,
        "device_status": status,
        "input_generation_s": round(t_gen, 1),
    }
    if rk_entry is not None:
        result["roofline"] = {"bound": "hbm", "kernel": names[rk], "achieved": rk_entry.get("gbps"), "peak": 8000.0,
                              "unit": "GB/s", "frac": rk_entry["gbps"] / 8000.0 if "gbps" in rk_entry else None,
                              "traffic": recorded_traffic(names[rk], workload_id),
                              "avg_launch_us": rk_entry["avg_us"], "launches_per_step": rk_entry["launches_per_step"],
                              "share_of_step": rk_entry.get("share_of_step"),
                              "ms_per_step_while_timed": rk_region_ms,
                              "bytes_per_launch": rk_entry["bytes_per_launch"]}
    if shape.n_layers < full_layers:
        scale = full_layers / shape.n_layers
        lm_ms = breakdown.get("lm_head", {}).get("avg_us", 0.0) / 1e3 if lm else 0.0
        stack_ms = ms_per_step - lm_ms
        full_ms = stack_ms * scale + lm_ms
        result["extrapolated"] = {
            "layers": full_layers, "ms_per_step": full_ms, "tokens_per_s": batch * 1000.0 / full_ms,
            "hbm_gbps": (stack_bytes * scale + lm_bytes) / (full_ms * 1e-3) / 1e9,
            "how": f"the first {shape.n_layers} layers at the full shape, timed; the step time less the LM head "
                   f"scaled by {full_layers}/{shape.n_layers}"}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(shape, wdtype, lm)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
