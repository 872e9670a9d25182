"""Benchmark: quantized-KV decode attention on one MI355X.

Workload: Llama-3-8B-shaped decode step, 32 layers, batch 16, context 32768,
8 KV heads x 4 query heads, head_dim 128, bf16 inputs, 4-bit K and 4-bit V
(token-wise asymmetric INT4 after a 128-wide block-diagonal Hadamard
rotation), paged 16-token blocks with a randomly permuted page table.

One step = for every layer: quantize-append the new token of each sequence
(kvq_quantize_append), then decode attention over the 32768 cached tokens
(kvq_decode_partial + kvq_decode_merge). The cache is prefilled before the
timed region; each step rewrites position 32767 with the new token, so every
step attends over exactly 32768 tokens. All inputs are seeded synthetic data
resident in HBM when timing starts.

Prints one JSON line. `roofline` is for the dominant kernel (the split-K
partial decode kernel): algorithmic bytes per launch over its average
duration from HIP events recorded around each launch on the launch stream.
`roofline.traffic` is the kernel's measured HBM bytes per launch from two
rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE), each scaled by what the same
counter reads for a 1 GiB device copy; it is read from the committed summary
under profiles/ and reported only while the kernel source still has the hash
recorded there (else null). `cpu_baseline` times the CPU oracle on a bounded
sample of the same step.

    python bench.py [--steps K] [--warmup W] [--layers L] [--cpu-units U]
    python bench.py --summarize-pmc FETCH_CSV WRITE_CSV   # writes the traffic summary to stdout
    python bench.py --summarize-trace KERNEL_TRACE_CSV    # per-kernel durations of a kernel trace
"""

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
DECODE_SRC = os.path.join(ROOT, "quantized_decode_attention_03_amd", "csrc", "kvq_decode.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_partial_k4v4_d128_b16_ctx32k_traffic.md")
PARTIAL_KERNEL = "decode_partial_kernel<4, 4, 128>"
COPY_BYTES = 1 << 30

B, T, HKV, G, D, HAD = 16, 32768, 8, 4, 128, 128
BITS_K, BITS_V = 4, 4
LAYERS = 32
SEED_BASE = 2000

WORKLOAD = ("llama3-8b-shaped decode: 32 layers, batch 16, ctx 32768, 8 kv heads x 4 q heads, "
            "head_dim 128, K4/V4 token-wise INT4, hadamard 128, 16-token pages, permuted page table")


def source_hash():
    with open(DECODE_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """Bytes per launch of the partial kernel from the committed counter summary, if current."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if line.startswith("- ") and ": " in line)
    if fields.get("- kernel source sha256/16") != source_hash():
        return None
    return int(fields["- traffic bytes per launch"])


def _pmc_rows(path, counter):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def summarize_pmc(fetch_csv, write_csv):
    """Traffic summary from a FETCH_SIZE pass and a WRITE_SIZE pass (KiB per dispatch)."""
    out = []
    factors, per_launch = {}, {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _pmc_rows(path, counter)
        copy = max(v for k, v in rows if "copyBuffer" in k or "copy" in k.lower())
        factors[counter] = COPY_BYTES / (copy * 1024.0)
        part = [v for k, v in rows if PARTIAL_KERNEL in k]
        per_launch[counter] = float(np.mean(part)) * 1024.0 * factors[counter]
        out.append(f"- {counter} of the 1 GiB copy (KiB): {copy:.0f}")
        out.append(f"- {counter} scale factor: {factors[counter]:.4f}")
        out.append(f"- {counter} partial-kernel launches: {len(part)}, mean KiB {np.mean(part):.0f}, "
                   f"scaled bytes {per_launch[counter]:.0f}")
    traffic = per_launch["FETCH_SIZE"] + per_launch["WRITE_SIZE"]
    out.append(f"- kernel source sha256/16: {source_hash()}")
    out.append(f"- algorithmic bytes per launch: {bytes_per_layer()}")
    out.append(f"- traffic bytes per launch: {traffic:.0f}")
    out.append(f"- traffic / algorithmic: {traffic / bytes_per_layer():.4f}")
    return "\n".join(out) + "\n"


def summarize_trace(trace_csv):
    """Per-kernel durations of the library's kernels from a rocprofv3 kernel trace.

    Launches are grouped by kernel and grid size, so the prefill appends (one
    token per lane group, 32768 tokens) and the per-step appends (one token)
    are told apart.
    """
    groups = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "kvq::" not in name:
                continue
            m = re.search(r"(\w+_kernel(<[^>]*>)?)", name)
            short = m.group(1) if m else name
            key = (short, int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
            groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = ["| kernel | grid threads | launches | mean us | min us | max us |", "|---|---|---|---|---|---|"]
    for (short, grid), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        d = np.asarray(d) / 1e3
        out.append(f"| {short} | {grid} | {len(d)} | {d.mean():.2f} | {d.min():.2f} | {d.max():.2f} |")
    return "\n".join(out) + "\n"


def bytes_per_layer():
    """Algorithmic HBM bytes of the partial decode kernel for one layer."""
    row = D * BITS_K // 8 + D * BITS_V // 8 + 16   # codes K + V + fp32 {s, mn} x 2 per token-head
    cache = B * HKV * T * row
    table = B * (T // 16) * 4
    q = B * HKV * G * D * 2
    return cache + table + q


def cpu_baseline(units, seed=77):
    """Time the CPU oracle on `units` (sequence, KV head, layer) units of one step."""
    from threadpoolctl import threadpool_limits

    from oracle import kvq_oracle as O
    from quantized_decode_attention_03_amd import synth

    lay = O.Layout(1, G, D, HAD, [BITS_K], [BITS_V])
    nb = T // 16
    table = np.arange(nb, dtype=np.int32)[None]
    elapsed = 0.0
    with threadpool_limits(limits=1):
        for u in range(units):
            k, v, q = synth.llama_layer_np(seed=seed + u, batch=1, tokens=T, hkv=1)
            pool = np.zeros((nb, lay.block_bytes), np.uint8)
            O.quantize_append(lay, pool, table, np.array([0]), k[:, :T - 1], v[:, :T - 1])  # prefill, untimed
            t0 = time.perf_counter()
            O.quantize_append(lay, pool, table, np.array([T - 1]), k[:, T - 1:], v[:, T - 1:])
            O.decode_attention([(lay, pool, table, np.array([T]))], q[:, :G].astype(np.float64))
            elapsed += time.perf_counter() - t0
    per_unit = elapsed / units
    step_s = per_unit * B * HKV * LAYERS
    return {"value": B / step_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{units} (sequence, kv head, layer) units of the step (append 1 token + decode over "
                      f"{T} tokens each, {elapsed:.1f} s on 1 host thread), scaled x{B * HKV * LAYERS // units} "
                      f"to the full step ({B * HKV * LAYERS} units)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--cpu-units", type=int, default=48, help="oracle units timed for cpu_baseline (0: skip)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the traffic summary of two counter passes and exit")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="print per-kernel durations from a rocprofv3 kernel trace and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        sys.stdout.write(summarize_pmc(*args.summarize_pmc))
        return
    if args.summarize_trace:
        sys.stdout.write(summarize_trace(args.summarize_trace))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_decode_attention_03_amd import kvq, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = kvq.kvq_layout_init(HKV, G, D, HAD, [BITS_K] * HKV, [BITS_V] * HKV)
    pages = T // 16
    n_blocks = B * pages
    start = torch.full((B,), T - 1, dtype=torch.int32, device=dev)
    zeros = torch.zeros((B,), dtype=torch.int32, device=dev)
    lens = torch.full((B,), T, dtype=torch.int32, device=dev)

    layers = []
    for l in range(args.layers):
        seed = SEED_BASE + l
        free = synth.free_list(n_blocks, seed)
        table_np = np.full((B, pages), -1, np.int32)
        kvq.kvq_page_alloc(free, 0, np.zeros(B, np.int32), np.full(B, T, np.int32), table_np)
        table = torch.from_numpy(table_np).to(dev)
        pool = torch.empty((n_blocks, L.block_bytes), dtype=torch.uint8, device=dev)
        k, v, q = synth.llama_layer_torch(seed, B, T, HKV, G, D, device=dev)
        kvq.kvq_quantize_append(L, pool, table, zeros, k, v)      # prefill all T positions
        new_k = k[:, T - 1:T].contiguous()
        new_v = v[:, T - 1:T].contiguous()
        del k, v
        seg = [kvq.Segment(L, pool, table, lens, T)]
        layers.append({"pool": pool, "table": table, "seg": seg, "q": q, "new_k": new_k, "new_v": new_v})
    torch.cuda.synchronize()

    ws = kvq.decode_workspace(layers[0]["seg"], B, dev)
    out = torch.empty((B, HKV * G, D), dtype=torch.float32, device=dev)
    calls = []
    for ly in layers:
        calls.append((kvq.prepare_quantize_append(L, ly["pool"], ly["table"], start, ly["new_k"], ly["new_v"]),
                      kvq.prepare_decode_partial(ly["seg"], ly["q"], ws),
                      kvq.prepare_decode_merge(ly["seg"], B, out, ws)))

    n_ev = args.layers * args.steps
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

    def step(record=None):
        for i, (app, part, merge) in enumerate(calls):
            app()
            if record is not None:
                ev_a[record + i].record()
            part()
            if record is not None:
                ev_b[record + i].record()
            merge()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(record=s * args.layers)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    part_ms = [a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]
    part_us = 1e3 * float(np.mean(part_ms))
    ms_per_step = 1e3 * elapsed / args.steps
    tokens_per_s = B * args.steps / elapsed
    layer_bytes = bytes_per_layer()
    achieved = layer_bytes / (part_us * 1e-6) / 1e9
    step_bytes = layer_bytes * args.layers

    if args.copy_calib:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if args.cpu_units > 0:
        cpu = cpu_baseline(args.cpu_units)

    line = {
        "metric": "quantized-KV decode attention: tokens/s and HBM GB/s (% of peak) at 32k ctx",
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "layers": args.layers, "batch": B, "ctx": T, "kv_heads": HKV,
                   "q_per_kv": G, "head_dim": D, "bits_k": BITS_K, "bits_v": BITS_V, "had_block": HAD},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "decode_partial_kernel<4,4,128>", "avg_us": round(part_us, 3),
                     "bytes_per_launch": layer_bytes},
        "step_hbm_gbs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
