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
PARTIAL_KERNEL = "decode_partial_kernel<4, 4, 128, false>"
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


def summarize_counters(csv_paths, match):
    """Mean per dispatch of every counter in rocprofv3 --pmc CSVs, for kernels whose name contains `match`."""
    vals, names = {}, set()
    for path in csv_paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                if match not in r["Kernel_Name"]:
                    continue
                m = re.search(r"(\w+_kernel(<[^>]*>)?)", r["Kernel_Name"])
                short = m.group(1) if m else r["Kernel_Name"]
                key = (short, int(r["Grid_Size"]))
                vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                names.add(r["Counter_Name"])
    names = sorted(names)
    out = ["| kernel | grid threads | dispatches | " + " | ".join(names) + " |",
           "|---|---|---|" + "---|" * len(names)]
    for (short, grid), cnt in sorted(vals.items()):
        n = max(len(v) for v in cnt.values())
        out.append(f"| {short} | {grid} | {n} | " +
                   " | ".join(f"{np.mean(cnt[c]):.4g}" if c in cnt else "-" for c in names) + " |")
    return "\n".join(out) + "\n"


def bytes_per_layer():
    """Algorithmic HBM bytes of the partial decode kernel for one layer."""
    row = D * BITS_K // 8 + D * BITS_V // 8 + 16   # codes K + V + fp32 {s, mn} x 2 per token-head
    cache = B * HKV * T * row
    table = B * (T // 16) * 4
    q = B * HKV * G * D * 2
    return cache + table + q


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_workers():
    """Worker processes for the oracle: the host cores this process may use, at most 16 (one GPU's
    share of a shared box)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_worker(units, barrier, out_q):
    """One host process: build its units' caches (untimed), wait for every worker, then time the
    append of one token + decode over T tokens for each of its units."""
    from threadpoolctl import threadpool_limits

    from oracle import kvq_oracle as O
    from quantized_decode_attention_03_amd import synth

    lay = O.Layout(1, G, D, HAD, [BITS_K], [BITS_V])
    nb = T // 16
    table = np.arange(nb, dtype=np.int32)[None]
    with threadpool_limits(limits=1):
        work = []
        for u in units:
            k, v, q = synth.llama_layer_np(seed=77 + u, batch=1, tokens=T, hkv=1)
            pool = np.zeros((nb, lay.block_bytes), np.uint8)
            O.quantize_append(lay, pool, table, np.array([0]), k[:, :T - 1], v[:, :T - 1])  # prefill, untimed
            work.append((pool, k[:, T - 1:], v[:, T - 1:], q[:, :G].astype(np.float64)))
        barrier.wait()
        t0 = time.time()
        for pool, nk, nv, q in work:
            O.quantize_append(lay, pool, table, np.array([T - 1]), nk, nv)
            O.decode_attention([(lay, pool, table, np.array([T]))], q)
        t1 = time.time()
    out_q.put((t0, t1, len(units)))


def cpu_baseline(units_per_worker):
    """Time the CPU oracle on a sample of (sequence, KV head, layer) units of one step, on every host core
    this process may use (one process per core, one thread each), and scale it to the full step.

    Runs before the GPU is touched; the workers are fresh interpreters (spawn) that load only numpy and
    the oracle."""
    import multiprocessing as mp

    workers = host_workers()
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(workers)
    out_q = ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker,
                         args=(list(range(w * units_per_worker, (w + 1) * units_per_worker)), barrier, out_q))
             for w in range(workers)]
    for p in procs:
        p.start()
    res = [out_q.get() for _ in procs]
    for p in procs:
        p.join()
    wall = max(r[1] for r in res) - min(r[0] for r in res)
    units = sum(r[2] for r in res)
    step_units = B * HKV * LAYERS
    step_s = wall / units * step_units
    return {"value": B / step_s, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "cpu_model": host_cpu_model(),
            "sample": f"{units} (sequence, kv head, layer) units of the step (append 1 token + decode over {T} "
                      f"tokens each) on {workers} host processes of one thread, {wall:.1f} s wall, scaled "
                      f"x{step_units / units:.1f} to the full step ({step_units} units)"}


def decode_bytes(batch, tokens, bits_k, bits_v, d=D, meta=8):
    """Algorithmic bytes the partial kernels read for one layer of one segment: codes + metadata
    (`meta` bytes per row, none at 16 bits) per token and head, and the page table."""
    per_tok = sum(d * bk // 8 + (meta if bk != 16 else 0) + d * bv // 8 + (meta if bv != 16 else 0)
                  for bk, bv in zip(bits_k, bits_v))
    return batch * tokens * per_tok + batch * (-(-tokens // 16)) * 4


def make_pool(kvq, torch, dev, L, batch, tokens, seed):
    pages = -(-tokens // 16)
    n_blocks = batch * pages
    table_np = np.full((batch, pages), -1, np.int32)
    kvq.kvq_page_alloc(synth_mod().free_list(n_blocks, seed), 0, np.zeros(batch, np.int32),
                       np.full(batch, tokens, np.int32), table_np)
    return (torch.empty((n_blocks, L.block_bytes), dtype=torch.uint8, device=dev),
            torch.from_numpy(table_np).to(dev))


def window_in_merge():
    """Whether the library attends to a short bf16 segment inside the merge kernel (its default)."""
    return os.environ.get("KVQ_WINDOW_IN_MERGE", "1") != "0"


def long_kernel_label():
    if window_in_merge():
        return ("decode_partial_multi_kernel<128> (the 4-bit and 2-bit segments, one launch; the bf16 window "
                "is read by decode_merge_kernel and its bytes are not counted here)")
    return "decode_partial_multi_kernel<128> (4-bit and 2-bit segments) + decode_partial_kernel<16,16,128>"


def synth_mod():
    from quantized_decode_attention_03_amd import synth
    return synth


def build_decode_layers(args, kvq, torch, dev):
    """Per layer: segments (layout, pool, table, lens, tokens), q, the new token's K/V and the
    segment it is appended to; plus the config and the algorithmic bytes per layer."""
    synth = synth_mod()
    layers = []
    if args.workload == "mixed32k":
        batch, tokens = 8, 32768
        args.dtype_detail = ("2/3/4/8-bit K/V codes with fp32 {scale, min} per row, bf16 queries and new rows; "
                             "scores on int8 MFMA for 2-, 4- and 8-bit keys (the query as three signed-byte digits "
                             "of a 24-bit fixed-point number per head, exact int32 sums) and on fp16 MFMA (hi+lo "
                             "pairs) for 3-bit keys; PV on fp16 MFMA (weights as hi+lo pairs, ~22 bits); fp32 "
                             "softmax and accumulation")
        w_k = synth.sensitivities(LAYERS, HKV, seed=3).ravel()
        w_v = synth.sensitivities(LAYERS, HKV, seed=33).ravel()
        budget = 3 * LAYERS * HKV
        bk_all = kvq.kvq_plan_bits(w_k, 1.0, 3.6, [2, 3, 4, 8], budget)[0].reshape(LAYERS, HKV)
        bv_all = kvq.kvq_plan_bits(w_v, 1.0, 5.3, [2, 3, 4, 8], budget)[0].reshape(LAYERS, HKV)
        total_bytes = 0
        for l in range(args.layers):
            bk, bv = [int(x) for x in bk_all[l]], [int(x) for x in bv_all[l]]
            L = kvq.kvq_layout_init(HKV, G, D, HAD, bk, bv)
            pool, table = make_pool(kvq, torch, dev, L, batch, tokens, 3000 + l)
            k, v, q = synth.llama_layer_torch(3000 + l, batch, tokens, HKV, G, D, device=dev)
            kvq.kvq_quantize_append(L, pool, table, torch.zeros(batch, dtype=torch.int32, device=dev), k, v)
            lens = torch.full((batch,), tokens, dtype=torch.int32, device=dev)
            layers.append({"segs": [(L, pool, table, lens, tokens)], "q": q, "app": 0,
                           "new_k": k[:, -1:].contiguous(), "new_v": v[:, -1:].contiguous(),
                           "pos": tokens - 1})
            total_bytes += decode_bytes(batch, tokens, bk, bv)
            del k, v
        config = {"workload": "mixed-precision decode: 32 layers, batch 8, ctx 32768, 8 kv heads x 4 q heads, "
                              "head_dim 128, per-head K/V bits from kvq_plan_bits (ladder {2,3,4,8}, average 3, "
                              "beta_K 3.6, beta_V 5.3), hadamard 128",
                  "layers": args.layers, "batch": batch, "ctx": tokens}
        return layers, config, batch, total_bytes / args.layers, (
            "decode_partial_multi_kernel<128> (the 2/3/4-bit heads of a layer, one launch) + "
            "decode_partial_kernel<8,*,128> beside it for the layers with an 8-bit head")
    if args.workload == "long131k":
        args.dtype_detail = ("2- and 4-bit K/V codes with fp32 {scale, min} per row and a bf16 window, bf16 queries "
                             "and new rows; scores of the coded tokens on int8 MFMA (the query as three signed-byte "
                             "digits of a 24-bit fixed-point number per head, exact int32 sums), PV on fp16 MFMA "
                             "(weights as hi+lo pairs); the window scored and weighted in fp32 by the merge kernel")
        batch, tokens, window = 1, 131072, 128
        cls = kvq.kvq_logquant_classes(tokens, window)
        idx_all = [torch.from_numpy(np.flatnonzero(cls == c)).to(dev) for c in range(3)]
        counts = [int(i.numel()) for i in idx_all]
        total_bytes = 0
        for l in range(args.layers):
            k, v, q = synth.llama_layer_torch(4000 + l, batch, tokens, HKV, G, D, device=dev)
            segs = []
            for c, bits in enumerate((16, 4, 2)):
                L = kvq.kvq_layout_init(HKV, G, D, 32, [bits] * HKV, [bits] * HKV)
                pool, table = make_pool(kvq, torch, dev, L, batch, counts[c], 40 + c + 10 * l)
                kvq.kvq_quantize_append(L, pool, table, torch.zeros(batch, dtype=torch.int32, device=dev),
                                        k[:, idx_all[c]].contiguous(), v[:, idx_all[c]].contiguous())
                segs.append((L, pool, table, torch.full((batch,), counts[c], dtype=torch.int32, device=dev),
                             counts[c]))
                if bits != 16 or not window_in_merge():
                    total_bytes += decode_bytes(batch, counts[c], [bits] * HKV, [bits] * HKV)
            # the new token goes into the bf16 window (its last slot is rewritten each step)
            layers.append({"segs": segs, "q": q, "app": 0, "new_k": k[:, -1:].contiguous(),
                           "new_v": v[:, -1:].contiguous(), "pos": counts[0] - 1})
            del k, v
        config = {"workload": "long-context decode: batch 1, ctx 131072, 8 kv heads x 4 q heads, head_dim 128, "
                              "hadamard 32; segments: bf16 window 128, log-spaced 4-bit subset 1280, 2-bit 129664; "
                              "layers back to back (each layer's cache evicted from the MALL by the others)",
                  "layers": args.layers, "batch": batch, "ctx": tokens}
        return layers, config, batch, total_bytes / args.layers, long_kernel_label()
    # default: Llama-3-8B-shaped 32k decode (bf16_32k: the same shape with 16-bit rows, the unquantized
    # baseline the 4-bit cache is compared with)
    batch, tokens = B, T
    bk, bv = (16, 16) if args.workload == "bf16_32k" else (BITS_K, BITS_V)
    m16 = args.workload == "llama32k_m16"
    kc = args.workload == "kivi32k"
    L = kvq.kvq_layout_init(HKV, G, D, HAD, [bk] * HKV, [bv] * HKV, meta_fp16=m16, key_per_channel=kc)
    for l in range(args.layers):
        seed = SEED_BASE + l
        pool, table = make_pool(kvq, torch, dev, L, batch, tokens, seed)
        k, v, q = synth.llama_layer_torch(seed, batch, tokens, HKV, G, D, device=dev)
        kvq.kvq_quantize_append(L, pool, table, torch.zeros(batch, dtype=torch.int32, device=dev), k, v)
        lens = torch.full((batch,), tokens, dtype=torch.int32, device=dev)
        layers.append({"segs": [(L, pool, table, lens, tokens)], "q": q, "app": 0,
                       "new_k": k[:, T - 1:T].contiguous(), "new_v": v[:, T - 1:T].contiguous(), "pos": T - 1,
                       "new_k_block": k[:, T - 16:T].contiguous() if kc else None,
                       "new_v_block": v[:, T - 16:T].contiguous() if kc else None})
        del k, v
    if kc:
        # per-channel keys cannot take single tokens: the step's new token is written as the block that
        # holds it (its 16 tokens re-quantized), the cost a KIVI-style cache pays when a block completes
        for ly in layers:
            ly["new_k"] = ly["new_k_block"]
            ly["new_v"] = ly["new_v_block"]
            ly["pos"] = T - 16
        config = {"workload": WORKLOAD.replace("K4/V4 token-wise INT4", "K4 per channel over each 16-token block, "
                                               "V4 per token"),
                  "layers": args.layers, "batch": B, "ctx": T, "kv_heads": HKV, "q_per_kv": G, "head_dim": D,
                  "bits_k": BITS_K, "bits_v": BITS_V, "had_block": HAD, "keys": "per channel"}
        per_tok = D * BITS_K // 8 + D * 8 // 16 + D * BITS_V // 8 + 8
        args.dtype = "f16"
        args.dtype_detail = ("int4 codes (keys with fp32 {scale, min} per channel and block, values per row), bf16 "
                             "queries; scores and PV on fp16 MFMA (codes exact, query and weights as fp16 hi+lo "
                             "pairs, ~22 bits), fp32 softmax and accumulation")
        return (layers, config, batch, B * HKV * T * per_tok + B * (T // 16) * 4 + B * HKV * G * D * 2,
                "decode_partial_kc_kernel<4,4,128>")
    if m16:
        config = {"workload": WORKLOAD.replace("K4/V4 token-wise INT4", "K4/V4 token-wise INT4 with float16 {s, mn}"),
                  "layers": args.layers, "batch": B, "ctx": T, "kv_heads": HKV, "q_per_kv": G, "head_dim": D,
                  "bits_k": BITS_K, "bits_v": BITS_V, "had_block": HAD, "meta": "fp16"}
        return (layers, config, batch, decode_bytes(B, T, [BITS_K] * HKV, [BITS_V] * HKV, meta=4) + B * HKV * G * D * 2,
                "decode_partial_kernel<4,4,128,fp16 meta>")
    if args.workload == "bf16_32k":
        args.dtype = "bf16"
        args.dtype_detail = ("bf16 K/V rows (rotated), bf16 queries; scores and PV on bf16 MFMA (the query and the "
                             "weights as bf16 hi+lo pairs), fp32 softmax and accumulation")
        config = {"workload": "bf16 paged decode baseline: " + WORKLOAD.replace("K4/V4 token-wise INT4", "bf16 K/V rows (rotated, no metadata)"),
                  "layers": args.layers, "batch": B, "ctx": T, "kv_heads": HKV, "q_per_kv": G, "head_dim": D,
                  "bits_k": 16, "bits_v": 16, "had_block": HAD}
        return (layers, config, batch, decode_bytes(B, T, [16] * HKV, [16] * HKV) + B * HKV * G * D * 2,
                "decode_partial_kernel<16,16,128>")
    config = {"workload": WORKLOAD, "layers": args.layers, "batch": B, "ctx": T, "kv_heads": HKV,
              "q_per_kv": G, "head_dim": D, "bits_k": BITS_K, "bits_v": BITS_V, "had_block": HAD}
    return layers, config, batch, bytes_per_layer(), "decode_partial_kernel<4,4,128>"


def run_decode(args, torch, dev, kvq):
    """One step = per layer: append the new token and decode. By default one library call per layer does
    both (kvq_append_decode_partial, then kvq_append_decode_merge, which quantizes, stores and attends to
    the new token); --separate-append makes the append a launch of its own (kvq_quantize_append)."""
    layers, config, batch, layer_bytes, kernel = build_decode_layers(args, kvq, torch, dev)
    torch.cuda.synchronize()
    seg_objs = [[kvq.Segment(L, pool, table, lens, n) for (L, pool, table, lens, n) in ly["segs"]] for ly in layers]
    # one workspace for every layer: the largest any layer needs (split counts follow the bit widths)
    ws_bytes = max(kvq.kvq_decode_workspace_bytes(sg, batch) for sg in seg_objs)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    kvq.kvq_decode_workspace_init(ws)
    out = torch.empty((batch, HKV * G, D), dtype=torch.float32, device=dev)
    calls = []
    fused_any = False
    for ly, segs in zip(layers, seg_objs):
        L, pool, table, _, _ = ly["segs"][ly["app"]]
        start = torch.full((batch,), ly["pos"], dtype=torch.int32, device=dev)
        if not args.separate_append and not L.key_per_channel and ly["new_k"].shape[1] == 1:
            fused_any = True
            nk, nv = ly["new_k"][:, 0].contiguous(), ly["new_v"][:, 0].contiguous()
            calls.append((None, kvq.prepare_append_decode_partial(segs, ly["app"], start, nk, nv, ly["q"], ws),
                          kvq.prepare_append_decode_merge(segs, ly["app"], start, batch, out, ws)))
        else:
            calls.append((kvq.prepare_quantize_append(L, pool, table, start, ly["new_k"], ly["new_v"]),
                          kvq.prepare_decode_partial(segs, ly["q"], ws),
                          kvq.prepare_decode_merge(segs, batch, out, ws)))
    config = dict(config, step=("per layer one call: the new token's append fused into the decode "
                                "(kvq_append_decode_partial + kvq_append_decode_merge)") if fused_any else
                  "per layer: kvq_quantize_append, kvq_decode_partial, kvq_decode_merge")

    n_ev = args.layers * args.steps
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

    def step(record=None):
        for i, (app, part, merge) in enumerate(calls):
            if app is not None:
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
    # eager timed steps: per-launch events around every partial call
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(record=s * args.layers)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    eager_elapsed = elapsed
    if args.graph:
        # the same K steps captured once as one HIP graph and replayed: the
        # step rate comes from the replay (events cannot be graph nodes here,
        # so the kernel's duration stays the eager pass's)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for s in range(args.steps):
                step()
        graph.replay()  # first replay (uploads the graph)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0

    # the decode kernel's own load pattern with no compute (kvq_measure_read_paged, same grid and split
    # plan), over the layers in turn so no layer's pages are still in the 256 MB cache in front of HBM
    pattern_gbs = None
    try:
        def seg_bytes_of(sg):
            if sg.layout.key_per_channel:
                return layer_bytes - batch * HKV * G * D * 2
            return decode_bytes(batch, sg.max_len, list(sg.layout.bits_k[:HKV]), list(sg.layout.bits_v[:HKV]),
                                meta=4 if sg.layout.meta_fp16 else 8)
        # the segment holding most of a layer's bytes (the 2-bit one at long context)
        si = max(range(len(seg_objs[0])), key=lambda i: seg_bytes_of(seg_objs[0][i]))
        seg0 = seg_objs[0][si]
        sink = torch.empty(1 << 20, dtype=torch.int32, device=dev)
        per_layer = [segs[si] for segs in seg_objs]
        kvq.kvq_measure_read_paged(per_layer, batch, sink)
        # one library call launches the layers' reads back to back, so the two events span GPU work only
        # (timed one launch at a time, the host's enqueue of each call falls inside the interval)
        pat_ms = []
        for _ in range(3):
            p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            p0.record()
            kvq.kvq_measure_read_paged(per_layer, batch, sink)
            p1.record()
            torch.cuda.synchronize()
            pat_ms.append(p0.elapsed_time(p1) / len(per_layer))
        pattern_gbs = seg_bytes_of(seg0) / (float(np.median(pat_ms)) * 1e-3) / 1e9
    except kvq.KvqError:  # a layout outside what the probe covers (16-bit rows, 8-bit codes at head_dim 128)
        pass
    part_ms = [a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]
    part_us = 1e3 * float(np.mean(part_ms))
    p10, p50, p90 = (1e3 * float(x) for x in np.percentile(part_ms, [10, 50, 90]))
    ms_per_step = 1e3 * elapsed / args.steps
    achieved = layer_bytes / (part_us * 1e-6) / 1e9
    extra = {}
    if args.graph:
        config = dict(config, launch="hip graph of the timed steps")
        extra["eager_tokens_per_s"] = round(batch * args.steps / eager_elapsed, 2)
    if getattr(args, "dtype", None):
        extra["dtype"] = args.dtype
    if getattr(args, "dtype_detail", None):
        extra["dtype_detail"] = args.dtype_detail
    return {**extra,
        "value": round(batch * args.steps / elapsed, 2),
        "unit": "tokens/s",
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "config": config,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "measured_load_pattern_gbs": round(pattern_gbs, 1) if pattern_gbs else None,
                     "frac_of_load_pattern": round(achieved / pattern_gbs, 4) if pattern_gbs else None,
                     "traffic": measured_traffic() if args.workload == "llama32k" else None,
                     "kernel": kernel, "avg_us": round(part_us, 3), "median_us": round(p50, 3),
                     "p10_us": round(p10, 3), "p90_us": round(p90, 3), "launches": len(part_ms),
                     "bytes_per_launch": int(layer_bytes)},
        "step_hbm_gbs": round(layer_bytes * args.layers / (ms_per_step * 1e-3) / 1e9, 1),
    }


def run_bulk_append(args, torch, dev, kvq):
    """One step = per layer: quantize-append 16384 new bf16 tokens of 4 sequences (K4/V2); then one decode
    step over the 16384 cached tokens is timed separately."""
    synth = synth_mod()
    batch, tokens = 4, 16384
    L = kvq.kvq_layout_init(HKV, G, D, HAD, [4] * HKV, [2] * HKV)
    layers = []
    for l in range(args.layers):
        pool, table = make_pool(kvq, torch, dev, L, batch, tokens, 5000 + l)
        k, v, q = synth.llama_layer_torch(5000 + l, batch, tokens, HKV, G, D, device=dev)
        layers.append((pool, table, k, v, q))
    zeros = torch.zeros(batch, dtype=torch.int32, device=dev)
    calls = [kvq.prepare_quantize_append(L, pool, table, zeros, k, v) for (pool, table, k, v, q) in layers]
    rows = batch * tokens * HKV
    app_bytes = 2 * rows * D * 2 + rows * (D * 4 // 8 + 8) + rows * (D * 2 // 8 + 8)
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        for c in calls:
            c()
    e1.record()
    torch.cuda.synchronize()
    app_us = e0.elapsed_time(e1) * 1e3 / (args.steps * args.layers)
    # one decode step over the whole cache
    lens = torch.full((batch,), tokens, dtype=torch.int32, device=dev)
    segs = [[kvq.Segment(L, pool, table, lens, tokens)] for (pool, table, k, v, q) in layers]
    ws = kvq.decode_workspace(segs[0], batch, dev)
    out = torch.empty((batch, HKV * G, D), dtype=torch.float32, device=dev)
    dcalls = [(kvq.prepare_decode_partial(sg, ly[4], ws), kvq.prepare_decode_merge(sg, batch, out, ws))
              for sg, ly in zip(segs, layers)]
    for p, m in dcalls:
        p(); m()
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    for _ in range(args.steps):
        for p, m in dcalls:
            p(); m()
    d1.record()
    torch.cuda.synchronize()
    dec_us = d0.elapsed_time(d1) * 1e3 / (args.steps * args.layers)
    achieved = app_bytes / (app_us * 1e-6) / 1e9
    return {
        "metric": "quantized-KV bulk append: GB/s (bf16 read + packed write), then one decode step",
        "dtype": "f64",
        "dtype_detail": "bf16 rows rotated in fp64 (exact sums), rounded to fp32; fp32 min/max, scale and "
                        "round-half-even codes; 4-bit K and 2-bit V codes with fp32 {scale, min} written",
        "value": round(achieved, 1),
        "unit": "GB/s",
        "ms_per_step": round(app_us * args.layers / 1e3, 4),
        "higher_is_better": True,
        "config": {"workload": "prefill-time bulk quantize-append: 32 layers, batch 4, 16384 new tokens per "
                               "sequence, 8 kv heads, head_dim 128, bf16 inputs, K4/V2, hadamard 128, then one "
                               "decode step (x4 q heads) over the 16384 cached tokens",
                   "layers": args.layers, "batch": batch, "new_tokens": tokens},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "append_kernel<4,2,128>", "avg_us": round(app_us, 3), "bytes_per_launch": app_bytes},
        "decode_after": {"us_per_layer": round(dec_us, 3),
                         "gb_s": round(decode_bytes(batch, tokens, [4] * HKV, [2] * HKV) / (dec_us * 1e-6) / 1e9, 1)},
    }


def run_calib(args, torch, dev, kvq):
    """Distortion calibration of the key quantizer: mean squared error at widths 2..6 over the K rows of a
    16-sequence x 2048-token calibration batch, every layer and KV head pooled (one kvq_quant_mse call),
    then the fit of alpha, beta."""
    synth = synth_mod()
    seqs, tokens = 16, 2048
    ks = []
    for l in range(args.layers):
        k, _, _ = synth.llama_layer_torch(6000 + l, seqs, tokens, HKV, G, D, device=dev)
        ks.append(k.reshape(-1, D))
        del _
    x = torch.cat(ks)
    del ks
    widths = [2, 3, 4, 5, 6]
    out = torch.empty(len(widths), dtype=torch.float64, device=dev)
    for _ in range(args.warmup):
        kvq.kvq_quant_mse(x, HAD, widths, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        kvq.kvq_quant_mse(x, HAD, widths, out=out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    alpha, beta, r2 = kvq.kvq_fit_distortion(widths, out.cpu().numpy())
    rows = int(x.shape[0])
    nbytes = rows * D * 2
    achieved = nbytes / (us * 1e-6) / 1e9
    return {
        "metric": "distortion calibration: rows/s through rotate + quantize at 5 widths (kvq_quant_mse)",
        "value": round(rows / (us * 1e-6), 1),
        "unit": "rows/s",
        "ms_per_step": round(us / 1e3, 4),
        "higher_is_better": True,
        "dtype": "f64",
        "config": {"workload": f"key-quantizer calibration: {args.layers} layers x 8 kv heads x 16 sequences x "
                               f"2048 tokens = {rows} bf16 rows of 128, hadamard 128, widths 2..6",
                   "layers": args.layers, "rows": rows},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "quant_mse_kernel<128>", "avg_us": round(us, 3), "bytes_per_launch": nbytes},
        "fit": {"alpha": alpha, "beta": beta, "r2": r2},
    }


def run_long_dynamic(args, torch, dev, kvq):
    """The 131k long-context decode grown token by token with LogQuant's dynamic adjustment: per step the
    host plans the class changes once (kvq_logquant_advance, shared by every layer), then per layer the
    moved rows are re-encoded (kvq_logquant_requant), the new token goes into the bf16 window ring, and the
    three segments are decoded (partials + merge). Eager: the plan is made on the host every step."""
    synth = synth_mod()
    batch, tokens, window = 1, 131072, 128
    extra = args.steps + args.warmup + 16
    cls = kvq.kvq_logquant_dynamic_classes(tokens, window)
    idx_all = [torch.from_numpy(np.flatnonzero(cls == c)).to(dev) for c in range(3)]
    counts = [int(i.numel()) for i in idx_all]
    caps = [window, counts[1] + extra, counts[2] + extra]
    lens = [torch.full((batch,), counts[c], dtype=torch.int32, device=dev) for c in range(3)]
    layers = []
    total_bytes = 0
    for l in range(args.layers):
        k, v, q = synth.llama_layer_torch(4000 + l, batch, tokens + extra, HKV, G, D, device=dev)
        segs = []
        for c, bits in enumerate((16, 4, 2)):
            L = kvq.kvq_layout_init(HKV, G, D, 32, [bits] * HKV, [bits] * HKV)
            pool, table = make_pool(kvq, torch, dev, L, batch, caps[c], 40 + c + 10 * l)
            # positions ascend within each class; the window's 128 positions fill ring slots p mod 128 = 0..127
            kvq.kvq_quantize_append(L, pool, table, torch.zeros(batch, dtype=torch.int32, device=dev),
                                    k[:, idx_all[c]].contiguous(), v[:, idx_all[c]].contiguous())
            segs.append(kvq.Segment(L, pool, table, lens[c], caps[c]))
            if bits != 16 or not window_in_merge():
                total_bytes += decode_bytes(batch, counts[c], [bits] * HKV, [bits] * HKV)
        layers.append({"segs": segs, "q": q, "new_k": k[:, tokens:].contiguous(), "new_v": v[:, tokens:].contiguous()})
        del k, v
    st = kvq.LogQuantStates(batch, window, cap_mid=caps[1])
    st.init(0, tokens)
    ws = kvq.decode_workspace(layers[0]["segs"], batch, dev)
    out = torch.empty((batch, HKV * G, D), dtype=torch.float32, device=dev)
    start = torch.zeros((batch,), dtype=torch.int32, device=dev)
    fused = not args.separate_append
    prepared = [(None if fused else kvq.prepare_decode_partial(ly["segs"], ly["q"], ws),
                 kvq.prepare_append_decode_merge(ly["segs"], 0, start, batch, out, ws) if fused else
                 kvq.prepare_decode_merge(ly["segs"], batch, out, ws))
                for ly in layers]
    n_ev = args.layers * args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(3)]

    # Calls marshalled once: the requant reads the planner's move array when it runs, and each
    # step's append (fused into the merge, or a launch of its own) has its own prepared call (its
    # token's rows) writing at the start position filled in per step.
    requants = [kvq.prepare_logquant_requant(ly["segs"][0], ly["segs"][1], ly["segs"][2], batch, st.moves)
                for ly in layers]
    if fused:
        appends = [[kvq.prepare_append_decode_partial(ly["segs"], 0, start, ly["new_k"][:, i].contiguous(),
                                                      ly["new_v"][:, i].contiguous(), ly["q"], ws)
                    for i in range(args.warmup + args.steps)] for ly in layers]
    else:
        appends = [[kvq.prepare_quantize_append(ly["segs"][0].layout, ly["segs"][0].pool,
                                                ly["segs"][0].block_table, start, ly["new_k"][:, i:i + 1],
                                                ly["new_v"][:, i:i + 1])
                    for i in range(args.warmup + args.steps)] for ly in layers]

    def step(i, record=None):
        st.advance()
        mv = st.move_array()
        # (fill kernels take the value as an argument, so no host buffer is shared between steps)
        for c, n_c in enumerate((window, st.states[0].n_mid, st.states[0].n_low)):
            lens[c].fill_(int(n_c))
        start.fill_(int(mv[0, 4]))
        for li, (part, merge) in enumerate(prepared):
            if record is not None:
                ev[0][record + li].record()
            requants[li]()
            if not fused:
                appends[li][i]()
            if record is not None:
                ev[1][record + li].record()
            if fused:
                appends[li][i]()  # the partials, this step's token appended by their split-0 waves
            else:
                part()
            if record is not None:
                ev[2][record + li].record()
            merge()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(args.warmup + s_, record=s_ * args.layers)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    upd_us = 1e3 * float(np.mean([a.elapsed_time(b) for a, b in zip(ev[0], ev[1])]))
    part_us = 1e3 * float(np.mean([a.elapsed_time(b) for a, b in zip(ev[1], ev[2])]))
    layer_bytes = total_bytes / args.layers
    achieved = layer_bytes / (part_us * 1e-6) / 1e9
    return {
        "value": round(batch * args.steps / elapsed, 2),
        "unit": "tokens/s",
        "ms_per_step": round(1e3 * elapsed / args.steps, 4),
        "higher_is_better": True,
        "config": {"workload": "long-context decode with LogQuant's dynamic adjustment: batch 1, ctx 131072 "
                               "growing one token per step, 8 kv heads x 4 q heads, head_dim 128, hadamard 32; "
                               "segments: bf16 window ring 128, log-spaced 4-bit subset, 2-bit rest; per layer "
                               "per step: requant of the moved rows, then the partials and the merge with the new "
                               "token's append fused into it (--separate-append: its own launch) (eager)",
                   "layers": args.layers, "batch": batch, "ctx": tokens},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": long_kernel_label(), "avg_us": round(part_us, 3),
                     "bytes_per_launch": int(layer_bytes)},
        "update_us_per_layer": round(upd_us, 3),
        "final_state": {"total": int(st.states[0].total), "n_mid": int(st.states[0].n_mid),
                        "n_low": int(st.states[0].n_low)},
    }


def run_tiny(args, torch, dev, kvq):
    """The 1024-token tiny layer: append all tokens, then decode; latency per decode call."""
    synth = synth_mod()
    k, v, q = synth.tiny_layer(seed=1)
    L = kvq.kvq_layout_init(4, 4, 64, 64, [4] * 4, [2] * 4)
    pool, table = make_pool(kvq, torch, dev, L, 1, 1024, 1)
    kvq.kvq_quantize_append(L, pool, table, torch.zeros(1, dtype=torch.int32, device=dev),
                            torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev))
    lens = torch.full((1,), 1024, dtype=torch.int32, device=dev)
    seg = [kvq.Segment(L, pool, table, lens, 1024)]
    qt = torch.from_numpy(q).to(dev)
    ws = kvq.decode_workspace(seg, 1, dev)
    out = torch.empty((1, 16, 64), dtype=torch.float32, device=dev)
    p, m = kvq.prepare_decode_partial(seg, qt, ws), kvq.prepare_decode_merge(seg, 1, out, ws)
    for _ in range(max(args.warmup, 3)):
        p(); m()
    torch.cuda.synchronize()
    n = max(args.steps, 1) * 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        p(); m()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    nbytes = decode_bytes(1, 1024, [4] * 4, [2] * 4, d=64)
    return {
        "metric": "tiny-layer decode latency (launch-bound)",
        "value": round(us, 3),
        "unit": "us",
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": False,
        "config": {"workload": "tiny layer: batch 1, 1024 tokens, 4 kv heads x 4 q heads, head_dim 64, "
                               "hadamard 64, K4/V2, fp32 inputs", "layers": 1, "batch": 1, "ctx": 1024},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 5), "traffic": None,
                     "kernel": "decode_partial_kernel<4,2,64> + decode_merge_kernel<64>", "avg_us": round(us, 3),
                     "bytes_per_launch": nbytes},
    }


WORKLOADS = ("llama32k", "mixed32k", "long131k", "bulk16k", "tiny", "bf16_32k", "calib", "long131k_dyn",
             "llama32k_m16", "kivi32k")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--workload", choices=WORKLOADS, default="llama32k",
                    help="llama32k (default, the headline): batch 16, 32k decode, K4/V4; mixed32k: per-head "
                         "bits from the planner; long131k: batch 1, three precision segments; bulk16k: "
                         "prefill append; tiny: the 1024-token layer; bf16_32k: the llama32k shape with "
                         "16-bit rows (the unquantized baseline); calib: kvq_quant_mse over a key "
                         "calibration set; long131k_dyn: long131k grown one token per step with LogQuant's "
                         "dynamic adjustment; llama32k_m16: llama32k with float16 metadata; kivi32k: llama32k "
                         "with keys quantized per channel over each block")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=True,
                    help="decode workloads: after the eager timed steps (which give the partial kernel's "
                         "per-launch times), capture the same steps as one HIP graph and take the step rate "
                         "from its replay (default on)")
    ap.add_argument("--cpu-units", type=int, default=6,
                    help="oracle units per host worker timed for cpu_baseline (0: skip)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the traffic summary of two counter passes and exit")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="print per-kernel durations from a rocprofv3 kernel trace and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="COUNTER_CSV",
                    help="print per-dispatch means of the counters in rocprofv3 --pmc CSVs (kernels matching "
                         "--match) and exit")
    ap.add_argument("--match", default="kvq::", help="kernel-name filter for --summarize-counters")
    ap.add_argument("--separate-append", action="store_true",
                    help="decode steps append the new token with a launch of its own (kvq_quantize_append) "
                         "instead of fusing it into the decode call")
    args = ap.parse_args()
    if args.summarize_pmc:
        sys.stdout.write(summarize_pmc(*args.summarize_pmc))
        return
    if args.summarize_trace:
        sys.stdout.write(summarize_trace(args.summarize_trace))
        return
    if args.summarize_counters:
        sys.stdout.write(summarize_counters(args.summarize_counters, args.match))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    # the oracle's CPU baseline first, before anything touches the GPU (its workers are spawned processes)
    cpu = None
    if args.cpu_units > 0 and args.workload == "llama32k":
        cpu = cpu_baseline(args.cpu_units)

    import torch

    from quantized_decode_attention_03_amd import kvq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "bulk16k":
        res = run_bulk_append(args, torch, dev, kvq)
    elif args.workload == "tiny":
        res = run_tiny(args, torch, dev, kvq)
    elif args.workload == "calib":
        res = run_calib(args, torch, dev, kvq)
    elif args.workload == "long131k_dyn":
        res = run_long_dynamic(args, torch, dev, kvq)
    else:
        res = run_decode(args, torch, dev, kvq)

    # streaming ceiling on this machine: a 1 GiB device-to-device copy (1 GiB read + 1 GiB written), the median
    # of 10 timed copies; --copy-calib adds one untimed copy that the counter passes scale HBM bytes by
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    if args.copy_calib:
        dst.copy_(src)
        torch.cuda.synchronize()
    copy_ms = []
    for _ in range(10):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        copy_ms.append(c0.elapsed_time(c1))
    copy_gbs = 2 * COPY_BYTES / (float(np.median(copy_ms)) * 1e-3) / 1e9
    # streaming-read ceiling: one read of 1 GiB by kvq_measure_read_stream, the median of 10
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    kvq.kvq_measure_read_stream(src, sink)
    rd_ms = []
    for i in range(10):
        buf = src if i % 2 == 0 else dst  # alternate buffers, 1 GiB each: no reuse from the 256 MB cache
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        kvq.kvq_measure_read_stream(buf, sink)
        c1.record()
        torch.cuda.synchronize()
        rd_ms.append(c0.elapsed_time(c1))
    read_gbs = COPY_BYTES / (float(np.median(rd_ms)) * 1e-3) / 1e9
    del src, dst
    rl = res.setdefault("roofline", {})
    rl["measured_copy_gbs"] = round(copy_gbs, 1)
    rl["measured_stream_read_gbs"] = round(read_gbs, 1)
    rl["frac_of_stream_read"] = round(rl.get("achieved", 0.0) / read_gbs, 4)

    line = {
        "metric": res.pop("metric", "quantized-KV decode attention: tokens/s and HBM GB/s (% of peak) at 32k ctx"),
        "value": res.pop("value"),
        "unit": res.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res.pop("ms_per_step"),
        "higher_is_better": res.pop("higher_is_better"),
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res.pop("dtype", "i8+f16"),
        "dtype_detail": res.pop("dtype_detail", "int4 K/V codes with fp32 {scale, min} per row, bf16 queries and new "
                                                "rows; scores on int8 MFMA (codes exact as bytes, the query as three "
                                                "signed-byte digits of a 24-bit fixed-point number per head, exact "
                                                "int32 sums), PV on fp16 MFMA (centred codes exact, weights as fp16 "
                                                "hi+lo pairs, ~22 bits), fp32 softmax and accumulation"),
        "data": "synthetic",
        "config": res.pop("config"),
        "roofline": res.pop("roofline"),
    }
    line.update(res)
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
