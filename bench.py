"""MSA decode benchmark on one MI355X: query-tokens/s per layer at 128K context.

Workload (the headline configuration): batch 8, context 131,072 tokens (1,024 blocks of 128),
4 query tokens per sequence (speculative verify, causal within the last block), 64 query heads,
4 KV heads, head_dim 128, NVFP4 K/V/index-key caches in 128-token pages under a random page
permutation, top-16 selection. Synthetic, seeded data (msa_inputs, recipe 3).

A step is one layer's whole decode path: NVFP4 insert of the step's 32 new tokens, indexer over
the full context, block top-16 and sparse attention, as two launches: insert and indexer
(msa_insert_indexer_score), then selection, attention and the split merge
(msa_select_attn_decode). The same step as three calls (insert, indexer, selection + attention)
and as four is timed too (config.ms_per_step_three_calls, config.ms_per_step_four_calls).
Each step runs on the next
of L layers whose caches live in separate memory, so the index-key working set (L x 75.5 MB)
exceeds the 256 MB Infinity Cache and the scan streams from HBM, as a multi-layer decode does.
Each layer's step is captured once in a HIP graph; the timed region replays K steps.

Kernel durations for the roofline come from HIP events around graphs of L back-to-back launches
of one kernel (one per layer), recorded on the stream the kernels run on.

Beside the headline line: "side" repeats the step on the batched workload (32 x 32,768 tokens,
1 query token), the ragged one (6 sequences of 8K to 512K tokens, 1 query token) and 32
sequences at 128K with 4 query tokens (which takes the union attention kernel), each with its
two launches against the HBM peak; "hbm_read_ceiling_gbs" is the GPU's measured streaming-read
rate for a 76 MB and a 2 GiB working set; "prefill" times the chunked-prefill workload's calls
against the matrix-core peak; "side" also holds the prefix-sharing workload (prefix64) and the
headline workload with the window knobs of the selection (window64: top-64, init and local
blocks, attention over 64 ids per row); "cpu_baseline" times the oracle on the host.

Output: one JSON line (see the keys below). --gpus N > 1 exits: the path runs on one GPU.
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

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix-core peak, TFLOP/s
COPY_BYTES = 512 << 20  # calibration copy for the HBM traffic counters (read and written once)
METRIC = "MSA decode query-tokens/s per layer at 128K ctx; achieved HBM GB/s vs peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8000)
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--kernel-reps", type=int, default=20, help="graph replays per kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-workload side measurement")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the side lines (batched 32K, ragged to 512K, 32 sequences at 128K)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle CPU time")
    ap.add_argument("--only", default="", help="profiling aid: run a calibration copy of "
                    f"{COPY_BYTES >> 20} MiB, then only this call in a loop "
                    "(insert|indexer|insert_indexer|topk|attention|select_attention), and exit; "
                    "'prefill', 'prefix' and 'window' run only that side measurement")
    ap.add_argument("--workload", default="spec128k",
                    choices=("spec128k", "union32x128k", "batched32k", "ragged512k"),
                    help="decode workload of an --only run")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs of '--only insert_indexer' "
                         "(FETCH_SIZE, WRITE_SIZE) into "
                         "profiles/insert_indexer_spec128k_traffic.json and exit")
    ap.add_argument("--counters-from", metavar="CSV",
                    help="summarize a rocprofv3 --pmc counter CSV per kernel (mean per dispatch, "
                         "duration, matrix-core figures) as a markdown table and exit")
    ap.add_argument("--trace-from", metavar="CSV",
                    help="per-kernel duration statistics of a rocprofv3 kernel-trace CSV and exit")
    return ap.parse_args()


def source_digest(*names):
    """Digest of the kernel sources with comments and blank lines removed: a change of the code
    changes it, a change of a comment does not."""
    import re
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_sparse_attention_nvfp4_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def load_traffic(kernel, digest):
    """HBM bytes per launch measured with rocprofv3 counters for this exact kernel source, if any."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_spec128k_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_rows(path):
    """(kernel name, counter value) per dispatch of a rocprofv3 counter-collection CSV."""
    import csv
    with open(path) as f:
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(f)]


# the dominant kernel of the step (insert + indexer launch), its sources and its dispatch name
ROOF_KERNEL = "insert_indexer"
ROOF_SOURCES = ("indexer.hip", "nvfp4_quant.hpp", "device_common.hpp")
ROOF_DISPATCH = "indexer_kernel<true>"


def traffic_from(fetch_csv, write_csv):
    """HBM bytes per insert + indexer launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the calibration copy: the largest runtime
    copy-kernel dispatch of the run, which moves COPY_BYTES in and COPY_BYTES out."""
    rec = {"source_digest": source_digest(*ROOF_SOURCES), "copy_bytes": COPY_BYTES,
           "kernel": ROOF_DISPATCH}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path)
        idx = [v for k, v in rows if ROOF_DISPATCH in k]
        copies = [v for k, v in rows if "copyBuffer" in k]
        assert idx and copies, (counter, sorted(set(k for k, _ in rows))[:20])
        copy_kib = max(copies)
        factor = copy_kib * 1024.0 / COPY_BYTES
        assert 0.25 <= factor <= 4.0, (counter, copy_kib)
        mean_kib = sum(idx) / len(idx)
        scaled = mean_kib * 1024.0 / factor
        rec[counter] = {"kib_per_dispatch": round(mean_kib, 1), "dispatches": len(idx),
                        "copy_kib": copy_kib, "factor": round(factor, 5),
                        "bytes_scaled": round(scaled)}
        total += scaled
    rec["hbm_bytes_per_launch"] = round(total)
    path = os.path.join(ROOT, "profiles", f"{ROOF_KERNEL}_spec128k_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def short_name(k):
    """Kernel name of a rocprofv3 record without return type, namespaces and argument list."""
    k = k.replace("(anonymous namespace)::", "")
    k = k[5:] if k.startswith("void ") else k
    depth = 0
    for i, ch in enumerate(k):
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            k = k[:i]
            break
    return k.replace("msa::", "")


def trace_from(path, last=160):
    """Per-kernel duration statistics of a rocprofv3 kernel-trace CSV over each kernel's last
    `last` dispatches (for the decode kernels: the event-timed replays of its timing graph).
    Only the library's kernels and the read probe are listed (torch's input generation is not)."""
    import csv
    by = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if "msa::" not in r["Kernel_Name"] and "stream_read_kernel" not in r["Kernel_Name"]:
                continue
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            by.setdefault(short_name(r["Kernel_Name"]), []).append(us)
    w = max(len(k) for k in by)
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        t = sorted(v[-last:])
        print(f"  {k:{w}s} calls {len(v):6d}  last {len(t):3d}: mean {sum(t) / len(t):8.2f} us  "
              f"median {t[len(t) // 2]:8.2f}  p10 {t[len(t) // 10]:8.2f}  p90 {t[(9 * len(t)) // 10]:8.2f}")


def counters_from(path, min_dispatches=2):
    """Per-kernel means of a rocprofv3 counter CSV (one row per dispatch and counter), with the
    dispatch duration from its timestamps and two matrix-core figures: the fp16 + bf16 matrix
    flops the hardware counted (SQ_INSTS_VALU_MFMA_MOPS_* are in units of 512 flops) over the
    duration, and SQ_VALU_MFMA_BUSY_CYCLES over SQ_BUSY_CU_CYCLES (the share of busy-CU cycles
    in which a matrix core was busy, summed over the CU's four SIMDs, so 4.0 is the ceiling).
    Only the library's kernels, the read probe and the runtime's copy kernel are listed."""
    import csv
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))
    durs = defaultdict(dict)
    with open(path) as f:
        for r in csv.DictReader(f):
            k = r["Kernel_Name"]
            if not any(n in k for n in ("msa::", "stream_read_kernel", "copyBuffer")):
                continue
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                durs[k][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
    names = sorted({c for k in vals for c in vals[k]})
    print("| kernel | dispatches | mean us | " + " | ".join(names) +
          " | counted matrix TFLOP/s | MFMA busy / busy CU cycles |")
    print("|" + "---|" * (len(names) + 5))
    for k in sorted(vals, key=lambda k: -sum(durs[k].values())):
        n = max(len(v) for v in vals[k].values())
        if n < min_dispatches:
            continue
        mean = {c: sum(v) / len(v) for c, v in vals[k].items()}
        us = sorted(durs[k].values())[len(durs[k]) // 2] if durs[k] else float("nan")
        mops = mean.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + mean.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        tflops = 512.0 * mops / (us * 1e-6) / 1e12 if us == us and us > 0 else float("nan")
        busy = (mean["SQ_VALU_MFMA_BUSY_CYCLES"] / mean["SQ_BUSY_CU_CYCLES"]
                if mean.get("SQ_BUSY_CU_CYCLES") else float("nan"))
        print(f"| `{short_name(k)}` | {n} | {us:.2f} | " + " | ".join(f"{mean.get(c, float('nan')):.4g}" for c in names)
              + f" | {tflops:.1f} | {busy:.3f} |")


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.counters_from:
        counters_from(args.counters_from)
        return
    if args.trace_from:
        trace_from(args.trace_from)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the MSA decode path "
              "here runs on a single device (its indexer shards run on one GPU; the exchange "
              "between devices is not implemented).", file=sys.stderr)
        sys.exit(2)

    import torch

    import msa_inputs as mi

    torch.cuda.set_device(0)
    w = mi.full_workload(3)
    if args.only == "prefill":
        print(json.dumps(prefill_side(args)), flush=True)
        return
    if args.only == "prefix":
        print(json.dumps(prefix_side(args)), flush=True)
        return
    if args.only == "window":
        print(json.dumps(window_side(args)), flush=True)
        return
    if args.only:
        ow = {"spec128k": w, "union32x128k": mi.make_workload(3, batch=32),
              "batched32k": mi.full_workload(2), "ragged512k": mi.full_workload(4)}[args.workload]
        decode_measure(ow, args.layers, args, only=args.only)
        return
    m = decode_measure(w, args.layers, args, full=True)
    B, q, T = w.batch, w.q_len, w.ctx_lens[0]
    kernel_us = m["kernels_us"]
    value = B * q / (m["ms_per_step"] * 1e-3)
    roof_gbs = m["roof_bytes"] / (kernel_us[ROOF_KERNEL] * 1e-6) / 1e9
    idx_gbs = m["idx_bytes"] / (kernel_us["indexer"] * 1e-6) / 1e9
    attn_gbs = m["attn_bytes"] / (kernel_us["select_attention"] * 1e-6) / 1e9
    traffic = load_traffic(ROOF_KERNEL, source_digest(*ROOF_SOURCES))

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "spec128k: batch 8 x context 131072 tokens, 4 query tokens each "
                        "(speculative verify), 64 q heads / 4 kv heads / head_dim 128, "
                        "NVFP4 K/V/index caches, 128-token pages, top-16",
            "batch": B, "context": T, "query_tokens": q, "cache_dtype": "nvfp4",
            "layers_rotated": args.layers, "graph": f"{args.layers} layer steps per graph replay",
            "device_ms_per_step": round(m["device_ms_per_step"], 5),
            "step_us_p10_p50_p90": m["step_us_p10_p50_p90"],
            "step_calls": "msa_insert_indexer_score, msa_select_attn_decode",
            "ms_per_step_three_calls": round(m["alt_ms"]["three"], 5),
            "ms_per_step_four_calls": round(m["alt_ms"]["four"], 5),
        },
        "kernels_us": {k: round(v, 3) for k, v in kernel_us.items()},
        "roofline": {
            "bound": "hbm",
            "kernel": ROOF_KERNEL,
            "achieved": round(roof_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(roof_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": m["roof_bytes"],
        },
        "indexer_alone": {"achieved_gbs": round(idx_gbs, 1), "frac": round(idx_gbs / PEAK_HBM_GBS, 4),
                          "algorithmic_bytes": m["idx_bytes"]},
        "attention_gather": {"achieved_gbs": round(attn_gbs, 1), "frac": round(attn_gbs / PEAK_HBM_GBS, 4),
                             "algorithmic_bytes": m["attn_bytes"]},
    }
    torch.cuda.empty_cache()
    result["hbm_read_ceiling_gbs"] = read_ceiling()
    if not args.no_side:
        side = {}
        for name, sw, layers in (("batched32k", mi.full_workload(2), args.layers),
                                 ("ragged512k", mi.full_workload(4), args.layers),
                                 ("union32x128k", mi.make_workload(3, batch=32), 4)):
            print(f"# side line {name}", file=sys.stderr, flush=True)
            side[name] = side_line(sw, layers, args)
            torch.cuda.empty_cache()
        result["side"] = side
    if not args.no_prefill:
        torch.cuda.empty_cache()
        result["prefill"] = prefill_side(args)
    if not args.no_side:
        torch.cuda.empty_cache()
        print("# side line prefix64", file=sys.stderr, flush=True)
        result["side"]["prefix64"] = prefix_side(args)
        torch.cuda.empty_cache()
        print("# side line window64", file=sys.stderr, flush=True)
        result["side"]["window64"] = window_side(args)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def layer_caches(w, L):
    """Caches of L layers for workload w: layer 0 built from the generator through the insert
    kernel (every token but the q query tokens of each sequence), layers 1..L-1 copies of it in
    their own memory, so the index-key working set is L times one layer's."""
    import torch

    import block_sparse_attention_nvfp4_amd as msa

    dev = "cuda"
    q = w.q_len
    cache0 = msa.Cache.allocate(w.num_pages, dev)
    chunk = 1 << 15
    for b in range(w.batch):
        T = w.ctx_lens[b]
        for t0 in range(0, T - q, chunk):
            t1 = min(T - q, t0 + chunk)
            slots = torch.from_numpy(w.slots(b, t0, t1)).to(dev)
            msa.msa_kv_insert_nvfp4(cache0, slots, w.kv_rows("k", b, t0, t1, dev),
                                    w.kv_rows("v", b, t0, t1, dev), w.ik_rows(b, t0, t1, dev))
    return [cache0] + [msa.Cache(cache0.k.clone(), cache0.v.clone(), cache0.ik.clone())
                       for _ in range(L - 1)]


def decode_measure(w, L, args, full=False, only=""):
    """The decode step of workload w on L rotated layers: one graph runs the step of every
    layer in turn (as a decode pass runs its layers); K layer-steps are timed between
    synchronizations (wall clock), then again in ten chunks of HIP events for the spread, and
    each kernel alone with HIP events around graphs of L back-to-back launches (the median of
    five series). full: also the step as three and as four calls, and every separate call."""
    import numpy as np
    import torch

    import block_sparse_attention_nvfp4_amd as msa

    dev = "cuda"
    B, q = w.batch, w.q_len
    t_setup = time.time()
    caches = layer_caches(w, L)
    table = torch.from_numpy(w.block_table).to(dev)
    ctx = torch.tensor(w.ctx_lens, dtype=torch.int32, device=dev)
    batch = msa.Batch(table, ctx, q)
    toks = [(b, w.ctx_lens[b] - q, w.ctx_lens[b]) for b in range(B)]
    new_slots = torch.from_numpy(np.concatenate([w.slots(b, t0, t1) for b, t0, t1 in toks])).to(dev)
    new_k = torch.cat([w.kv_rows("k", b, t0, t1, dev) for b, t0, t1 in toks])
    new_v = torch.cat([w.kv_rows("v", b, t0, t1, dev) for b, t0, t1 in toks])
    new_ik = torch.cat([w.ik_rows(b, t0, t1, dev) for b, t0, t1 in toks])
    q_idx, qq = w.q_idx.to(dev), w.q.to(dev)
    steps = [msa.DecodeStep(c, batch, dev) for c in caches]
    scale = msa.default_softmax_scale()
    torch.cuda.synchronize()
    print(f"# setup {time.time() - t_setup:.1f}s: {w.name} batch {B}, {L} layers x {w.num_pages} "
          f"pages, {torch.cuda.memory_allocated() / 2**30:.2f} GiB allocated",
          file=sys.stderr, flush=True)

    calls = {
        "insert": lambda s: msa.msa_kv_insert_nvfp4(s.cache, new_slots, new_k, new_v, new_ik),
        "indexer": lambda s: msa.msa_indexer_score(s.cache, batch, q_idx, s.block_scores),
        "insert_indexer": lambda s: msa.msa_insert_indexer_score(s.cache, batch, new_k, new_v,
                                                                 new_ik, q_idx, s.block_scores),
        "topk": lambda s: msa.msa_block_topk(s.block_scores, batch, 16, s.block_ids),
        "attention": lambda s: msa.msa_sparse_attn_decode(s.cache, batch, qq, s.block_ids, scale,
                                                          s.out, s.workspace),
        "select_attention": lambda s: msa.msa_select_attn_decode(s.cache, batch, s.block_scores, 16,
                                                                 s.block_ids, qq, scale, s.out,
                                                                 s.workspace),
    }
    STEP = ("insert_indexer", "select_attention")               # the timed step: two launches
    THREE_CALLS = ("insert", "indexer", "select_attention")     # the same step as three calls
    FOUR_CALLS = ("insert", "indexer", "topk", "attention")     # and as four
    timed_calls = list(calls) if full else list(STEP)

    def full_step(s, names=STEP):
        for name in names:
            calls[name](s)

    # eager warmup (also fills every layer's scores/ids used by single-kernel timings)
    for s in steps:
        full_step(s)
    torch.cuda.synchronize()

    if only:
        # profiling aid: a plain copy of known size (counter calibration), then the chosen
        # kernel alone, L launches per round, no graphs
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        for _ in range(args.kernel_reps):
            for s in steps:
                calls[only](s)
        torch.cuda.synchronize()
        print(f"# ran {args.kernel_reps * L} launches of {only}", file=sys.stderr)
        return None

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        layers_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(layers_graph, stream=stream):
            for s in steps:
                full_step(s)
        alt_graphs = {}
        if full:
            for key, names in (("three", THREE_CALLS), ("four", FOUR_CALLS)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for s in steps:
                        full_step(s, names)
                alt_graphs[key] = g
        graphs = []  # single-layer steps for a step count that is not a multiple of L
        for s in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                full_step(s)
            graphs.append(g)
        kgraphs = {}
        for name in timed_calls:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for s in steps:
                    calls[name](s)
            kgraphs[name] = g
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            graphs[i % L].replay()
        torch.cuda.synchronize()
        ev0, ev1 = ev(), ev()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps // L):       # exactly `steps` layer steps
            layers_graph.replay()
        for i in range(args.steps % L):
            graphs[i].replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        dev_ms = ev0.elapsed_time(ev1)

        # the spread: the same replays in ten chunks, each bracketed by events
        per_chunk = max(1, args.steps // L // 10)
        chunk_us = []
        for _ in range(10):
            e0, e1 = ev(), ev()
            e0.record(stream)
            for _ in range(per_chunk):
                layers_graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            chunk_us.append(e0.elapsed_time(e1) * 1e3 / (per_chunk * L))

        alt_ms = {}
        for key, g in alt_graphs.items():
            g.replay()
            torch.cuda.synchronize()
            e4s, e4e = ev(), ev()
            e4s.record(stream)
            for _ in range(max(1, args.steps // L)):
                g.replay()
            e4e.record(stream)
            torch.cuda.synchronize()
            alt_ms[key] = e4s.elapsed_time(e4e) / (max(1, args.steps // L) * L)

        kernel_us = {}
        for name, g in kgraphs.items():
            g.replay()
            torch.cuda.synchronize()
            series = []
            for _ in range(5):
                es, ee = ev(), ev()
                es.record(stream)
                for _ in range(args.kernel_reps):
                    g.replay()
                ee.record(stream)
                torch.cuda.synchronize()
                series.append(es.elapsed_time(ee) * 1e3 / (args.kernel_reps * L))
            kernel_us[name] = sorted(series)[2]

    # algorithmic bytes per launch: the insert + indexer reads every index-key byte of the
    # context (72 B per token), the index queries, writes the block scores, and the insert's
    # fp32 inputs (9 vectors of 128 per new token) and NVFP4 outputs; the selection + attention
    # launch reads the block scores, gathers the K + V of each selected (sequence, group, block)
    # once per distinct block over the query tokens (144 B per valid token), reads the queries
    # and writes the outputs
    sum_T = sum(w.ctx_lens)
    idx_bytes = sum_T * 72 + B * q * 4 * 128 * 2 + B * q * 4 * w.max_blocks * 4
    ins_bytes = B * q * 9 * (128 * 4 + 72)
    ids = steps[0].block_ids.cpu().numpy().reshape(B, q, 4, 16)
    gathered_tokens = 0
    for b in range(B):
        T = w.ctx_lens[b]
        for g in range(4):
            for blk in set(int(x) for x in ids[b, :, g].ravel() if x >= 0):
                gathered_tokens += max(0, min(128, T - blk * 128))
    attn_bytes = gathered_tokens * 144 + 2 * B * q * 64 * 128 * 2 + B * q * 4 * w.max_blocks * 4
    ms_per_step = wall * 1e3 / args.steps
    pct = np.percentile(np.array(chunk_us), [10, 50, 90])
    out = {"ms_per_step": ms_per_step, "device_ms_per_step": dev_ms / args.steps,
           "step_us_p10_p50_p90": [round(float(x), 2) for x in pct],
           "kernels_us": kernel_us, "alt_ms": alt_ms, "idx_bytes": idx_bytes,
           "roof_bytes": idx_bytes + ins_bytes, "attn_bytes": attn_bytes}
    del steps, caches, kgraphs, alt_graphs, graphs, layers_graph
    return out


def side_line(w, L, args):
    """A decode step on another workload, reported beside the headline: query-tokens/s per layer
    and the two launches against the HBM peak."""
    m = decode_measure(w, L, args)
    ku = m["kernels_us"]
    B, q = w.batch, w.q_len
    return {
        "workload": f"{w.name}: batch {B}, contexts {min(w.ctx_lens)}..{max(w.ctx_lens)} tokens, "
                    f"{q} query token(s) each, {L} layers rotated",
        "query_tokens_per_s": round(B * q / (m["ms_per_step"] * 1e-3), 1),
        "ms_per_step": round(m["ms_per_step"], 5),
        "step_us_p10_p50_p90": m["step_us_p10_p50_p90"],
        "kernels_us": {k: round(v, 3) for k, v in ku.items()},
        "insert_indexer": {"algorithmic_bytes": m["roof_bytes"],
                           "frac": round(m["roof_bytes"] / (ku["insert_indexer"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "attention_gather": {"algorithmic_bytes": m["attn_bytes"],
                             "frac": round(m["attn_bytes"] / (ku["select_attention"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
    }


def prefix_side(args, L=4):
    """The prefix-sharing workload (64 requests sharing a 32,768-token prefix, each with its own
    1K-8K suffix, 1 query token): the decode step as the per-request path runs it (fused insert
    + indexer, then selection + attention) and as the shared-prefix path runs it (insert; the
    indexer scoring each shared page once for all requests; selection; the attention
    dequantizing each selected shared block once for all requests that selected it), on L
    rotated layers, with every call timed alone and the blocks each attention dequantizes."""
    import numpy as np
    import torch

    import block_sparse_attention_nvfp4_amd as msa
    import msa_inputs as mi

    dev = "cuda"
    w = mi.make_workload(6)
    B, q, P = w.batch, w.q_len, w.prefix_tokens // 128
    caches = layer_caches(w, L)
    batch = msa.Batch(torch.from_numpy(w.block_table).to(dev),
                      torch.tensor(w.ctx_lens, dtype=torch.int32, device=dev), q)
    toks = [(b, w.ctx_lens[b] - q, w.ctx_lens[b]) for b in range(B)]
    new_slots = torch.from_numpy(np.concatenate([w.slots(b, t0, t1) for b, t0, t1 in toks])).to(dev)
    new_k = torch.cat([w.kv_rows("k", b, t0, t1, dev) for b, t0, t1 in toks])
    new_v = torch.cat([w.kv_rows("v", b, t0, t1, dev) for b, t0, t1 in toks])
    new_ik = torch.cat([w.ik_rows(b, t0, t1, dev) for b, t0, t1 in toks])
    q_idx, qq = w.q_idx.to(dev), w.q.to(dev)
    steps = [msa.DecodeStep(c, batch, dev) for c in caches]
    ws = torch.empty(msa.msa_sparse_attn_shared_prefix_workspace_bytes(batch), dtype=torch.uint8,
                     device=dev)
    scale = msa.default_softmax_scale()
    calls = {
        "insert_indexer": lambda s: msa.msa_insert_indexer_score(s.cache, batch, new_k, new_v,
                                                                 new_ik, q_idx, s.block_scores),
        "select_attention": lambda s: msa.msa_select_attn_decode(s.cache, batch, s.block_scores, 16,
                                                                 s.block_ids, qq, scale, s.out,
                                                                 s.workspace),
        "insert": lambda s: msa.msa_kv_insert_nvfp4(s.cache, new_slots, new_k, new_v, new_ik),
        "indexer": lambda s: msa.msa_indexer_score(s.cache, batch, q_idx, s.block_scores),
        "indexer_shared_prefix": lambda s: msa.msa_indexer_score_shared_prefix(
            s.cache, batch, q_idx, P, s.block_scores),
        "topk": lambda s: msa.msa_block_topk(s.block_scores, batch, 16, s.block_ids),
        "attention": lambda s: msa.msa_sparse_attn_decode(s.cache, batch, qq, s.block_ids, scale,
                                                          s.out, s.workspace),
        "attention_shared_prefix": lambda s: msa.msa_sparse_attn_decode_shared_prefix(
            s.cache, batch, qq, s.block_ids, P, scale, s.out, ws),
    }
    paths = {"per_request": ("insert_indexer", "select_attention"),
             "shared_prefix": ("insert", "indexer_shared_prefix", "topk", "attention_shared_prefix")}
    for s in steps:
        for name in paths["per_request"]:
            calls[name](s)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graphs = {}
    with torch.cuda.stream(stream):
        for key, names in list(paths.items()) + [(n, (n,)) for n in calls]:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for s in steps:
                    for name in names:
                        calls[name](s)
            graphs[key] = g
    torch.cuda.synchronize()
    us = {}
    with torch.cuda.stream(stream):
        for key, g in graphs.items():
            g.replay()
            series = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(args.kernel_reps):
                    g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                series.append(e0.elapsed_time(e1) * 1e3 / (args.kernel_reps * L))
            us[key] = round(sorted(series)[2], 3)
    # blocks each attention dequantizes (one layer): the per-request kernel every usable
    # (row, group, slot); the shared-prefix one each selected shared (group, block) once plus
    # every usable private slot
    ids = steps[0].block_ids.cpu().numpy().reshape(B, q, 4, 16)
    pos = np.array(w.ctx_lens)[:, None] - q + np.arange(q)[None, :]
    usable = (ids >= 0) & (ids * 128 <= pos[:, :, None, None])
    shared = usable & (ids < P)
    uniq = sum(len(set(ids[:, :, g][shared[:, :, g]].tolist())) for g in range(4))
    per_row = int(usable.sum())
    return {
        "workload": f"prefix: {B} requests sharing {P * 128} prefix tokens, own suffixes "
                    f"{min(w.ctx_lens) - P * 128}..{max(w.ctx_lens) - P * 128} tokens, {q} query "
                    f"token each, 64 q heads / 4 kv heads / head_dim 128, NVFP4 caches, top-16, "
                    f"{L} layers rotated",
        "us": us,
        "query_tokens_per_s": {k: round(B * q / (us[k] * 1e-6), 1) for k in paths},
        "attention_dequantized_blocks": {"per_request": per_row, "shared_prefix": uniq + per_row - int(shared.sum())},
        "shared_slots": int(shared.sum()),
    }


def window_side(args, topk=64, init=1, local=2, L=4):
    """The headline workload (8 x 131,072 tokens, 4 query tokens) with the window knobs of the
    selection: top-`topk` blocks with the first `init` and the last `local` blocks kept, then
    attention over those rows of `topk` ids. The step as msa_decode_step_window (three launches:
    insert + indexer, the window selection, the attention) on L rotated layers, every call also
    timed alone; the attention's gather against the HBM peak (144 B per valid token of each
    distinct selected (sequence, group, block), the scores, queries and outputs)."""
    import numpy as np
    import torch

    import block_sparse_attention_nvfp4_amd as msa
    import msa_inputs as mi

    dev = "cuda"
    w = mi.full_workload(3)
    B, q = w.batch, w.q_len
    caches = layer_caches(w, L)
    batch = msa.Batch(torch.from_numpy(w.block_table).to(dev),
                      torch.tensor(w.ctx_lens, dtype=torch.int32, device=dev), q)
    toks = [(b, w.ctx_lens[b] - q, w.ctx_lens[b]) for b in range(B)]
    new_k = torch.cat([w.kv_rows("k", b, t0, t1, dev) for b, t0, t1 in toks])
    new_v = torch.cat([w.kv_rows("v", b, t0, t1, dev) for b, t0, t1 in toks])
    new_ik = torch.cat([w.ik_rows(b, t0, t1, dev) for b, t0, t1 in toks])
    q_idx, qq = w.q_idx.to(dev), w.q.to(dev)
    steps = [msa.DecodeStep(c, batch, dev) for c in caches]
    ids = [torch.full((B * q, 4, topk), -1, dtype=torch.int32, device=dev) for _ in steps]
    scale = msa.default_softmax_scale()
    calls = {
        "step": lambda i, s: msa.msa_decode_step_window(s.cache, batch, new_k, new_v, new_ik, q_idx,
                                                        qq, topk, init, local, scale,
                                                        s.block_scores, ids[i], s.out, s.workspace),
        "insert_indexer": lambda i, s: msa.msa_insert_indexer_score(s.cache, batch, new_k, new_v,
                                                                    new_ik, q_idx, s.block_scores),
        "topk_window": lambda i, s: msa.msa_block_topk_window(s.block_scores, batch, topk, init,
                                                              local, ids[i]),
        "attention_topk": lambda i, s: msa.msa_sparse_attn_decode_topk(s.cache, batch, qq, ids[i],
                                                                       scale, s.out, s.workspace),
    }
    for i, s in enumerate(steps):
        calls["step"](i, s)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graphs = {}
    with torch.cuda.stream(stream):
        for key, names in [(n, (n,)) for n in calls]:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i, s in enumerate(steps):
                    for name in names:
                        calls[name](i, s)
            graphs[key] = g
    torch.cuda.synchronize()
    us = {}
    with torch.cuda.stream(stream):
        for key, g in graphs.items():
            g.replay()
            series = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(args.kernel_reps):
                    g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                series.append(e0.elapsed_time(e1) * 1e3 / (args.kernel_reps * L))
            us[key] = round(sorted(series)[2], 3)
    sel = ids[0].cpu().numpy().reshape(B, q, 4, topk)
    gathered = 0
    for b in range(B):
        T = w.ctx_lens[b]
        for g in range(4):
            for blk in set(int(x) for x in sel[b, :, g].ravel() if x >= 0):
                gathered += max(0, min(128, T - blk * 128))
    attn_bytes = gathered * 144 + 2 * B * q * 64 * 128 * 2 + B * q * 4 * topk * 4
    return {
        "workload": f"spec128k with window selection: batch {B} x context {w.ctx_lens[0]} tokens, "
                    f"{q} query tokens each, top-{topk} with init {init} and local {local} "
                    f"blocks, {L} layers rotated",
        "us": us,
        "query_tokens_per_s": round(B * q / (us["step"] * 1e-6), 1),
        "attention_gather": {"algorithmic_bytes": attn_bytes,
                             "frac": round(attn_bytes / (us["attention_topk"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
    }


def read_ceiling():
    """Measured streaming-read rate of this GPU for two working sets, by the library's read probe
    (include/msa_probe.h: each workgroup streams one contiguous share): 76 MB (one layer's
    index keys at the headline workload; eight buffers in turn, 608 MB, so they miss the 256 MB
    Infinity Cache) and 2 GiB. HIP events around repeated launches; the best of five series, in
    GB/s."""
    import torch

    import block_sparse_attention_nvfp4_amd as msa

    sink = torch.zeros(msa.msa_probe_sink_words(), dtype=torch.int32, device="cuda")
    out = {}
    for label, nbytes, nbuf, reps in (("76MB", 76 << 20, 8, 10), ("2GiB", 2 << 30, 2, 4)):
        bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda") for _ in range(nbuf)]
        for bf in bufs:
            msa.msa_probe_stream_read(bf, sink)
        torch.cuda.synchronize()
        best = 0.0
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                for bf in bufs:
                    msa.msa_probe_stream_read(bf, sink)
            e1.record()
            torch.cuda.synchronize()
            gbs = nbytes * nbuf * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
            best = max(best, gbs)
        out[label] = round(best, 1)
        del bufs
        torch.cuda.empty_cache()
    return out


def prefill_side(args):
    """The chunked-prefill workload (2 sequences, 65,536 cached tokens + a 2,048-token chunk):
    the same calls with q_len = 2,048, which take the score-GEMM indexer and the token-tile
    attention. Reported beside the decode metric, against the bf16 matrix-core peak."""
    import numpy as np
    import torch

    import block_sparse_attention_nvfp4_amd as msa
    import msa_inputs as mi

    dev = "cuda"
    w = mi.full_workload(5)
    B, q = w.batch, w.q_len
    cache = msa.Cache.allocate(w.num_pages, dev)
    for b in range(B):
        T = w.ctx_lens[b]
        for t0 in range(0, T - q, 1 << 15):
            t1 = min(T - q, t0 + (1 << 15))
            slots = torch.from_numpy(w.slots(b, t0, t1)).to(dev)
            msa.msa_kv_insert_nvfp4(cache, slots, w.kv_rows("k", b, t0, t1, dev),
                                    w.kv_rows("v", b, t0, t1, dev), w.ik_rows(b, t0, t1, dev))
    batch = msa.Batch(torch.from_numpy(w.block_table).to(dev),
                      torch.tensor(w.ctx_lens, dtype=torch.int32, device=dev), q)
    toks = [(b, w.ctx_lens[b] - q, w.ctx_lens[b]) for b in range(B)]
    new_k = torch.cat([w.kv_rows("k", b, t0, t1, dev) for b, t0, t1 in toks])
    new_v = torch.cat([w.kv_rows("v", b, t0, t1, dev) for b, t0, t1 in toks])
    new_ik = torch.cat([w.ik_rows(b, t0, t1, dev) for b, t0, t1 in toks])
    q_idx, qq = w.q_idx.to(dev), w.q.to(dev)
    st = msa.DecodeStep(cache, batch, dev, mode="separate")
    scale = msa.default_softmax_scale()
    calls = {
        "insert_indexer": lambda: msa.msa_insert_indexer_score(cache, batch, new_k, new_v, new_ik,
                                                               q_idx, st.block_scores),
        "indexer": lambda: msa.msa_indexer_score(cache, batch, q_idx, st.block_scores),
        "topk": lambda: msa.msa_block_topk(st.block_scores, batch, 16, st.block_ids),
        "attention": lambda: msa.msa_sparse_attn_decode(cache, batch, qq, st.block_ids, scale,
                                                        st.out, st.workspace),
    }
    for name in ("insert_indexer", "topk", "attention"):
        calls[name]()
    torch.cuda.synchronize()
    us = {}
    for name, fn in calls.items():
        series = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                fn()
            e1.record()
            torch.cuda.synchronize()
            series.append(e0.elapsed_time(e1) * 1e3 / 5)
        us[name] = round(sorted(series)[1], 2)
    # algorithmic flops: the indexer multiplies every (row, visible key) pair once (2 x 128 per
    # pair, 4 rows per query token); the attention does QK and PV for 16 heads over every
    # visible key of the selected blocks (2 x 2 x 128 x 16 per (token, group, key))
    ctx = np.array(w.ctx_lens, dtype=np.int64)
    pos = (ctx[:, None] - q + np.arange(q)[None, :])  # [B][q]
    idx_flops = float(2 * 128 * 4 * (pos + 1).sum())
    ids = st.block_ids.cpu().numpy().reshape(B, q, 4, 16).astype(np.int64)
    vis = np.clip(pos[:, :, None, None] + 1 - 128 * ids, 0, 128) * (ids >= 0)
    att_flops = float(2 * 2 * 128 * 16 * vis.sum())
    peak = PEAK_BF16_TFLOPS
    return {
        "workload": "prefill: batch 2 x (65,536 cached + 2,048 chunk tokens), q_len 2,048, "
                    "64 q heads / 4 kv heads / head_dim 128, NVFP4 caches, top-16",
        "us": us,
        "step_us": round(us["insert_indexer"] + us["topk"] + us["attention"], 2),
        "indexer": {"bound": "mfma", "tflops": round(idx_flops / us["indexer"] / 1e6, 1),
                    "peak": peak, "frac": round(idx_flops / us["indexer"] / 1e6 / peak, 4),
                    "flops": idx_flops},
        "attention": {"bound": "mfma", "tflops": round(att_flops / us["attention"] / 1e6, 1),
                      "peak": peak, "frac": round(att_flops / us["attention"] / 1e6 / peak, 4),
                      "flops": att_flops},
    }


def cpu_baseline(w, target_seconds):
    """The oracle (single-threaded, fp64) on whole sequences of the same workload: quantize the
    step's new tokens, score every index key, select, attend. Cache quantization of the
    already-cached context is setup and untimed."""
    import numpy as np

    import msa_inputs as mi
    import oracle

    q = w.q_len
    done_tokens, spent, seqs = 0, 0.0, 0
    for b in range(w.batch):
        T = w.ctx_lens[b]
        ik = w.ik_rows(b, 0, T).numpy()
        ikc, iks = oracle.quantize(ik[:T - q])
        qi = mi.bf16_bits(w.q_idx[b * q:(b + 1) * q])
        qb = mi.bf16_bits(w.q[b * q:(b + 1) * q])
        # untimed: which K/V blocks the attention will read, quantized ahead as cache contents
        pre_c, pre_s = oracle.quantize(ik[T - q:])
        ids0, _ = oracle.select_sequence(
            oracle.index_scores(qi, np.concatenate([ikc, pre_c]), np.concatenate([iks, pre_s]),
                                T, q, w.max_blocks), T, q)
        blocks = sorted(set(int(x) for x in ids0.ravel() if x >= 0))
        kc = np.zeros((T, 4, 64), np.uint8)
        ks = np.zeros((T, 4, 8), np.uint8)
        vc, vs = np.zeros_like(kc), np.zeros_like(ks)
        for blk in blocks:
            t0, t1 = blk * 128, min(T - q, blk * 128 + 128)
            if t1 > t0:
                kc[t0:t1], ks[t0:t1] = oracle.quantize(w.kv_rows("k", b, t0, t1).numpy())
                vc[t0:t1], vs[t0:t1] = oracle.quantize(w.kv_rows("v", b, t0, t1).numpy())
        new_ik = ik[T - q:]
        new_k = w.kv_rows("k", b, T - q, T).numpy()
        new_v = w.kv_rows("v", b, T - q, T).numpy()
        t0 = time.perf_counter()
        c, s = oracle.quantize(new_ik)                                        # insert
        kc[T - q:], ks[T - q:] = oracle.quantize(new_k)
        vc[T - q:], vs[T - q:] = oracle.quantize(new_v)
        full_c, full_s = np.concatenate([ikc, c]), np.concatenate([iks, s])
        scores = oracle.index_scores(qi, full_c, full_s, T, q, w.max_blocks)  # indexer
        ids, _ = oracle.select_sequence(scores, T, q)                          # top-k
        for j in range(q):                                                    # attention
            oracle.sparse_attention_token(qb[j], kc, ks, vc, vs, T, ids[j], T - q + j,
                                          oracle.default_scale())
        spent += time.perf_counter() - t0
        done_tokens += q
        seqs += 1
        if spent >= target_seconds:
            break
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), model)
    except OSError:
        pass
    return {
        "value": round(done_tokens / spent, 3),
        "unit": "query-tokens/s",
        "cores": 1,
        "nproc": os.cpu_count(),
        "cpus_allowed": len(os.sched_getaffinity(0)),
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"{seqs} of {w.batch} sequences of the same workload (full 131072-token context, "
                  f"{q} query tokens each); {spent:.1f} s single-threaded; cache quantization of "
                  "the context untimed",
    }


if __name__ == "__main__":
    main()
