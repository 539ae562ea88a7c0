"""Benchmark of the Domino draft-block rollout on one MI355X.

One step = one whole rollout (LM-head logits, first proposal, [pool], GRU
prefix, 14 correction steps with feedback) for one batch of synthetic
requests whose inputs are already resident in HBM, replayed from the
library's HIP graph.  The default workload is the Qwen3-8B-shaped rollout
at batch 1 with full-vocabulary correction (K = 0); ``--workload`` and
``--k`` select the other cells of the matrix (8B at B = 1/8/64 with K = 0 or
2048, 27B-class at B = 64); ``--in-library-s`` has the library form the
per-step projector offsets from the hiddens inside the timed step instead of
taking them as an input.

Prints one JSON line: ms per block (lower is better), the roofline figure of
the dominant kernel (its average duration from HIP events stamped by each of
its launches' own dispatch, in eager runs right after the timed region on the
same stream), and the CPU oracle's time on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix
FP32_PEAK_TFLOPS = 157.3


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic(shape, B, K, union_sizes=None, proposals=15):
    """Algorithmic bytes / flops per launch of each kernel class (the unit
    figures of the design notes times the units one launch processes).
    union_sizes: rows of each request group's pool union when the pool
    correction streams the unions."""
    V, H, e, g, r = shape.vocab, shape.hidden, shape.emb_dim, shape.gru_hidden, shape.proj_dim
    wb = 2 if shape.dtype == "bf16" else 4
    pool = 0 < K < V
    if pool and union_sizes is not None:
        # each group's union rows (fc2 row + 16-byte record), the members'
        # base values, u as hi/lo planes
        correct_bytes = sum(int(n) for n in union_sizes) * (r * wb + 16) + B * K * 4 + B * r * 4
    elif pool:
        # gathered fc2 rows + their biases, compact base values, pool ids, u
        correct_bytes = B * K * (r * wb + wb + 4 + 4) + B * r * 4
    else:
        # the whole fc2 and b2, one base row per request, u
        correct_bytes = V * r * wb + V * wb + B * V * 4 + B * r * 4
    lm_bytes = V * H * wb + B * 15 * H * wb + 15 * B * V * 4
    lm_flops = 2.0 * 15 * B * H * V
    # GRU update + projector layer 1 of one correction step: the stacked
    # [fc1; W_hh] rows once, the gate inputs (row G[token], c = W_hh h, h),
    # the new h and c, u with its bf16 planes and s; the last step has no
    # W_hh rows and no c.  Average per step launch over the P - 1 steps.
    gates_in = B * (3 * g * 4 + 3 * g * 4 + g * 4)
    full = (r + 3 * g) * g * wb + gates_in + B * (g * 4 + 3 * g * 4 + r * (4 + 2 + 2) + r * 4)
    last = r * g * wb + gates_in + B * (g * 4 + r * (4 + 2 + 2) + r * 4)
    nsteps = max(proposals - 1, 1)
    step_bytes = ((nsteps - 1) * full + last) / nsteps
    return {"correct_bytes": correct_bytes, "lm_bytes": lm_bytes, "lm_flops": lm_flops,
            "step_bytes": step_bytes}


def _code_only(text):
    """Source text without comments, trailing blanks and empty lines, so that
    a comment edit does not mark recorded counters as stale."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gru_corrected_draft_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def read_counter(kernel, workload, digest, field="hbm_bytes_per_launch"):
    """A figure recorded from rocprofv3 counters (HBM bytes per launch, or
    the matrix-core busy fraction), if they were taken on the current kernel
    sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_d = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    m_t = re.search(field + r":\s*([0-9.eE+]+)", text)
    if not m_d or not m_t or m_d.group(1) != digest:
        return None
    return float(m_t.group(1))


def read_traffic(kernel, workload, digest):
    return read_counter(kernel, workload, digest)


def host_info():
    """CPU model, BLAS build and the BLAS thread count the oracle runs with."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = None, None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')}, " \
                       f"{i.get('threading_layer')})"
                threads = int(i.get("num_threads", 1))
                break
    except Exception:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"cpu_model": model, "blas": blas, "numpy": np.__version__,
            "threads": threads or affinity, "host_cpus": affinity}


def cpu_baseline(f32, shape, B, K, input_seed, budget_s, proposals=None, in_library_s=False,
                 max_blocks=20):
    """The oracle, as it stands, on whole blocks of the same workload until
    about budget_s seconds of work; ms per block (with in_library_s the
    oracle also forms the step offsets from the hiddens, inside the timing)."""
    import oracle
    from gru_corrected_draft_amd import synth
    info = host_info()
    times = []
    t_start = time.perf_counter()
    trial = 0
    while True:
        inp = synth.make_inputs(shape, B, input_seed, trial)
        X = inp.hidden_f32()
        t0 = time.perf_counter()
        s = (oracle.step_offsets(X, f32["fc1_x_w"], f32["fc1_b"]) if in_library_s
             else inp.step_s)
        oracle.rollout(f32, X, s, inp.verified, K, proposals=proposals)
        times.append(time.perf_counter() - t0)
        trial += 1
        if time.perf_counter() - t_start > budget_s or trial >= max_blocks:
            break
    return {"value": round(1e3 * float(np.median(times)), 3), "unit": "ms/block",
            "cores": int(info["threads"]), "kind": "oracle",
            "sample": f"{trial} whole blocks (trials 0..{trial - 1}) of the same workload, "
                      f"NumPy fp32 oracle, median",
            "cpu_model": info["cpu_model"], "blas": info["blas"], "numpy": info["numpy"],
            "host_cpus": info["host_cpus"]}


def one_thread_baseline(f32, shape, B, K, input_seed):
    """The same oracle on one BLAS thread, one block (ms)."""
    import oracle
    from gru_corrected_draft_amd import synth
    inp = synth.make_inputs(shape, B, input_seed, 0)
    X = inp.hidden_f32()
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        return None
    with threadpool_limits(limits=1, user_api="blas"):
        t0 = time.perf_counter()
        oracle.rollout(f32, X, inp.step_s, inp.verified, K)
        return round(1e3 * (time.perf_counter() - t0), 3)


def lower_bound_ms(alg, shape, B, K, P):
    """max(LM-head bytes / HBM peak, LM-head flops / bf16 peak) plus every
    other algorithmic byte of the block over HBM peak (no launch or sync
    latency): the block's roofline time."""
    steps = max(P - 1, 0)
    lm_ms = max(alg["lm_bytes"] / (HBM_PEAK_GBS * 1e9), alg["lm_flops"] / (BF16_PEAK_TFLOPS * 1e12)) * 1e3
    other = steps * (alg["correct_bytes"] + alg["step_bytes"])
    return lm_ms + other / (HBM_PEAK_GBS * 1e9) * 1e3


# the metric's cells: the 8B-shaped rollout at B = 1/8/64 with K = 0 and 2048,
# and the 27B-class one at B = 64, K = 2048 (first: the headline cell)
MATRIX = [("8b_b1", 0), ("8b_b1", 2048), ("8b_b8", 0), ("8b_b8", 2048), ("8b_b64", 0),
          ("8b_b64", 2048), ("27b_b64", 2048)]


def time_cell(h, shape, wl_name, B, K, args, hid, s, ver, digest):
    """One cell: W warm-up replays, exactly K timed graph replays between
    synchronisations, a spread of 5 x 20 replays, and the per-kernel
    durations of K eager runs on the same stream.  Returns the cell's record
    (without the CPU baseline) and the replayed tokens."""
    import torch
    from gru_corrected_draft_amd import rollout as R
    P = args.proposals
    prop = None if P == 15 else P
    out_t = torch.empty((B, P), dtype=torch.int32, device="cuda")
    out_l = torch.empty((B, P), dtype=torch.float32, device="cuda")

    # warm-up (the first call captures the graph)
    for _ in range(args.warmup):
        h.run(hid, s, ver, K, out_tokens=out_t, out_top1=out_l, graph=True, proposals=prop)
    torch.cuda.synchronize()
    ref_tokens = out_t.clone()

    # timed region: graph replays on torch's current stream
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        h.run(hid, s, ver, K, out_tokens=out_t, out_top1=out_l, graph=True, proposals=prop)
    ev1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    ms_step = ev0.elapsed_time(ev1) / args.steps
    assert torch.equal(out_t, ref_tokens), "graph replays disagree"

    # spread: rounds of back-to-back replays (median, p10, p90 of the
    # per-block time of each round), outside the timed region
    rounds = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            h.run(hid, s, ver, K, out_tokens=out_t, out_top1=out_l, graph=True, proposals=prop)
        e1.record()
        torch.cuda.synchronize()
        rounds.append(e0.elapsed_time(e1) / 20)
    spread = {"rounds": 5, "replays_per_round": 20,
              "median_ms": round(float(np.median(rounds)), 4),
              "p10_ms": round(float(np.percentile(rounds, 10)), 4),
              "p90_ms": round(float(np.percentile(rounds, 90)), 4)}
    flushed = None
    if args.flushed:
        # each replay timed alone after streaming 512 MB, so the memory-side
        # cache holds none of the weights the block reads
        junk = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        per = []
        for _ in range(20):
            junk.add_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            h.run(hid, s, ver, K, out_tokens=out_t, out_top1=out_l, graph=True, proposals=prop)
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1))
        del junk
        flushed = {"replays": 20, "median_ms": round(float(np.median(per)), 4),
                   "p10_ms": round(float(np.percentile(per, 10)), 4),
                   "p90_ms": round(float(np.percentile(per, 90)), 4)}
    assert torch.equal(out_t, ref_tokens), "graph replays disagree"

    # per-kernel durations: HIP events stamped by each kernel's dispatch, eager runs, same stream
    h.set_timing(True)
    h.reset_kernel_times()
    for _ in range(args.steps):
        h.run(hid, s, ver, K, out_tokens=out_t, out_top1=out_l, proposals=prop)
    torch.cuda.synchronize()
    kt = h.kernel_times()
    h.set_timing(False)
    assert torch.equal(out_t, ref_tokens), "eager run disagrees with graph replay"
    avg = {k: (ms / n if n else None) for k, (ms, n) in kt.items()}
    log(f"[bench] {wl_name} K={K}: {ms_step:.4f} ms/block; per-launch ms: " +
        ", ".join(f"{k}={v:.4f}" for k, v in avg.items() if v))

    union_sizes = None
    if 0 < K < shape.vocab:
        try:
            union_sizes = h.read_workspace(3).cpu().tolist()
        except R.DominoError:
            union_sizes = None
    alg = algorithmic(shape, B, K, union_sizes, P)
    corr_ms = avg["correct"]
    lm_ms = avg["lmhead"]
    corr_total = (corr_ms or 0.0) * max(P - 1, 0)
    lm_bound_mfma = 15 * B > 128
    wkey = f"{wl_name}_k{K}"
    if corr_ms is None or (lm_bound_mfma and lm_ms > corr_total):
        # the LM-head dominates (always when no correction step runs)
        if lm_bound_mfma:
            achieved = alg["lm_flops"] / (lm_ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "kernel": "lmhead_gemm", "achieved": round(achieved, 1),
                    "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
        else:
            achieved = alg["lm_bytes"] / (lm_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "kernel": "lmhead_gemm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        roof["traffic"] = read_traffic("lmhead", wkey, digest)
        if lm_bound_mfma:  # rocprofv3 MfmaUtil of the same kernel, when recorded
            roof["mfma_util_counter"] = read_counter("lmhead", wkey, digest, "mfma_util")
        dominant_ms = lm_ms
    else:
        achieved = alg["correct_bytes"] / (corr_ms * 1e-3) / 1e9
        kind = ("union" if union_sizes is not None else "pool") if 0 < K < shape.vocab else "full"
        roof = {"bound": "hbm", "kernel": "correct_" + kind,
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": read_traffic("correct", wkey, digest)}
        dominant_ms = corr_ms
    roof["launch_ms"] = round(dominant_ms, 5)
    phases = {k: {"ms_per_launch": round(v, 5), "launches_per_block": kt[k][1] // args.steps}
              for k, v in avg.items() if v}
    # achieved algorithmic bandwidth of the HBM-bound phases (the step product
    # is latency bound: ~8 MB per launch against a few-microsecond launch)
    for k, nbytes in (("correct", alg["correct_bytes"]), ("step", alg["step_bytes"])):
        if k in phases:
            gbs = nbytes / (avg[k] * 1e-3) / 1e9
            phases[k]["alg_gb_s"] = round(gbs, 1)
            phases[k]["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    if "lmhead" in phases:
        if lm_bound_mfma:
            phases["lmhead"]["alg_tflop_s"] = round(alg["lm_flops"] / (lm_ms * 1e-3) / 1e12, 1)
        phases["lmhead"]["alg_gb_s"] = round(alg["lm_bytes"] / (lm_ms * 1e-3) / 1e9, 1)
    # one correction step as a whole: its correction launch plus the GRU
    # update and projector launches that feed the next step (the prefix
    # launch included), algorithmic bytes of both over their summed time
    per_step = None
    if P > 1 and "correct" in phases:
        t_ms = sum(avg[k] * kt[k][1] / args.steps for k in ("correct", "step", "gru") if avg.get(k))
        t_ms /= P - 1
        nbytes = alg["correct_bytes"] + alg["step_bytes"]
        per_step = {"ms": round(t_ms, 5), "alg_gb_s": round(nbytes / (t_ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(nbytes / (t_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "bytes": "correction + stacked [fc1; W_hh] rows + gate inputs (the W_ih "
                             "product is read as one row of the per-id table G, 3g floats per "
                             "request, not as W_ih itself)"}
    lb = lower_bound_ms(alg, shape, B, K, P)
    cell = {"workload": wl_name, "model": shape.name, "batch": B, "K": K, "proposals": P,
            "ms_per_block": round(ms_step, 4), "wall_ms_per_block": round(wall_ms / args.steps, 4),
            "lower_bound_ms": round(lb, 4), "frac_of_lower_bound": round(lb / ms_step, 4),
            "spread": spread, "roofline": roof, "per_step": per_step, "phases": phases}
    if flushed:
        cell["flushed"] = flushed
    if union_sizes is not None:
        cell["pool_union_rows"] = union_sizes
    return cell, ref_tokens


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    help="one cell only (8b_b1, 8b_b8, 8b_b64, 27b_b64, tiny_b1); default: the "
                         "headline cell 8b_b1 K=0 plus every cell of the metric's matrix")
    ap.add_argument("--k", type=int, default=None, help="pool size (0 = full vocabulary)")
    ap.add_argument("--batch", type=int, default=None,
                    help="requests per block (default: the workload's batch)")
    ap.add_argument("--proposals", type=int, default=15,
                    help="proposals per block (< 15: truncated rollout, e.g. 8 for b8 serving)")
    ap.add_argument("--in-library-s", action="store_true",
                    help="form the per-step projector offsets in the library from the hiddens "
                         "(run without step_s)")
    ap.add_argument("--step-path", type=int, default=0, choices=(0, 1, 2, 3),
                    help="GRU/projector step: 0 auto, 1 fused gates + rows, 2 gate kernel + rows, "
                         "3 gate kernel + matrix cores")
    ap.add_argument("--pool-strategy", type=int, default=0, choices=(0, 1, 2),
                    help="pool correction at 17-64 requests: 0 automatic, 1 per-request "
                         "gather, 2 group unions")
    ap.add_argument("--flushed", action="store_true",
                    help="also time replays one by one after streaming 512 MB (cold memory-side cache)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the headline cell's baseline")
    ap.add_argument("--cell-cpu-budget", type=float, default=3.0,
                    help="seconds of oracle work for each other cell's baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times "
                         "(reference for the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py times one GPU: the rollout runs on a single MI355X, and --gpus above 1 "
              "is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    from gru_corrected_draft_amd import rollout as R
    from gru_corrected_draft_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "bytes_written": n, "launches": 3}))
        return

    if args.workload is None:
        cells = list(MATRIX)
    else:
        wl = synth.WORKLOADS[args.workload]
        cells = [(args.workload, wl.ks[0] if args.k is None else args.k)]
    digest = kernel_source_digest()
    records = []
    head_line = None
    model_cache = {}
    for ci, (wl_name, K) in enumerate(cells):
        wl = synth.WORKLOADS[wl_name]
        shape = synth.MODELS[wl.model]
        B = wl.batch if (args.batch is None or args.workload is None) else args.batch
        if wl.model not in model_cache:
            for old in model_cache.values():   # one model's weights on the device at a time
                old["h"].close()
            model_cache.clear()
            t0 = time.time()
            w = synth.make_weights(shape)
            dev = R.device_weights(w)
            # one handle per model, sized like the parity tests' (64 requests, pools of 2048)
            h = R.DominoRollout(dev, max_batch=64, max_k=2048)
            h.set_pool_strategy(args.pool_strategy)
            h.set_step_path(args.step_path)
            model_cache[wl.model] = {"w": w, "dev": dev, "h": h}
            log(f"[bench] {shape.name}: weights and handle ready in {time.time() - t0:.1f}s")
        m = model_cache[wl.model]
        inp = synth.make_inputs(shape, B, wl.input_seed, 0)
        hid, s, ver = R.device_inputs(inp)
        if args.in_library_s:
            assert m["h"].has_offsets, "the weight set has no fc1_x_w / fc1_b"
            s = None
        cell, _ = time_cell(m["h"], shape, wl_name, B, K, args, hid, s, ver, digest)
        if not args.no_cpu_baseline:
            f32 = {n: m["w"].f32(n) for n in m["w"].raw}
            budget = args.cpu_budget if ci == 0 else args.cell_cpu_budget
            log(f"[bench] cpu baseline {wl_name} K={K} (~{budget:.0f}s)")
            cb = cpu_baseline(f32, shape, B, K, wl.input_seed, budget,
                              None if args.proposals == 15 else args.proposals, args.in_library_s,
                              max_blocks=20 if ci == 0 else 5)
            if ci == 0 and args.proposals == 15 and not args.in_library_s:
                cb["one_thread_ms"] = one_thread_baseline(f32, shape, B, K, wl.input_seed)
                cb["one_thread_sample"] = "trial 0 of the same workload on one BLAS thread"
            cell["cpu_baseline"] = cb
        else:
            cell["cpu_baseline"] = None
        records.append(cell)
        if ci == 0:
            head_line = cell
    for mc in model_cache.values():
        mc["h"].close()

    head = head_line
    P = args.proposals
    K0 = head["K"]
    line = {
        "metric": f"Domino rollout ms/block ({P} proposals)",
        "value": head["ms_per_block"],
        "unit": "ms/block",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_block"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if synth.MODELS[synth.WORKLOADS[head["workload"]].model].dtype == "bf16"
        else "f32",
        "data": "synthetic",
        "config": {"workload": f"{head['model']}-shaped Domino rollout, batch {head['batch']}, "
                               f"{'full-vocabulary correction (K=0)' if K0 == 0 else f'pool K={K0}'}",
                   "batch": head["batch"], "K": K0,
                   "vocab": synth.MODELS[synth.WORKLOADS[head["workload"]].model].vocab,
                   "block_size": 16, "proposals": P,
                   "step_offsets": "in library" if args.in_library_s else "input",
                   "pool_strategy": ("auto", "gather", "unions")[args.pool_strategy],
                   "step_path": ("auto", "fused", "gates+rows", "gates+mfma")[args.step_path],
                   "accumulate": "fp32", "mode": "hip graph replay"},
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "per_step": head["per_step"],
        "phases": head["phases"],
        "spread": head["spread"],
        "cells": [{k: v for k, v in c.items()} for c in records],
        "kernel_source_digest": digest,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
