"""Benchmark of the batch-1 decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 8b_4k] [--no-cpu-baseline]

A step is one whole decode step (all layers, one kernel launch) over synthetic bf16
weights and KV cache already resident in HBM. Prints ONE JSON line. --launch stages|graph
times the same step split into one launch per stage (eagerly, or replayed from a HIP graph),
the launch-per-operator execution the persistent engine replaces. --verify M times a
verification step of M tokens (one launch; value = microseconds per token, the step's time / M).
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "bs=1 decode latency (us/token) + achieved HBM GB/s as % of 8 TB/s peak"
WORKLOADS = {
    "8b_4k": "Llama-3-8B-shaped decoder (32 layers, hidden 4096, 32x128 q heads, 8 KV heads, SwiGLU 14336, "
             "vocab 128256), batch 1, one decode token over a 4096-position KV cache",
    "8b_32k": "Llama-3-8B-shaped decoder, batch 1, one decode token over a 32768-position KV cache",
    "mla_8k": "MLA decoder stack (8 layers, hidden 7168, 16 heads, q/kv ranks 1536/512, 128+64 qk, v 128, "
              "SwiGLU 18432), batch 1, one decode token over an 8192-position latent cache",
    "moe_4k": "MLA + MoE decoder stack (4 layers, hidden 7168, MLA as above, 256 routed experts of 2048 + 1 "
              "shared, sigmoid top-8), batch 1, one decode token over a 4096-position latent cache",
    "tiny": "tiny decoder (2 layers, hidden 256), batch 1, KV 128",
    "8b_4k_fp8": "the 8B-shaped decoder with every linear matrix in FP8 E4M3 (one fp32 scale per row), "
                 "batch 1, one decode token over a 4096-position bf16 KV cache",
    "mla_8k_fp8": "the MLA stack with every linear matrix but the absorption matrices in FP8 E4M3 (one fp32 scale "
                  "per row), batch 1, one decode token over an 8192-position bf16 latent cache",
    "moe_4k_fp8": "the MLA + MoE stack with every linear matrix but the absorption matrices and the router in FP8 "
                  "E4M3 (one fp32 scale per row), batch 1, one decode token over a 4096-position bf16 latent cache",
    "mla_32k": "the MLA decoder stack (8 layers, hidden 7168, 16 heads) at batch 1, one decode token over a "
               "32768-position latent cache (dense attention)",
    "mla_32k_sparse": "the MLA decoder stack (8 layers, hidden 7168, 16 heads) with a sparse indexer (64 index heads of "
                      "128, top 2048 positions), batch 1, one decode token over a 32768-position cache",
    "moe_4k_mxfp4": "the MLA + MoE stack with every expert matrix in MXFP4 (E2M1 elements, one E8M0 scale per "
                    "32), other weights bf16, batch 1, one decode token over a 4096-position latent cache",
}
# Sources whose content decides the engine's memory traffic: a stored counter reading is
# reported only while their hash matches.
TRAFFIC_SOURCES = ["persistent_tile_scheduled_amd/csrc/engine.hip", "persistent_tile_scheduled_amd/csrc/plan_types.h",
                   "persistent_tile_scheduled_amd/csrc/planner.cpp"]


def source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(config):
    """HBM bytes per launch from the committed counter summary of this workload
    (profiles/dec_engine_<config>_traffic.md: a line `traffic_bytes_per_launch: N` and a line
    `source_hash: H`), or None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"dec_engine_{config}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip().strip("`")
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_hash") != source_hash() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(vals["traffic_bytes_per_launch"])


def copy_calibration(nbytes, reps):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters:
    each launch reads and writes `nbytes`."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "copy_calibration_bytes_written": nbytes,
                      "launches": reps}), flush=True)


def stream_read(nbytes_list, reps):
    """The HBM read ceiling for the engine's loads (dec_stream_read): GB/s per buffer size,
    the mean over `reps` launches timed with events on one stream."""
    import torch
    from persistent_tile_scheduled_amd import binding as B
    n_cu = B.device_query().n_cu
    sink = torch.empty(n_cu * 512, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    rows = []
    for nbytes in nbytes_list:
        buf = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
        for _ in range(3):
            B.stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), sink.numel() * 4, stream.cuda_stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            B.stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), sink.numel() * 4, stream.cuda_stream)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        rows.append({"bytes": nbytes, "us_per_launch": round(us, 2), "GB_s": round(nbytes / us / 1e3, 1)})
        print(f"[bench] stream read {nbytes / 2**20:.0f} MiB: {nbytes / us / 1e3:.1f} GB/s", file=sys.stderr, flush=True)
        del buf
    best = max(r["GB_s"] for r in rows)
    print(json.dumps({"metric": "HBM stream-read rate with the engine's loads (dec_stream_read)", "value": best,
                      "unit": "GB/s", "higher_is_better": True, "peak": HBM_PEAK_GBS,
                      "frac": round(best / HBM_PEAK_GBS, 4), "launches_per_size": reps, "sizes": rows}), flush=True)


def cpu_baseline(cfg, w, x, kv, eng=None, budget_s=10.0):
    """The fp64 oracle, as it stands, timed on a bounded sample of the same step: layers 0,
    1, ... in order (each from the previous layer's oracle output) until about `budget_s`
    seconds of oracle time or the whole stack, then the final norm + LM head; the per-token
    figure extrapolates the mean layer time to all layers. Weights are copied to the host
    before each layer's timed region."""
    import numpy as np
    import torch

    import oracle
    import workloads

    def W(name, index=None):
        t = w[name] if index is None else w[name][index]
        return workloads.bf16_bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()

    cache = {}

    def Wc(name, index=None):
        k = (name, index)
        if k not in cache:
            cache[k] = W(name, index)
        return cache[k]

    n = cfg["kv_len"]
    specs = workloads.weight_specs(cfg)
    xo = oracle.widen_bf16(workloads.bf16_bits(x))
    layer_s, done = 0.0, 0
    for l in range(cfg["n_layers"]):
        # host copies first (not timed). Routed experts: those the GPU selected for this
        # layer (the oracle fetches any other it picks itself)
        cache.clear()
        for s in specs:
            if s.name.startswith(f"layers.{l}.") and not s.name.startswith(f"layers.{l}.experts."):
                Wc(s.name)
        if eng is not None and cfg["arch"] == "moe":
            k = cfg["top_k"]
            for e in eng.buffer(f"layers.{l}.topk")[:k].view(torch.int32).cpu().tolist():
                for m in ("w_gate", "w_up", "w_down"):
                    Wc(f"layers.{l}.experts.{m}", int(e))
        kvl = workloads.bf16_bits(kv[l])
        t0 = time.perf_counter()
        xo, _ = oracle.layer(cfg, Wc, l, xo, kvl, n)
        layer_s += time.perf_counter() - t0
        done += 1
        if layer_s >= budget_s:
            break
    head_s = 0.0
    has_head = cfg.get("vocab", 0) > 0
    if has_head:
        cache.clear()
        for s in specs:
            if s.name.startswith("final_norm") or s.name.startswith("lm_head"):
                Wc(s.name)
        t0 = time.perf_counter()
        oracle.head(cfg, Wc, xo)
        head_s = time.perf_counter() - t0
    per_token = layer_s / done * cfg["n_layers"] + head_s
    return {"value": per_token * 1e6, "unit": "us/token", "kind": "oracle",
            "sample": f"layers 0..{done - 1} of {cfg['n_layers']} ({layer_s:.2f} s) extrapolated x{cfg['n_layers'] / done:.2f}"
                      + (f" + final norm and LM head ({head_s:.2f} s)" if has_head else "")}


def host_description():
    """The host the oracle runs on: core counts, CPU model, BLAS library and its threads."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", None
    try:
        import threadpoolctl
        for i in threadpoolctl.threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')}"
                threads = i.get("num_threads")
                break
    except Exception:
        pass
    return {"cpu_model": model, "cores_online": os.cpu_count(), "cores_available": len(os.sched_getaffinity(0)),
            "blas": blas, "blas_threads": threads}


def cpu_baselines(cfg, w, x, kv, eng, budget_s):
    """The oracle timed twice on the host: with every BLAS thread the process may use, and
    with one thread (each on its own bounded sample of the same step)."""
    import threadpoolctl
    host = host_description()
    run_all = cpu_baseline(cfg, w, x, kv, eng, budget_s)
    with threadpoolctl.threadpool_limits(limits=1, user_api="blas"):
        run_one = cpu_baseline(cfg, w, x, kv, eng, budget_s)
    threads = host["blas_threads"] or host["cores_available"]
    out = dict(run_all, cores=int(threads), threads=int(threads), **host)
    out["one_thread"] = {"value": run_one["value"], "unit": "us/token", "cores": 1, "sample": run_one["sample"]}
    return out


def generation(args, cfg, w, kv, x):
    """Greedy generation with one plan for the largest position: T steps issued back to back,
    each at the position and with the token the previous step left in the device state. A
    model without an LM head (vocab 0) has no token to feed back: its steps take the same
    input vector x at advancing positions."""
    import torch
    import workloads
    from persistent_tile_scheduled_amd.engine import DecodeEngine

    T, W = args.generate, args.warmup
    n = cfg["kv_len"]
    if T + W > n:
        raise SystemExit("--generate T needs T + warmup <= kv_len")
    greedy = cfg.get("vocab", 0) > 0
    if greedy:
        w["embed"] = workloads.generate_embedding(cfg, seed=args.seed, device="cuda")
    xin = None if greedy else x
    eng = DecodeEngine(cfg, w, max_len=n)
    p0 = n - T - W if args.start_pos is None else args.start_pos
    if not 0 <= p0 <= n - T - W:
        raise SystemExit("--start-pos P needs 0 <= P <= kv_len - T - warmup")
    eng.set_state(p0, 0)
    for _ in range(W):
        eng.step_dynamic(kv, xin)
    torch.cuda.synchronize()
    eng.status()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(eng.stream)
    for _ in range(T):
        eng.step_dynamic(kv, xin)
    b.record(eng.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eng.status()
    st = eng.read_state()
    assert st[0] == p0 + T + W and st[2] == T + W, st
    gpu_us = a.elapsed_time(b) * 1e3 / T
    us = wall * 1e6 / T
    print(json.dumps({
        "metric": ("greedy generation latency (us/token), steps issued back to back" if greedy else
                   "decode latency at advancing positions (us/token), steps issued back to back"),
        "value": round(us, 2), "unit": "us/token", "n_gpus": 1, "steps": T, "warmup": W,
        "higher_is_better": False, "tokens_per_s": round(1e6 / us, 1),
        "gpu_us_per_token": round(gpu_us, 2),
        "config": {"workload": f"{args.config}: {WORKLOADS.get(args.config, args.config)}",
                   "positions": [p0 + W, p0 + W + T - 1], "max_len": n, "batch": 1},
        "launch": "dynamic plan (max_len = kv_len), one launch per token, no host work between tokens",
        "dtype": "bf16", "data": "synthetic"}), flush=True)
    teardown(eng)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="8b_4k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, metavar="S",
                    help="seconds of oracle layer time per CPU-baseline run (all cores, one thread)")
    ap.add_argument("--launch", choices=["persistent", "stages", "graph"], default="persistent",
                    help="persistent: the step as one engine launch (the product); stages: one launch per "
                         "stage of the same tasks; graph: those launches replayed from a HIP graph")
    ap.add_argument("--start-pos", type=int, default=None, metavar="P",
                    help="with --generate: the position of the first warm-up step (default kv_len - T - warmup, "
                         "so that the timed steps end at the plan's largest position)")
    ap.add_argument("--generate", type=int, default=0, metavar="T",
                    help="time T greedy steps of a plan with a per-step length, issued back to back "
                         "(positions kv_len - T .. kv_len - 1, each step's token from the last)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--verify", type=int, default=1, metavar="M",
                    help="time a verification step of M tokens (2..4, GQA bf16 workloads) instead of a "
                         "one-token decode step; no CPU baseline")
    ap.add_argument("--stream-read", action="store_true",
                    help="only measure the HBM stream-read rate of the engine's loads (dec_stream_read) "
                         "over 256 MiB, 1 GiB and 4 GiB buffers")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this engine has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(args.steps, 1))
        return
    if args.stream_read:
        stream_read([256 << 20, 1 << 30, 4 << 30], max(args.steps, 1))
        return

    import workloads
    from persistent_tile_scheduled_amd.engine import DecodeEngine

    cfg = dict(workloads.get_config(args.config))
    m = args.verify
    name = args.config
    if m > 1:
        if args.launch != "persistent" or args.generate:
            print("--verify times whole persistent steps only", file=sys.stderr)
            sys.exit(2)
        cfg["verify"] = m
        name = f"{args.config}_verify{m}"
        args.no_cpu_baseline = True
    print(f"[bench] generating {name} inputs on cuda:0", file=sys.stderr, flush=True)
    w, x, kv = workloads.generate(cfg, seed=args.seed, device="cuda")
    if args.generate:
        generation(args, cfg, w, kv, x)
        return
    eng = DecodeEngine(cfg, w)
    alg_bytes = eng.sizes["algorithmic_bytes_per_step"]
    stream = eng.stream
    if args.launch == "persistent":
        run = lambda: eng.step(x, kv)
    else:
        run = lambda: eng.step_stages(x, kv)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    eng.status()
    if args.launch == "graph":
        graph = eng.capture_stages(x, kv)
        run = graph.replay
        run()
        torch.cuda.synchronize()
        eng.status()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eng.status()
    per = [a.elapsed_time(b) * 1e3 for a, b in ev]  # us per launch
    mean_us = statistics.mean(per)
    med_us = statistics.median(per)
    us_per_step = wall * 1e6 / args.steps
    us_per_token = us_per_step / m
    achieved = alg_bytes / (mean_us * 1e-6) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on a bounded sample (all cores, then one thread)", file=sys.stderr, flush=True)
        cpu = cpu_baselines(cfg, w, x, kv, eng, args.cpu_budget)

    line = {
        "metric": METRIC,
        "value": round(us_per_token, 2),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_step / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8", "mxfp4": "mxfp4"}.get(cfg.get("weights"), "bf16"),
        "data": "synthetic (seeded N(0,0.02) " + {"fp8": "weights quantised per row to FP8 E4M3",
                                                  "mxfp4": "bf16 weights, expert matrices quantised per block of 32 to MXFP4"
                                                  }.get(cfg.get("weights"), "bf16 weights") + ", N(0,1) bf16 KV and input)",
        "config": {"workload": f"{name}: {WORKLOADS.get(args.config, args.config)}" +
                   (f"; a verification step of {m} tokens at positions kv_len .. kv_len + {m - 1}" if m > 1 else ""),
                   "kv_len": cfg["kv_len"], "batch": 1, "tokens_per_step": m},
        "launch": args.launch if args.launch == "persistent" else
        f"{args.launch}: {eng.n_stages} launches per step",
        "tokens_per_s": round(1e6 / us_per_token, 1),
        "us_per_step": round(us_per_step, 2),
        "kernel_us_mean": round(mean_us, 2),
        "kernel_us_median": round(med_us, 2),
        "kernel_us_p10": round(sorted(per)[len(per) // 10], 2),
        "kernel_us_p90": round(sorted(per)[(len(per) * 9) // 10], 2),
        "algorithmic_bytes_per_step": alg_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(name)},
        "source_hash": source_hash(),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    teardown(eng)


def teardown(eng):
    """Release the plan and the engine's device memory before the interpreter exits, with the
    device idle: nothing of the engine is left to interpreter shutdown (profilers that hook the
    runtime tear down in exit handlers)."""
    import torch
    torch.cuda.synchronize()
    eng.plan.close()
    del eng
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
