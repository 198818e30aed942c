#!/usr/bin/env python3
"""Benchmark of the MI355X GR00T action head (flow-matching DiT, System 1).

One step = one get_action call: K Euler steps of the 32-block DiT over one batch of
synthetic inputs already resident in HBM (prologue, graph of the K steps, output).
Default workload: B = 64, ragged VL lengths 200..400 padded to 400, mixed embodiment
ids, K = 4 (chunks/s). A second leg times get_action at B = 1 (300 VL tokens, 256
image + 44 text) for the p50 latency. The dominant kernel class is timed live with
HIP events on the call's stream (library launch timing) for the roofline, and the
CPU oracle is timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0  # dense e4m3 MFMA (the W8A8 GEMMs)
METRIC = "action chunks/sec at B=64 and get_action p50 latency (ms) at B=1, 32-layer DiT"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_per_launch(cls, w, inputs):
    """Algorithmic (flops, bytes) of one launch of a kernel class, and its bound.

    Counts only what the method must compute or move: valid VL tokens, weights read
    once, activations read and written once (bf16 activations, fp32 residual)."""
    c = w.cfg
    B, H, D, F, E = w.batch, c.action_horizon, c.hidden, c.ff_dim, c.vl_dim
    S = H + 1
    M = B * S
    L = w.vl_len
    Nc = (c.num_layers + 1) // 2
    wb = 1 if c.precision in ("fp8", "fp8a8") else 2  # e4m3 weight bytes
    valid = np.ones((B, L), bool) if inputs["vl_mask"] is None else inputs["vl_mask"].astype(bool)
    nvalid = int(valid.sum())
    if cls in ("qkv_proj", "q_proj", "o_proj", "out_proj", "ff_up", "ff_down"):
        n, k = {"qkv_proj": (3 * D, D), "q_proj": (D, D), "o_proj": (D, D), "out_proj": (D, D),
                "ff_up": (F, D), "ff_down": (D, F)}[cls]
        out_b = 8 if cls in ("o_proj", "ff_down") else 2  # residual add reads and writes fp32
        return 2.0 * M * n * k, n * k * wb + M * k * 2 + M * n * out_b, "mfma"
    if cls == "kv_proj":
        n = Nc * 2 * D
        return 2.0 * nvalid * E * n, n * E * wb + nvalid * E * 2 + nvalid * n * 2, "mfma"
    if cls == "attn_cross":
        # keys admitted per (sample, cross block); half the blocks use text/image splits
        # only with an image mask (none in this workload): every block reads all valid keys
        return 4.0 * S * D * nvalid, nvalid * 2 * D * 2 + 2 * M * D * 2, "hbm"
    if cls == "attn_self":
        return 4.0 * B * S * S * D, 4 * M * D * 2, "hbm"
    if cls in ("adaln", "norm3"):
        return 8.0 * M * D, M * D * 4 + M * D * 2, "hbm"
    if cls == "vlln":
        return 8.0 * B * L * E, B * L * E * 4, "hbm"
    return None


def gpu_leg(args, w, weights, inputs, noise, H, synth):
    import torch
    from dataclasses import replace
    b1 = synth.WORKLOADS[args.b1_workload]
    if b1.cfg != w.cfg and b1.cfg.num_layers == w.cfg.num_layers and b1.cfg.hidden == w.cfg.hidden:
        # the same model in another precision: the B=1 leg takes the handle's configuration
        b1 = replace(b1, name=f"{b1.name}_{w.cfg.precision}", cfg=w.cfg)
    assert b1.cfg == w.cfg, "the B=1 leg reuses the handle: same model required"
    max_vl = max(w.vl_len, b1.vl_len)
    h = H.Gr00tHead(w.cfg, max_batch=w.batch, max_vl_len=max_vl, flags=H.FLAG_USE_GRAPH)
    t = time.time()
    h.load_weights(weights).finalize()
    h.prepare(w.batch, w.vl_len)
    log(f"[bench] loaded + finalized + captured in {time.time() - t:.1f}s; device bytes {h.device_bytes() / 2**30:.2f} GiB")
    d = H.device_inputs(inputs, noise, h.act_torch_dtype)
    out = torch.empty((w.batch, w.cfg.action_horizon, w.cfg.action_dim), dtype=torch.float32, device="cuda:0")
    for _ in range(args.warmup):
        h.get_action(**d, out=out)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    first = None
    h.profile(2)  # launches outside the captured graph (prologue: VL LayerNorm, K/V projection) are timed live
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        h.get_action(**d, out=out)
        evs[i][1].record()
        if i == 0:
            first = out.clone()
    torch.cuda.synchronize()
    total_s = time.perf_counter() - t0
    per_call = [a.elapsed_time(b) for a, b in evs]
    prof_live = h.profile_read()
    h.profile(False)
    log(f"[bench] {w.name}: {args.steps} calls in {total_s * 1e3:.1f} ms; per call p50 {statistics.median(per_call):.3f} ms")

    # the same batch again with the VL key/value caches of the last full call reused (several
    # action chunks drawn from one backbone output)
    reuse = lambda: h.get_action_reuse_vl(w.batch, w.vl_len, d["state"], d["embodiment_id"], noise=d["noise"],
                                          action_mask=d["action_mask"], out=out)
    for _ in range(2):
        reuse()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        reuse()
    torch.cuda.synchronize()
    reuse_s = (time.perf_counter() - t0) / args.steps
    log(f"[bench] {w.name} reusing the VL caches: {reuse_s * 1e3:.3f} ms per call")

    # flow-matching training forward and loss on the same batch (seeded draws: t ~ Beta(1.5, 1),
    # actions ~ N(0, 1)); forward only
    rng = np.random.default_rng(5)
    acts = torch.from_numpy(rng.standard_normal(tuple(out.shape)).astype(np.float32)).cuda()
    tt = torch.from_numpy(rng.beta(1.5, 1.0, w.batch).astype(np.float32)).cuda()
    train = lambda: h.train_forward(d["vl_features"], d["vl_mask"], d["image_mask"], d["state"], d["embodiment_id"],
                                    acts, tt, d["noise"], action_mask=d["action_mask"], v_pred=False)
    for _ in range(2):
        train()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        loss = train()[0]
    torch.cuda.synchronize()
    train_s = (time.perf_counter() - t0) / args.steps
    log(f"[bench] {w.name} training forward: {train_s * 1e3:.3f} ms per batch, loss {float(loss.item()):.4f}")

    # live launch timing of every kernel class (eager, HIP events on the call's stream)
    h.profile(True)
    for _ in range(args.profile_calls):
        h.get_action(**d, out=out)
    torch.cuda.synchronize()
    prof = h.profile_read()
    h.profile(False)

    # B = 1 latency leg on the same handle
    bi, bn = synth.make_inputs(b1), synth.make_noise(b1)
    h.prepare(b1.batch, b1.vl_len)
    d1 = H.device_inputs(bi, bn, h.act_torch_dtype)
    out1 = torch.empty((1, b1.cfg.action_horizon, b1.cfg.action_dim), dtype=torch.float32, device="cuda:0")
    for _ in range(3 if args.b1_steps else 0):
        h.get_action(**d1, out=out1)
    torch.cuda.synchronize()
    lat_wall, lat_dev = [], []
    h.profile(True)
    h.get_action(**d1, out=out1)
    torch.cuda.synchronize()
    prof_b1 = h.profile_read()
    h.profile(False)
    for _ in range(args.b1_steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t = time.perf_counter()
        e0.record()
        h.get_action(**d1, out=out1)
        e1.record()
        torch.cuda.synchronize()
        lat_wall.append((time.perf_counter() - t) * 1e3)
        lat_dev.append(e0.elapsed_time(e1))
    h.close()
    return total_s, per_call, prof, first.cpu().numpy(), lat_wall, lat_dev, prof_b1, prof_live, reuse_s, train_s


# Horizon and step-count variants of the same 32-block model (the weights do not depend on
# either): the base N1.7 horizon of 40 and K in {1, 2, 8, 16} Euler steps.
VARIANTS = [("dit32_bf16_b1", 40, 4), ("dit32_bf16_b1", 16, 1), ("dit32_bf16_b1", 16, 2),
            ("dit32_bf16_b1", 16, 8), ("dit32_bf16_b1", 16, 16), ("dit32_bf16_b64", 40, 4),
            # B = 256 with e4m3 DiT weights (W8A16) and with per-row e4m3 GEMM inputs (W8A8)
            ("dit32_fp8_b256", 16, 4), ("dit32_w8a8_b256", 16, 4)]


def variants_leg(weights, H, synth, calls=20):
    """get_action p50 of each horizon / step-count variant (graph replays, inputs in HBM)."""
    from dataclasses import replace

    import torch
    out = []
    for name, hz, k in VARIANTS:
        base = synth.WORKLOADS[name]
        w = replace(base, name=f"{name}_h{hz}_k{k}", cfg=replace(base.cfg, action_horizon=hz, num_steps=k))
        inputs, noise = synth.make_inputs(w), synth.make_noise(w)
        h = H.Gr00tHead(w.cfg, max_batch=w.batch, max_vl_len=w.vl_len, flags=H.FLAG_USE_GRAPH)
        h.load_weights(weights).finalize()
        h.prepare(w.batch, w.vl_len)
        d = H.device_inputs(inputs, noise, h.act_torch_dtype)
        o = torch.empty((w.batch, hz, w.cfg.action_dim), dtype=torch.float32, device="cuda:0")
        for _ in range(3):
            h.get_action(**d, out=o)
        torch.cuda.synchronize()
        ts = []
        for _ in range(calls):
            t = time.perf_counter()
            h.get_action(**d, out=o)
            torch.cuda.synchronize()
            ts.append((time.perf_counter() - t) * 1e3)
        h.close()
        p50 = statistics.median(ts)
        out.append({"workload": w.name, "batch": w.batch, "precision": w.cfg.precision, "horizon": hz,
                    "euler_steps": k, "p50_ms": round(p50, 4),
                    "chunks_per_s": round(w.batch / p50 * 1e3, 1)})
        log(f"[bench] variant {w.name}: p50 {p50:.3f} ms")
    return out


def stats(xs):
    xs = sorted(xs)
    return {"p50_ms": round(statistics.median(xs), 4), "mean_ms": round(statistics.fmean(xs), 4),
            "std_ms": round(statistics.pstdev(xs), 4), "min_ms": round(xs[0], 4), "max_ms": round(xs[-1], 4),
            "p90_ms": round(xs[min(len(xs) - 1, int(0.9 * len(xs)))], 4)}


def cpu_leg(args, w, weights, inputs, noise, gpu_out):
    from threadpoolctl import threadpool_info

    from flow_matching_dit_amd import synth
    from oracle import gr00t_oracle as O
    t = time.time()
    P = O.effective_params(w.cfg.as_dict(), weights)
    log(f"[bench] oracle parameters ready in {time.time() - t:.1f}s")
    idx = list(range(args.cpu_samples))
    sub, nz = synth.take_samples(inputs, noise, idx)
    t = time.perf_counter()
    ref = O.get_action(w.cfg.as_dict(), weights, sub, nz, params=P)
    dt = time.perf_counter() - t
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    err = O.rel_l2(gpu_out[idx], ref)
    log(f"[bench] oracle: {len(idx)} samples in {dt:.1f}s; GPU vs oracle rel_l2 {err:.3e}")
    return {"value": round(len(idx) / dt, 5), "unit": "chunks/s", "cores": int(threads), "kind": "oracle",
            "sample": f"samples {idx[0]}..{idx[-1]} of the {w.batch}-sample {w.name} batch (full depth, "
                      f"same weights and inputs; samples are independent), one get_action",
            "seconds": round(dt, 2)}, err


def roofline(prof, w, inputs, profile_calls, prof_live):
    """Roofline of the dominant kernel class (largest summed duration in the per-launch
    profile). Its average launch duration is taken from the timed region itself when the
    class runs outside the captured graph (prof_live), else from the per-launch pass."""
    best, best_ms = None, -1.0
    for cls, (n, ms) in prof.items():
        if n > 0 and ms > best_ms and work_per_launch(cls, w, inputs) is not None:
            best, best_ms = cls, ms
    live = prof_live.get(best, (0, 0.0))[0] > 0
    n, ms = prof_live[best] if live else prof[best]
    flops, byts, bound = work_per_launch(best, w, inputs)
    avg_s = ms / n * 1e-3
    if bound == "mfma":
        # W8A8: the class's e4m3 x e4m3 contraction (its row quantisation inside the timed launch)
        peak = FP8_PEAK_TFLOPS if w.cfg.precision == "fp8a8" else BF16_PEAK_TFLOPS
        achieved, unit = flops / avg_s / 1e12, "TFLOP/s"
    else:
        achieved, peak, unit = byts / avg_s / 1e9, HBM_PEAK_GBS, "GB/s"
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{best}_{w.name}.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            t = json.load(f)
        from flow_matching_dit_amd.measure import kernel_source_hash
        if t.get("kernel_source_hash") == kernel_source_hash():
            traffic = t.get("bytes_per_launch")
    breakdown = {c: {"launches_per_call": v[0] // profile_calls, "ms_per_call": round(v[1] / profile_calls, 4)}
                 for c, v in prof.items() if v[0] > 0}
    return {"kernel": best, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "avg_launch_ms": round(ms / n, 5), "launches": n,
            "timed_in": "timed region (outside the graph)" if live else "per-launch pass (eager, same kernels)",
            "algorithmic_per_launch": {"flops": flops, "bytes": byts}}, breakdown


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dit32_bf16_b64")
    ap.add_argument("--b1-workload", default="dit32_bf16_b1")
    ap.add_argument("--b1-steps", type=int, default=30)
    ap.add_argument("--profile-calls", type=int, default=2)
    ap.add_argument("--cpu-samples", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variants", action="store_true",
                    help="also time the horizon 40 and K = 1, 2, 8, 16 variants and the B = 256 e4m3 and "
                         "W8A8 configurations (p50 per get_action)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (reference for HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "every sample of a get_action batch is independent, so more GPUs would each run "
              "their own share of the batch with no exchange.", file=sys.stderr)
        sys.exit(2)

    import torch

    from flow_matching_dit_amd import head as H
    from flow_matching_dit_amd import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = args.copy_calibration * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4}))
        return
    H.load_library()
    w = synth.WORKLOADS[args.workload]
    t = time.time()
    weights, inputs, noise = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    log(f"[bench] synthetic weights and inputs for {w.name} in {time.time() - t:.1f}s")
    (total_s, per_call, prof, first, lat_wall, lat_dev, prof_b1, prof_live, reuse_s,
     train_s) = gpu_leg(args, w, weights, inputs, noise, H, synth)
    value = w.batch * args.steps / total_s
    roof, breakdown = roofline(prof, w, inputs, args.profile_calls, prof_live)
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "chunks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total_s / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": {"bf16": "bf16", "fp8": "fp8e4m3-w/bf16", "fp8a8": "fp8e4m3", "fp32": "f32"}[w.cfg.precision],
        "data": "synthetic (seeded N(0,1) VL features/state/noise, N(0,0.02) weights)",
        "config": {"workload": w.name, "batch": w.batch, "vl_len_pad": w.vl_len, "layers": w.cfg.num_layers,
                   "hidden": w.cfg.hidden, "heads": w.cfg.num_heads, "ff": w.cfg.ff_dim,
                   "horizon": w.cfg.action_horizon, "action_dim": w.cfg.action_dim, "euler_steps": w.cfg.num_steps,
                   "graph": True},
        "per_call": stats(per_call),
        "latency_b1": (dict(workload=args.b1_workload, **stats(lat_wall), device=stats(lat_dev),
                            breakdown={c: {"launches": v[0], "ms": round(v[1], 4)} for c, v in prof_b1.items() if v[0]})
                       if lat_wall else None),
        "roofline": roof,
        "breakdown": breakdown,
        "reuse_vl": {"ms_per_call": round(reuse_s * 1e3, 4), "chunks_per_s": round(w.batch / reuse_s, 2),
                     "what": "gr00t_get_action_reuse_vl on the same batch: VL LayerNorm, key masks and K/V "
                             "projection of the previous full call reused"},
        "train_forward": {"ms_per_batch": round(train_s * 1e3, 4), "samples_per_s": round(w.batch / train_s, 2),
                          "what": "gr00t_train_forward on the same batch: x_t, one DiT forward with per-sample "
                                  "timesteps, masked MSE (forward only)"},
    }
    if args.variants:
        result["variants"] = variants_leg(weights, H, synth)
    if not args.no_cpu_baseline:
        cpu, err = cpu_leg(args, w, weights, inputs, noise, first)
        result["cpu_baseline"] = cpu
        result["parity_rel_l2_sampled"] = round(err, 6)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
