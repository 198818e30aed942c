#!/usr/bin/env python3
"""Benchmark of the MI355X GR00T action head (flow-matching DiT, System 1).

One step = one get_action call: K Euler steps of the 32-block DiT over one batch of
synthetic inputs already resident in HBM (prologue, graph of the K steps, output).
Headline workload: B = 64, ragged VL lengths 200..400 padded to 400, mixed embodiment
ids, K = 4 (chunks/s, calls enqueued back to back with launch timing off). Further legs:

* B = 1 latency (300 VL tokens, 256 image + 44 text): p50 of synchronised calls, with the
  algorithmic HBM bytes of one call over that time against the 8 TB/s peak;
* the other configurations (tiny fp32 B = 1; B = 16 with horizon 64, 1024 VL tokens and
  K = 8; B = 256 with e4m3 DiT weights): p50, chunks/s and a phase-roofline fraction;
* an eager per-launch pass (HIP events around every launch on the call's stream) for the
  per-class breakdown, the dominant kernel's roofline and the DiT GEMMs against bf16 peak;
* the CPU oracle on the full headline batch.

Phase roofline of a configuration: for every kernel class with a work model, its launches
per call times max(flops / peak, algorithmic bytes / 8 TB/s), summed; the fraction is that
lower bound over the measured p50.
"""
import argparse
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0    # dense e4m3 MFMA (the W8A8 GEMMs)
FP32_PEAK_TFLOPS = 157.3    # fp32 vector (the fp32 configuration's GEMMs)
METRIC = "action chunks/sec at B=64 and get_action p50 latency (ms) at B=1, 32-layer DiT"
GEMM_CLASSES = ("qkv_proj", "q_proj", "o_proj", "ff_up", "ff_down")
# configurations timed besides the headline (B = 64) and latency (B = 1) legs
OTHER_CONFIGS = ("tiny_fp32_b1", "dit32_bf16_b16_h64", "dit32_fp8_b256")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_per_launch(cls, w, inputs):
    """Algorithmic (flops, bytes) of one launch of a kernel class, and its bound.

    Counts only what the method must compute or move: valid VL tokens, weights read once
    (per-embodiment tables once per category present), activations read and written once
    (bf16 activations, fp32 residual). The per-embodiment classes average their per-step
    launches (action encoder: 3 per step, decoder: 2, state encoder: 2 per call)."""
    c = w.cfg
    B, H, D, F, E, A = w.batch, c.action_horizon, c.hidden, c.ff_dim, c.vl_dim, c.action_dim
    S = H + 1
    M = B * S
    L = w.vl_len
    Nc = (c.num_layers + 1) // 2
    wb = {"fp32": 4, "bf16": 2, "fp8": 1, "fp8a8": 1}[c.precision]   # DiT weight bytes
    ab = 4 if c.precision == "fp32" else 2                              # activation / table bytes
    valid = np.ones((B, L), bool) if inputs["vl_mask"] is None else inputs["vl_mask"].astype(bool)
    nvalid = int(valid.sum())
    ncat = len(np.unique(inputs["embodiment_id"]))
    if cls in ("qkv_proj", "q_proj", "o_proj", "out_proj", "ff_up", "ff_down"):
        n, k = {"qkv_proj": (3 * D, D), "q_proj": (D, D), "o_proj": (D, D), "out_proj": (D, D),
                "ff_up": (F, D), "ff_down": (D, F)}[cls]
        w_b = ab if cls == "out_proj" else wb
        out_b = 8 if cls in ("o_proj", "ff_down") else ab  # residual add reads and writes fp32
        return 2.0 * M * n * k, n * k * w_b + M * k * ab + M * n * out_b, "mfma"
    if cls == "kv_proj":
        n = Nc * 2 * D
        return 2.0 * nvalid * E * n, n * E * wb + nvalid * E * ab + nvalid * n * ab, "mfma"
    if cls == "attn_cross":
        # a cross block reads the keys and values of its admitted tokens: every valid token, or
        # with an image/text split the image or the text tokens, the blocks alternating between
        # the two sets (on average half the valid tokens per block)
        keys = nvalid if inputs.get("image_mask") is None else nvalid / 2
        return 4.0 * S * D * keys, keys * 2 * D * ab + 2 * M * D * ab, "hbm"
    if cls == "attn_self":
        return 4.0 * B * S * S * D, 4 * M * D * ab, "hbm"
    if cls in ("adaln", "norm3"):
        return 8.0 * M * D, M * D * 4 + M * D * ab, "hbm"
    if cls == "vlln":
        return 8.0 * B * L * E, B * L * E * (ab + ab), "hbm"
    if cls == "action_enc":   # W1 [A -> D], W2's action half [D -> D], W3 [D -> D]; 3 launches per step
        R = B * H
        return (2.0 * R * (A * D + 2 * D * D) / 3, (ncat * (A * D + 2 * D * D) * ab + R * (A * 4 + 3 * D * ab)) / 3,
                "hbm")
    if cls == "decoder":      # W1 [D -> D], W2 [D -> A] with the Euler update; 2 launches per step
        R = B * H
        return 2.0 * R * (D * D + D * A) / 2, (ncat * (D * D + D * A) * ab + R * (2 * D * ab + 3 * A * 4)) / 2, "hbm"
    if cls == "state_enc":    # W1 [state -> D], W2 [D -> D]; 2 launches per call
        sd = c.state_dim
        return 2.0 * B * (sd * D + D * D) / 2, (ncat * (sd * D + D * D) * ab + B * (sd * 4 + 2 * D * 4)) / 2, "hbm"
    return None


def mfma_peak(w):
    return {"fp32": FP32_PEAK_TFLOPS, "fp8a8": FP8_PEAK_TFLOPS}.get(w.cfg.precision, BF16_PEAK_TFLOPS)


def phase_roofline(prof, w, inputs, calls):
    """Lower bound (ms per call) over the classes with a work model, and the algorithmic bytes
    and flops per call behind it."""
    t_ms, byts, flops, modeled = 0.0, 0.0, 0.0, []
    for cls, (n, _) in prof.items():
        m = work_per_launch(cls, w, inputs) if n > 0 else None
        if m is None:
            continue
        f, b, _bound = m
        per_call = n / calls
        t_ms += per_call * max(f / (mfma_peak(w) * 1e12), b / (HBM_PEAK_GBS * 1e9)) * 1e3
        byts += per_call * b
        flops += per_call * f
        modeled.append(cls)
    return {"roofline_ms": round(t_ms, 4), "bytes_per_call": byts, "flops_per_call": flops,
            "classes": sorted(modeled)}


def gemm_aggregate(prof, w, inputs, calls, classes=GEMM_CLASSES):
    """Summed flops over summed per-launch time of the DiT GEMM classes (eager per-launch pass)."""
    fl, ms = 0.0, 0.0
    for cls in classes:
        n, t = prof.get(cls, (0, 0.0))
        if n == 0:
            continue
        fl += n * work_per_launch(cls, w, inputs)[0]
        ms += t
    if ms == 0.0:
        return None
    tf = fl / (ms * 1e-3) / 1e12
    return {"classes": list(classes), "tflop_per_call": round(fl / calls / 1e12, 4),
            "ms_per_call": round(ms / calls, 4), "tflops": round(tf, 1), "peak": mfma_peak(w),
            "frac": round(tf / mfma_peak(w), 4), "timed_in": "eager per-launch pass (HIP events)"}


def stats(xs):
    xs = sorted(xs)
    return {"p50_ms": round(statistics.median(xs), 4), "mean_ms": round(statistics.fmean(xs), 4),
            "std_ms": round(statistics.pstdev(xs), 4), "min_ms": round(xs[0], 4), "max_ms": round(xs[-1], 4),
            "p90_ms": round(xs[min(len(xs) - 1, int(0.9 * len(xs)))], 4)}


def timed_calls(call, n):
    """Wall-clock and device (HIP events on the current stream) ms of n synchronised calls."""
    import torch
    wall, dev = [], []
    for _ in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t = time.perf_counter()
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        wall.append((time.perf_counter() - t) * 1e3)
        dev.append(e0.elapsed_time(e1))
    return wall, dev


def per_launch_pass(h, call, calls):
    """Eager pass with HIP events around every launch: {class: (launches, total ms)}."""
    import torch
    h.profile(True)
    for _ in range(calls):
        call()
    torch.cuda.synchronize()
    prof = h.profile_read()
    h.profile(False)
    return prof


def headline_leg(args, w, weights, inputs, noise, H, synth):
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
    call = lambda: h.get_action(**d, out=out)
    for _ in range(args.warmup):
        call()
    call()
    torch.cuda.synchronize()
    first = out.clone()
    # the timed region: calls enqueued back to back, launch timing off
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    total_s = time.perf_counter() - t0
    log(f"[bench] {w.name}: {args.steps} calls in {total_s * 1e3:.1f} ms ({w.batch * args.steps / total_s:.1f} chunks/s)")
    # per-call latency of the same workload: synchronised calls
    wall, dev = timed_calls(call, args.latency_calls)
    log(f"[bench] {w.name}: synchronised call p50 {statistics.median(wall):.3f} ms")

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

    # per-launch pass of the headline workload
    prof = per_launch_pass(h, call, args.profile_calls)

    # B = 1 latency leg on the same handle
    b1_res = None
    if args.b1_steps:
        bi, bn = synth.make_inputs(b1), synth.make_noise(b1)
        h.prepare(b1.batch, b1.vl_len)
        d1 = H.device_inputs(bi, bn, h.act_torch_dtype)
        out1 = torch.empty((1, b1.cfg.action_horizon, b1.cfg.action_dim), dtype=torch.float32, device="cuda:0")
        call1 = lambda: h.get_action(**d1, out=out1)
        for _ in range(3):
            call1()
        torch.cuda.synchronize()
        lat_wall, lat_dev = timed_calls(call1, args.b1_steps)
        prof_b1 = per_launch_pass(h, call1, 1)
        b1_res = (b1, bi, lat_wall, lat_dev, prof_b1)
    h.close()
    return total_s, wall, dev, prof, first.cpu().numpy(), reuse_s, train_s, b1_res


def persist_leg(args, weights, H, synth):
    """B = 1 latency with the opt-in persistent block kernel (GR00T_FLAG_PERSIST: every DiT block
    of an Euler step in one launch): wall / device times of synchronised calls and the per-launch
    pass."""
    import torch
    b1 = synth.WORKLOADS[args.b1_workload]
    inputs, noise = synth.make_inputs(b1), synth.make_noise(b1)
    h = H.Gr00tHead(b1.cfg, max_batch=1, max_vl_len=b1.vl_len, flags=H.FLAG_USE_GRAPH | H.FLAG_PERSIST)
    h.load_weights(weights).finalize()
    h.prepare(1, b1.vl_len)
    d = H.device_inputs(inputs, noise, h.act_torch_dtype)
    o = torch.empty((1, b1.cfg.action_horizon, b1.cfg.action_dim), dtype=torch.float32, device="cuda:0")
    call = lambda: h.get_action(**d, out=o)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    wall, dev = timed_calls(call, args.b1_steps)
    prof = per_launch_pass(h, call, 1)
    h.close()
    log(f"[bench] {b1.name} with GR00T_FLAG_PERSIST: p50 {statistics.median(wall):.3f} ms")
    return wall, dev, prof


def sub_categories(weights, C):
    """The first C categories of every per-embodiment table (leading category axis)."""
    out = {}
    for k, v in weights.items():
        out[k] = v[:C] if k.split(".")[0] in ("state_enc", "action_enc", "action_dec") else v
    return out


def config_leg(name, weights_for, H, synth, calls):
    """p50 and phase roofline of one configuration (graph replays, inputs in HBM)."""
    import torch
    w = synth.WORKLOADS[name]
    inputs, noise = synth.make_inputs(w), synth.make_noise(w)
    h = H.Gr00tHead(w.cfg, max_batch=w.batch, max_vl_len=w.vl_len, flags=H.FLAG_USE_GRAPH)
    h.load_weights(weights_for(w)).finalize()
    h.prepare(w.batch, w.vl_len)
    d = H.device_inputs(inputs, noise, h.act_torch_dtype)
    o = torch.empty((w.batch, w.cfg.action_horizon, w.cfg.action_dim), dtype=torch.float32, device="cuda:0")
    call = lambda: h.get_action(**d, out=o)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    wall, dev = timed_calls(call, calls)
    prof = per_launch_pass(h, call, 1)
    h.close()
    return config_record(w, inputs, wall, dev, prof, 1)


def config_record(w, inputs, wall, dev, prof, prof_calls):
    p50 = statistics.median(wall)
    roof = phase_roofline(prof, w, inputs, prof_calls)
    rec = {"workload": w.name, "batch": w.batch, "precision": w.cfg.precision, "horizon": w.cfg.action_horizon,
           "euler_steps": w.cfg.num_steps, "vl_len_pad": w.vl_len, **stats(wall), "device": stats(dev),
           "chunks_per_s": round(w.batch / p50 * 1e3, 2),
           "phase_roofline": dict(roof, frac=round(roof["roofline_ms"] / p50, 4),
                                  achieved_gbs=round(roof["bytes_per_call"] / (p50 * 1e-3) / 1e9, 1),
                                  achieved_tflops=round(roof["flops_per_call"] / (p50 * 1e-3) / 1e12, 2))}
    log(f"[bench] {w.name}: p50 {p50:.3f} ms, {rec['chunks_per_s']} chunks/s, phase roofline "
        f"{roof['roofline_ms']:.3f} ms ({rec['phase_roofline']['frac']:.3f})")
    return rec


# Horizon and step-count variants of the same 32-block model (the weights do not depend on
# either): the base N1.7 horizon of 40 and K in {1, 2, 8, 16} Euler steps.
VARIANTS = [("dit32_bf16_b1", 40, 4), ("dit32_bf16_b1", 16, 1), ("dit32_bf16_b1", 16, 2),
            ("dit32_bf16_b1", 16, 8), ("dit32_bf16_b1", 16, 16), ("dit32_bf16_b64", 40, 4),
            ("dit32_w8a8_b256", 16, 4)]


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
        call = lambda: h.get_action(**d, out=o)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        wall, _ = timed_calls(call, calls)
        h.close()
        p50 = statistics.median(wall)
        out.append({"workload": w.name, "batch": w.batch, "precision": w.cfg.precision, "horizon": hz,
                    "euler_steps": k, "p50_ms": round(p50, 4),
                    "chunks_per_s": round(w.batch / p50 * 1e3, 1)})
        log(f"[bench] variant {w.name}: p50 {p50:.3f} ms")
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_leg(args, w, weights, inputs, noise, gpu_out):
    from threadpoolctl import threadpool_info

    from flow_matching_dit_amd import synth
    from oracle import gr00t_oracle as O
    t = time.time()
    P = O.effective_params(w.cfg.as_dict(), weights)
    log(f"[bench] oracle parameters ready in {time.time() - t:.1f}s")
    n = w.batch if args.cpu_samples <= 0 else min(args.cpu_samples, w.batch)
    idx = list(range(n))
    sub, nz = synth.take_samples(inputs, noise, idx)
    t = time.perf_counter()
    ref = O.get_action(w.cfg.as_dict(), weights, sub, nz, params=P)
    dt = time.perf_counter() - t
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    err = O.rel_l2(gpu_out[idx], ref)
    log(f"[bench] oracle: {n} samples in {dt:.1f}s; GPU vs oracle rel_l2 {err:.3e}")
    whole = "the whole" if n == w.batch else f"samples {idx[0]}..{idx[-1]} of the"
    return {"value": round(n / dt, 5), "unit": "chunks/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{whole} {w.batch}-sample {w.name} batch (full depth, same weights and inputs), "
                      f"one get_action",
            "seconds": round(dt, 2), "cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
            "threads_note": "cores = BLAS threads the fp64 NumPy oracle ran on (threadpoolctl)"}, err


def dominant_roofline(prof, w, inputs, calls):
    """Roofline of the dominant kernel class (largest summed duration in the per-launch pass),
    with its average launch duration from that pass (HIP events around each launch on the call's
    stream); the committed kernel trace of the same command gives the kernel-only duration."""
    best, best_ms = None, -1.0
    for cls, (n, ms) in prof.items():
        if n > 0 and ms > best_ms and work_per_launch(cls, w, inputs) is not None:
            best, best_ms = cls, ms
    n, ms = prof[best]
    flops, byts, bound = work_per_launch(best, w, inputs)
    avg_s = ms / n * 1e-3

    def rate(sec):
        return flops / sec / 1e12 if bound == "mfma" else byts / sec / 1e9

    peak, unit = (mfma_peak(w), "TFLOP/s") if bound == "mfma" else (HBM_PEAK_GBS, "GB/s")
    achieved = rate(avg_s)
    from flow_matching_dit_amd.measure import kernel_source_hash
    src = kernel_source_hash()
    traffic, trace = None, None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{best}_{w.name}.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            t = json.load(f)
        if t.get("kernel_source_hash") == src:
            traffic = t.get("bytes_per_launch")
    kpath = os.path.join(ROOT, "profiles", f"trace_{best}_{w.name}.json")
    if os.path.exists(kpath):
        with open(kpath) as f:
            t = json.load(f)
        if t.get("kernel_source_hash") == src:
            tr_s = t["avg_us"] * 1e-6
            trace = {"avg_launch_ms": round(t["avg_us"] * 1e-3, 5), "achieved": round(rate(tr_s), 2),
                     "frac": round(rate(tr_s) / peak, 4),
                     "event_gap_pct": round(100.0 * (avg_s - tr_s) / tr_s, 1),
                     "source": os.path.relpath(kpath, ROOT)}
    breakdown = {c: {"launches_per_call": v[0] // calls, "ms_per_call": round(v[1] / calls, 4)}
                 for c, v in prof.items() if v[0] > 0}
    return {"kernel": best, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "avg_launch_ms": round(ms / n, 5), "launches": n,
            "timed_in": "eager per-launch pass: HIP events around each launch on the call's stream",
            "kernel_trace": trace,
            "algorithmic_per_launch": {"flops": flops, "bytes": byts}}, breakdown


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dit32_bf16_b64")
    ap.add_argument("--b1-workload", default="dit32_bf16_b1")
    ap.add_argument("--b1-steps", type=int, default=30)
    ap.add_argument("--latency-calls", type=int, default=10,
                    help="synchronised calls of the headline workload for its per-call statistics")
    ap.add_argument("--config-calls", type=int, default=10,
                    help="synchronised calls per other configuration (0: skip those legs)")
    ap.add_argument("--profile-calls", type=int, default=2)
    ap.add_argument("--no-b1-persist", dest="b1_persist", action="store_false",
                    help="skip the B = 1 leg with the opt-in persistent block kernel")
    ap.add_argument("--cpu-samples", type=int, default=0, help="oracle samples (0: the whole batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variants", action="store_true",
                    help="also time the horizon 40 and K = 1, 2, 8, 16 variants and W8A8 at B = 256")
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
    total_s, wall, dev, prof, first, reuse_s, train_s, b1_res = headline_leg(args, w, weights, inputs, noise, H,
                                                                             synth)
    value = w.batch * args.steps / total_s
    roof, breakdown = dominant_roofline(prof, w, inputs, args.profile_calls)
    configs = {"headline": config_record(w, inputs, wall, dev, prof, args.profile_calls)}
    latency_b1 = None
    if b1_res is not None:
        b1, bi, lat_wall, lat_dev, prof_b1 = b1_res
        rec = config_record(b1, bi, lat_wall, lat_dev, prof_b1, 1)
        configs["latency_b1"] = rec
        p50 = rec["p50_ms"]
        byts = rec["phase_roofline"]["bytes_per_call"]
        latency_b1 = dict(workload=b1.name, **stats(lat_wall), device=stats(lat_dev),
                          hbm={"algorithmic_bytes": byts, "achieved_gbs": round(byts / (p50 * 1e-3) / 1e9, 1),
                               "peak_gbs": HBM_PEAK_GBS, "frac": round(byts / (p50 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                               "roofline_ms": round(byts / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
                               "what": "weights of every layer read once per Euler step, the K/V projection "
                                       "weights and the VL features once per call, activations once"},
                          breakdown={c: {"launches": v[0], "ms": round(v[1], 4)} for c, v in prof_b1.items() if v[0]})
        if args.b1_persist:
            pw, pd, pprof = persist_leg(args, weights, H, synth)
            pp50 = statistics.median(pw)
            n, ms = pprof.get("blocks_b1", (0, 0.0))
            latency_b1["persistent"] = dict(
                flags="GR00T_FLAG_PERSIST", **stats(pw), device=stats(pd),
                hbm={"algorithmic_bytes": byts, "achieved_gbs": round(byts / (pp50 * 1e-3) / 1e9, 1),
                     "frac": round(byts / (pp50 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                blocks_kernel={"launches_per_call": n, "avg_launch_ms": round(ms / n, 4) if n else None,
                               "what": "one launch per Euler step running every DiT block (eager per-launch "
                                       "pass)"},
                breakdown={c: {"launches": v[0], "ms": round(v[1], 4)} for c, v in pprof.items() if v[0]})
    if args.config_calls:
        c3_w = {}

        def weights_for(cw):
            if cw.cfg.num_layers != w.cfg.num_layers or cw.cfg.hidden != w.cfg.hidden:
                return synth.make_weights(cw)       # the tiny model: its own draws
            if cw.cfg.num_categories != w.cfg.num_categories:
                if cw.name not in c3_w:
                    c3_w[cw.name] = sub_categories(weights, cw.cfg.num_categories)
                return c3_w[cw.name]
            return weights                          # same shapes (fp8 weights are quantised at load)

        for name in OTHER_CONFIGS:
            configs[name] = config_leg(name, weights_for, H, synth, args.config_calls)
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "chunks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total_s / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8e4m3-w/bf16", "fp8a8": "fp8e4m3", "fp32": "f32"}[w.cfg.precision],
        "data": "synthetic (seeded N(0,1) VL features/state/noise, N(0,0.02) weights)",
        "config": {"workload": w.name, "batch": w.batch, "vl_len_pad": w.vl_len, "layers": w.cfg.num_layers,
                   "hidden": w.cfg.hidden, "heads": w.cfg.num_heads, "ff": w.cfg.ff_dim,
                   "horizon": w.cfg.action_horizon, "action_dim": w.cfg.action_dim, "euler_steps": w.cfg.num_steps,
                   "graph": True},
        "per_call": stats(wall),
        "latency_b1": latency_b1,
        "roofline": roof,
        "dit_gemms": gemm_aggregate(prof, w, inputs, args.profile_calls),
        "configs": configs,
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
