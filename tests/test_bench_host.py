"""Host logic of bench.py (no GPU): the one-GPU refusal and the algorithmic work per launch
that the roofline divides by."""
import os
import subprocess
import sys
from dataclasses import replace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from flow_matching_dit_amd import synth  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                           env=dict(os.environ, **env), timeout=120)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr and r.stdout == ""


def test_work_per_launch_of_the_gemm_classes():
    w = synth.WORKLOADS["dit32_bf16_b64"]
    inputs = synth.make_inputs(w)
    M, D, F = w.batch * (w.cfg.action_horizon + 1), w.cfg.hidden, w.cfg.ff_dim
    flops, byts, bound = bench.work_per_launch("ff_up", w, inputs)
    assert bound == "mfma" and flops == 2.0 * M * D * F
    assert byts == F * D * 2 + M * D * 2 + M * F * 2          # bf16 weights, input and output
    flops, byts, _ = bench.work_per_launch("ff_down", w, inputs)
    assert byts == D * F * 2 + M * F * 2 + M * D * 8          # residual add reads and writes fp32
    for prec in ("fp8", "fp8a8"):                             # e4m3 weights: one byte each
        wq = replace(w, cfg=replace(w.cfg, precision=prec))
        assert bench.work_per_launch("ff_up", wq, inputs)[1] == F * D + M * D * 2 + M * F * 2


def test_work_per_launch_counts_only_valid_vl_tokens():
    w = synth.WORKLOADS["dit32_bf16_b64"]
    inputs = synth.make_inputs(w)
    nvalid = int(np.sum(inputs["vl_mask"]))
    assert 0 < nvalid < w.batch * w.vl_len                    # ragged lengths
    Nc, D, E = (w.cfg.num_layers + 1) // 2, w.cfg.hidden, w.cfg.vl_dim
    flops, _, bound = bench.work_per_launch("kv_proj", w, inputs)
    assert bound == "mfma" and flops == 2.0 * nvalid * E * Nc * 2 * D
    assert bench.work_per_launch("steps_graph", w, inputs) is None


def _b1_profile():
    """Launches of one B = 1 get_action per kernel class (launch path, 32 blocks, K = 4)."""
    return {"q_proj": (64, 1.0), "qkv_proj": (64, 1.0), "o_proj": (128, 1.0), "ff_up": (128, 1.0),
            "ff_down": (128, 1.0), "out_proj": (4, 1.0), "adaln": (132, 1.0), "attn_self": (64, 1.0),
            "attn_cross": (64, 1.0), "action_enc": (12, 1.0), "decoder": (8, 1.0), "state_enc": (2, 1.0),
            "kv_proj": (1, 1.0), "vlln": (1, 1.0), "small": (9, 1.0), "steps_graph": (0, 0.0)}


def test_b1_algorithmic_bytes_are_the_weight_stream():
    """B = 1 moves the DiT weights once per Euler step plus the K/V projection weights once:
    the phase model's bytes per call sit just above that sum (activations, tables)."""
    w = synth.WORKLOADS["dit32_bf16_b1"]
    inputs = synth.make_inputs(w)
    r = bench.phase_roofline(_b1_profile(), w, inputs, 1)
    D, F, E, N, K = w.cfg.hidden, w.cfg.ff_dim, w.cfg.vl_dim, w.cfg.num_layers, w.cfg.num_steps
    per_step = (N // 2) * (3 * D * D) + (N // 2) * D * D + N * (D * D + 2 * D * F)   # qkv / q, o, MLP
    weights = 2 * (K * per_step + (N // 2) * 2 * D * E)                               # bf16
    assert weights < r["bytes_per_call"] < 1.06 * weights
    assert "small" not in r["classes"] and "steps_graph" not in r["classes"]
    # the bound of a weight stream: bytes over 8 TB/s
    assert abs(r["roofline_ms"] - r["bytes_per_call"] / 8e12 * 1e3) < 0.02 * r["roofline_ms"]


def test_phase_roofline_takes_the_larger_of_compute_and_memory_per_class():
    w = synth.WORKLOADS["dit32_bf16_b64"]
    inputs = synth.make_inputs(w)
    prof = {"ff_up": (256, 7.0), "adaln": (10, 1.0)}
    r = bench.phase_roofline(prof, w, inputs, 2)
    f_up, b_up, _ = bench.work_per_launch("ff_up", w, inputs)
    f_ln, b_ln, _ = bench.work_per_launch("adaln", w, inputs)
    want = 128 * max(f_up / 2.5e15, b_up / 8e12) + 5 * max(f_ln / 2.5e15, b_ln / 8e12)
    assert abs(r["roofline_ms"] - want * 1e3) < 1e-3
    assert f_up / 2.5e15 > b_up / 8e12                         # B = 64 MLP: compute bound


def test_gemm_aggregate_is_summed_flops_over_summed_time():
    w = synth.WORKLOADS["dit32_bf16_b64"]
    inputs = synth.make_inputs(w)
    prof = {"ff_up": (128, 4.0), "o_proj": (128, 2.0), "adaln": (132, 9.0)}
    g = bench.gemm_aggregate(prof, w, inputs, 1)
    fl = 128 * bench.work_per_launch("ff_up", w, inputs)[0] + 128 * bench.work_per_launch("o_proj", w, inputs)[0]
    assert abs(g["tflops"] - fl / 6e-3 / 1e12) < 0.1 and g["ms_per_call"] == 6.0
    assert abs(g["frac"] - g["tflops"] / 2500.0) < 1e-4


def test_sub_categories_keeps_the_first_tables():
    w = synth.small_variant(synth.WORKLOADS["dit32_bf16_b64"], num_categories=4)
    wt = synth.make_weights(w)
    sub = bench.sub_categories(wt, 2)
    for k, v in wt.items():
        if k.split(".")[0] in ("state_enc", "action_enc", "action_dec"):
            assert sub[k].shape[0] == 2 and np.array_equal(sub[k], v[:2])
        else:
            assert sub[k] is v
