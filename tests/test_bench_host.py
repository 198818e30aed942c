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
