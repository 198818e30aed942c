"""Helpers of the GPU tests: run the HIP library through its C ABI on seeded inputs."""
import sys

import numpy as np

from flow_matching_dit_amd import head as H
from flow_matching_dit_amd import synth

TOL = {"fp32": 1e-4, "bf16": 2e-2, "fp8": 5e-2, "fp8a8": 5e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def build_head(w, weights, flags=0, max_batch=None, max_vl=None):
    h = H.Gr00tHead(w.cfg, max_batch or w.batch, max_vl or w.vl_len, flags)
    h.load_weights(weights)
    h.finalize()
    return h


def gpu_action(h, inputs, noise, prepare=False, state_out=False):
    import torch
    d = H.device_inputs(inputs, noise, h.act_torch_dtype)
    B, L = d["vl_features"].shape[:2]
    if prepare:
        h.prepare(B, L)
    sf = None
    if state_out:
        sf = torch.empty((B, 1, h._c.hidden), dtype=torch.float32, device="cuda:0")
    out = h.get_action(**d, state_features_out=sf)
    torch.cuda.synchronize()
    if state_out:
        return out.cpu().numpy(), sf.cpu().numpy()
    return out.cpu().numpy()


def gpu_velocity(h, inputs, noise, k):
    import torch
    d = H.device_inputs(inputs, noise, h.act_torch_dtype)
    d.pop("action_mask")
    v = h.velocity(**d, step_k=k)
    torch.cuda.synchronize()
    return v.cpu().numpy()


def small(name, **kw):
    """Reduced-width variant of a named workload (4 blocks: text, self, image, self)."""
    base = synth.WORKLOADS[name]
    args = dict(num_layers=4, hidden=192, num_heads=4, head_dim=48, ff_dim=768)
    args.update(kw)
    return synth.small_variant(base, **args)
