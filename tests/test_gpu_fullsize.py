"""Full-size parity: each 32-block workload runs its whole batch through the captured
graph (the launch configuration the benchmark times); the oracle recomputes a few
samples one by one (samples are independent), which are compared at the stated
tolerance."""
import gc

import numpy as np
import pytest

from flow_matching_dit_amd import head as H
from flow_matching_dit_amd import synth
from gpu_util import TOL, TOL_DISP, build_head, check_parity, gpu_action, say
from oracle import gr00t_oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(400)]

CASES = [
    ("dit32_bf16_b1", [0]),
    ("dit32_bf16_b64", [0, 17, 63]),
    ("dit32_bf16_b16_h64", [0, 6, 15]),
    ("dit32_fp8_b256", [0, 200, 255]),
    ("dit32_w8a8_b256", [0, 128, 255]),
]


@pytest.mark.parametrize("name,samples", CASES, ids=[c[0] for c in CASES])
def test_full_size_sampled_parity(name, samples):
    w = synth.WORKLOADS[name]
    say(f"[fullsize] {name}: B={w.batch} L={w.vl_len} H={w.cfg.action_horizon} K={w.cfg.num_steps} "
        f"prec={w.cfg.precision} samples={samples}")
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    h = build_head(w, wt, flags=H.FLAG_USE_GRAPH | H.FLAG_STRICT)
    y = gpu_action(h, inp, nz, prepare=True)
    h.close()
    say(f"[fullsize] {name}: GPU done, running the oracle")
    assert y.shape == (w.batch, w.cfg.action_horizon, w.cfg.action_dim)
    assert np.all(np.isfinite(y))
    if inp["action_mask"] is not None:
        assert np.all(y[inp["action_mask"] == 0] == 0)
    sub, nzs = synth.take_samples(inp, nz, samples)
    ref = O.get_action(w.cfg.as_dict(), wt, sub, nzs)
    del wt
    gc.collect()
    check_parity(y[samples], ref, nzs, sub["action_mask"], TOL[w.cfg.precision], f"{name} samples {samples}",
                 TOL_DISP[w.cfg.precision])
