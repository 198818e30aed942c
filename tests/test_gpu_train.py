"""Flow-matching training forward and loss on the GPU (gr00t_train_forward) against the
oracle: the loss and the predicted velocity on seeded draws (t ~ Beta(1.5, 1), noise and
actions ~ N(0, 1)); at t = k/K the forward is the inference velocity of step k at x_t."""
from dataclasses import replace

import numpy as np
import pytest

from flow_matching_dit_amd import head as H
from flow_matching_dit_amd import synth
from gpu_util import TOL, TOL_DISP, build_head, gpu_velocity, say, small
from oracle import gr00t_oracle as O

pytestmark = pytest.mark.gpu


def _draws(w, seed):
    rng = np.random.default_rng(seed)
    shape = (w.batch, w.cfg.action_horizon, w.cfg.action_dim)
    return (rng.standard_normal(shape).astype(np.float32), rng.beta(1.5, 1.0, w.batch).astype(np.float32))


def _gpu_train(h, inp, noise, actions, t):
    import torch
    d = H.device_inputs(inp, noise, h.act_torch_dtype)
    a = torch.from_numpy(actions).cuda()
    tt = torch.from_numpy(t).cuda()
    loss, vp = h.train_forward(d["vl_features"], d["vl_mask"], d["image_mask"], d["state"], d["embodiment_id"], a, tt,
                               d["noise"], action_mask=d["action_mask"])
    torch.cuda.synchronize()
    return float(loss.cpu().numpy()[0]), vp.cpu().numpy()


@pytest.mark.parametrize("name,kw", [
    ("tiny_fp32_b1", None),
    ("dit32_bf16_b1", dict(batch=3)),                                             # image / text split
    ("dit32_bf16_b64", dict(batch=8)),                                            # ragged VL, action mask
    ("dit32_bf16_b64", dict(batch=8, num_layers=2, hidden=1536, num_heads=32, ff_dim=6144)),  # full width
    ("dit32_w8a8_b256", dict(batch=8)),                                           # W8A8 GEMMs
])
def test_train_forward_matches_oracle(name, kw):
    w = synth.WORKLOADS[name] if kw is None else small(name, **kw)
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    actions, t = _draws(w, 11)
    h = build_head(w, wt)
    loss, vp = _gpu_train(h, inp, nz, actions, t)
    h.close()
    ref_loss, ref_vp = O.training_loss(w.cfg.as_dict(), wt, inp, actions, nz, t)
    err = O.rel_l2(vp, ref_vp)
    per = [O.rel_l2(vp[b], ref_vp[b]) for b in range(w.batch)]
    lerr = abs(loss - ref_loss) / ref_loss
    say(f"[train] {w.name} B={w.batch}: loss {loss:.6f} (oracle {ref_loss:.6f}, rel {lerr:.2e}), "
        f"v_pred rel_l2 {err:.2e}, worst sample {max(per):.2e}")
    # v_pred is a velocity: no noise passes through it, so it is gated like a displacement
    tol, tol_v = TOL[w.cfg.precision], TOL_DISP[w.cfg.precision]
    assert lerr < tol and err < tol_v and max(per) < tol_v


def test_train_forward_on_the_grid_is_the_inference_velocity():
    w = small("dit32_bf16_b64", batch=4)
    w = replace(w, cfg=replace(w.cfg, num_steps=4))
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    actions, _ = _draws(w, 12)
    ks = [0, 3, 1, 2]
    t = np.array([k / 4 for k in ks], np.float32)
    h = build_head(w, wt)
    _, vp = _gpu_train(h, inp, nz, actions, t)
    x_t = ((1.0 - t)[:, None, None] * nz + t[:, None, None] * actions).astype(np.float32)
    for b, k in enumerate(ks):
        v = gpu_velocity(h, inp, x_t, k)
        err = O.rel_l2(vp[b], v[b])
        say(f"[train] sample {b} on step {k}: rel_l2 vs the inference velocity {err:.2e}")
        assert err < 1e-5
    h.close()


def test_train_forward_bad_id_gives_nan_loss():
    w = small("dit32_bf16_b64", batch=2)
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    inp = dict(inp, embodiment_id=np.array([0, w.cfg.num_categories + 3], np.int32))
    actions, t = _draws(w, 13)
    h = build_head(w, wt)
    loss, _ = _gpu_train(h, inp, nz, actions, t)
    assert np.isnan(loss)
    h.close()
