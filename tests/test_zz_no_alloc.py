"""gr00t_train_forward_noalloc, the training forward that allocates nothing (its per-sample
tables live in the library's fixed scratch area), through the C ABI: bitwise the same loss
and predicted velocity as gr00t_train_forward on two calls in a row, the second with fewer
samples (the area keeps the first call's contents), both within the oracle's tolerance; and
a batch whose tables exceed the area is refused before anything is enqueued."""
import numpy as np
import pytest

from flow_matching_dit_amd import head as H
from flow_matching_dit_amd import synth
from gpu_util import TOL, TOL_DISP, build_head, say, small
from oracle import gr00t_oracle as O

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20  # the area's size as the header states it


def _table_bytes(cfg, rows):
    """Per-sample tables of `rows` samples as the header states them: seven fp32 tables, each
    rounded up to 256 bytes."""
    n = [rows * cfg.time_freq_dim] + [rows * cfg.hidden] * 5 + [rows * (cfg.num_layers + 1) * 2 * cfg.hidden]
    return sum((4 * k + 255) // 256 * 256 for k in n)


def _train(h, fn, sub, nzs, actions, t):
    import torch
    d = H.device_inputs(sub, nzs, h.act_torch_dtype)
    B = actions.shape[0]
    a = torch.from_numpy(actions).cuda()
    tt = torch.from_numpy(t).cuda()
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda:0")
    vp = torch.full(actions.shape, float("nan"), dtype=torch.float32, device="cuda:0")
    args = (d["vl_features"], d["vl_mask"], d["image_mask"], d["state"], d["embodiment_id"], a, tt, d["noise"])
    if fn == "noalloc":
        h.train_forward_noalloc(*args, loss=loss, v_pred=vp, action_mask=d["action_mask"])
    else:
        loss, vp = h.train_forward(*args, action_mask=d["action_mask"])
    torch.cuda.synchronize()
    assert vp.shape == (B, h._c.action_horizon, h._c.action_dim)
    return float(loss.cpu().numpy()[0]), vp.cpu().numpy()


def test_noalloc_equals_train_forward_on_two_calls_the_second_smaller():
    w = small("dit32_bf16_b64", batch=6)  # ragged VL lengths, action mask, mixed categories
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    rng = np.random.default_rng(21)
    actions = rng.standard_normal(nz.shape).astype(np.float32)
    t = rng.beta(1.5, 1.0, w.batch).astype(np.float32)
    h = build_head(w, wt)
    for B in (6, 3):
        say(f"[noalloc] {w.name}: call with B={B}")
        sub, nzs = synth.take_samples(inp, nz, list(range(B)))
        loss_n, vp_n = _train(h, "noalloc", sub, nzs, actions[:B], t[:B])
        loss_r, vp_r = _train(h, "train_forward", sub, nzs, actions[:B], t[:B])
        assert np.all(np.isfinite(vp_n)) and np.isfinite(loss_n)
        assert loss_n == loss_r and np.array_equal(vp_n, vp_r)
        ref_loss, ref_vp = O.training_loss(w.cfg.as_dict(), wt, sub, actions[:B], nzs, t[:B])
        err = O.rel_l2(vp_n, ref_vp)
        lerr = abs(loss_n - ref_loss) / ref_loss
        say(f"[noalloc] B={B}: bitwise equal to gr00t_train_forward; vs oracle loss {lerr:.2e}, v_pred {err:.2e}")
        assert lerr < TOL[w.cfg.precision] and err < TOL_DISP[w.cfg.precision]
    h.close()


def test_noalloc_refuses_a_batch_past_the_scratch_area():
    import torch
    w = small("dit32_bf16_b64", batch=1, num_layers=2, hidden=1536, num_heads=32, ff_dim=6144, num_categories=2)
    fit = SCRATCH_BYTES // _table_bytes(w.cfg, 1)
    while _table_bytes(w.cfg, fit + 1) <= SCRATCH_BYTES:
        fit += 1
    B = fit + 1
    say(f"[noalloc] {w.name}: {fit} samples fit the area, calling with B={B}")
    wt = synth.make_weights(w)
    h = build_head(w, wt, max_batch=B, max_vl=1)
    c = w.cfg
    dev = "cuda:0"
    vl = torch.zeros((B, 1, c.vl_dim), dtype=h.act_torch_dtype, device=dev)
    ones = torch.ones((B, 1), dtype=torch.uint8, device=dev)
    st = torch.zeros((B, 1, c.state_dim), dtype=torch.float32, device=dev)
    ids = torch.zeros((B,), dtype=torch.int32, device=dev)
    act = torch.zeros((B, c.action_horizon, c.action_dim), dtype=torch.float32, device=dev)
    tt = torch.zeros((B,), dtype=torch.float32, device=dev)
    loss = torch.zeros((1,), dtype=torch.float32, device=dev)
    with pytest.raises(H.Gr00tError) as ei:
        h.train_forward_noalloc(vl, ones, None, st, ids, act, tt, act.clone(), loss=loss)
    torch.cuda.synchronize()
    say(f"[noalloc] refused: {ei.value}")
    assert ei.value.status == "E_SHAPE" and "scratch" in str(ei.value)
    assert float(loss.cpu()[0]) == 0.0  # nothing was enqueued
    h.close()
