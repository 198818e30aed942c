"""Invariants and edge cases of the HIP path, through the C ABI.

Bitwise: repeated calls, graph vs eager replay,
perturbed masked VL tokens, a zero velocity field. Closed forms: a constant
velocity field, K = 1. Error paths: strict-mode ids, unprepared shapes, the
deferred report of a bad id, the library's own noise."""
import ctypes
from dataclasses import replace

import numpy as np
import pytest

from flow_matching_dit_amd import head as H
from flow_matching_dit_amd import synth
from gpu_util import TOL, build_head, gpu_action, gpu_velocity, say, small
from oracle import gr00t_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wl():
    w = small("dit32_bf16_b64", batch=8)
    return w, synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)


def test_repeat_and_graph_bitwise(wl):
    w, wt, inp, nz = wl
    h = build_head(w, wt, flags=H.FLAG_USE_GRAPH)
    y_eager = gpu_action(h, inp, nz)           # not prepared: eager
    y_g1 = gpu_action(h, inp, nz, prepare=True)
    y_g2 = gpu_action(h, inp, nz)
    h.close()
    assert np.array_equal(y_g1, y_g2)
    assert np.array_equal(y_eager, y_g1)


def test_w8a8_graph_replays_and_masked_tokens_bitwise():
    # W8A8 on the ragged B=64 recipe: eager, then three graph replays with eager work of the
    # same handle (a velocity call) and synchronisations between them, all bitwise equal; and
    # masked VL tokens changed to huge values leave the result bitwise unchanged (they are
    # neither quantised nor projected)
    w = small("dit32_bf16_b64", batch=8)
    w = replace(w, name=w.name + "_fp8a8", cfg=replace(w.cfg, precision="fp8a8"))
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    h = build_head(w, wt, flags=H.FLAG_USE_GRAPH)
    y_eager = gpu_action(h, inp, nz)
    ys = [gpu_action(h, inp, nz, prepare=True)]
    for k in (1, 2):
        gpu_velocity(h, inp, nz, k)
        ys.append(gpu_action(h, inp, nz))
    for y in ys:
        assert np.array_equal(y, y_eager)
    inp2 = dict(inp)
    vl = inp["vl_features"].copy()
    vl[inp["vl_mask"] == 0] = 1000.0
    inp2["vl_features"] = vl
    assert np.array_equal(gpu_action(h, inp2, nz), y_eager)
    h.close()


def test_w8a8_bad_id_stays_in_its_sample():
    # non-strict mode, W8A8: the NaN rows of a sample with an invalid id are quantised row by
    # row, so the other samples are bitwise those of the clean call
    w = small("dit32_bf16_b64", batch=8)
    w = replace(w, name=w.name + "_fp8a8", cfg=replace(w.cfg, precision="fp8a8"))
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    h = build_head(w, wt)
    y = gpu_action(h, inp, nz)
    bad = dict(inp)
    bad["embodiment_id"] = inp["embodiment_id"].copy()
    bad["embodiment_id"][5] = w.cfg.num_categories
    yb = gpu_action(h, bad, nz)
    assert np.all(np.isnan(yb[5]))
    keep = [b for b in range(w.batch) if b != 5]
    assert np.array_equal(yb[keep], y[keep])
    with pytest.raises(H.Gr00tError) as e:
        gpu_action(h, inp, nz)
    assert e.value.status == "E_DEVICE_ERROR"
    h.close()


def test_batch_independence(wl):
    # a sample alone equals the same sample inside the batch; the GEMM tiling and split-K
    # depth depend on the batch size, so only the fp32 summation order may differ
    w, wt, inp, nz = wl
    h = build_head(w, wt)
    y = gpu_action(h, inp, nz)
    for b in (0, 5, 7):
        sub, n1 = synth.take_samples(inp, nz, [b])
        yb = gpu_action(h, sub, n1)
        assert np.max(np.abs(yb[0] - y[b])) <= 1e-4 * np.max(np.abs(y[b])), b
    h.close()


def test_masked_vl_tokens_bitwise(wl):
    w, wt, inp, nz = wl
    h = build_head(w, wt)
    y = gpu_action(h, inp, nz)
    inp2 = dict(inp)
    vl = inp["vl_features"].copy()
    vl[inp["vl_mask"] == 0] = 1000.0
    inp2["vl_features"] = vl
    assert np.array_equal(gpu_action(h, inp2, nz), y)
    h.close()


def test_zero_and_constant_velocity(wl):
    w, wt, inp, nz = wl
    wt = {k: v.copy() for k, v in wt.items()}
    wt["action_dec.w2"][:] = 0
    wt["action_dec.b2"][:] = 0
    inp = dict(inp)
    inp["action_mask"] = None
    h = build_head(w, wt)
    assert np.array_equal(gpu_action(h, inp, nz), nz)
    h.close()
    wt["action_dec.b2"][:] = 0.5
    h = build_head(w, wt)
    y = gpu_action(h, inp, nz)
    h.close()
    # four fp32 additions of dt * 0.5 = 0.125
    assert np.max(np.abs(y - (nz.astype(np.float64) + 0.5))) < 4 * 2.0 ** -23 * (np.abs(nz).max() + 1)


def test_k1_is_noise_plus_one_velocity():
    w = small("dit32_bf16_b64", batch=4)
    w = replace(w, cfg=replace(w.cfg, num_steps=1))
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    inp["action_mask"] = None
    h = build_head(w, wt)
    y = gpu_action(h, inp, nz)
    v = gpu_velocity(h, inp, nz, 0)
    h.close()
    assert np.max(np.abs(y - (nz + v))) <= 2.0 ** -22 * (np.abs(nz + v).max() + 1)
    ref = O.get_action(w.cfg.as_dict(), wt, inp, nz)
    assert O.rel_l2(y, ref) < TOL["bf16"]


def test_empty_text_set_and_single_token():
    # one sample whose tokens are all image tokens: its text blocks see no key (output 0)
    w = small("dit32_bf16_b1", batch=3)
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    inp = dict(inp)
    im = np.zeros((3, w.vl_len), np.uint8)
    im[:, :256] = 1
    im[1, :] = 1
    inp["image_mask"] = im
    h = build_head(w, wt)
    y = gpu_action(h, inp, nz)
    h.close()
    ref = O.get_action(w.cfg.as_dict(), wt, inp, nz)
    assert O.rel_l2(y, ref) < TOL["bf16"]
    # a single VL token
    w1 = replace(w, vl_len=1, image_tokens=None, batch=2)
    wt1, inp1, nz1 = synth.make_weights(w1), synth.make_inputs(w1), synth.make_noise(w1)
    h = build_head(w1, wt1)
    y1 = gpu_action(h, inp1, nz1)
    h.close()
    assert O.rel_l2(y1, O.get_action(w1.cfg.as_dict(), wt1, inp1, nz1)) < TOL["bf16"]


def test_strict_mode_rejects_bad_id_and_unprepared_shape(wl):
    w, wt, inp, nz = wl
    h = build_head(w, wt, flags=H.FLAG_STRICT | H.FLAG_USE_GRAPH)
    bad = dict(inp)
    bad["embodiment_id"] = inp["embodiment_id"].copy()
    bad["embodiment_id"][3] = w.cfg.num_categories
    h.prepare(w.batch, w.vl_len)
    with pytest.raises(H.Gr00tError) as e:
        gpu_action(h, bad, nz)
    assert e.value.status == "E_EMBODIMENT"
    sub, n1 = synth.take_samples(inp, nz, [0, 1])
    with pytest.raises(H.Gr00tError) as e:
        gpu_action(h, sub, n1)                  # (B=2, L) was never prepared
    assert e.value.status == "E_UNCAPTURED"
    h.close()


def test_nonstrict_bad_id_gives_nan_rows_and_deferred_error(wl):
    w, wt, inp, nz = wl
    h = build_head(w, wt)
    y = gpu_action(h, inp, nz)
    bad = dict(inp)
    bad["embodiment_id"] = inp["embodiment_id"].copy()
    bad["embodiment_id"][2] = -1
    yb = gpu_action(h, bad, nz)
    assert np.all(np.isnan(yb[2]))
    keep = [b for b in range(w.batch) if b != 2]
    assert np.array_equal(yb[keep], y[keep])
    with pytest.raises(H.Gr00tError) as e:
        gpu_action(h, inp, nz)
    assert e.value.status == "E_DEVICE_ERROR"
    assert np.array_equal(gpu_action(h, inp, nz), y)   # reported once
    h.close()


def test_deferred_error_survives_pipelined_calls(wl):
    """A bad-id call followed by clean calls enqueued back to back with no synchronisation:
    the invalid id is reported exactly once, by whichever later call first finds a completed
    copy of the device's count (not lost when later calls overwrite the report), and the
    clean calls' results are unaffected."""
    import torch
    w, wt, inp, nz = wl
    h = build_head(w, wt)
    bad = dict(inp)
    bad["embodiment_id"] = inp["embodiment_id"].copy()
    bad["embodiment_id"][1] = w.cfg.num_categories + 3
    db = H.device_inputs(bad, nz, h.act_torch_dtype)
    dg = H.device_inputs(inp, nz, h.act_torch_dtype)
    yb = h.get_action(**db)          # bad id, not synchronised
    reports, outs = [], []
    for _ in range(6):               # clean calls enqueued behind it
        try:
            outs.append(h.get_action(**dg))
        except H.Gr00tError as e:
            reports.append(e)
    torch.cuda.synchronize()
    for _ in range(2):               # after the stream drained: report it now if not yet done
        try:
            outs.append(h.get_action(**dg))
        except H.Gr00tError as e:
            reports.append(e)
    torch.cuda.synchronize()
    assert len(reports) == 1, [str(e) for e in reports]
    assert reports[0].status == "E_DEVICE_ERROR" and "1 embodiment id" in str(reports[0])
    assert np.all(np.isnan(yb.cpu().numpy()[1]))
    ys = [o.cpu().numpy() for o in outs]
    assert len(ys) == 7 and all(np.array_equal(y, ys[0]) for y in ys) and np.all(np.isfinite(ys[0]))
    h.close()


def test_library_noise_is_standard_normal():
    w = synth.small_variant(synth.WORKLOADS["dit32_bf16_b64"], batch=64, num_layers=2)
    wt, inp = synth.make_weights(w), synth.make_inputs(w)
    wt = {k: v.copy() for k, v in wt.items()}
    wt["action_dec.w2"][:] = 0
    wt["action_dec.b2"][:] = 0
    inp = dict(inp)
    inp["action_mask"] = None
    h = build_head(w, wt)
    a = gpu_action(h, inp, None)
    b = gpu_action(h, inp, None)
    h.close()
    x = a.ravel().astype(np.float64)
    say(f"[noise] mean {x.mean():.4f} std {x.std():.4f} n={x.size}")
    assert abs(x.mean()) < 0.03 and abs(x.std() - 1) < 0.03
    assert not np.array_equal(a, b)


def test_horizon_permutation_equivariance(wl):
    # the head has no positional term: permuting the action rows of the noise (and of the
    # action mask) permutes action_pred the same way; self attention sums its keys in
    # another order, so equality holds to fp32 rounding
    w, wt, inp, nz = wl
    h = build_head(w, wt)
    y = gpu_action(h, inp, nz)
    perm = np.random.default_rng(5).permutation(w.cfg.action_horizon)
    inp2 = dict(inp)
    if inp["action_mask"] is not None:
        inp2["action_mask"] = np.ascontiguousarray(inp["action_mask"][:, perm])
    yp = gpu_action(h, inp2, np.ascontiguousarray(nz[:, perm]))
    h.close()
    assert np.max(np.abs(yp - y[:, perm])) <= 1e-4 * np.max(np.abs(y))


def test_unused_category_weights_do_not_matter(wl):
    w, wt, inp, nz = wl
    h = build_head(w, wt)
    y = gpu_action(h, inp, nz)
    h.close()
    unused = sorted(set(range(w.cfg.num_categories)) - set(int(i) for i in inp["embodiment_id"]))
    assert unused
    wt2 = {k: v.copy() for k, v in wt.items()}
    for name in ("state_enc.w1", "action_enc.w2", "action_dec.w1", "action_dec.b2"):
        wt2[name][unused] = 7.0
    h = build_head(w, wt2)
    y2 = gpu_action(h, inp, nz)
    h.close()
    assert np.array_equal(y, y2)
