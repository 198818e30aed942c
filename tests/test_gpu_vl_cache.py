"""The VL key/value cache across calls (gr00t_get_action_reuse_vl): a call that reuses the
VL LayerNorm, key masks and K/V projection of the last full call equals a full call with
those VL inputs (bitwise) and the oracle; a shape without a cache is refused."""
import numpy as np
import pytest

from flow_matching_dit_amd import head as H
from flow_matching_dit_amd import synth
from gpu_util import TOL, TOL_DISP, build_head, check_parity, say, small
from oracle import gr00t_oracle as O

pytestmark = pytest.mark.gpu


def _other(inputs, noise, seed):
    """the same VL input with another state, ids, noise and action mask"""
    rng = np.random.default_rng(seed)
    inp = dict(inputs)
    inp["state"] = rng.standard_normal(inputs["state"].shape).astype(np.float32)
    inp["embodiment_id"] = rng.permutation(inputs["embodiment_id"]).astype(np.int32)
    if inputs["action_mask"] is not None:
        inp["action_mask"] = inputs["action_mask"][::-1].copy()
    return inp, rng.standard_normal(noise.shape).astype(np.float32)


@pytest.mark.parametrize("name,graph", [("dit32_bf16_b1", False), ("dit32_bf16_b1", True), ("dit32_w8a8_b256", True)],
                         ids=["eager", "graph", "w8a8-graph"])
def test_reuse_vl_equals_full_call(name, graph):
    import torch
    # 3 samples (the bf16 case with the image/text split: text blocks and image blocks use
    # different key masks); W8A8: the cached keys and values come from e4m3 VL rows
    w = small(name, batch=3)
    say(f"[vl-cache] {w.name} B={w.batch} L={w.vl_len} graph={graph}")
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    flags = H.FLAG_USE_GRAPH if graph else 0
    h = build_head(w, wt, flags=flags)
    if graph:
        h.prepare(w.batch, w.vl_len)
    d = H.device_inputs(inp, nz, h.act_torch_dtype)
    y1 = h.get_action(**d)
    inp2, nz2 = _other(inp, nz, 7)
    d2 = H.device_inputs(inp2, nz2, h.act_torch_dtype)
    y2 = h.get_action_reuse_vl(w.batch, w.vl_len, d2["state"], d2["embodiment_id"], noise=d2["noise"],
                               action_mask=d2["action_mask"])
    y3 = h.get_action(**d2)  # the full call with the cached call's VL input
    torch.cuda.synchronize()
    y1, y2, y3 = y1.cpu().numpy(), y2.cpu().numpy(), y3.cpu().numpy()
    assert np.array_equal(y2, y3)
    assert not np.array_equal(y1, y2)
    ref = O.get_action(w.cfg.as_dict(), wt, inp2, nz2)
    check_parity(y2, ref, nz2, inp2["action_mask"], TOL[w.cfg.precision], f"{w.name} reusing the VL caches",
                 TOL_DISP[w.cfg.precision])
    h.close()


def test_reuse_vl_needs_a_full_call_of_the_same_shape():
    import torch
    w = small("dit32_bf16_b64", batch=4)
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    h = build_head(w, wt)
    d = H.device_inputs(inp, nz, h.act_torch_dtype)
    with pytest.raises(RuntimeError, match="E_NO_VL_CACHE"):  # no full call yet
        h.get_action_reuse_vl(w.batch, w.vl_len, d["state"], d["embodiment_id"], noise=d["noise"])
    y = h.get_action(**d)
    y_again = h.get_action_reuse_vl(w.batch, w.vl_len, d["state"], d["embodiment_id"], noise=d["noise"],
                                    action_mask=d["action_mask"])
    with pytest.raises(RuntimeError, match="E_NO_VL_CACHE"):  # another padded length
        h.get_action_reuse_vl(w.batch, w.vl_len - 32, d["state"], d["embodiment_id"], noise=d["noise"])
    # a full call of another shape replaces the cache
    sub, nzs = synth.take_samples(inp, nz, [0, 1])
    ds = H.device_inputs(sub, nzs, h.act_torch_dtype)
    h.get_action(**ds)
    with pytest.raises(RuntimeError, match="E_NO_VL_CACHE"):
        h.get_action_reuse_vl(w.batch, w.vl_len, d["state"], d["embodiment_id"], noise=d["noise"])
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y_again.cpu().numpy())  # same inputs: same chunk
    h.close()
