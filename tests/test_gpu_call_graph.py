"""Whole-call graphs: with GR00T_FLAG_USE_GRAPH, a prepared shape and caller noise, a get_action
whose buffers repeat those of the previous call is captured once as one graph (prologue, K
Euler steps, output) and replayed from then on ("Single-GPU inference for GR00T-N1.7", Prepare
a request and construct the engine: the engine replays captured profiles). Checked through the
C ABI: bitwise equality with the uncaptured path, live reads of changed buffer contents, the
VL caches that a replay leaves for gr00t_get_action_reuse_vl, eviction past eight graphs, and
the deferred invalid-id report."""
import numpy as np
import pytest

from flow_matching_dit_amd import head as H
from flow_matching_dit_amd import synth
from gpu_util import build_head, gpu_action, say, small

pytestmark = pytest.mark.gpu


def _call(h, d, out):
    import torch
    h.profile(2)  # the graphs are kept; their launches are counted
    h.get_action(**d, out=out)
    torch.cuda.synchronize()
    prof = h.profile_read()
    h.profile(False)
    return out.cpu().numpy().copy(), prof.get("call_graph", (0, 0.0))[0]


@pytest.fixture(scope="module")
def wl():
    w = small("dit32_bf16_b64", batch=4)
    return w, synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)


def test_repeated_buffers_replay_one_graph_of_the_call(wl):
    import torch
    w, wt, inp, nz = wl
    ref = gpu_action(build_head(w, wt), inp, nz)  # no graphs at all
    h = build_head(w, wt, flags=H.FLAG_USE_GRAPH)
    h.prepare(w.batch, w.vl_len)
    d = H.device_inputs(inp, nz, h.act_torch_dtype)
    out = torch.empty((w.batch, w.cfg.action_horizon, w.cfg.action_dim), dtype=torch.float32, device="cuda:0")
    runs = [_call(h, d, out) for _ in range(3)]
    say(f"[call graph] whole-call graph launches per call: {[n for _, n in runs]}")
    assert [n for _, n in runs] == [0, 1, 1]  # new buffers, then the repetition is captured and replayed
    for y, _ in runs:
        assert np.array_equal(y, ref)
    # the graph reads the buffers' contents live: change them in place
    d["vl_features"].mul_(0.5)
    d["noise"].copy_(torch.flip(d["noise"], dims=[0]))
    y2, n2 = _call(h, d, out)
    inp2 = dict(inp, vl_features=inp["vl_features"] * 0.5)
    ref2 = gpu_action(build_head(w, wt), inp2, np.ascontiguousarray(nz[::-1]))
    assert n2 == 1 and np.array_equal(y2, ref2)
    # a replay leaves the VL caches of its inputs for the reuse entry point
    yr = h.get_action_reuse_vl(w.batch, w.vl_len, d["state"], d["embodiment_id"], noise=d["noise"],
                               action_mask=d["action_mask"])
    torch.cuda.synchronize()
    assert np.array_equal(yr.cpu().numpy(), ref2)
    h.close()


def test_more_buffer_sets_than_kept_graphs(wl):
    import torch
    w, wt, inp, nz = wl
    ref = gpu_action(build_head(w, wt), inp, nz)
    h = build_head(w, wt, flags=H.FLAG_USE_GRAPH)
    h.prepare(w.batch, w.vl_len)
    d = H.device_inputs(inp, nz, h.act_torch_dtype)
    outs = [torch.empty((w.batch, w.cfg.action_horizon, w.cfg.action_dim), dtype=torch.float32, device="cuda:0")
            for _ in range(10)]
    counts = []
    for o in outs + outs[:2]:   # ten buffer sets, each called twice (captured), then the first two again
        for _ in range(2):
            y, n = _call(h, d, o)
            counts.append(n)
            assert np.array_equal(y, ref)
    say(f"[call graph] launches: {counts}")
    assert counts[:20] == [0, 1] * 10
    assert counts[20:] == [0, 1, 0, 1]  # evicted (eight kept), captured again on repetition
    h.close()


def test_invalid_id_is_still_reported_after_a_replay(wl):
    import torch
    w, wt, inp, nz = wl
    h = build_head(w, wt, flags=H.FLAG_USE_GRAPH)
    h.prepare(w.batch, w.vl_len)
    bad = dict(inp, embodiment_id=inp["embodiment_id"].copy())
    bad["embodiment_id"][2] = w.cfg.num_categories + 1
    d = H.device_inputs(bad, nz, h.act_torch_dtype)
    out = torch.empty((w.batch, w.cfg.action_horizon, w.cfg.action_dim), dtype=torch.float32, device="cuda:0")
    _, n0 = _call(h, d, out)           # uncaptured: its invalid id is reported by the next call
    with pytest.raises(H.Gr00tError) as e:
        _call(h, d, out)
    assert e.value.status == "E_DEVICE_ERROR"
    y, n1 = _call(h, d, out)           # the buffers repeat: captured and replayed
    assert (n0, n1) == (0, 1) and np.all(np.isnan(y[2]))
    with pytest.raises(H.Gr00tError) as e:  # the replay's report
        _call(h, d, out)
    assert e.value.status == "E_DEVICE_ERROR"
    h.close()
