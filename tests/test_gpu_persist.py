"""The persistent kernel that runs every DiT block of an Euler step in one launch at B = 1
(full model width: 32 heads of 48, MLP 6144), through the C ABI: parity with the oracle, and
agreement with the launch-per-step path of the same configuration without GR00T_FLAG_PERSIST,
over horizons (one or two 16-token tiles), VL lengths and key masks (image/text split, a
single admitted token, an empty text set), eager and in the captured graph."""
from dataclasses import replace

import numpy as np
import pytest

from flow_matching_dit_amd import head as H
from flow_matching_dit_amd import synth
from gpu_util import TOL, TOL_DISP, build_head, check_parity, gpu_action, say
from oracle import gr00t_oracle as O

pytestmark = pytest.mark.gpu


def _b1(num_layers=4, horizon=16, vl_len=300, image_tokens=256, steps=4, name="dit32_bf16_b1"):
    base = synth.WORKLOADS[name]
    w = synth.small_variant(base, num_layers=num_layers, hidden=1536, num_heads=32, head_dim=48, ff_dim=6144)
    w = replace(w, name=f"{w.name}_n{num_layers}_h{horizon}_l{vl_len}", vl_len=vl_len,
                image_tokens=None if image_tokens is None else min(image_tokens, vl_len),
                cfg=replace(w.cfg, action_horizon=horizon, num_steps=steps))
    return w


def _ran_persistent(h, inp, nz):
    """Whether a call on this handle runs its DiT blocks in the persistent kernel."""
    h.profile(True)
    gpu_action(h, inp, nz)
    prof = h.profile_read()
    h.profile(False)
    return prof.get("blocks_b1", (0, 0.0))[0] > 0


def _run(w, flags, graph):
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    h = build_head(w, wt, flags=flags | (H.FLAG_USE_GRAPH if graph else 0))
    y = gpu_action(h, inp, nz, prepare=graph)
    assert _ran_persistent(h, inp, nz) == bool(flags & H.FLAG_PERSIST)
    h.close()
    return y, wt, inp, nz


@pytest.mark.parametrize("layers,horizon,vl_len,image,graph", [
    (4, 16, 300, 256, False),   # the B = 1 recipe: text / self / image / self blocks, two token tiles
    (4, 16, 300, 256, True),    # the same replayed from the captured graph
    (2, 8, 300, None, False),   # one token tile (9 rows), no image/text split
    (2, 31, 64, None, True),    # 32 rows, the largest horizon the kernel takes
    (4, 16, 1, None, False),    # a single VL token
    (4, 16, 40, 40, False),     # every token an image token: text blocks admit no key (output 0)
    (4, 16, 1000, 700, False),  # long VL input: the score loop takes two passes of the workgroup
])
def test_persistent_blocks_match_oracle_and_launch_path(layers, horizon, vl_len, image, graph):
    w = _b1(layers, horizon, vl_len, image)
    say(f"[persist] {w.name}: N={layers} H={horizon} L={vl_len} image={image} graph={graph}")
    y, wt, inp, nz = _run(w, H.FLAG_PERSIST, graph)
    y_ref, _, _, _ = _run(w, 0, graph)
    ref = O.get_action(w.cfg.as_dict(), wt, inp, nz)
    check_parity(y, ref, nz, inp["action_mask"], TOL["bf16"], f"{w.name} persistent", TOL_DISP["bf16"])
    gap = O.rel_l2(y, y_ref)
    say(f"[persist] {w.name}: persistent vs launch-per-step rel_l2 {gap:.3e}")
    assert gap < 5e-3  # the two paths sum the same products in another order


def test_persistent_blocks_repeat_bitwise():
    """Fixed summation order: the same call twice gives the same bits (eager and graph)."""
    w = _b1(2, 16, 300, 256)
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    h = build_head(w, wt, flags=H.FLAG_USE_GRAPH | H.FLAG_PERSIST)
    assert _ran_persistent(h, inp, nz)
    ya = gpu_action(h, inp, nz)
    yb = gpu_action(h, inp, nz)
    yg = [gpu_action(h, inp, nz, prepare=True) for _ in range(3)]
    h.close()
    assert np.array_equal(ya, yb)
    for y in yg:
        assert np.array_equal(y, ya)


def test_persistent_timeout_falls_back_to_launch_path(monkeypatch):
    """Failure handling, forced from the host: with a poll budget of one (GR00T_PERSIST_SPIN=1 at
    create) the persistent kernel's waits give up at once and every workgroup leaves its loop,
    so the call's result is invalid. The next call reports E_DEVICE_ERROR; from then on the
    handle runs the blocks launch by launch, also from the graphs it had captured with the
    persistent kernel (they are captured again), bitwise as a handle without the flag."""
    w = _b1(2, 16, 300, 256)
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    say(f"[persist] {w.name}: forced timeout, fallback")
    ref_h = build_head(w, wt, flags=H.FLAG_USE_GRAPH)
    y_ref = gpu_action(ref_h, inp, nz, prepare=True)
    ref_h.close()
    monkeypatch.setenv("GR00T_PERSIST_SPIN", "1")
    h = build_head(w, wt, flags=H.FLAG_USE_GRAPH | H.FLAG_PERSIST)
    monkeypatch.delenv("GR00T_PERSIST_SPIN")
    gpu_action(h, inp, nz, prepare=True)  # its waits give up: an invalid result, reported next
    with pytest.raises(H.Gr00tError) as e:
        gpu_action(h, inp, nz)
    assert e.value.status == "E_DEVICE_ERROR" and "persistent" in str(e.value)
    y = gpu_action(h, inp, nz)  # the recaptured step graph: launch by launch
    assert not _ran_persistent(h, inp, nz)
    y_again = gpu_action(h, inp, nz)
    h.close()
    assert np.array_equal(y, y_ref)
    assert np.array_equal(y_again, y_ref)
