"""Category buckets of the per-embodiment linears at B >= 128 ("Model architecture",
Embodiment-specific projectors, CategorySpecificLinear): the samples are sorted by embodiment
id on the device and each bucket of up to 8 samples of one category reads its weights once.
Checked through the C ABI against the oracle on sampled samples, and against the per-sample
weight gather of the same handle configuration (GR00T_FLAG_NO_BUCKETS), over id patterns:
every category present, one category for all samples, runs that are not multiples of the
bucket size with absent categories, a batch that is not a multiple of 8, and an invalid id."""
import numpy as np
import pytest

from flow_matching_dit_amd import head as H
from flow_matching_dit_amd import synth
from gpu_util import TOL, TOL_DISP, build_head, check_parity, gpu_action, say, small
from oracle import gr00t_oracle as O

pytestmark = pytest.mark.gpu


def _ids(pattern, B, C, rng):
    if pattern == "uniform":
        return rng.integers(0, C, B).astype(np.int32)
    if pattern == "one_category":
        return np.full(B, 5, np.int32)
    if pattern == "ragged_runs":   # 3 categories with 1, 9 and B - 10 samples, the rest absent, shuffled
        ids = np.array([2] + [7] * 9 + [30] * (B - 10), np.int32)
        return ids[rng.permutation(B)]
    raise ValueError(pattern)


@pytest.mark.parametrize("pattern,B", [("uniform", 128), ("one_category", 128), ("ragged_runs", 131)])
def test_buckets_match_oracle_and_per_sample_gather(pattern, B):
    w = small("dit32_bf16_b64", batch=B)   # 32 categories, ragged VL, action mask
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    inp = dict(inp, embodiment_id=_ids(pattern, B, w.cfg.num_categories, np.random.default_rng(3)))
    say(f"[buckets] {w.name}: {pattern} B={B}, {len(np.unique(inp['embodiment_id']))} categories present")
    h = build_head(w, wt, flags=H.FLAG_USE_GRAPH)
    y = gpu_action(h, inp, nz, prepare=True)
    h.close()
    h = build_head(w, wt, flags=H.FLAG_USE_GRAPH | H.FLAG_NO_BUCKETS)
    y_ps = gpu_action(h, inp, nz, prepare=True)
    h.close()
    gap = O.rel_l2(y, y_ps)
    say(f"[buckets] buckets vs per-sample gather rel_l2 {gap:.2e}")
    assert gap < 5e-3  # the same products summed in another order (and bf16 roundings between them)
    samples = [0, 1, B // 2, B - 1]
    sub, nzs = synth.take_samples(inp, nz, samples)
    ref = O.get_action(w.cfg.as_dict(), wt, sub, nzs)
    check_parity(y[samples], ref, nzs, sub["action_mask"], TOL["bf16"], f"{w.name} {pattern} samples {samples}",
                 TOL_DISP["bf16"])


def test_buckets_invalid_id_leaves_the_other_samples_unchanged():
    """Non-strict mode: an invalid id gives its sample NaN rows; it is sorted into category 0's
    buckets as its sanitised id, and every other sample is bitwise what it is without it (a
    sample's rows are its own rows of the bucket tiles, whatever the tile position)."""
    B = 128
    w = small("dit32_bf16_b64", batch=B)
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    h = build_head(w, wt)
    y = gpu_action(h, inp, nz)
    bad = dict(inp, embodiment_id=inp["embodiment_id"].copy())
    bad["embodiment_id"][17] = w.cfg.num_categories + 4
    yb = gpu_action(h, bad, nz)
    assert np.all(np.isnan(yb[17]))
    keep = [b for b in range(B) if b != 17]
    assert np.array_equal(yb[keep], y[keep])
    with pytest.raises(H.Gr00tError) as e:   # the deferred report of the invalid id
        gpu_action(h, inp, nz)
    assert e.value.status == "E_DEVICE_ERROR"
    h.close()


def test_buckets_training_forward_matches_per_sample_gather():
    B = 128
    w = small("dit32_bf16_b64", batch=B)
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    rng = np.random.default_rng(9)
    actions = rng.standard_normal(nz.shape).astype(np.float32)
    t = rng.beta(1.5, 1.0, B).astype(np.float32)
    import torch
    res = []
    for flags in (0, H.FLAG_NO_BUCKETS):
        h = build_head(w, wt, flags=flags)
        d = H.device_inputs(inp, nz, h.act_torch_dtype)
        loss, vp = h.train_forward(d["vl_features"], d["vl_mask"], d["image_mask"], d["state"], d["embodiment_id"],
                                   torch.from_numpy(actions).cuda(), torch.from_numpy(t).cuda(), d["noise"],
                                   action_mask=d["action_mask"])
        torch.cuda.synchronize()
        res.append((float(loss.cpu()[0]), vp.cpu().numpy()))
        h.close()
    gap = O.rel_l2(res[0][1], res[1][1])
    say(f"[buckets] training forward: loss {res[0][0]:.6f} vs {res[1][0]:.6f}, v_pred rel_l2 {gap:.2e}")
    assert gap < 5e-3 and abs(res[0][0] - res[1][0]) < 5e-3 * abs(res[1][0])
