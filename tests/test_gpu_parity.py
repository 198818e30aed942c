"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded inputs.

Tolerances (relative L2 over every entry, float64; gated on action_pred, on the displacement
action_pred - noise and on every sample on its own):
fp32 path 1e-4, bf16 2e-2, fp8 e4m3 weights 5e-2, W8A8 (e4m3 weights and per-row e4m3 GEMM
inputs, against the oracle's W8A8 mode) 5e-2.
"""
from dataclasses import replace

import numpy as np
import pytest

from flow_matching_dit_amd import head as H
from flow_matching_dit_amd import synth
from gpu_util import TOL, TOL_DISP, build_head, check_parity, gpu_action, gpu_velocity, say, small
from oracle import gr00t_oracle as O

pytestmark = pytest.mark.gpu


def _parity(w, flags=0, prepare=False, samples=None):
    say(f"[parity] {w.name} B={w.batch} L={w.vl_len} D={w.cfg.hidden} N={w.cfg.num_layers} "
        f"prec={w.cfg.precision}")
    wt = synth.make_weights(w)
    inp = synth.make_inputs(w)
    nz = synth.make_noise(w)
    h = build_head(w, wt, flags=flags)
    y = gpu_action(h, inp, nz, prepare=prepare)
    h.close()
    if samples is not None:
        inp, nz = synth.take_samples(inp, nz, samples)
        y = y[np.asarray(samples)]
    ref = O.get_action(w.cfg.as_dict(), wt, inp, nz)
    err, _, _ = check_parity(y, ref, nz, inp["action_mask"], TOL[w.cfg.precision], w.name,
                              TOL_DISP[w.cfg.precision])
    return err


def test_tiny_fp32_full_parity():
    _parity(synth.WORKLOADS["tiny_fp32_b1"])


def test_tiny_fp32_graph_parity():
    _parity(synth.WORKLOADS["tiny_fp32_b1"], flags=H.FLAG_USE_GRAPH, prepare=True)


@pytest.mark.parametrize("name,kw", [
    ("dit32_bf16_b1", {}),
    ("dit32_bf16_b64", dict(batch=8)),
    ("dit32_bf16_b16_h64", dict(batch=3)),
    ("dit32_fp8_b256", dict(batch=12)),
    ("dit32_w8a8_b256", dict(batch=12)),
])
def test_small_width_parity(name, kw):
    _parity(small(name, **kw))


@pytest.mark.parametrize("precision", ["fp8", "fp8a8"])
def test_ragged_vl_fp8_modes_parity(precision):
    # the B=64 recipe (ragged VL lengths, action mask) with e4m3 weights, and with W8A8: the
    # key/value projection then runs over the compacted valid rows only (device row count)
    w = small("dit32_bf16_b64", batch=8)
    w = replace(w, name=f"{w.name}_{precision}", cfg=replace(w.cfg, precision=precision))
    _parity(w, flags=H.FLAG_USE_GRAPH, prepare=True)


def test_full_width_batch64_two_blocks_parity():
    # 64 samples of 17 tokens at width 1536: every block GEMM runs at its full-size shape
    # (1088 rows; the MLP down projection in 4 K-splits); the oracle checks 3 samples
    _parity(small("dit32_bf16_b64", num_layers=2, hidden=1536, num_heads=32, ff_dim=6144),
            flags=H.FLAG_USE_GRAPH, prepare=True, samples=[0, 31, 63])


@pytest.mark.parametrize("name,batch", [
    ("dit32_bf16_b64", 2),    # 34 rows: skinny kernel, 4 row fragments, activations staged in LDS
    ("dit32_bf16_b64", 4),    # 68 rows: 64 x 128 and 128 x 64 tiles, the MLP down in 8 K-splits
    ("dit32_bf16_b64", 12),   # 204 rows: several row tiles, ragged last tile
    ("dit32_fp8_b256", 1),    # e4m3 weights, 17 rows: skinny e4m3 kernel
    ("dit32_fp8_b256", 4),    # e4m3 weights, 68 rows: 64 x 128 tiles of weight bytes
    ("dit32_fp8_b256", 64),   # e4m3 weights, 1088 rows: 256 x 128 and 128 x 64 tiles, split-K MLP down
    ("dit32_w8a8_b256", 1),   # W8A8, 17 rows: 64 x 128 fp8 x fp8 tiles, one ragged row tile
    ("dit32_w8a8_b256", 4),   # W8A8, 68 rows: 64 x 128 tiles
    ("dit32_w8a8_b256", 64),  # W8A8, 1088 rows: 256 x 128 and 128 x 64 tiles, split-K MLP down
])
def test_full_width_mid_batch_parity(name, batch):
    # the GEMM configurations between the B=1 and B=64 shapes, at the full width of 1536
    _parity(small(name, batch=batch, num_layers=2, hidden=1536, num_heads=32, ff_dim=6144),
            flags=H.FLAG_USE_GRAPH, prepare=True, samples=[0, 40, 63] if batch == 64 else None)


def test_full_width_batch256_bf16_parity():
    # 4352 rows: the MLP up and q,k,v projections take 256 x 256 tiles (GELU and head-major
    # epilogues), the narrow projections 256 x 128; the oracle checks 3 samples
    _parity(small("dit32_bf16_b64", batch=256, num_layers=2, hidden=1536, num_heads=32, ff_dim=6144),
            flags=H.FLAG_USE_GRAPH, prepare=True, samples=[0, 101, 255])


def test_full_width_batch256_w8a8_parity():
    # the W8A8 workload's shapes (4352 rows, 256 x 128 fp8 x fp8 tiles for every DiT GEMM,
    # 76800 VL rows into the key/value projection) against the oracle's W8A8 mode, 3 samples
    _parity(small("dit32_w8a8_b256", batch=256, num_layers=2, hidden=1536, num_heads=32, ff_dim=6144),
            flags=H.FLAG_USE_GRAPH, prepare=True, samples=[0, 101, 255])


@pytest.mark.parametrize("name,kw", [
    ("dit32_bf16_b64", dict(batch=64, num_heads=16, hidden=768, ff_dim=1536)),  # one wave per pair
    ("dit32_bf16_b1", {}),                                                        # workgroup per pair
])
def test_short_horizon_single_query_fragment_parity(name, kw):
    # horizon 8: 9 tokens, one 16-query fragment per (sample, head) in both attention kernels
    w = small(name, **kw)
    w = replace(w, cfg=replace(w.cfg, action_horizon=8))
    _parity(w, samples=[0, 63] if w.batch == 64 else None)


@pytest.mark.parametrize("name,hz,k", [
    ("dit32_bf16_b1", 40, 4),    # the base N1.7 horizon: 41 tokens, three query fragments
    ("dit32_bf16_b64", 40, 4),   # 2624 rows: 256 x 256 tiles for the MLP and q,k,v
    ("dit32_bf16_b1", 16, 1),
    ("dit32_bf16_b1", 16, 2),
    ("dit32_bf16_b1", 16, 16),
])
def test_horizon_and_step_variants_parity(name, hz, k):
    w = small(name, num_layers=2, hidden=1536, num_heads=32, ff_dim=6144)
    w = replace(w, cfg=replace(w.cfg, action_horizon=hz, num_steps=k))
    _parity(w, flags=H.FLAG_USE_GRAPH, prepare=True, samples=[0, 63] if w.batch == 64 else None)


def test_folded_layernorm_parity_b1():
    # at most 32 rows and a width of 1024..2048: the norms run inside the GEMMs that read them
    # and the residual projections add into h unsplit
    _parity(small("dit32_bf16_b1", hidden=1536, num_heads=32, ff_dim=3072), flags=H.FLAG_USE_GRAPH, prepare=True)


@pytest.mark.parametrize("hidden,heads,hz", [(1024, 16, 16), (1280, 20, 16), (1792, 28, 8), (2048, 32, 16)])
def test_folded_layernorm_widths_parity_b1(hidden, heads, hz):
    # the folded LayerNorm is compiled per width / 256 (4, 5, 7 and 8 here, 6 above; horizon 8:
    # 9 rows, one row fragment), and the skinny projections take their split depth, tile width
    # and k-steps per wave from the shape
    w = small("dit32_bf16_b1", hidden=hidden, num_heads=heads, head_dim=hidden // heads, ff_dim=2 * hidden)
    w = replace(w, cfg=replace(w.cfg, action_horizon=hz))
    _parity(w, flags=H.FLAG_USE_GRAPH, prepare=True)


def test_wave_per_head_attention_parity():
    # 64 samples x 16 heads of width 48: at >= 1024 (sample, head) pairs attention runs one
    # wave per pair (ragged VL lengths, skipped key tiles); the oracle runs on sampled rows
    _parity(small("dit32_bf16_b64", batch=64, num_heads=16, hidden=768, ff_dim=1536), samples=[0, 29, 63])


def test_small_width_graph_parity_ragged():
    _parity(small("dit32_bf16_b64", batch=8), flags=H.FLAG_USE_GRAPH | H.FLAG_STRICT, prepare=True)


def test_fp32_small_width_parity_many_tiles():
    # fp32 path at a width spanning several GEMM tiles, ragged masks and mixed ids
    w = small("dit32_bf16_b64", batch=5, num_categories=6)
    w = replace(w, cfg=replace(w.cfg, precision="fp32"), id_range=(0, 5))
    _parity(w)


def test_velocity_matches_oracle_each_step():
    w = small("dit32_bf16_b64", batch=4)
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    h = build_head(w, wt)
    P = O.effective_params(w.cfg.as_dict(), wt)
    for k in range(w.cfg.num_steps):
        v = gpu_velocity(h, inp, nz, k)
        ref = O.get_action(w.cfg.as_dict(), wt, inp, nz, params=P, return_velocity_at=k)
        err = O.rel_l2(v, ref)
        say(f"[velocity] k={k} rel_l2 = {err:.3e}")
        assert err < TOL["bf16"]
    h.close()


def test_state_features_output():
    w = small("dit32_bf16_b64", batch=4)
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    h = build_head(w, wt)
    _, sf = gpu_action(h, inp, nz, state_out=True)
    h.close()
    ref = O.state_features(w.cfg.as_dict(), wt, inp)
    assert O.rel_l2(sf, ref) < TOL["bf16"]
