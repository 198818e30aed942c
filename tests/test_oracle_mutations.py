"""Plant plausible mistakes in the CPU oracle and check that a pin catches each one.

Each case swaps one oracle function for a subtly wrong version (on the CPU only)
and runs the pin that is meant to catch it; the pin must fail.
"""
import math

import numpy as np
import pytest

import test_oracle as pins
from oracle import gr00t_oracle as O


def _gelu_tanh(x):
    return 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))


def _attention_no_temperature(q, k, v, admitted):
    return O.__dict__["_orig_attention"](q * math.sqrt(q.shape[-1]), k, v, admitted)


def _ada_swapped(P, prefix, h, temb):
    D = h.shape[-1]
    mod = O.linear(O.silu(temb), P[prefix + "ada.w"], P[prefix + "ada.b"])
    return O.layer_norm(h) * (1.0 + mod[D:]) + mod[:D]


def _block_without_residual(P, cfg, l, h, vl, key_masks, temb):
    return O.__dict__["_orig_block"](P, cfg, l, h, vl, key_masks, temb) - h


def _category_linear_no_bias(x, W, b, ids):
    return np.einsum("bti,bio->bto", x, W[ids])


def _category_linear_first_id(x, W, b, ids):
    return np.einsum("bti,io->bto", x, W[ids[0]]) + b[ids[0]][None, None, :]


def _bf16_truncate(a):
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def _euler_wrong_dt(x0, vfn, K, buckets=1000):
    _, tau, _ = O.timestep_grid(K, buckets)
    x = np.array(x0, dtype=np.float64)
    for k in range(K):
        x = x + (1.0 / (K + 1)) * vfn(x, k, tau[k])
    return x


def _grid_shifted(K, buckets=1000):
    return [(k + 1) / K for k in range(K)], [(buckets * (k + 1)) // K for k in range(K)], 1.0 / K


def _mask_swapped(cfg, l, valid, image):
    if image is None:
        return valid
    if l % (2 * cfg["attend_text_every_n_blocks"]) == 0:
        return valid & image
    return valid & ~image


def _layer_norm_unbiased(x, gamma=None, beta=None, eps=O.LN_EPS):
    mu = x.mean(axis=-1, keepdims=True)
    var = x.var(axis=-1, ddof=1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * gamma
    if beta is not None:
        y = y + beta
    return y


def _sinusoid_cos_first(tau, dim):
    s = O.__dict__["_orig_sinusoid"](tau, dim)
    half = dim // 2
    return np.concatenate([s[..., half:], s[..., :half]], axis=-1)


def _e4m3_ties_away(v):
    v = np.asarray(v, dtype=np.float64)
    mag = np.minimum(np.abs(v), 448.0)
    hi = np.clip(np.searchsorted(O._E4M3_POS, mag, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    pick_lo = np.abs(mag - O._E4M3_POS[lo]) < np.abs(O._E4M3_POS[hi] - mag)
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def _velocity_decode_all_rows(P, cfg, vl, valid, image, s, x, tau, ids):
    temb = O.timestep_encoder(P, cfg, tau)
    af = O.action_encoder(P, cfg, x, tau, ids)
    y = O.dit(P, cfg, np.concatenate([af, s], axis=1), vl, valid, image, temb)
    return O.action_decoder(P, y[:, 1:, :], ids)


def _rows_quantised_per_column(x):
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-2, keepdims=True).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return O.e4m3_decode(O.e4m3_encode((x32 / scale).astype(np.float32))) * scale.astype(np.float64)


def _interp_swapped(actions, noise, t):
    t = np.asarray(t, np.float64)[:, None, None]
    return t * np.asarray(noise, np.float64) + (1.0 - t) * np.asarray(actions, np.float64)


def _bucket_rounded(t, buckets=1000):
    return np.rint(np.asarray(t, np.float32) * np.float32(buckets)).astype(np.int64)


def _training_target_sign(cfg, weights, inputs, actions, noise, t, params=None):
    # the target velocity taken as noise - action
    return O.__dict__["_orig_training_loss"](cfg, weights, inputs, noise, actions, 1.0 - np.asarray(t), params)


def _timestep_encoder_no_silu(P, cfg, tau):
    e = O.sinusoid(np.array(float(tau)), cfg["time_freq_dim"])
    return O.linear(O.linear(e, P["time.w1"], P["time.b1"]), P["time.w2"], P["time.b2"])


def _action_encoder_concat_swapped(P, cfg, x, tau, ids):
    B, H, _ = x.shape
    a = O.category_linear(x, P["action_enc.w1"], P["action_enc.b1"], ids)
    te = np.broadcast_to(O.sinusoid(np.array(float(tau)), cfg["hidden"]), (B, H, cfg["hidden"]))
    z = O.silu(O.category_linear(np.concatenate([te, a], axis=-1), P["action_enc.w2"], P["action_enc.b2"], ids))
    return O.category_linear(z, P["action_enc.w3"], P["action_enc.b3"], ids)


def _action_encoder_swish_after_w3(P, cfg, x, tau, ids):
    B, H, _ = x.shape
    a = O.category_linear(x, P["action_enc.w1"], P["action_enc.b1"], ids)
    te = np.broadcast_to(O.sinusoid(np.array(float(tau)), cfg["hidden"]), (B, H, cfg["hidden"]))
    z = O.category_linear(np.concatenate([a, te], axis=-1), P["action_enc.w2"], P["action_enc.b2"], ids)
    return O.silu(O.category_linear(z, P["action_enc.w3"], P["action_enc.b3"], ids))


def _state_encoder_no_relu(P, state, ids):
    z = O.category_linear(state, P["state_enc.w1"], P["state_enc.b1"], ids)
    return O.category_linear(z, P["state_enc.w2"], P["state_enc.b2"], ids)


def _action_decoder_no_relu(P, y, ids):
    z = O.category_linear(y, P["action_dec.w1"], P["action_dec.b1"], ids)
    return O.category_linear(z, P["action_dec.w2"], P["action_dec.b2"], ids)


def _dit_plain_final_norm(P, cfg, sa_embs, vl, valid, image, temb):
    h = sa_embs
    for l in range(cfg["num_layers"]):
        masks = None if l % 2 else [O.cross_layer_mask(cfg, l, valid[b], None if image is None else image[b])
                                    for b in range(h.shape[0])]
        h = O.transformer_block(P, cfg, l, h, vl, masks, temb)
    return O.dit_linear(cfg, O.layer_norm(h), P["out.proj.w"], P["out.proj.b"])


def _dit_no_output_projection(P, cfg, sa_embs, vl, valid, image, temb):
    h = sa_embs
    for l in range(cfg["num_layers"]):
        masks = None if l % 2 else [O.cross_layer_mask(cfg, l, valid[b], None if image is None else image[b])
                                    for b in range(h.shape[0])]
        h = O.transformer_block(P, cfg, l, h, vl, masks, temb)
    return O.ada_layer_norm(P, "out.", h, temb)


def _dit_linear_unrounded_a8(cfg, x, w, b):
    if cfg["precision"] == "fp8a8":
        x = O.quantize_e4m3_rows(x)
    return O.linear(x, w, b)


CASES = [
    ("gelu", _gelu_tanh, pins.test_gelu_textbook_values),
    ("attention", _attention_no_temperature, pins.test_attention_temperature),
    ("ada_layer_norm", _ada_swapped, pins.test_ada_layer_norm_scale_shift_order),
    ("transformer_block", _block_without_residual,
     pins.test_block_with_zero_output_projections_is_identity),
    ("category_linear", _category_linear_no_bias, pins.test_category_linear_brute_force_integer_exact),
    ("category_linear", _category_linear_first_id, pins.test_category_linear_brute_force_integer_exact),
    ("round_bf16", _bf16_truncate, pins.test_bf16_rounding_ties_and_library),
    ("euler", _euler_wrong_dt, lambda: pins.test_euler_closed_forms(4)),
    ("timestep_grid", _grid_shifted, pins.test_time_grid_matches_page),
    ("cross_layer_mask", _mask_swapped, pins.test_alternate_schedule),
    ("layer_norm", _layer_norm_unbiased, pins.test_layer_norm_statistics),
    ("sinusoid", _sinusoid_cos_first, pins.test_sinusoid_values),
    ("e4m3_encode", _e4m3_ties_away, pins.test_e4m3_roundtrip_all_codes_and_ties),
    ("velocity", _velocity_decode_all_rows, pins.test_horizon_permutation_equivariance),
    ("flow_interp", _interp_swapped, pins.test_flow_interp_endpoints),
    ("discretize_t", _bucket_rounded, pins.test_training_bucket_matches_inference_grid),
    ("training_loss", _training_target_sign, pins.test_training_loss_closed_form),
    ("quantize_e4m3_rows", _rows_quantised_per_column, pins.test_row_quantisation),
    ("timestep_encoder", _timestep_encoder_no_silu, pins.test_timestep_encoder_closed_form),
    ("action_encoder", _action_encoder_concat_swapped, pins.test_action_encoder_concat_order_and_swish),
    ("action_encoder", _action_encoder_swish_after_w3, pins.test_action_encoder_concat_order_and_swish),
    ("state_encoder", _state_encoder_no_relu, pins.test_state_encoder_relu_between_linears),
    ("action_decoder", _action_decoder_no_relu, pins.test_action_decoder_relu_between_linears),
    ("dit", _dit_plain_final_norm, pins.test_dit_output_head_is_modulated_norm_then_projection),
    ("dit", _dit_no_output_projection, pins.test_dit_output_head_is_modulated_norm_then_projection),
    ("dit_linear", _dit_linear_unrounded_a8, pins.test_w8a8_linear_quantises_the_bf16_activation),
]


@pytest.mark.parametrize("name,bad,pin", CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_planted_mistake_is_caught(monkeypatch, name, bad, pin):
    monkeypatch.setitem(O.__dict__, "_orig_attention", O.attention)
    monkeypatch.setitem(O.__dict__, "_orig_block", O.transformer_block)
    monkeypatch.setitem(O.__dict__, "_orig_sinusoid", O.sinusoid)
    monkeypatch.setitem(O.__dict__, "_orig_training_loss", O.training_loss)
    monkeypatch.setattr(O, name, bad)
    with pytest.raises(AssertionError):
        pin()
