"""Plain CPU oracle of the GR00T flow-matching DiT action head (System 1).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code, header, table or constant generator
with the HIP library; it sees the same seeded input arrays and nothing else.

Everything is computed in float64 with plain NumPy (a matmul, an einsum and
scipy's erf are the only library primitives). Weights and inputs are first
rounded to the precision the GPU path stores them in (bf16 round-to-nearest-even,
or OCP e4m3 with a per-output-channel fp32 scale), so the comparison measures the
GPU's arithmetic and nothing else.

Sources (page titles as printed; sections in quotes):
  [ARCH]   "Model architecture" (GR00T N1.6): "Action head architecture",
           "Diffusion transformer (DiT)", "Transformer block structure",
           "AlternateVLDiT variant", "Flow matching diffusion" / "Inference
           (denoising)", "Embodiment-specific projectors", "Model configuration".
  [MODEL]  "GR00T model class": "get_action", "Training configuration"
           (tune_vlln), "Flow matching diffusion" (num_timestep_buckets).
  [WS1]    "Single-GPU inference for GR00T-N1.7": "Architecture" (request path:
           masked normalized action chunk), "Prepare a request" (optional noise).

Readings adopted where the pages are silent (each listed with its reason in the
design notes): one width D for encoders, DiT and decoder; the DiT ends in a
final adaptive LayerNorm and a D->D projection; the discretised timestep is
floor(buckets*k/K); sinusoids are [sin | cos] with frequencies 10000^(-i/half);
the timestep encoder is sin256 -> Linear -> SiLU -> Linear; adaLN is
LN(h)*(1+scale)+shift with [scale | shift] = Linear(SiLU(temb)); norm3 and the
final norm carry no affine; attention has no mask besides the key mask and no
positional term; an empty key set gives a zero output; the feed-forward is
Linear -> exact-erf GELU -> Linear; the per-embodiment MLPs use ReLU; only the
H action rows are decoded; the vision-language LayerNorm (vlln) has gain and
bias; action_mask multiplies the final chunk only. Training forward: the loss is
the elementwise squared error times action_mask, summed, over the mask's sum plus
1e-6; the training timestep bucket is floor(t * buckets) in float32. W8A8 mode
("fp8a8"): the input rows of every e4m3-weight GEMM, the bf16 activations of that mode, are
quantised to e4m3 per row (scale = row amax / 448), the code decided in float32 from the bf16 value.

Parity: pinned by closed forms and invariants in tests/test_oracle.py; the
whole network has no printed worked example on the pages, so beyond those pins
the end-to-end value is "parity unpinned".
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Dict, Optional

import numpy as np
from scipy.special import erf

LN_EPS = 1e-5

# --------------------------------------------------------------------------
# Number formats (storage precision of the GPU path)
# --------------------------------------------------------------------------


def round_bf16(a) -> np.ndarray:
    """fp32 -> bf16 with round-to-nearest, ties-to-even, returned as float64.

    bf16 keeps the top 16 bits of an IEEE binary32 value; the dropped 16 bits
    decide the rounding (greater than half: up; exactly half: to the even
    neighbour)."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lower = u & 0xFFFF
    upper = u >> 16
    half = 0x8000
    round_up = (lower > half) | ((lower == half) & ((upper & 1) == 1))
    upper = upper + round_up.astype(np.uint64)
    out = (upper << 16).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """OCP 8-bit float E4M3 (the 'fn' variant: no infinities, S.1111.111 is NaN).

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits. Exponent field 0
    holds subnormals m * 2^-9. Largest finite magnitude 1.75 * 2^8 = 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.power(2.0, e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


_E4M3_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # codes 0x00..0x7E, increasing


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code, ties to the even code, magnitudes above 448 saturate to 448."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.minimum(np.abs(v), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, mag, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = np.abs(_E4M3_POS[hi] - mag)
    d_lo = np.abs(mag - _E4M3_POS[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def quantize_e4m3_columns(w32: np.ndarray):
    """Per-output-channel e4m3 weights of an [.., in, out] fp32 matrix.

    scale[o] = fp32(max_i |W[i,o]|) / fp32(448) (fp32 division; 1 where the column
    is all zero), code = e4m3(fp32(W / scale)), dequantised W = decode(code)*scale.
    The code is decided on fp32 operands, the precision the library uses."""
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=-2, keepdims=True).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = (w32 / scale).astype(np.float32)
    codes = e4m3_encode(q)
    deq = e4m3_decode(codes) * scale.astype(np.float64)
    return deq, codes, scale


def quantize_e4m3_rows(x) -> np.ndarray:
    """Per-row e4m3 activations of the W8A8 mode ("fp8a8"): the input rows of a GEMM with
    e4m3 weights. scale[r] = fp32(max_k |x[r,k]|) / fp32(448) (fp32 division; 1 for an all-zero
    row), code = e4m3(fp32(x / scale)) decided on fp32 operands, dequantised x = decode(code) *
    scale: the column quantisation of the weights applied along the rows."""
    codes, scale = quantize_e4m3_rows_codes(x)
    return e4m3_decode(codes) * scale.astype(np.float64)[..., None]


def quantize_e4m3_rows_codes(x):
    """The codes [.., rows, cols] (uint8) and fp32 scales [.., rows] of quantize_e4m3_rows."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1, keepdims=True).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = e4m3_encode((x32 / scale).astype(np.float32))
    return codes, scale[..., 0]


# --------------------------------------------------------------------------
# Building blocks
# --------------------------------------------------------------------------


def layer_norm(x, gamma=None, beta=None, eps=LN_EPS):
    """LayerNorm over the last axis: (x - mean) / sqrt(var + eps), population variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * gamma
    if beta is not None:
        y = y + beta
    return y


def silu(x):
    """x * sigmoid(x); also the 'swish' of the action encoder [ARCH, encoder forward]."""
    return x / (1.0 + np.exp(-x))


def relu(x):
    return np.maximum(x, 0.0)


def gelu(x):
    """Exact GELU: x * Phi(x) = x * (1 + erf(x / sqrt 2)) / 2 (MLP with GELU, [ARCH])."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def sinusoid(tau, dim: int) -> np.ndarray:
    """[sin(tau*w_i) | cos(tau*w_i)], w_i = 10000^(-i/half), i < half = dim/2.

    Used for the diffusion timestep both in the timestep encoder (width 256) and in
    the action encoder's positional encoding of the timestep (width D) [ARCH]."""
    half = dim // 2
    i = np.arange(half, dtype=np.float64)
    w = np.power(10000.0, -i / half)
    arg = np.asarray(tau, dtype=np.float64)[..., None] * w
    return np.concatenate([np.sin(arg), np.cos(arg)], axis=-1)


def linear(x, w, b):
    return x @ w + b


def dit_linear(cfg, x, w, b):
    """A linear whose weight is an e4m3 matrix in the fp8 modes (is_fp8_matrix); in the W8A8
    mode ("fp8a8") its input rows are quantised to e4m3 first (quantize_e4m3_rows). The rows
    quantised are the bf16 activations of that mode (bf16 activations, as in the e4m3-weight
    workload), so the input is rounded to bf16 before its row scale and codes are decided."""
    if cfg["precision"] == "fp8a8":
        x = quantize_e4m3_rows(round_bf16(x))
    return linear(x, w, b)


def category_linear(x, W, b, ids):
    """Per-embodiment linear: y_b = x_b @ W[id_b] + b[id_b] ([ARCH], CategorySpecificLinear:
    weights gathered by category id, then a batched product). x [B,T,in], W [C,in,out]."""
    return np.einsum("bti,bio->bto", x, W[ids]) + b[ids][:, None, :]


def attention(q, k, v, admitted):
    """softmax(q k^T / sqrt(d)) v over the admitted keys, per head.

    q [S,h,d], k/v [L,h,d], admitted [L] bool. A query with no admitted key yields 0.
    Every softmax row is checked to sum to 1."""
    S, nh, d = q.shape
    out = np.zeros((S, nh, d))
    idx = np.flatnonzero(admitted)
    if idx.size == 0:
        return out
    kk, vv = k[idx], v[idx]
    scores = np.einsum("shd,lhd->hsl", q, kk) / math.sqrt(d)
    scores = scores - scores.max(axis=-1, keepdims=True)
    p = np.exp(scores)
    p = p / p.sum(axis=-1, keepdims=True)
    assert np.allclose(p.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    return np.einsum("hsl,lhd->shd", p, vv)


# --------------------------------------------------------------------------
# The action head
# --------------------------------------------------------------------------


def timestep_grid(K: int, buckets: int = 1000):
    """Inference grid [ARCH, Inference]: t_cont = k/K for k = 0..K-1, dt = 1/K, and the
    discretised timestep floor(buckets * k / K) in integer arithmetic."""
    t_cont = [k / K for k in range(K)]
    tau = [(buckets * k) // K for k in range(K)]
    return t_cont, tau, 1.0 / K


def timestep_encoder(P, cfg, tau):
    """temb = Linear2(SiLU(Linear1(sin256(tau)))) (TimestepEncoder of width inner_dim)."""
    e = sinusoid(np.array(float(tau)), cfg["time_freq_dim"])
    return linear(silu(linear(e, P["time.w1"], P["time.b1"])), P["time.w2"], P["time.b2"])


def ada_layer_norm(P, prefix, h, temb):
    """Adaptive LayerNorm conditioned on the timestep: LN(h)*(1+scale)+shift with
    [scale | shift] = Linear(SiLU(temb)); LN without affine."""
    D = h.shape[-1]
    mod = linear(silu(temb), P[prefix + "ada.w"], P[prefix + "ada.b"])
    scale, shift = mod[:D], mod[D:]
    return layer_norm(h) * (1.0 + scale) + shift


def cross_layer_mask(cfg, l, valid, image):
    """AlternateVLDiT key mask for even (cross-attention) block l [ARCH]:
    text = valid & ~image on blocks with l % (2n) == 0, image = valid & image otherwise,
    n = attend_text_every_n_blocks. With no image mask every cross block uses valid."""
    if image is None:
        return valid
    if l % (2 * cfg["attend_text_every_n_blocks"]) == 0:
        return valid & ~image
    return valid & image


def transformer_block(P, cfg, l, h, vl, key_masks, temb):
    """One BasicTransformerBlock [ARCH]: h += attn(norm1(h, temb)); h += ff(norm3(h)).

    Odd l: self-attention over the S state+action tokens. Even l: cross-attention
    to the vision-language tokens admitted by key_masks[b]."""
    B, S, D = h.shape
    nh, hd = cfg["num_heads"], cfg["head_dim"]
    p = f"blocks.{l}."
    n = ada_layer_norm(P, p, h, temb)
    out = np.empty_like(h)
    for b in range(B):
        q = dit_linear(cfg, n[b], P[p + "attn.wq"], P[p + "attn.bq"]).reshape(S, nh, hd)
        if l % 2 == 1:
            src, admitted = n[b], np.ones(S, bool)
        else:
            src, admitted = vl[b], key_masks[b]
        k = dit_linear(cfg, src, P[p + "attn.wk"], P[p + "attn.bk"]).reshape(-1, nh, hd)
        v = dit_linear(cfg, src, P[p + "attn.wv"], P[p + "attn.bv"]).reshape(-1, nh, hd)
        out[b] = attention(q, k, v, admitted).reshape(S, D)
    h = h + dit_linear(cfg, out, P[p + "attn.wo"], P[p + "attn.bo"])
    u = gelu(dit_linear(cfg, layer_norm(h), P[p + "ff.w1"], P[p + "ff.b1"]))
    return h + dit_linear(cfg, u, P[p + "ff.w2"], P[p + "ff.b2"])


def dit(P, cfg, sa_embs, vl, valid, image, temb):
    """AlternateVLDiT: the blocks in order, then final adaLN and the D->D output projection."""
    h = sa_embs
    B = h.shape[0]
    for l in range(cfg["num_layers"]):
        masks = None
        if l % 2 == 0:
            masks = [cross_layer_mask(cfg, l, valid[b],
                                      None if image is None else image[b]) for b in range(B)]
        h = transformer_block(P, cfg, l, h, vl, masks, temb)
    y = ada_layer_norm(P, "out.", h, temb)
    return dit_linear(cfg, y, P["out.proj.w"], P["out.proj.b"])


def state_encoder(P, state, ids):
    """CategorySpecificMLP on the state: Linear_c -> ReLU -> Linear_c, one state token."""
    z = relu(category_linear(state, P["state_enc.w1"], P["state_enc.b1"], ids))
    return category_linear(z, P["state_enc.w2"], P["state_enc.b2"], ids)


def action_encoder(P, cfg, x, tau, ids):
    """MultiEmbodimentActionEncoder [ARCH]: a = W1(x); cat with the sinusoidal encoding of
    the timestep broadcast over the horizon; swish(W2(.)); W3(.)."""
    B, H, _ = x.shape
    a = category_linear(x, P["action_enc.w1"], P["action_enc.b1"], ids)
    te = np.broadcast_to(sinusoid(np.array(float(tau)), cfg["hidden"]), (B, H, cfg["hidden"]))
    z = silu(category_linear(np.concatenate([a, te], axis=-1),
                             P["action_enc.w2"], P["action_enc.b2"], ids))
    return category_linear(z, P["action_enc.w3"], P["action_enc.b3"], ids)


def action_decoder(P, y, ids):
    """CategorySpecificMLP decoder: Linear_c -> ReLU -> Linear_c to action_dim."""
    z = relu(category_linear(y, P["action_dec.w1"], P["action_dec.b1"], ids))
    return category_linear(z, P["action_dec.w2"], P["action_dec.b2"], ids)


def velocity(P, cfg, vl, valid, image, s, x, tau, ids):
    """Predicted velocity at Euler state x and discretised timestep tau: encode actions,
    prepend the state token, run the DiT, decode the H action rows."""
    temb = timestep_encoder(P, cfg, tau)
    af = action_encoder(P, cfg, x, tau, ids)
    sa = np.concatenate([s, af], axis=1)
    y = dit(P, cfg, sa, vl, valid, image, temb)
    return action_decoder(P, y[:, 1:, :], ids)


def euler(x0, vfn: Callable, K: int, buckets: int = 1000):
    """x <- x + dt * v(x, k) for k = 0..K-1, dt = 1/K, starting at the noise x0."""
    _, tau, dt = timestep_grid(K, buckets)
    x = np.array(x0, dtype=np.float64)
    for k in range(K):
        x = x + dt * vfn(x, k, tau[k])
    return x


# --------------------------------------------------------------------------
# Precision of stored operands, and the entry point
# --------------------------------------------------------------------------

FP8_MATRIX_SUFFIXES = ("attn.wq", "attn.wk", "attn.wv", "attn.wo", "ff.w1", "ff.w2")


def is_fp8_matrix(name: str) -> bool:
    """DiT matrices stored as e4m3 in fp8 mode: every block's q/k/v/o and MLP matrices
    and the output projection. Embodiment MLPs, time/adaLN linears, norms stay bf16."""
    if name == "out.proj.w":
        return True
    return name.startswith("blocks.") and name.endswith(FP8_MATRIX_SUFFIXES)


def effective_params(cfg, weights: Dict[str, np.ndarray], threads: int = 8) -> Dict[str, np.ndarray]:
    """Parameters as float64 values of what the GPU path stores (tensors are converted
    independently, on several threads)."""
    prec = cfg["precision"]

    def convert(item):
        name, w = item
        if prec == "fp32":
            return name, np.asarray(w, dtype=np.float64)
        if prec in ("fp8", "fp8a8") and is_fp8_matrix(name):
            return name, quantize_e4m3_columns(w)[0]
        return name, round_bf16(w)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return dict(ex.map(convert, list(weights.items())))


def effective_vl(cfg, vl_features):
    return (np.asarray(vl_features, np.float64) if cfg["precision"] == "fp32"
            else round_bf16(vl_features))


def get_action(cfg, weights, inputs, noise, params=None, return_velocity_at=None):
    """action_pred (B, H, A) of one get_action call [MODEL get_action; ARCH Inference].

    cfg: dict of HeadConfig fields; weights: fp32 masters by name; inputs: the dict of
    make_inputs (vl_features, vl_mask, image_mask, state, embodiment_id, action_mask);
    noise: x_0 [B,H,A]. ``params`` may carry effective_params(cfg, weights)."""
    P = params if params is not None else effective_params(cfg, weights)
    vl_raw = effective_vl(cfg, inputs["vl_features"])
    B, L, _ = vl_raw.shape
    vl = layer_norm(vl_raw, P["vlln.gamma"], P["vlln.beta"])
    valid = (np.ones((B, L), bool) if inputs.get("vl_mask") is None
             else np.asarray(inputs["vl_mask"]).astype(bool))
    image = (None if inputs.get("image_mask") is None
             else np.asarray(inputs["image_mask"]).astype(bool))
    ids = np.asarray(inputs["embodiment_id"]).astype(np.int64)
    state = np.asarray(inputs["state"], np.float64)
    s = state_encoder(P, state, ids)

    def vfn(x, k, tau):
        return velocity(P, cfg, vl, valid, image, s, x, tau, ids)

    if return_velocity_at is not None:
        _, tau, _ = timestep_grid(cfg["num_steps"], cfg["num_timestep_buckets"])
        k = return_velocity_at
        return vfn(np.asarray(noise, np.float64), k, tau[k])
    x = euler(noise, vfn, cfg["num_steps"], cfg["num_timestep_buckets"])
    if inputs.get("action_mask") is not None:
        x = x * np.asarray(inputs["action_mask"], np.float64)
    return x


def flow_interp(actions, noise, t):
    """Noisy trajectory of flow-matching training [MODEL Flow matching diffusion, Training;
    ARCH Training objective]: x_t = (1 - t) * noise + t * action, t [B] broadcast over (H, A)."""
    t = np.asarray(t, np.float64)[:, None, None]
    return (1.0 - t) * np.asarray(noise, np.float64) + t * np.asarray(actions, np.float64)


def discretize_t(t, buckets: int = 1000) -> np.ndarray:
    """Training timestep bucket floor(t * buckets) per sample (the inference grid's
    discretisation applied to a continuous t), decided in float32."""
    t32 = np.asarray(t, np.float32)
    return np.floor(t32 * np.float32(buckets)).astype(np.int64)


def training_loss(cfg, weights, inputs, actions, noise, t, params=None):
    """Flow-matching training forward and loss [MODEL Flow matching diffusion, Training;
    ARCH Training objective]. The draws are inputs: t [B] (t ~ Beta(1.5, 1) on the pages)
    and noise [B,H,A] (N(0,1)).

    x_t = (1 - t) noise + t action; target velocity v = action - noise; v_pred = the head's
    velocity at x_t and the sample's bucket floor(t * buckets) (samples are independent, so
    each runs with its own timestep); loss = sum(mask (v_pred - v)^2) / (sum(mask) + 1e-6)
    with mask = action_mask (ones if absent). Returns (loss, v_pred)."""
    P = params if params is not None else effective_params(cfg, weights)
    vl_raw = effective_vl(cfg, inputs["vl_features"])
    B, L, _ = vl_raw.shape
    vl = layer_norm(vl_raw, P["vlln.gamma"], P["vlln.beta"])
    valid = (np.ones((B, L), bool) if inputs.get("vl_mask") is None
             else np.asarray(inputs["vl_mask"]).astype(bool))
    image = (None if inputs.get("image_mask") is None
             else np.asarray(inputs["image_mask"]).astype(bool))
    ids = np.asarray(inputs["embodiment_id"]).astype(np.int64)
    s = state_encoder(P, np.asarray(inputs["state"], np.float64), ids)
    x_t = flow_interp(actions, noise, t)
    v = np.asarray(actions, np.float64) - np.asarray(noise, np.float64)
    tau = discretize_t(t, cfg["num_timestep_buckets"])
    v_pred = np.concatenate([
        velocity(P, cfg, vl[b:b + 1], valid[b:b + 1], None if image is None else image[b:b + 1],
                 s[b:b + 1], x_t[b:b + 1], int(tau[b]), ids[b:b + 1]) for b in range(B)], axis=0)
    mask = (np.ones_like(v) if inputs.get("action_mask") is None
            else np.asarray(inputs["action_mask"], np.float64))
    loss = float(np.sum(mask * (v_pred - v) ** 2) / (np.sum(mask) + 1e-6))
    return loss, v_pred


def state_features(cfg, weights, inputs, params=None):
    """The encoded state token [B,1,D] (an optional get_action output)."""
    P = params if params is not None else effective_params(cfg, weights)
    ids = np.asarray(inputs["embodiment_id"]).astype(np.int64)
    return state_encoder(P, np.asarray(inputs["state"], np.float64), ids)


def rel_l2(y, y_ref) -> float:
    """||y - y_ref||_2 / ||y_ref||_2 over all entries, in float64."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    den = np.linalg.norm(y_ref.ravel())
    return float(np.linalg.norm((y - y_ref).ravel()) / (den if den > 0 else 1.0))
