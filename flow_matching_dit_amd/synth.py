"""Seeded synthetic workloads for the GR00T flow-matching DiT action head.

This module only draws random numbers and shapes them. It holds none of the
head's arithmetic: no rounding, no quantisation, no layer math. Both the CPU
oracle's tests and the HIP path's tests, and the benchmark, take their inputs
from here, so the two implementations see the same arrays.

Workload shapes follow the pages:
  * "Model architecture" (GR00T N1.6), section "Action head architecture" and
    "Model configuration": VL features [B, seq, 2048], state, embodiment ids,
    action horizon and action dim.
  * "GR00T model class", section "get_action": action_pred (B, horizon, dim).
  * "Single-GPU inference for GR00T-N1.7", step "Prepare a request": noise is
    an optional input used for deterministic regression checks.

Random streams: NumPy PCG64 seeded with SeedSequence([seed, workload_id,
tensor_index]); weights use seed 0, inputs seed 1, noise seed 2. Every matrix
and bias is N(0, 0.02^2); the vision-language LayerNorm gain is 1 + N(0, 0.02^2).
"""
from __future__ import annotations

from collections import OrderedDict
from concurrent.futures import ThreadPoolExecutor
from dataclasses import asdict, dataclass, replace
from typing import Dict, Optional

import numpy as np

WEIGHT_SEED = 0
INPUT_SEED = 1
NOISE_SEED = 2


@dataclass(frozen=True)
class HeadConfig:
    """Hyper-parameters of the action head (names follow the pages' config)."""

    num_layers: int
    hidden: int            # D = num_heads * head_dim (inner dim, embedding dim)
    num_heads: int
    head_dim: int
    ff_dim: int            # F, width of the GELU MLP
    state_dim: int
    action_dim: int
    action_horizon: int    # H
    num_categories: int    # C, embodiment tables
    num_steps: int         # K Euler steps
    vl_dim: int = 2048     # backbone_embedding_dim
    num_timestep_buckets: int = 1000
    attend_text_every_n_blocks: int = 2
    time_freq_dim: int = 256
    precision: str = "bf16"  # "fp32" | "bf16" | "fp8" (e4m3 DiT matrices) | "fp8a8" (and e4m3 inputs)

    def as_dict(self) -> dict:
        return asdict(self)


@dataclass(frozen=True)
class Workload:
    """One synthetic get_action workload: a model plus a batch recipe."""

    name: str
    wid: int               # workload id, part of every seed
    cfg: HeadConfig
    batch: int
    vl_len: int            # L_pad
    len_range: Optional[tuple] = None     # (lo, hi) inclusive valid lengths; None = all valid
    image_tokens: Optional[int] = None    # first n positions are image tokens (text after)
    id_range: tuple = (0, 0)              # embodiment ids drawn from U{lo..hi}
    fixed_id: Optional[int] = None
    mask_tail_range: Optional[tuple] = None  # action_mask zeroes a tail of U{lo..hi} dims


def _full_model(**kw) -> HeadConfig:
    base = dict(num_layers=32, hidden=1536, num_heads=32, head_dim=48, ff_dim=6144,
                state_dim=64, action_dim=32, action_horizon=16, num_categories=32,
                num_steps=4, precision="bf16")
    base.update(kw)
    return HeadConfig(**base)


TINY = HeadConfig(num_layers=2, hidden=256, num_heads=4, head_dim=64, ff_dim=1024,
                  state_dim=64, action_dim=32, action_horizon=16, num_categories=2,
                  num_steps=4, precision="fp32")

WORKLOADS: Dict[str, Workload] = OrderedDict()
WORKLOADS["tiny_fp32_b1"] = Workload("tiny_fp32_b1", 0, TINY, batch=1, vl_len=32, fixed_id=1)
WORKLOADS["dit32_bf16_b1"] = Workload("dit32_bf16_b1", 1, _full_model(), batch=1, vl_len=300,
                                      image_tokens=256, id_range=(0, 31))
WORKLOADS["dit32_bf16_b64"] = Workload("dit32_bf16_b64", 2, _full_model(), batch=64, vl_len=400,
                                       len_range=(200, 400), id_range=(0, 31),
                                       mask_tail_range=(0, 25))
WORKLOADS["dit32_bf16_b16_h64"] = Workload("dit32_bf16_b16_h64", 3,
                                           _full_model(action_horizon=64, num_steps=8),
                                           batch=16, vl_len=1024, id_range=(0, 7))
WORKLOADS["dit32_fp8_b256"] = Workload("dit32_fp8_b256", 4, _full_model(precision="fp8"),
                                       batch=256, vl_len=300, id_range=(0, 31))
# W8A8 variant of the high-batch workload: e4m3 DiT weights and per-row e4m3 GEMM inputs
WORKLOADS["dit32_w8a8_b256"] = Workload("dit32_w8a8_b256", 5, _full_model(precision="fp8a8"),
                                        batch=256, vl_len=300, id_range=(0, 31))
WORKLOAD_BY_INDEX = list(WORKLOADS.values())


def small_variant(w: Workload, *, num_layers: int = 2, hidden: int = 192, num_heads: int = 4,
                  head_dim: int = 48, ff_dim: int = 768, batch: Optional[int] = None,
                  num_categories: Optional[int] = None, wid_offset: int = 100) -> Workload:
    """Same recipe as ``w`` at a reduced width/depth, for parity at oracle-friendly sizes."""
    cfg = replace(w.cfg, num_layers=num_layers, hidden=hidden, num_heads=num_heads,
                  head_dim=head_dim, ff_dim=ff_dim,
                  num_categories=num_categories or w.cfg.num_categories)
    return replace(w, name=w.name + "_small", wid=w.wid + wid_offset, cfg=cfg,
                   batch=batch if batch is not None else w.batch)


def _rng(seed: int, wid: int, idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wid, idx])))


def weight_shapes(cfg: HeadConfig) -> "OrderedDict[str, tuple]":
    """Canonical parameter names and shapes, in generation order.

    Every linear is stored as [in, out] (x @ W), the layout of the per-embodiment
    linear on the "Model architecture" page (section "CategorySpecificLinear").
    Per-embodiment tables carry a leading category axis C.
    """
    D, F, C = cfg.hidden, cfg.ff_dim, cfg.num_categories
    s = OrderedDict()
    s["vlln.gamma"] = (cfg.vl_dim,)
    s["vlln.beta"] = (cfg.vl_dim,)
    s["time.w1"] = (cfg.time_freq_dim, D)
    s["time.b1"] = (D,)
    s["time.w2"] = (D, D)
    s["time.b2"] = (D,)
    s["state_enc.w1"] = (C, cfg.state_dim, D)
    s["state_enc.b1"] = (C, D)
    s["state_enc.w2"] = (C, D, D)
    s["state_enc.b2"] = (C, D)
    s["action_enc.w1"] = (C, cfg.action_dim, D)
    s["action_enc.b1"] = (C, D)
    s["action_enc.w2"] = (C, 2 * D, D)
    s["action_enc.b2"] = (C, D)
    s["action_enc.w3"] = (C, D, D)
    s["action_enc.b3"] = (C, D)
    for l in range(cfg.num_layers):
        din = cfg.vl_dim if l % 2 == 0 else D
        p = f"blocks.{l}."
        s[p + "ada.w"] = (D, 2 * D)
        s[p + "ada.b"] = (2 * D,)
        s[p + "attn.wq"] = (D, D)
        s[p + "attn.bq"] = (D,)
        s[p + "attn.wk"] = (din, D)
        s[p + "attn.bk"] = (D,)
        s[p + "attn.wv"] = (din, D)
        s[p + "attn.bv"] = (D,)
        s[p + "attn.wo"] = (D, D)
        s[p + "attn.bo"] = (D,)
        s[p + "ff.w1"] = (D, F)
        s[p + "ff.b1"] = (F,)
        s[p + "ff.w2"] = (F, D)
        s[p + "ff.b2"] = (D,)
    s["out.ada.w"] = (D, 2 * D)
    s["out.ada.b"] = (2 * D,)
    s["out.proj.w"] = (D, D)
    s["out.proj.b"] = (D,)
    s["action_dec.w1"] = (C, D, D)
    s["action_dec.b1"] = (C, D)
    s["action_dec.w2"] = (C, D, cfg.action_dim)
    s["action_dec.b2"] = (C, cfg.action_dim)
    return s


def make_weights(w: Workload, seed: int = WEIGHT_SEED, threads: int = 8) -> "OrderedDict[str, np.ndarray]":
    """fp32 master weights, N(0, 0.02^2) each; LayerNorm gain 1 + N(0, 0.02^2).

    Each tensor has its own stream, so drawing them on several threads gives the
    same arrays as drawing them in order."""
    items = list(weight_shapes(w.cfg).items())

    def draw(idx):
        name, shape = items[idx]
        a = _rng(seed, w.wid, idx).standard_normal(shape, dtype=np.float32)
        a *= np.float32(0.02)
        if name == "vlln.gamma":
            a += np.float32(1.0)
        return a

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        arrays = list(ex.map(draw, range(len(items))))
    return OrderedDict((name, a) for (name, _), a in zip(items, arrays))


def make_inputs(w: Workload, seed: int = INPUT_SEED) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of one get_action call.

    vl_features [B, L_pad, vl_dim] f32 ~ N(0,1) (padded positions are random too);
    vl_mask [B, L_pad] u8 or None (all valid); image_mask [B, L_pad] u8 or None
    (no image/text split); state [B, 1, state_dim] f32; embodiment_id [B] i32;
    action_mask [B, H, A] u8 or None.
    """
    cfg, B, L = w.cfg, w.batch, w.vl_len
    vl = _rng(seed, w.wid, 0).standard_normal((B, L, cfg.vl_dim), dtype=np.float32)
    vl_mask = None
    if w.len_range is not None:
        lens = _rng(seed, w.wid, 1).integers(w.len_range[0], w.len_range[1] + 1, size=B)
        vl_mask = (np.arange(L)[None, :] < lens[:, None]).astype(np.uint8)
    image_mask = None
    if w.image_tokens is not None:
        image_mask = np.zeros((B, L), np.uint8)
        image_mask[:, : w.image_tokens] = 1
    state = _rng(seed, w.wid, 2).standard_normal((B, 1, cfg.state_dim), dtype=np.float32)
    if w.fixed_id is not None:
        ids = np.full((B,), w.fixed_id, np.int32)
    else:
        ids = _rng(seed, w.wid, 3).integers(w.id_range[0], w.id_range[1] + 1,
                                             size=B).astype(np.int32)
    action_mask = None
    if w.mask_tail_range is not None:
        tail = _rng(seed, w.wid, 4).integers(w.mask_tail_range[0], w.mask_tail_range[1] + 1,
                                              size=B)
        keep = cfg.action_dim - tail
        am = (np.arange(cfg.action_dim)[None, :] < keep[:, None]).astype(np.uint8)
        action_mask = np.ascontiguousarray(
            np.broadcast_to(am[:, None, :], (B, cfg.action_horizon, cfg.action_dim)))
    return dict(vl_features=vl, vl_mask=vl_mask, image_mask=image_mask, state=state,
                embodiment_id=ids, action_mask=action_mask)


def make_noise(w: Workload, seed: int = NOISE_SEED) -> np.ndarray:
    """Initial Euler state x_0 ~ N(0,1), [B, H, A] f32."""
    cfg = w.cfg
    return _rng(seed, w.wid, 0).standard_normal(
        (w.batch, cfg.action_horizon, cfg.action_dim), dtype=np.float32)


def take_samples(inputs: dict, noise: np.ndarray, idx) -> tuple:
    """Restrict a batch to the samples ``idx`` (used with batch independence)."""
    idx = np.asarray(idx)
    sub = {k: (None if v is None else np.ascontiguousarray(v[idx])) for k, v in inputs.items()}
    return sub, np.ascontiguousarray(noise[idx])
