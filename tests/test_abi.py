"""C-ABI checks that need no GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments before any device work (gr00t_create and
gr00t_load_weights touch no device; the other entry points validate first)."""
import ctypes
import os
import re
from dataclasses import replace

import numpy as np
import pytest

from flow_matching_dit_amd import head as H
from flow_matching_dit_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _cfg(**kw):
    return replace(synth.TINY, **kw)


def _header_functions():
    src = open(os.path.join(ROOT, "include", "gr00t_head.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gr00t_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = H.load_library()
    declared = _header_functions()
    assert set(declared) == set(H.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_struct_layouts_match_header():
    # gr00t_config: 16 int32 + 2 enums + uint32 flags + uint64 seed (8-aligned)
    assert ctypes.sizeof(H.Gr00tConfig) == 16 * 4 + 2 * 4 + 4 + 4 + 8
    assert H.Gr00tConfig.noise_seed.offset == 80
    # gr00t_inputs: two int32 then eight pointers
    assert ctypes.sizeof(H.Gr00tInputs) == 8 + 8 * 8


@pytest.mark.parametrize("kw,frag", [
    (dict(hidden=250), "hidden must equal"),
    (dict(head_dim=80, hidden=320, num_heads=4), "head_dim"),
    (dict(num_steps=0), "num_steps"),
    (dict(action_horizon=65), "action_horizon"),
    (dict(precision="bf16"), None),
])
def test_create_validates_config(kw, frag):
    if frag is None:
        h = H.Gr00tHead(_cfg(**kw), max_batch=2, max_vl_len=8)
        h.close()
        return
    with pytest.raises(H.Gr00tError) as e:
        H.Gr00tHead(_cfg(**kw), max_batch=2, max_vl_len=8)
    assert e.value.status == "E_INVALID_ARG" and frag in str(e.value)


def test_create_rejects_mixed_precisions_and_capacity():
    lib = H.load_library()
    c = H.make_config(synth.TINY, 1, 8)
    c.act_dtype = H.BF16
    out = ctypes.c_void_p()
    assert lib.gr00t_create(ctypes.byref(c), 0, ctypes.byref(out)) == -1
    assert b"F32 weights" in lib.gr00t_last_error(None)
    assert out.value is None
    c = H.make_config(synth.TINY, 0, 8)
    assert lib.gr00t_create(ctypes.byref(c), 0, ctypes.byref(out)) == -1
    assert lib.gr00t_create(None, 0, ctypes.byref(out)) == -1


def test_create_w8a8_flag_needs_fp8_weights():
    lib = H.load_library()
    out = ctypes.c_void_p()
    c = H.make_config(_cfg(precision="bf16"), 1, 8, flags=H.FLAG_W8A8)
    assert lib.gr00t_create(ctypes.byref(c), 0, ctypes.byref(out)) == -1
    assert b"W8A8 needs FP8_E4M3" in lib.gr00t_last_error(None)
    assert out.value is None
    c = H.make_config(_cfg(precision="fp8a8"), 1, 8)
    assert c.flags & H.FLAG_W8A8 and c.weight_dtype == H.FP8_E4M3
    h = H.Gr00tHead(_cfg(precision="fp8a8"), max_batch=2, max_vl_len=8)
    h.close()


def test_load_weights_errors():
    w = synth.WORKLOADS["tiny_fp32_b1"]
    h = H.Gr00tHead(w.cfg, max_batch=1, max_vl_len=32)
    with pytest.raises(H.Gr00tError) as e:
        h.load_weight("blocks.9.attn.wq", np.zeros((256, 256), np.float32))
    assert e.value.status == "E_UNKNOWN_WEIGHT"
    with pytest.raises(H.Gr00tError) as e:
        h.load_weight("blocks.0.attn.wk", np.zeros((256, 256), np.float32))  # cross block: [2048, 256]
    assert e.value.status == "E_SHAPE" and "[2048,256]" in str(e.value)
    with pytest.raises(H.Gr00tError) as e:
        h.load_weight("time.w1", np.zeros((256, 256), np.uint16), dtype=H.BF16)  # fp32 handle
    assert e.value.status == "E_INVALID_ARG"
    with pytest.raises(H.Gr00tError) as e:
        h.load_weight("vlln.gamma", np.zeros((2048,), np.float32), dtype=7)
    assert e.value.status == "E_INVALID_ARG"
    h.close()


def test_finalize_reports_missing_weight_without_device():
    w = synth.WORKLOADS["tiny_fp32_b1"]
    h = H.Gr00tHead(w.cfg, max_batch=1, max_vl_len=32)
    weights = synth.make_weights(w)
    for name in list(weights)[:-1]:
        h.load_weight(name, weights[name])
    with pytest.raises(H.Gr00tError) as e:
        h.finalize()
    assert e.value.status == "E_MISSING_WEIGHT" and "action_dec.b2" in str(e.value)
    h.close()


def test_fp8_matrices_refuse_raw_bf16():
    cfg = _cfg(precision="fp8")
    h = H.Gr00tHead(cfg, max_batch=1, max_vl_len=8)
    with pytest.raises(H.Gr00tError) as e:
        h.load_weight("blocks.1.attn.wq", np.zeros((256, 256), np.uint16), dtype=H.BF16)
    assert e.value.status == "E_INVALID_ARG"
    h.load_weight("blocks.1.ada.w", np.zeros((256, 512), np.uint16), dtype=H.BF16)  # bf16 matrix: accepted
    h.close()


def _fake_inputs(B, L):
    p = ctypes.c_void_p(0x1000)
    return H.Gr00tInputs(B, L, p, None, None, p, p, None, None, None)


def test_get_action_validates_before_device_work():
    lib = H.load_library()
    h = H.Gr00tHead(synth.TINY, max_batch=2, max_vl_len=32)
    out = ctypes.c_void_p(0x2000)
    cases = [(_fake_inputs(3, 8), -2, b"batch 3"), (_fake_inputs(1, 33), -2, b"vl_len 33"),
             (_fake_inputs(0, 8), -2, b"batch 0"), (_fake_inputs(1, 8), -4, b"not finalized")]
    for inp, code, msg in cases:
        assert lib.gr00t_get_action(h.h, ctypes.byref(inp), out, None) == code
        assert msg in lib.gr00t_last_error(h.h)
    bad = _fake_inputs(1, 8)
    bad.state = None
    assert lib.gr00t_get_action(h.h, ctypes.byref(bad), out, None) == -1
    assert lib.gr00t_get_action(h.h, None, out, None) == -1
    assert lib.gr00t_get_action(h.h, ctypes.byref(_fake_inputs(1, 8)), None, None) == -1
    assert lib.gr00t_get_action(None, ctypes.byref(_fake_inputs(1, 8)), out, None) == -1
    nz = _fake_inputs(1, 8)
    assert lib.gr00t_velocity(h.h, ctypes.byref(nz), 0, out, None) == -4
    assert lib.gr00t_prepare(h.h, 1, 8) == -4
    assert lib.gr00t_device_bytes(h.h) == 0
    h.close()


def test_reuse_vl_validates_before_device_work():
    lib = H.load_library()
    h = H.Gr00tHead(synth.TINY, max_batch=2, max_vl_len=32)
    out = ctypes.c_void_p(0x2000)
    novl = _fake_inputs(1, 8)
    novl.vl_features = None
    assert lib.gr00t_get_action(h.h, ctypes.byref(novl), out, None) == -1  # a full call reads the VL input
    assert lib.gr00t_get_action_reuse_vl(h.h, ctypes.byref(novl), out, None) == -4  # ... a reuse call does not
    assert b"not finalized" in lib.gr00t_last_error(h.h)
    assert lib.gr00t_get_action_reuse_vl(h.h, ctypes.byref(_fake_inputs(3, 8)), out, None) == -2
    assert lib.gr00t_get_action_reuse_vl(h.h, ctypes.byref(_fake_inputs(1, 8)), None, None) == -1
    assert lib.gr00t_get_action_reuse_vl(None, ctypes.byref(_fake_inputs(1, 8)), out, None) == -1
    h.close()


def test_train_forward_validates_before_device_work():
    lib = H.load_library()
    h = H.Gr00tHead(synth.TINY, max_batch=2, max_vl_len=32)
    loss = ctypes.c_void_p(0x2000)
    act, t = ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000)
    inp = _fake_inputs(1, 8)
    assert lib.gr00t_train_forward(h.h, ctypes.byref(inp), act, t, None, None, None) == -1  # no loss output
    assert lib.gr00t_train_forward(h.h, ctypes.byref(inp), None, t, loss, None, None) == -4  # not finalized first
    assert lib.gr00t_train_forward(h.h, ctypes.byref(_fake_inputs(3, 8)), act, t, loss, None, None) == -2
    assert lib.gr00t_train_forward(None, ctypes.byref(inp), act, t, loss, None, None) == -1
    h.close()


def test_quantize_validates_before_device_work():
    lib = H.load_library()
    h = H.Gr00tHead(synth.TINY, max_batch=1, max_vl_len=8)
    x, q, sc = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    cases = [((None, 16, 2, 16, q, sc), b"NULL"), ((x, 16, 2, 16, q, None), b"NULL"),
             ((ctypes.c_void_p(0x1008), 16, 2, 16, q, sc), b"aligned"),
             ((x, 16, 2, 16, ctypes.c_void_p(0x2004), sc), b"aligned"),
             ((x, 16, -1, 16, q, sc), b"rows >= 0"), ((x, 16, 2, 12, q, sc), b"multiple of 8"),
             ((x, 16, 2, 0, q, sc), b"multiple of 8"), ((x, 8, 2, 16, q, sc), b"ld_x"),
             ((x, 20, 2, 16, q, sc), b"ld_x")]
    for args, msg in cases:
        assert lib.gr00t_quantize_e4m3_rows(h.h, *args, None) == -1
        assert msg in lib.gr00t_last_error(h.h)
    assert lib.gr00t_quantize_e4m3_rows(h.h, x, 16, 0, 16, q, sc, None) == 0  # no rows: no device work
    assert lib.gr00t_quantize_e4m3_rows(None, x, 16, 1, 16, q, sc, None) == -1
    h.close()


def test_destroy_null_and_last_error_null():
    lib = H.load_library()
    lib.gr00t_destroy(None)
    assert isinstance(lib.gr00t_last_error(None), bytes)


def test_canonical_weight_names_are_accepted():
    w = synth.small_variant(synth.WORKLOADS["dit32_bf16_b64"], num_layers=3)
    h = H.Gr00tHead(w.cfg, max_batch=2, max_vl_len=16)
    for name, shape in synth.weight_shapes(w.cfg).items():
        h.load_weight(name, np.zeros(shape, np.float32))
    h.close()


def test_binding_checks_dtype_shape_and_device_before_the_call():
    """The binding refuses tensors the library would misread: an int64 id tensor (read as int32
    it would give every sample after the first the wrong category), a vl_features of the wrong
    width or dtype, short buffers, and host tensors. No library call is made (this runs on the
    CPU, with a handle that was never finalised)."""
    import torch
    w = synth.WORKLOADS["tiny_fp32_b1"]
    h = H.Gr00tHead(w.cfg, max_batch=2, max_vl_len=w.vl_len)
    try:
        B, L, c = 2, w.vl_len, w.cfg
        ok = dict(vl_features=torch.zeros(B, L, c.vl_dim), vl_mask=None, image_mask=None,
                  state=torch.zeros(B, 1, c.state_dim), embodiment_id=torch.zeros(B, dtype=torch.int32),
                  noise=torch.zeros(B, c.action_horizon, c.action_dim))
        bad_cases = [
            (dict(embodiment_id=torch.zeros(B, dtype=torch.int64)), "embodiment_id has dtype torch.int64"),
            (dict(vl_features=torch.zeros(B, L, c.vl_dim - 16)), "vl_features has shape"),
            (dict(vl_features=torch.zeros(B, L, c.vl_dim, dtype=torch.bfloat16)), "vl_features has dtype"),
            (dict(state=torch.zeros(B, c.state_dim)), "state has shape"),
            (dict(noise=torch.zeros(B, c.action_horizon, c.action_dim - 1)), "noise has shape"),
            (dict(vl_mask=torch.zeros(B, L - 1, dtype=torch.uint8)), "vl_mask has shape"),
            (dict(embodiment_id=torch.zeros(B + 1, dtype=torch.int32)), "embodiment_id has shape"),
            ({}, "is on cpu"),
        ]
        for change, frag in bad_cases:
            with pytest.raises(ValueError) as e:
                h.get_action(**{**ok, **change})
            assert frag in str(e.value), (change.keys(), str(e.value))
        with pytest.raises(ValueError, match="t has shape"):
            h.train_forward(ok["vl_features"], None, None, ok["state"], ok["embodiment_id"],
                            torch.zeros(B, c.action_horizon, c.action_dim), torch.zeros(B + 1), ok["noise"])
        with pytest.raises(ValueError, match="noise is required"):
            h.velocity(ok["vl_features"], None, None, ok["state"], ok["embodiment_id"], None, step_k=0)
        with pytest.raises(ValueError, match="state has dtype"):
            h.get_action_reuse_vl(B, L, ok["state"].double(), ok["embodiment_id"])
    finally:
        h.close()


@pytest.mark.parametrize("mb,ml,frag", [
    (1024, 1024, "VL features"),            # 1024 * 1024 * 2048 * 2 bytes
    (64, 1 << 20, "VL features"),
    (1 << 17, 300, "VL features"),
])
def test_create_refuses_capacities_past_32_bit_buffer_ranges(mb, ml, frag):
    """Every GEMM operand, cache layer and workspace buffer is addressed through 32-bit buffer
    descriptors: a capacity that would need a larger one is refused at create, not computed wrongly."""
    cfg = synth.WORKLOADS["dit32_bf16_b64"].cfg
    with pytest.raises(H.Gr00tError) as e:
        H.Gr00tHead(cfg, max_batch=mb, max_vl_len=ml)
    assert e.value.status == "E_INVALID_ARG" and "capacity too large" in str(e.value) and frag in str(e.value)
    # the largest benchmarked capacity is accepted
    H.Gr00tHead(cfg, max_batch=256, max_vl_len=1024).close()


def test_create_refuses_oversized_mlp_width():
    cfg = replace(synth.WORKLOADS["dit32_bf16_b64"].cfg, ff_dim=1 << 20)
    with pytest.raises(H.Gr00tError, match="one MLP weight matrix"):
        H.Gr00tHead(cfg, max_batch=1, max_vl_len=8)


def test_create_accepts_every_declared_flag_and_refuses_others():
    """Every GR00T_FLAG_* the header declares is accepted at create (W8A8 with e4m3 weights);
    a bit it does not declare is refused."""
    src = open(os.path.join(ROOT, "include", "gr00t_head.h")).read()
    flags = {m.group(1): int(m.group(2), 16) for m in re.finditer(r"#define GR00T_FLAG_(\w+) (0x[0-9a-fA-F]+)u", src)}
    assert {"STRICT", "USE_GRAPH", "W8A8", "PERSIST", "NO_BUCKETS"} <= set(flags)
    lib = H.load_library()
    for name, bit in flags.items():
        assert getattr(H, "FLAG_" + name) == bit
        c = H.make_config(_cfg(precision="fp8a8" if name == "W8A8" else "bf16"), 1, 8, flags=bit)
        out = ctypes.c_void_p()
        assert lib.gr00t_create(ctypes.byref(c), 0, ctypes.byref(out)) == 0, (name, lib.gr00t_last_error(None))
        lib.gr00t_destroy(out)
    undeclared = 1
    while undeclared in flags.values():
        undeclared <<= 1
    c = H.make_config(_cfg(precision="bf16"), 1, 8, flags=undeclared)
    out = ctypes.c_void_p()
    assert lib.gr00t_create(ctypes.byref(c), 0, ctypes.byref(out)) == -1
    assert b"unknown flag bits" in lib.gr00t_last_error(None)
