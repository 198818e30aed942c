"""ctypes binding of libgr00t_head.so (C ABI declared in include/gr00t_head.h).

Argument marshalling only: every step of get_action runs in the HIP library.
torch supplies device memory and the current HIP stream. A missing library is an
error (there is no other implementation to fall back to).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int, c_int32, c_int64, c_size_t, c_uint32, c_uint64, c_void_p
from typing import Dict, Optional

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libgr00t_head.so")

F32, BF16, FP8_E4M3, U8, I32 = 0, 1, 2, 3, 4
FLAG_STRICT = 0x1
FLAG_USE_GRAPH = 0x2
FLAG_W8A8 = 0x4
FLAG_PERSIST = 0x8
FLAG_NO_BUCKETS = 0x10

STATUS = {
    0: "OK", -1: "E_INVALID_ARG", -2: "E_SHAPE", -3: "E_EMBODIMENT", -4: "E_NOT_FINALIZED",
    -5: "E_UNKNOWN_WEIGHT", -6: "E_UNCAPTURED", -7: "E_HIP", -8: "E_OOM", -9: "E_MISSING_WEIGHT",
    -10: "E_DEVICE_ERROR",
    -11: "E_NO_VL_CACHE",
}

# Every exported symbol of include/gr00t_head.h.
EXPORTS = ("gr00t_create", "gr00t_load_weights", "gr00t_finalize", "gr00t_prepare", "gr00t_get_action",
           "gr00t_get_action_reuse_vl", "gr00t_train_forward", "gr00t_train_forward_noalloc", "gr00t_velocity",
           "gr00t_quantize_e4m3_rows",
           "gr00t_destroy",
           "gr00t_last_error", "gr00t_device_bytes", "gr00t_profile_enable", "gr00t_profile_read",
           "gr00t_profile_class_name")


class Gr00tConfig(ctypes.Structure):
    _fields_ = [("num_layers", c_int32), ("hidden", c_int32), ("num_heads", c_int32), ("head_dim", c_int32),
                ("ff_dim", c_int32), ("vl_dim", c_int32), ("state_dim", c_int32), ("action_dim", c_int32),
                ("action_horizon", c_int32), ("num_categories", c_int32), ("num_steps", c_int32),
                ("num_timestep_buckets", c_int32), ("attend_text_every_n_blocks", c_int32),
                ("time_freq_dim", c_int32), ("max_batch", c_int32), ("max_vl_len", c_int32),
                ("weight_dtype", c_int), ("act_dtype", c_int), ("flags", c_uint32), ("noise_seed", c_uint64)]


class Gr00tInputs(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("vl_len", c_int32), ("vl_features", c_void_p), ("vl_mask", c_void_p),
                ("image_mask", c_void_p), ("state", c_void_p), ("embodiment_id", c_void_p), ("noise", c_void_p),
                ("action_mask", c_void_p), ("state_features_out", c_void_p)]


class Gr00tError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code
        self.status = STATUS.get(code, str(code))


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open the HIP library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m flow_matching_dit_amd.build`")
    # torch (device memory and streams of the callers) ships its own HIP runtime; it is loaded
    # before the library's, which otherwise initialises the device first and leaves torch's
    # runtime without a GPU
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    lib.gr00t_create.argtypes = [POINTER(Gr00tConfig), c_int, POINTER(c_void_p)]
    lib.gr00t_create.restype = c_int
    lib.gr00t_load_weights.argtypes = [c_void_p, c_char_p, c_void_p, c_int, POINTER(c_int64), c_int]
    lib.gr00t_load_weights.restype = c_int
    lib.gr00t_finalize.argtypes = [c_void_p]
    lib.gr00t_finalize.restype = c_int
    lib.gr00t_prepare.argtypes = [c_void_p, c_int32, c_int32]
    lib.gr00t_prepare.restype = c_int
    lib.gr00t_get_action.argtypes = [c_void_p, POINTER(Gr00tInputs), c_void_p, c_void_p]
    lib.gr00t_get_action.restype = c_int
    lib.gr00t_get_action_reuse_vl.argtypes = [c_void_p, POINTER(Gr00tInputs), c_void_p, c_void_p]
    lib.gr00t_get_action_reuse_vl.restype = c_int
    lib.gr00t_train_forward.argtypes = [c_void_p, POINTER(Gr00tInputs), c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p]
    lib.gr00t_train_forward_noalloc.argtypes = lib.gr00t_train_forward.argtypes
    lib.gr00t_train_forward_noalloc.restype = c_int
    lib.gr00t_train_forward.restype = c_int
    lib.gr00t_velocity.argtypes = [c_void_p, POINTER(Gr00tInputs), c_int32, c_void_p, c_void_p]
    lib.gr00t_velocity.restype = c_int
    lib.gr00t_quantize_e4m3_rows.argtypes = [c_void_p, c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p,
                                             c_void_p]
    lib.gr00t_quantize_e4m3_rows.restype = c_int
    lib.gr00t_destroy.argtypes = [c_void_p]
    lib.gr00t_destroy.restype = None
    lib.gr00t_last_error.argtypes = [c_void_p]
    lib.gr00t_last_error.restype = c_char_p
    lib.gr00t_device_bytes.argtypes = [c_void_p]
    lib.gr00t_device_bytes.restype = c_size_t
    lib.gr00t_profile_enable.argtypes = [c_void_p, c_int]
    lib.gr00t_profile_enable.restype = c_int
    lib.gr00t_profile_read.argtypes = [c_void_p, c_int, POINTER(c_int64), POINTER(ctypes.c_double)]
    lib.gr00t_profile_read.restype = c_int
    lib.gr00t_profile_class_name.argtypes = [c_int]
    lib.gr00t_profile_class_name.restype = c_char_p
    _lib = lib
    return lib


def make_config(cfg, max_batch: int, max_vl_len: int, flags: int = 0, noise_seed: int = 0) -> Gr00tConfig:
    """Gr00tConfig from a HeadConfig-like object (attributes or dict keys of the same names)."""
    get = (lambda k: cfg[k]) if isinstance(cfg, dict) else (lambda k: getattr(cfg, k))
    prec = get("precision")
    wdt = {"fp32": F32, "bf16": BF16, "fp8": FP8_E4M3, "fp8a8": FP8_E4M3}[prec]
    if prec == "fp8a8":  # W8A8: e4m3 weights and per-row e4m3 inputs of their GEMMs
        flags |= FLAG_W8A8
    return Gr00tConfig(get("num_layers"), get("hidden"), get("num_heads"), get("head_dim"), get("ff_dim"),
                       get("vl_dim"), get("state_dim"), get("action_dim"), get("action_horizon"),
                       get("num_categories"), get("num_steps"), get("num_timestep_buckets"),
                       get("attend_text_every_n_blocks"), get("time_freq_dim"), max_batch, max_vl_len,
                       wdt, F32 if prec == "fp32" else BF16, flags, noise_seed)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _expect(name, t, shape, dtypes, device, optional=False):
    """Raise ValueError unless tensor t has this shape, one of these dtypes, is contiguous and
    lives on `device` (the library reads raw pointers: a wrong dtype or a short buffer would be
    read as garbage or past its end)."""
    import torch
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the head's device is {device}")


class Gr00tHead:
    """One library handle: create -> load_weights -> finalize -> [prepare] -> get_action."""

    def __init__(self, cfg, max_batch: int, max_vl_len: int, flags: int = 0, device: int = 0,
                 noise_seed: int = 0):
        self.lib = load_library()
        self.cfg = cfg
        self._c = make_config(cfg, max_batch, max_vl_len, flags, noise_seed)
        h = c_void_p()
        rc = self.lib.gr00t_create(ctypes.byref(self._c), device, ctypes.byref(h))
        if rc != 0:
            raise Gr00tError(rc, self.lib.gr00t_last_error(None).decode())
        self.h = h
        self.device = device

    def _check(self, rc: int):
        if rc != 0:
            raise Gr00tError(rc, self.lib.gr00t_last_error(self.h).decode())

    @property
    def act_torch_dtype(self):
        import torch
        return torch.float32 if self._c.act_dtype == F32 else torch.bfloat16

    def load_weight(self, name: str, arr: np.ndarray, dtype: int = F32):
        arr = np.ascontiguousarray(arr)
        shape = (c_int64 * arr.ndim)(*arr.shape)
        self._check(self.lib.gr00t_load_weights(self.h, name.encode(), arr.ctypes.data_as(c_void_p), dtype,
                                                shape, arr.ndim))

    def load_weights(self, weights: Dict[str, np.ndarray]):
        for name, arr in weights.items():
            self.load_weight(name, np.asarray(arr, dtype=np.float32))
        return self

    def finalize(self):
        self._check(self.lib.gr00t_finalize(self.h))
        return self

    def prepare(self, batch: int, vl_len: int):
        self._check(self.lib.gr00t_prepare(self.h, batch, vl_len))
        return self

    @property
    def torch_device(self):
        import torch
        return torch.device("cuda", self.device)

    def _check_inputs(self, B, L, vl_features, vl_mask, image_mask, state, embodiment_id, noise, action_mask,
                      state_features_out=None, need_vl=True, need_noise=False):
        """Shapes, dtypes and device of one call's tensors against the handle's configuration."""
        import torch
        c = self._c
        u8 = (torch.uint8, torch.bool)
        H, A = c.action_horizon, c.action_dim
        # shapes and dtypes of every tensor first, then the device
        for dev in (None, self.torch_device):
            _expect("vl_features", vl_features, (B, L, c.vl_dim), (self.act_torch_dtype,), dev, optional=not need_vl)
            _expect("vl_mask", vl_mask, (B, L), u8, dev, optional=True)
            _expect("image_mask", image_mask, (B, L), u8, dev, optional=True)
            _expect("state", state, (B, 1, c.state_dim), (torch.float32,), dev)
            _expect("embodiment_id", embodiment_id, (B,), (torch.int32,), dev)
            _expect("noise", noise, (B, H, A), (torch.float32,), dev, optional=not need_noise)
            _expect("action_mask", action_mask, (B, H, A), u8, dev, optional=True)
            _expect("state_features_out", state_features_out, (B, 1, c.hidden), (torch.float32,), dev,
                    optional=True)

    def _inputs(self, vl_features, vl_mask, image_mask, state, embodiment_id, noise, action_mask,
                state_features_out, need_noise=False) -> Gr00tInputs:
        if getattr(vl_features, "dim", lambda: 0)() != 3:
            raise ValueError("vl_features must be a 3-D tensor [B, L, vl_dim]")
        B, L = int(vl_features.shape[0]), int(vl_features.shape[1])
        self._check_inputs(B, L, vl_features, vl_mask, image_mask, state, embodiment_id, noise, action_mask,
                           state_features_out, need_noise=need_noise)
        return Gr00tInputs(B, L, _ptr(vl_features), _ptr(vl_mask), _ptr(image_mask), _ptr(state),
                           _ptr(embodiment_id), _ptr(noise), _ptr(action_mask), _ptr(state_features_out))

    def _stream(self, stream):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        return c_void_p(s.cuda_stream)

    def get_action(self, vl_features, vl_mask, image_mask, state, embodiment_id, noise=None,
                   action_mask=None, out=None, state_features_out=None, stream=None):
        """action_pred [B, H, A] f32 on the device (enqueued on the current stream)."""
        import torch
        B = int(vl_features.shape[0])
        inp = self._inputs(vl_features, vl_mask, image_mask, state, embodiment_id, noise, action_mask,
                           state_features_out)
        if out is None:
            out = torch.empty((B, self._c.action_horizon, self._c.action_dim), dtype=torch.float32,
                              device=vl_features.device)
        for dev in (None, self.torch_device):
            _expect("out", out, (B, self._c.action_horizon, self._c.action_dim), (torch.float32,), dev)
        self._check(self.lib.gr00t_get_action(self.h, ctypes.byref(inp), c_void_p(out.data_ptr()),
                                              self._stream(stream)))
        return out

    def get_action_reuse_vl(self, batch: int, vl_len: int, state, embodiment_id, noise=None, action_mask=None,
                            out=None, state_features_out=None, stream=None):
        """get_action with the VL key/value caches of the last full call of this (batch, vl_len)."""
        import torch
        self._check_inputs(batch, vl_len, None, None, None, state, embodiment_id, noise, action_mask,
                           state_features_out, need_vl=False)
        if out is None:
            out = torch.empty((batch, self._c.action_horizon, self._c.action_dim), dtype=torch.float32,
                              device=state.device)
        _expect("out", out, (batch, self._c.action_horizon, self._c.action_dim), (torch.float32,), self.torch_device)
        inp = Gr00tInputs(batch, vl_len, None, None, None, _ptr(state), _ptr(embodiment_id), _ptr(noise),
                          _ptr(action_mask), _ptr(state_features_out))
        self._check(self.lib.gr00t_get_action_reuse_vl(self.h, ctypes.byref(inp), c_void_p(out.data_ptr()),
                                                       self._stream(stream)))
        return out

    def train_forward(self, vl_features, vl_mask, image_mask, state, embodiment_id, actions, t, noise,
                      action_mask=None, v_pred=True, stream=None):
        """(loss [1] f32, v_pred [B, H, A] f32 or None) of the flow-matching training forward."""
        import torch
        B = int(vl_features.shape[0])
        for dev in (None, self.torch_device):
            _expect("actions", actions, (B, self._c.action_horizon, self._c.action_dim), (torch.float32,), dev)
            _expect("t", t, (B,), (torch.float32,), dev)
        inp = self._inputs(vl_features, vl_mask, image_mask, state, embodiment_id, noise, action_mask, None,
                           need_noise=True)
        loss = torch.empty(1, dtype=torch.float32, device=vl_features.device)
        vp = (torch.empty((B, self._c.action_horizon, self._c.action_dim), dtype=torch.float32,
                          device=vl_features.device) if v_pred else None)
        self._check(self.lib.gr00t_train_forward(self.h, ctypes.byref(inp), _ptr(actions), _ptr(t),
                                                 c_void_p(loss.data_ptr()), _ptr(vp), self._stream(stream)))
        return loss, vp

    def train_forward_noalloc(self, vl_features, vl_mask, image_mask, state, embodiment_id, actions, t, noise,
                              loss, v_pred=None, action_mask=None, stream=None):
        """The training forward into caller-provided outputs (loss [1] f32, optional v_pred
        [B, H, A] f32, both on the handle's device) through the entry point that allocates
        nothing: its per-sample tables live in the library's fixed scratch area."""
        import torch
        B = int(vl_features.shape[0])
        for dev in (None, self.torch_device):
            _expect("actions", actions, (B, self._c.action_horizon, self._c.action_dim), (torch.float32,), dev)
            _expect("t", t, (B,), (torch.float32,), dev)
            _expect("loss", loss, (1,), (torch.float32,), dev)
            _expect("v_pred", v_pred, (B, self._c.action_horizon, self._c.action_dim), (torch.float32,), dev,
                    optional=True)
        inp = self._inputs(vl_features, vl_mask, image_mask, state, embodiment_id, noise, action_mask, None,
                           need_noise=True)
        self._check(self.lib.gr00t_train_forward_noalloc(self.h, ctypes.byref(inp), _ptr(actions), _ptr(t),
                                                         _ptr(loss), _ptr(v_pred), self._stream(stream)))
        return loss, v_pred

    def velocity(self, vl_features, vl_mask, image_mask, state, embodiment_id, noise, step_k: int,
                 stream=None):
        import torch
        inp = self._inputs(vl_features, vl_mask, image_mask, state, embodiment_id, noise, None, None,
                           need_noise=True)
        B = int(vl_features.shape[0])
        out = torch.empty((B, self._c.action_horizon, self._c.action_dim), dtype=torch.float32,
                          device=vl_features.device)
        self._check(self.lib.gr00t_velocity(self.h, ctypes.byref(inp), step_k, c_void_p(out.data_ptr()),
                                            self._stream(stream)))
        return out

    def quantize_e4m3_rows(self, x, stream=None):
        """Per-row e4m3 codes [rows, cols] uint8 and fp32 scales [rows] of a bf16 device matrix
        [rows, cols] (the W8A8 mode's quantisation of a GEMM input)."""
        import torch
        if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16 or x.dim() != 2:
            raise ValueError("x must be a 2-D bfloat16 tensor")
        _expect("x", x, tuple(x.shape), (torch.bfloat16,), self.torch_device)
        rows, cols = int(x.shape[0]), int(x.shape[1])
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        scale = torch.empty((rows,), dtype=torch.float32, device=x.device)
        self._check(self.lib.gr00t_quantize_e4m3_rows(self.h, _ptr(x), cols, rows, cols, c_void_p(q.data_ptr()),
                                                      c_void_p(scale.data_ptr()), self._stream(stream)))
        return q, scale

    def profile(self, on=True):
        """on: False/0 off, True/1 every launch (eager), 2 graph kept (launches outside it timed)."""
        self._check(self.lib.gr00t_profile_enable(self.h, int(on)))

    def profile_read(self) -> dict:
        """{class name: (launches, total ms)} of the launches recorded since profile(True)."""
        out = {}
        k = 0
        while True:
            name = self.lib.gr00t_profile_class_name(k)
            if name is None:
                break
            n, ms = c_int64(), ctypes.c_double()
            self._check(self.lib.gr00t_profile_read(self.h, k, ctypes.byref(n), ctypes.byref(ms)))
            out[name.decode()] = (int(n.value), float(ms.value))
            k += 1
        return out

    def device_bytes(self) -> int:
        return int(self.lib.gr00t_device_bytes(self.h))

    def close(self):
        if getattr(self, "h", None) is not None and self.h.value is not None:
            self.lib.gr00t_destroy(self.h)
            self.h = c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def device_inputs(inputs: dict, noise: Optional[np.ndarray], act_dtype, device="cuda:0") -> dict:
    """Move a synth.make_inputs dict (and the noise) to the device in the library's dtypes."""
    import torch
    t = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)
    vl = torch.from_numpy(np.ascontiguousarray(inputs["vl_features"])).to(device).to(act_dtype)
    return dict(vl_features=vl.contiguous(), vl_mask=t(inputs["vl_mask"], torch.uint8),
                image_mask=t(inputs["image_mask"], torch.uint8), state=t(inputs["state"], torch.float32),
                embodiment_id=t(inputs["embodiment_id"], torch.int32), noise=t(noise, torch.float32),
                action_mask=t(inputs["action_mask"], torch.uint8))
