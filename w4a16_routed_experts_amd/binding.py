"""ctypes binding of the C ABI declared in include/moe_w4a16.h.

Functions carry the C names and arguments.  Tensor arguments are torch tensors
on the current HIP device (or None where the C argument is nullable); the
binding passes their data pointers and the current torch stream, nothing else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

from .build import LIB_PATH

PATH_AUTO, PATH_DECODE, PATH_CHUNK = 0, 1, 2
DEBUG_WAIT_GIVE_UP = 0x100  # dims.flags test hook: the few-token path's bounded waits give up at once
GIVE_UP_WORD_OFFSET = 1024  # byte offset in the workspace of the give-up counter

_STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_ALIGN",
           -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_LAUNCH", -6: "MOE_ERR_DEVICE", -7: "MOE_ERR_SCRATCH"}

# size of the static scratch array behind moe_forward_noalloc (MOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 8 << 20

WEIGHT_FIELDS = ("router_q", "router_s", "w13_q", "w13_s", "w2_q", "w2_s",
                 "sh13_q", "sh13_s", "sh2_q", "sh2_s", "w13_b", "w2_b")
FMT_AFFINE4 = 0x200  # dims.flags: affine int4 routed experts (unsigned codes, per-group scale and offset)
NORM_GAIN_PLUS_ONE = 0x400  # dims.flags: the norm gain holds w of a (1 + w) multiplier


class MoeDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("expert_inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32), ("group", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in WEIGHT_FIELDS]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({moe_status_string(status)})")


_lib = None


def library_path() -> str:
    return os.environ.get("MOE_W4A16_LIB", LIB_PATH)


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with w4a16_routed_experts_amd.build.build()")
        L = ctypes.CDLL(path)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        dims_p, w_p = ctypes.POINTER(MoeDims), ctypes.POINTER(MoeWeights)
        L.moe_workspace_bytes.argtypes = [dims_p, i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_route.argtypes = [dims_p, w_p, vp, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_route.restype = ctypes.c_int
        L.moe_experts_w4a16.argtypes = [dims_p, w_p, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_experts_w4a16.restype = ctypes.c_int
        L.moe_forward.argtypes = [dims_p, w_p, vp, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_forward.restype = ctypes.c_int
        if hasattr(L, "moe_forward_noalloc"):
            L.moe_forward_noalloc.argtypes = [dims_p, w_p, vp, i32, vp, vp, vp, vp, vp]
            L.moe_forward_noalloc.restype = ctypes.c_int
        if hasattr(L, "moe_block_forward"):  # a library without it raises when it is called
            L.moe_block_forward.argtypes = [dims_p, w_p, vp, vp, ctypes.c_float, i32, vp, vp, vp, vp, vp, sz, vp]
            L.moe_block_forward.restype = ctypes.c_int
        if hasattr(L, "moe_layers_forward"):
            L.moe_layers_workspace_bytes.argtypes = [dims_p, i32, i32]
            L.moe_layers_workspace_bytes.restype = sz
            L.moe_layers_forward.argtypes = [dims_p, w_p, vp, ctypes.c_int64, i32, ctypes.c_float, vp, i32, vp, vp,
                                             sz, vp]
            L.moe_layers_forward.restype = ctypes.c_int
        _lib = L
    return _lib


# ------------------------------------------------------------------ helpers


def make_dims(H, E, k, I, Is, G=64, flags=PATH_AUTO) -> MoeDims:
    return MoeDims(H, E, k, I, Is, G, flags)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _nbytes(ws) -> int:
    if ws is None:
        return 0
    return ws.numel() * ws.element_size()


def moe_workspace_bytes(dims: MoeDims, T: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(dims), T))


def moe_status_string(status: int) -> str:
    try:
        return lib().moe_status_string(status).decode()
    except Exception:  # the library may be the thing that is missing
        return _STATUS.get(status, "unknown")


def workspace(dims: MoeDims, T: int, device="cuda"):
    """A zero-filled workspace of the required size (uint8 tensor)."""
    import torch
    return torch.zeros(max(256, moe_workspace_bytes(dims, T)), dtype=torch.uint8, device=device)


def _check(status: int, where: str, raise_on_error: bool) -> int:
    if status != 0 and raise_on_error:
        raise MoeError(status, where)
    return status


def moe_route(dims, weights, x, T, ids, w, shared_gate=None, logits=None, ws=None, stream=None,
              raise_on_error=True) -> int:
    st = lib().moe_route(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), T, _ptr(ids), _ptr(w),
                         _ptr(shared_gate), _ptr(logits), _ptr(ws), _nbytes(ws), _stream(stream))
    return _check(st, "moe_route", raise_on_error)


def moe_experts_w4a16(dims, weights, x, T, ids, w, out, ws=None, stream=None, raise_on_error=True) -> int:
    st = lib().moe_experts_w4a16(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), T, _ptr(ids), _ptr(w),
                                 _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream))
    return _check(st, "moe_experts_w4a16", raise_on_error)


def moe_forward(dims, weights, x, T, out, ids=None, w=None, shared_gate=None, ws=None, stream=None,
                raise_on_error=True) -> int:
    st = lib().moe_forward(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), T, _ptr(out), _ptr(ids), _ptr(w),
                           _ptr(shared_gate), _ptr(ws), _nbytes(ws), _stream(stream))
    return _check(st, "moe_forward", raise_on_error)


def moe_forward_noalloc(dims, weights, x, T, out, ids=None, w=None, shared_gate=None, stream=None,
                        raise_on_error=True) -> int:
    st = lib().moe_forward_noalloc(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), T, _ptr(out), _ptr(ids),
                                   _ptr(w), _ptr(shared_gate), _stream(stream))
    return _check(st, "moe_forward_noalloc", raise_on_error)


def moe_block_forward(dims, weights, h, gain, eps, T, out, ids=None, w=None, shared_gate=None, ws=None, stream=None,
                      raise_on_error=True) -> int:
    st = lib().moe_block_forward(ctypes.byref(dims), ctypes.byref(weights), _ptr(h), _ptr(gain), float(eps), T,
                                 _ptr(out), _ptr(ids), _ptr(w), _ptr(shared_gate), _ptr(ws), _nbytes(ws),
                                 _stream(stream))
    return _check(st, "moe_block_forward", raise_on_error)


def moe_layers_workspace_bytes(dims: MoeDims, T: int, L: int) -> int:
    return int(lib().moe_layers_workspace_bytes(ctypes.byref(dims), T, L))


def layers_workspace(dims: MoeDims, T: int, L: int, device="cuda"):
    """A zero-filled workspace for moe_layers_forward (uint8 tensor)."""
    import torch
    return torch.zeros(max(256, moe_layers_workspace_bytes(dims, T, L)), dtype=torch.uint8, device=device)


def moe_layers_forward(dims, weights, gain, layer_stride, L, eps, h, T, out, ws=None, stream=None,
                       raise_on_error=True) -> int:
    st = lib().moe_layers_forward(ctypes.byref(dims), ctypes.byref(weights), _ptr(gain), int(layer_stride), L,
                                  float(eps), _ptr(h), T, _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream))
    return _check(st, "moe_layers_forward", raise_on_error)


class LayerStack:
    """L layers' weights and norm gains in one device buffer, every array of
    layer l at the same offset inside layer l's region and the regions a fixed
    stride apart: the layout moe_layers_forward reads.  `struct` and `gain`
    point into layer 0; `stride` is the region size in bytes."""

    def __init__(self, host_weights, gains, device="cuda"):
        import numpy as np
        import torch
        fields = [f for f in WEIGHT_FIELDS if getattr(host_weights[0], f, None) is not None]
        offs, o = {}, 0
        for f in fields + ["gain"]:
            a = gains[0] if f == "gain" else getattr(host_weights[0], f)
            offs[f] = o
            o = (o + a.nbytes + 255) // 256 * 256
        self.stride = o
        host = np.zeros((len(host_weights), o), dtype=np.uint8)
        for l, (W, g) in enumerate(zip(host_weights, gains)):
            for f in fields + ["gain"]:
                a = np.ascontiguousarray(g if f == "gain" else getattr(W, f))
                host[l, offs[f]:offs[f] + a.nbytes] = a.reshape(-1).view(np.uint8)
        self.buffer = torch.from_numpy(host).to(device)
        base = self.buffer.data_ptr()
        self.struct = MoeWeights(*[base + offs[f] if f in offs else None for f in WEIGHT_FIELDS])
        self.gain = base + offs["gain"]
        self.L = len(host_weights)


class DeviceWeights:
    """Device copies (torch tensors) of one layer's weights and the C struct over them."""

    def __init__(self, host_weights=None, device="cuda", tensors=None):
        import torch
        if tensors is None:
            tensors = {}
            for f in WEIGHT_FIELDS:
                a = getattr(host_weights, f, None)
                if a is not None:
                    tensors[f] = torch.from_numpy(a.view(_TORCH_VIEW[a.dtype.str])).to(device)
        self.tensors = tensors
        self.struct = MoeWeights(*[tensors[f].data_ptr() if tensors.get(f) is not None else None
                                   for f in WEIGHT_FIELDS])

    def clone(self) -> "DeviceWeights":
        return DeviceWeights(tensors={f: t.clone() for f, t in self.tensors.items()})

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.tensors.values())


# numpy dtype -> dtype torch can wrap without copying (uint16 bit patterns as int16)
_TORCH_VIEW = {"|i1": "int8", "|u1": "uint8", "<u2": "int16", "<i2": "int16"}
