"""The C ABI without a GPU: exported symbols, workspace sizes and refusals.

Every call made here is refused by host-side validation (or is a T = 0
no-op), so nothing reaches the device.  Pointers are fake addresses.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import w4a16_routed_experts_amd as m
from w4a16_routed_experts_amd.binding import MoeWeights, WEIGHT_FIELDS

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_w4a16.h")
REAL = dict(H=2048, E=256, k=8, I=512, Is=512)
FAKE = 1 << 20  # 1 MiB: a 256-byte aligned fake device address


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(m.library_path()):
        from w4a16_routed_experts_amd import build
        build.build()
    return m.lib()


def _dims(**kw):
    d = dict(REAL)
    d.update(kw)
    return m.make_dims(d["H"], d["E"], d["k"], d["I"], d["Is"], d.get("G", 64), d.get("flags", 0))


def _weights(addr=FAKE, **override):
    vals = {f: addr + 4096 * i for i, f in enumerate(WEIGHT_FIELDS)}
    vals.update(override)
    return MoeWeights(*[vals[f] for f in WEIGHT_FIELDS])


def test_every_declared_symbol_is_exported(L):
    text = open(HEADER).read()
    names = re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)
    assert set(names) == {"moe_workspace_bytes", "moe_route", "moe_experts_w4a16", "moe_forward", "moe_block_forward",
                          "moe_forward_noalloc", "moe_status_string", "moe_layers_workspace_bytes",
                          "moe_layers_forward"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert m.moe_status_string(code)
    assert m.moe_status_string(99) == "unknown status"


def test_workspace_bytes(L):
    d = _dims()
    assert m.moe_workspace_bytes(d, 0) == 0
    b1, b512 = m.moe_workspace_bytes(d, 1), m.moe_workspace_bytes(d, 512)
    assert 0 < b1 < b512
    # the 512-token chunk keeps y (T*k*H binary16) and the sorted h rows
    assert b512 >= 512 * 8 * 2048 * 2
    assert m.moe_workspace_bytes(_dims(G=32), 1) == 0
    assert m.moe_workspace_bytes(_dims(E=257), 1) == 0
    assert m.moe_workspace_bytes(_dims(k=9), 1) == 0
    assert m.moe_workspace_bytes(_dims(H=192), 1) == 0   # 64*3: neither 64*2^m nor a multiple of 2048
    assert m.moe_workspace_bytes(_dims(H=6144), 1) == 0  # above the 4096 limit
    assert m.moe_workspace_bytes(_dims(), -1) == 0
    assert m.moe_workspace_bytes(_dims(), 65537) == 0


def _forward(L, dims, W, x=FAKE, T=1, out=FAKE + 64, ws=FAKE, ws_bytes=1 << 30):
    return L.moe_forward(ctypes.byref(dims), ctypes.byref(W) if W is not None else None, x, T, out,
                         None, None, None, ws, ws_bytes, None)


def test_refusals_forward(L):
    d, W = _dims(), _weights()
    assert L.moe_forward(None, ctypes.byref(W), FAKE, 1, FAKE, None, None, None, FAKE, 1 << 30, None) == -1
    assert _forward(L, d, None) == -1                     # no weights struct
    assert _forward(L, d, _weights(w13_q=None)) == -1     # a weight array missing
    assert _forward(L, d, W, x=None) == -1
    assert _forward(L, d, W, out=None) == -1
    assert _forward(L, d, W, ws=None) == -1
    assert _forward(L, _dims(k=0), W) == -2
    assert _forward(L, _dims(E=4, k=8), W) == -2
    assert _forward(L, _dims(I=96), W) == -2
    assert _forward(L, _dims(flags=7), W) == -2
    assert _forward(L, _dims(flags=0x800), W) == -2                 # an unknown flag bit
    assert _forward(L, _dims(flags=0x103), W) == -2                 # an unknown path with the debug bit
    assert _forward(L, d, W, T=-1) == -2
    assert _forward(L, _dims(flags=m.PATH_DECODE), W, T=5) == -2  # few-token path holds at most 4 tokens
    assert _forward(L, d, W, x=FAKE + 2) == -3
    assert _forward(L, d, _weights(w2_s=FAKE + 8)) == -3
    assert _forward(L, d, W, ws=FAKE + 128) == -3
    need = m.moe_workspace_bytes(d, 7)
    assert _forward(L, d, W, T=7, ws_bytes=need - 1) == -4


def test_refusals_affine(L):
    aff = m.FMT_AFFINE4
    W = _weights()
    assert _forward(L, _dims(flags=aff), _weights(w13_b=None)) == -1  # offsets required with the flag
    assert _forward(L, _dims(flags=aff), _weights(w2_b=None)) == -1
    assert _forward(L, _dims(flags=aff), _weights(w2_b=FAKE + 4096 * 11 + 2)) == -3
    assert _forward(L, _dims(flags=aff | m.PATH_DECODE), W, T=5) == -2
    r = L.moe_experts_w4a16(ctypes.byref(_dims(flags=aff)), ctypes.byref(_weights(w13_b=None)), FAKE, 1, FAKE, FAKE,
                            FAKE, FAKE, 1 << 30, None)
    assert r == -1


def test_refusals_route_and_experts(L):
    d, W = _dims(), _weights()
    r = L.moe_route(ctypes.byref(d), ctypes.byref(W), FAKE, 1, None, FAKE, None, None, FAKE, 1 << 30, None)
    assert r == -1  # ids required
    r = L.moe_route(ctypes.byref(d), ctypes.byref(W), FAKE, 1, FAKE + 2, FAKE, None, None, FAKE, 1 << 30, None)
    assert r == -3
    r = L.moe_experts_w4a16(ctypes.byref(d), ctypes.byref(W), FAKE, 1, None, FAKE, FAKE, FAKE, 1 << 30, None)
    assert r == -1
    # the routed half does not need router or shared-expert arrays, but it does need the experts
    Wr = _weights(router_q=None, router_s=None, sh13_q=None, sh13_s=None, sh2_q=None, sh2_s=None, w2_q=None)
    r = L.moe_experts_w4a16(ctypes.byref(d), ctypes.byref(Wr), FAKE, 1, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert r == -1


def _block(L, dims, W, h=FAKE, gain=FAKE + (1 << 20), eps=1e-6, T=1, out=FAKE + (2 << 20), ws=FAKE, ws_bytes=1 << 30):
    return L.moe_block_forward(ctypes.byref(dims), ctypes.byref(W) if W is not None else None, h, gain, eps, T, out,
                               None, None, None, ws, ws_bytes, None)


def test_refusals_block_forward(L):
    d, W = _dims(), _weights()
    assert _block(L, d, W, gain=None) == -1
    assert _block(L, d, W, h=None) == -1
    assert _block(L, d, W, out=None) == -1
    assert _block(L, d, _weights(sh2_s=None)) == -1
    assert _block(L, d, W, gain=FAKE + (1 << 20) + 2) == -3
    assert _block(L, d, W, eps=-1.0) == -2
    assert _block(L, d, W, eps=float("nan")) == -2
    assert _block(L, d, W, eps=float("inf")) == -2
    assert _block(L, d, W, out=FAKE) == -2                          # out is the residual stream itself
    assert _block(L, d, W, T=4, out=FAKE + 2048 * 2 * 3) == -2      # out overlaps its last row
    assert _block(L, d, W, T=7, ws_bytes=m.moe_workspace_bytes(d, 7) - 1) == -4
    assert L.moe_block_forward(ctypes.byref(d), None, None, None, 0.0, 0, None, None, None, None, None, 0, None) == 0


def test_zero_tokens_is_a_noop(L):
    d = _dims()
    assert L.moe_forward(ctypes.byref(d), None, None, 0, None, None, None, None, None, 0, None) == 0
    assert L.moe_route(ctypes.byref(d), None, None, 0, None, None, None, None, None, 0, None) == 0
    assert L.moe_experts_w4a16(ctypes.byref(d), None, None, 0, None, None, None, None, 0, None) == 0


def test_valid_call_without_gpu_reports_device_error(L):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: a valid call with fake pointers would reach it")
    assert _forward(L, _dims(), _weights()) == -6


def _noalloc(L, dims, W, x=FAKE, T=1, out=FAKE, ids=None):
    return L.moe_forward_noalloc(ctypes.byref(dims) if dims is not None else None,
                                 ctypes.byref(W) if W is not None else None, x, T, out, ids, None, None, None)


def test_refusals_forward_noalloc(L):
    """The allocation-free variant refuses what moe_forward refuses, before any
    device call, and refuses calls that need more than its static scratch."""
    d, W = _dims(), _weights()
    assert _noalloc(L, None, W) == -1
    assert _noalloc(L, d, None) == -1
    assert _noalloc(L, d, W, x=None) == -1
    assert _noalloc(L, d, _weights(sh13_s=None)) == -1
    assert _noalloc(L, _dims(k=9), W) == -2
    assert _noalloc(L, _dims(flags=m.PATH_DECODE), W, T=5) == -2
    assert _noalloc(L, d, W, x=FAKE + 2) == -3
    assert _noalloc(L, d, W, ids=FAKE + 2) == -3
    assert _noalloc(L, d, W, T=0) == 0
    big = next(T for T in range(1, 4097) if m.moe_workspace_bytes(d, T) > m.NOALLOC_SCRATCH_BYTES)
    assert big > 128
    assert _noalloc(L, d, W, T=big) == -7
    assert _noalloc(L, d, W, T=512) == -7


def _layers(L, dims=None, W=None, gain=FAKE + 4096 * 20, stride=1 << 20, nl=2, eps=1e-6, h=FAKE + 4096 * 30, T=1,
            out=FAKE + 4096 * 40, ws=FAKE, ws_bytes=1 << 30):
    dims = dims if dims is not None else _dims()
    W = W if W is not None else _weights()
    return L.moe_layers_forward(ctypes.byref(dims), ctypes.byref(W), gain, stride, nl, eps, h, T, out, ws, ws_bytes,
                                None)


def test_layers_workspace_sizes(L):
    d = _dims()
    one = m.moe_workspace_bytes(d, 1)
    assert m.moe_layers_workspace_bytes(d, 1, 1) >= one
    # each layer of the persistent launch has its own hand-off zones
    assert m.moe_layers_workspace_bytes(d, 1, 8) > m.moe_layers_workspace_bytes(d, 1, 2)
    assert m.moe_layers_workspace_bytes(d, 1, 0) == 0
    assert m.moe_layers_workspace_bytes(d, 1, 257) == 0
    # T > 4: the grouped-GEMM path's workspace plus one [T][H] buffer
    assert m.moe_layers_workspace_bytes(d, 64, 3) >= m.moe_workspace_bytes(d, 64) + 64 * 2048 * 2


def test_refusals_layers(L):
    assert _layers(L, nl=0) == -2
    assert _layers(L, nl=257) == -2
    assert _layers(L, stride=8) == -3              # layer stride keeps 16-byte alignment
    assert _layers(L, gain=None) == -1
    assert _layers(L, W=_weights(sh2_s=None)) == -1
    assert _layers(L, h=FAKE + 4096 * 30 + 2) == -3
    assert _layers(L, out=FAKE + 4096 * 30) == -2  # out aliases h
    assert _layers(L, eps=float("nan")) == -2
    need = m.moe_layers_workspace_bytes(_dims(), 1, 2)
    assert _layers(L, ws_bytes=need - 1) == -4
    assert _layers(L, T=0) == 0
