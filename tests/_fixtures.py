"""Loaders for the text fixtures under tests/golden/."""
from __future__ import annotations

import os

import numpy as np

from workloads.gen import Dims, Weights, f16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                yield line.split()


def load_nibbles():
    codes = bytes_ = None
    for tok in _lines("int4_nibbles.txt"):
        if tok[0] == "codes":
            codes = np.array([int(v) for v in tok[1:]], dtype=np.int16)
        elif tok[0] == "bytes":
            bytes_ = np.array([int(v, 16) for v in tok[1:]], dtype=np.uint8)
    return codes, bytes_


def load_hand_case(name="hand_case_h64.txt"):
    """Build (dims, weights, x_bits, expect) from the sparse hand-derived fixture."""
    dims = None
    codes = {}
    scales = {}
    xs = []
    expect = {"ids": {}, "w": {}, "sigma": {}, "gap": {}, "out": {}}
    fills = {}
    for tok in _lines(name):
        kind = tok[0]
        if kind == "dims":
            H, E, k, I, Is, G = map(int, tok[1:])
            dims = Dims(H=H, E=E, k=k, I=I, Is=Is, G=G)
        elif kind == "fill":
            fills[tok[1]] = float(tok[2])
        elif kind == "x":
            xs.append((int(tok[1]), int(tok[2]), float(tok[3])))
        elif kind == "expect":
            idx = tuple(int(v) for v in tok[2:-1])
            expect[tok[1]][idx] = float(tok[-1])
        elif kind.endswith("_s"):
            scales.setdefault(kind, []).append((tuple(int(v) for v in tok[1:-1]), float(tok[-1])))
        else:
            codes.setdefault(kind, []).append((tuple(int(v) for v in tok[1:-1]), int(tok[-1])))
    H, E, I, Is, G = dims.H, dims.E, dims.I, dims.Is, dims.G
    shapes_q = {
        "router_q": (E + 1, H), "w13_q": (E, 2 * I, H), "w2_q": (E, H, I),
        "sh13_q": (2 * Is, H), "sh2_q": (H, Is),
    }
    shapes_s = {
        "router_s": (E + 1, H // G), "w13_s": (E, 2 * I, H // G), "w2_s": (E, H, I // G),
        "sh13_s": (2 * Is, H // G), "sh2_s": (H, Is // G),
    }
    q = {n: np.zeros(s, dtype=np.int16) for n, s in shapes_q.items()}
    for n, entries in codes.items():
        for idx, v in entries:
            q[n][idx] = v
    s = {n: np.full(sh, fills.get(n, 1.0)) for n, sh in shapes_s.items()}
    for n, entries in scales.items():
        for idx, v in entries:
            s[n][idx] = v

    def pack4(a):
        u = (a & 0xF).astype(np.uint8)
        return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)

    W = Weights(
        router_q=q["router_q"].astype(np.int8), router_s=f16_bits(s["router_s"]),
        w13_q=pack4(q["w13_q"]), w13_s=f16_bits(s["w13_s"]),
        w2_q=pack4(q["w2_q"]), w2_s=f16_bits(s["w2_s"]),
        sh13_q=q["sh13_q"].astype(np.int8), sh13_s=f16_bits(s["sh13_s"]),
        sh2_q=q["sh2_q"].astype(np.int8), sh2_s=f16_bits(s["sh2_s"]),
    )
    T = 1 + max(t for t, _, _ in xs)
    x = np.zeros((T, H))
    for t, j, v in xs:
        x[t, j] = v
    return dims, W, f16_bits(x), expect
