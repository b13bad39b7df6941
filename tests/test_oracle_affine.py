"""Pins of the oracle's affine int4 form (the routed experts as w = q s + b
with unsigned codes and one binary16 offset per group).

The affine form is tied to the symmetric form, which is pinned on its own: the
same signed codes stored as q + 8 with offset b = -8 s dequantise to exactly
the symmetric weights, so the two forwards agree bit for bit.  Hand values, an
independent nibble decode and a planted mistake complete the pins.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import ref
from workloads import gen
from workloads.gen import Dims, f16_bits

TINY = Dims(H=128, E=6, k=2, I=64, Is=64, G=64)


def test_unsigned_nibbles_every_byte_value():
    b = np.arange(256, dtype=np.uint8)
    q = ref.unpack_uint4(b[:, None])
    assert np.array_equal(q[:, 0], np.bitwise_and(b, 0x0F).astype(np.int16))
    assert np.array_equal(q[:, 1], np.right_shift(b, 4).astype(np.int16))


def test_unsigned_pack_roundtrip():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 16, size=(5, 4, 66))
    assert np.array_equal(ref.unpack_uint4(gen.pack_uint4(u)), u)


def test_affine_hand_values():
    codes = np.array([[0, 1, 15] + [7] * 61])
    s = f16_bits([[0.5]])
    b = f16_bits([[-3.0]])
    w = ref.dequant_affine(codes, s, b, 64)
    assert w[0, :3].tolist() == [-3.0, -2.5, 4.5]
    assert np.all(w[0, 3:] == 0.5)


def _as_affine(W):
    """The symmetric codes q stored as unsigned q + 8 with offsets -8 s."""
    def conv(q_bytes, s_bits):
        u = ref.unpack_int4(q_bytes) + 8
        b = f16_bits(-8.0 * ref.half_bits_to_f64(s_bits))
        return gen.pack_uint4(u), b
    w13_q, w13_b = conv(W.w13_q, W.w13_s)
    w2_q, w2_b = conv(W.w2_q, W.w2_s)
    from dataclasses import replace
    return replace(W, w13_q=w13_q, w2_q=w2_q, w13_b=w13_b, w2_b=w2_b)


def test_affine_reduces_to_symmetric_exactly():
    case = gen.make_case(TINY, 5, seed=41)
    Wa = _as_affine(case.weights)
    assert Wa.affine and not case.weights.affine
    for e in range(TINY.E):
        a13, a2 = ref.routed_expert_weights(Wa, TINY, e)
        s13, s2 = ref.routed_expert_weights(case.weights, TINY, e)
        assert np.array_equal(a13, s13) and np.array_equal(a2, s2)
    fa = ref.forward(case.x, Wa, TINY)
    fs = ref.forward(case.x, case.weights, TINY)
    assert np.array_equal(fa["out"], fs["out"])


def test_affine_offsets_change_the_result():
    # the generator's offsets are not -8 s: the affine layer differs from the
    # symmetric reading of the same bytes, and by the offsets' contribution
    case = gen.make_affine_case(TINY, 3, seed=42)
    sym = gen.replace(case.weights, w13_b=None, w2_b=None)
    fa = ref.forward(case.x, case.weights, TINY)["routed"]
    fu = ref.forward(case.x, sym, TINY)["routed"]
    assert np.abs(fa - fu).max() > 1e-3 * np.abs(fa).max()


def test_control_offset_dropped_is_caught(monkeypatch):
    """A planted mistake (the offset left out of the affine dequantisation)
    turns the reduction pin red."""
    case = gen.make_case(TINY, 2, seed=43)
    Wa = _as_affine(case.weights)
    good = ref.dequant_affine

    def no_offset(codes, s, b, G):
        return good(codes, s, np.zeros_like(b), G)

    monkeypatch.setattr(ref, "dequant_affine", no_offset)
    with pytest.raises(AssertionError):
        a13, _ = ref.routed_expert_weights(Wa, TINY, 0)
        s13, _ = ref.routed_expert_weights(case.weights, TINY, 0)
        assert np.array_equal(a13, s13)
