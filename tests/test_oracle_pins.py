"""Pins of the float64 oracle against facts fixed outside the oracle itself.

Every function of the oracle is checked against something other than its own
formula: a hand-derived worked case, brute-force enumeration, closed forms of
special cases, library routines, and invariants.  The controls at the end
plant plausible mistakes in the oracle (on the CPU) and check that the pins
turn red.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import pytest
import scipy.special

from oracle import ref
from tests import _fixtures
from workloads import gen
from workloads.gen import Dims, Weights, f16_bits

TINY = Dims(H=128, E=6, k=2, I=64, Is=64, G=64)


def _tiny_case(seed=5, T=3, dims=TINY):
    return gen.make_case(dims, T, seed)


# ---------------------------------------------------------------------------
# storage format
# ---------------------------------------------------------------------------


def test_int4_golden_bytes():
    codes, packed = _fixtures.load_nibbles()
    assert np.array_equal(gen.pack_int4(codes), packed)
    assert np.array_equal(ref.unpack_int4(packed), codes)


def test_int4_every_byte_value():
    # independent route to the signed nibbles: shift the nibble into the top of
    # an int8 and shift back arithmetically (sign extension)
    b = np.arange(256, dtype=np.uint8)
    lo = ((b << 4).astype(np.uint8).view(np.int8) >> 4).astype(np.int16)
    hi = ((b & 0xF0).view(np.int8) >> 4).astype(np.int16)
    q = ref.unpack_int4(b[:, None])
    assert np.array_equal(q[:, 0], lo) and np.array_equal(q[:, 1], hi)


def test_int4_roundtrip_random():
    rng = np.random.default_rng(0)
    q = rng.integers(-8, 8, size=(7, 3, 130))
    assert np.array_equal(ref.unpack_int4(gen.pack_int4(q)), q)


def test_dequant_group_indexing_and_exactness():
    rng = np.random.default_rng(1)
    G, rows, ngroups = 64, 3, 5
    s = f16_bits(rng.uniform(0.005, 0.02, size=(rows, ngroups)))
    q = rng.integers(-128, 128, size=(rows, G * ngroups))
    d = ref.dequant(q, s, G)
    sv = s.view(np.float16)
    for r in range(rows):
        for j in range(G * ngroups):
            # products of an 8-bit code and a binary16 scale are exact in fp32
            want = np.float32(q[r, j]) * np.float32(sv[r, j // G])
            assert d[r, j] == float(want)
    assert np.array_equal(np.rint(d / np.repeat(sv.astype(np.float64), G, axis=1)), q)


# ---------------------------------------------------------------------------
# the whole block on a hand-derived case
# ---------------------------------------------------------------------------


def _check_hand_case(fwd=None):
    dims, W, x, expect = _fixtures.load_hand_case()
    r = (fwd or ref.forward)(x, W, dims)
    for (t, i), v in expect["ids"].items():
        assert r["ids"][t, i] == int(v), ("ids", t, i)
    for (t, i), v in expect["w"].items():
        assert abs(r["w"][t, i] - v) < 1e-15, ("w", t, i)
    for (t,), v in expect["sigma"].items():
        assert abs(r["sigma"][t] - v) < 1e-15, ("sigma", t)
    for (t,), v in expect["gap"].items():
        assert r["gap"][t] == v, ("gap", t)
    want = np.zeros_like(r["out"])
    for (t, n), v in expect["out"].items():
        want[t, n] = v
    assert np.abs(r["out"] - want).max() < 1e-14


def test_hand_derived_block():
    _check_hand_case()


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------


def test_router_logits_brute_force():
    c = _tiny_case()
    dims, W = c.dims, c.weights
    got = ref.router_logits(c.x, W, dims)
    xs = c.x.view(np.float16)
    sv = W.router_s.view(np.float16)
    for t in range(c.T):
        for e in range(dims.E + 1):
            acc = math.fsum(float(xs[t, j]) * int(W.router_q[e, j]) * float(sv[e, j // dims.G])
                            for j in range(dims.H))
            assert abs(got[t, e] - acc) < 1e-12


@pytest.mark.parametrize("E,k", [(8, 2), (10, 3), (6, 1), (7, 7)])
def test_topk_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    for _ in range(200):
        # integer logits drawn from a small range make exact ties common
        lr = rng.integers(-3, 4, size=(1, E)).astype(np.float64)
        ids = ref.topk_ids(lr, k)[0]
        best = None
        for sub in itertools.combinations(range(E), k):
            key = (-sum(lr[0, list(sub)]), sub)  # max sum, then lexicographically smallest
            if best is None or key < best:
                best = key
        assert tuple(sorted(ids)) == best[1]
        # emitted order: descending logit, ties by ascending index
        keys = [(-lr[0, e], e) for e in ids]
        assert keys == sorted(keys)


def test_topk_identical_rows_pick_lowest_indices():
    lr = np.full((2, 9), 0.25)
    assert ref.topk_ids(lr, 4).tolist() == [[0, 1, 2, 3]] * 2


def test_renormalised_weights_closed_forms():
    rng = np.random.default_rng(3)
    lr = rng.normal(size=(50, 12))
    ids = ref.topk_ids(lr, 4)
    w = ref.softmax_renormalised(lr, ids)
    assert np.all(w > 0)
    assert np.abs(w.sum(axis=1) - 1).max() < 1e-15
    sel = np.take_along_axis(lr, ids, axis=1)
    assert np.abs(w - scipy.special.softmax(sel, axis=1)).max() < 1e-15
    # k = E: the textbook dense softmax, in descending order
    ids_all = ref.topk_ids(lr, 12)
    w_all = ref.softmax_renormalised(lr, ids_all)
    dense = scipy.special.softmax(lr, axis=1)
    assert np.abs(w_all - np.take_along_axis(dense, ids_all, axis=1)).max() < 1e-15


def test_gap_definition():
    lr = np.array([[0.5, 2.0, 1.0, 1.0, -1.0], [3.0, 3.0, 3.0, 0.0, 1.0]])
    # sorted rows: (2, 1, 1, 0.5, -1) and (3, 3, 3, 1, 0)
    assert ref.kth_gap(lr, 1).tolist() == [1.0, 0.0]
    assert ref.kth_gap(lr, 2).tolist() == [0.0, 0.0]
    assert ref.kth_gap(lr, 3).tolist() == [0.5, 2.0]
    assert np.isinf(ref.kth_gap(lr, 5)).all()


def test_sigmoid_and_silu_values():
    assert ref.sigmoid(0.0) == 0.5
    assert abs(ref.sigmoid(1.0) - math.e / (1 + math.e)) < 1e-16
    assert abs(ref.silu(2.0) - 2 * math.e ** 2 / (1 + math.e ** 2)) < 1e-15
    assert ref.silu(-800.0) == 0.0  # no overflow to nan for very negative input


# ---------------------------------------------------------------------------
# experts
# ---------------------------------------------------------------------------


def _identity_experts(dims, x_scale_gate=1.0):
    """Gate = identity, up = 2 x identity, down = cyclic shift by one."""
    H, E, I, Is, G = dims.H, dims.E, dims.I, dims.Is, dims.G
    w13 = np.zeros((E, 2 * I, H), dtype=np.int16)
    w2 = np.zeros((E, H, I), dtype=np.int16)
    for e in range(E):
        for j in range(I):
            w13[e, j, j] = 1
            w13[e, I + j, j] = 2
        for n in range(min(H, I)):
            w2[e, n, (n + 1) % I] = 1
    ones = lambda shape: f16_bits(np.ones(shape))  # noqa: E731
    return dict(w13_q=gen.pack_int4(w13), w13_s=ones((E, 2 * I, H // G)),
                w2_q=gen.pack_int4(w2), w2_s=ones((E, H, I // G)))


def test_swiglu_closed_form_identity_weights():
    dims = Dims(H=128, E=3, k=1, I=64, Is=64, G=64)
    c = gen.make_case(dims, 4, seed=11)
    W = c.weights
    for n, a in _identity_experts(dims).items():
        setattr(W, n, a)
    ids = np.zeros((c.T, 1), dtype=np.int64)
    w = np.ones((c.T, 1))
    y = ref.experts(c.x, ids, w, W, dims)
    xs = c.x.view(np.float16).astype(np.float64)
    for t in range(c.T):
        for n in range(dims.H):
            if n < dims.I:
                j = (n + 1) % dims.I
                z = xs[t, j]
                want = (z / (1.0 + math.exp(-z))) * (2.0 * z)
            else:
                want = 0.0
            assert abs(y[t, n] - want) < 1e-12


def test_identical_experts_reduce_to_one():
    dims = Dims(H=128, E=5, k=3, I=64, Is=64, G=64)
    c = gen.make_case(dims, 6, seed=12)
    W = c.weights
    W.w13_q[:] = W.w13_q[0]
    W.w13_s[:] = W.w13_s[0]
    W.w2_q[:] = W.w2_q[0]
    W.w2_s[:] = W.w2_s[0]
    r = ref.forward(c.x, W, dims)
    one = ref.swiglu_ffn(ref.half_bits_to_f64(c.x), *ref.routed_expert_weights(W, dims, 0), dims.I)
    assert np.abs(r["routed"] - one).max() < 1e-12 * max(1.0, np.abs(one).max())


@pytest.mark.parametrize("k", [1, 2])
def test_one_hot_router(k):
    dims = Dims(H=128, E=6, k=k, I=64, Is=64, G=64)
    c = gen.make_case(dims, 3, seed=13)
    W = c.weights
    star = 4
    # x_t . row = 30 for every token: put the mass on coordinate 0 and set x_0 = 1
    x = c.x.copy()
    x[:, 0] = f16_bits(1.0)
    W.router_q[:, :64] = 0
    W.router_q[star, 0] = 120
    W.router_s[star, 0] = f16_bits(0.25)
    W.router_q[star, 1:64] = 0
    r = ref.forward(x, W, dims)
    assert np.all(r["ids"][:, 0] == star)
    one = ref.swiglu_ffn(ref.half_bits_to_f64(x), *ref.routed_expert_weights(W, dims, star), dims.I)
    if k == 1:
        assert np.array_equal(r["routed"], one)
    else:
        assert np.abs(r["routed"] - one).max() < 1e-9 * np.abs(one).max()


def test_dense_mask_formulation_agrees():
    for seed, T in [(21, 5), (22, 9)]:
        c = gen.make_case(TINY, T, seed)
        a = ref.forward(c.x, c.weights, c.dims)["out"]
        b = ref.forward_dense(c.x, c.weights, c.dims)
        assert np.abs(a - b).max() < 1e-12 * np.abs(a).max()


def test_shared_gate_special_cases():
    c = _tiny_case(seed=31, T=4)
    dims, W = c.dims, c.weights
    r = ref.forward(c.x, W, dims)
    S = ref.shared_expert(c.x, W, dims)
    routed = ref.experts(c.x, r["ids"], r["w"], W, dims)
    assert np.abs((r["out"] - routed) - r["sigma"][:, None] * S).max() < 1e-12
    # zero gate row -> sigma exactly one half
    W.router_q[dims.E] = 0
    r0 = ref.forward(c.x, W, dims)
    assert np.all(r0["sigma"] == 0.5)
    # zero shared weights -> the output is the routed half alone
    W.sh2_q[:] = 0
    r1 = ref.forward(c.x, W, dims)
    assert np.array_equal(r1["out"], r1["routed"])


def test_near_tie_rows_of_the_512_token_chunk():
    case = gen.make_config(4)
    r = ref.route(case.x, case.weights, case.dims)
    tokens = case.meta["near_tie_tokens"]
    assert len(tokens) == 26
    assert np.all(r["gap"][tokens] < 1e-3)
    assert 26 <= int((r["gap"] < 1e-3).sum()) <= 40


# ---------------------------------------------------------------------------
# planted controls: each plausible mistake must turn at least one pin red
# ---------------------------------------------------------------------------


def _swapped_gate_up(X, w13, w2, inter):
    A = X @ w13.T
    return (A[:, :inter] * ref.silu(A[:, inter:])) @ w2.T


def _transposed_down(X, w13, w2, inter):
    A = X @ w13.T
    Hh = ref.silu(A[:, :inter]) * A[:, inter:]
    n = min(w2.shape)
    out = np.zeros((X.shape[0], w2.shape[0]))
    out[:, :n] = Hh[:, :n] @ w2[:n, :n]
    return out


def _no_renorm(lr, ids):
    p = np.exp(lr - lr.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, ids, axis=1)


def _high_index_ties(lr, k):
    E = lr.shape[1]
    return np.stack([np.lexsort((-np.arange(E), -row))[:k] for row in lr])


def _nibbles_swapped(packed):
    b = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int16)
    out[..., 1::2] = b & 0x0F
    out[..., 0::2] = (b >> 4) & 0x0F
    out[out >= 8] -= 16
    return out


def _gate_sign_flipped(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(z))


@pytest.mark.parametrize("name,attr,bad", [
    ("gate/up swapped", "swiglu_ffn", _swapped_gate_up),
    ("down projection transposed", "swiglu_ffn", _transposed_down),
    ("renormalisation dropped", "softmax_renormalised", _no_renorm),
    ("ties to the highest index", "topk_ids", _high_index_ties),
    ("nibble order swapped", "unpack_int4", _nibbles_swapped),
    ("sigmoid sign flipped", "sigmoid", _gate_sign_flipped),
])
def test_planted_mistakes_are_caught(monkeypatch, name, attr, bad):
    monkeypatch.setattr(ref, attr, bad)
    with pytest.raises(AssertionError):
        _check_hand_case(ref.forward)


# ---------------------------------------------------------------------------
# the MoE sub-block: post-attention RMSNorm -> block -> residual add
# ---------------------------------------------------------------------------


def _rmsnorm_pins(norm):
    # hand-derived: h = (3, 4), gain = (1, 2), eps = 0 -> mean of squares 12.5
    h = f16_bits(np.array([[3.0, 4.0]]))
    g = f16_bits(np.array([1.0, 2.0]))
    want = np.array([[3.0, 8.0]]) / math.sqrt(12.5)
    assert np.abs(norm(h, g, 0.0) - want).max() < 1e-15
    # constant row c with eps > 0: sign(c) * gain / sqrt(1 + eps / c^2)
    c, eps = -0.25, 1e-2
    hc = f16_bits(np.full((1, 64), c))
    gc = f16_bits(np.linspace(0.5, 1.5, 64))
    want_c = -ref.half_bits_to_f64(gc) / math.sqrt(1.0 + eps / c ** 2)
    assert np.abs(norm(hc, gc, eps)[0] - want_c).max() < 1e-15
    # with eps = 0 a power-of-two scaling of a row changes nothing, exactly
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 128))
    hx, hy = f16_bits(x), f16_bits(x * 8.0)
    gr = f16_bits(rng.uniform(0.5, 1.5, 128))
    assert np.array_equal(norm(hx, gr, 0.0), norm(hy, gr, 0.0))


def test_rmsnorm_pins():
    _rmsnorm_pins(ref.rmsnorm)


def _block_pins(block):
    case = _tiny_case(seed=21, T=4)
    d = case.dims
    # a row of +-1 has unit RMS: with gain 1 and eps 0 the normalised
    # activations are the row itself, so the sub-block is h + the block of h
    signs = np.where(np.random.default_rng(3).random((4, d.H)) < 0.5, -1.0, 1.0)
    h = f16_bits(signs)
    ones = f16_bits(np.ones(d.H))
    r = block(h, ones, 0.0, case.weights, d)
    assert np.array_equal(r["a_bits"], h)
    assert np.abs(r["out"] - (signs + ref.forward(h, case.weights, d)["out"])).max() < 1e-12
    # all-zero routed and shared weights: the output is the residual exactly
    W0 = Weights(**{f: (np.zeros_like(v) if f in ("w13_q", "w2_q", "sh13_q", "sh2_q") else v)
                    for f, v in case.weights.items()})
    h2 = f16_bits(np.random.default_rng(4).standard_normal((4, d.H)) * 3.0)
    r0 = block(h2, ones, 1e-6, W0, d)
    assert np.array_equal(r0["out"], ref.half_bits_to_f64(h2))


def test_block_forward_pins():
    _block_pins(ref.block_forward)


def _norm_sum_not_mean(h_bits, gain_bits, eps):
    X = ref.half_bits_to_f64(h_bits)
    return X / np.sqrt(np.sum(X * X, axis=1, keepdims=True) + eps) * ref.half_bits_to_f64(gain_bits)


def _norm_eps_outside(h_bits, gain_bits, eps):
    X = ref.half_bits_to_f64(h_bits)
    return X / (np.sqrt(np.mean(X * X, axis=1, keepdims=True)) + eps) * ref.half_bits_to_f64(gain_bits)


def _norm_no_gain(h_bits, gain_bits, eps):
    X = ref.half_bits_to_f64(h_bits)
    return X / np.sqrt(np.mean(X * X, axis=1, keepdims=True) + eps)


@pytest.mark.parametrize("name,bad", [
    ("sum of squares instead of mean", _norm_sum_not_mean),
    ("eps outside the square root", _norm_eps_outside),
    ("gain dropped", _norm_no_gain),
])
def test_planted_rmsnorm_mistakes_are_caught(monkeypatch, name, bad):
    monkeypatch.setattr(ref, "rmsnorm", bad)
    with pytest.raises(AssertionError):
        _rmsnorm_pins(ref.rmsnorm)


def test_planted_residual_mistake_is_caught():
    def no_residual(h_bits, gain_bits, eps, W, dims):
        r = ref.block_forward(h_bits, gain_bits, eps, W, dims)
        r["out"] = r["moe"]
        return r
    with pytest.raises(AssertionError):
        _block_pins(no_residual)


def _zero_layer(W):
    """The same arrays with every routed and shared code zero: the sub-block is the identity."""
    return Weights(**{f: (np.zeros_like(v) if f in ("w13_q", "w2_q", "sh13_q", "sh2_q") else v)
                      for f, v in W.items()})


def _layers_pins(layers):
    case = _tiny_case(seed=31, T=3)
    d = case.dims
    rng = np.random.default_rng(32)
    h = f16_bits(rng.standard_normal((3, d.H)) * 2.0)
    g1, g2 = f16_bits(rng.uniform(0.5, 1.5, d.H)), f16_bits(rng.uniform(0.5, 1.5, d.H))
    B = case.weights
    Z = _zero_layer(_tiny_case(seed=33, T=1).weights)
    one = ref.block_forward(h, g2, 1e-6, B, d)["out"]
    # one layer is the sub-block itself
    assert np.array_equal(layers(h, [g2], 1e-6, [B], d), one)
    # identity layers leave the residual stream exactly as it is
    assert np.array_equal(layers(h, [g1, g2, g1], 1e-6, [Z, Z, Z], d), ref.half_bits_to_f64(h))
    # an identity layer first: the second layer, with its own weights and gain, sees h itself
    assert np.array_equal(layers(h, [g1, g2], 1e-6, [Z, B], d), one)
    # an identity layer last: it returns what it reads, the binary16 value of the first layer's output
    want = ref.half_bits_to_f64(ref.f64_to_half_bits(one))
    assert np.array_equal(layers(h, [g2, g1], 1e-6, [B, Z], d), want)
    assert not np.array_equal(want, one)  # the case does exercise the rounding


def test_layers_forward_pins():
    _layers_pins(ref.layers_forward)


def _layers_unrounded(h_bits, gains, eps, Ws, dims):
    X = ref.half_bits_to_f64(h_bits)
    for g, W in zip(gains, Ws):
        X = X + ref.block_forward(ref.f64_to_half_bits(X), g, eps, W, dims)["moe"]
    return X


def _layers_first_weights(h_bits, gains, eps, Ws, dims):
    return ref.layers_forward(h_bits, gains, eps, [Ws[0]] * len(Ws), dims)


def _layers_first_gain(h_bits, gains, eps, Ws, dims):
    return ref.layers_forward(h_bits, [gains[0]] * len(gains), eps, Ws, dims)


@pytest.mark.parametrize("name,bad", [
    ("residual carried in float64 between layers", _layers_unrounded),
    ("every layer reads layer 0's weights", _layers_first_weights),
    ("every layer reads layer 0's gain", _layers_first_gain),
])
def test_planted_layer_mistakes_are_caught(name, bad):
    with pytest.raises(AssertionError):
        _layers_pins(bad)
