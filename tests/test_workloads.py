"""The seeded workloads: storage format, determinism and routing statistics."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import ref
from workloads import gen


def _check_format(case):
    d, W = case.dims, case.weights
    H, E, I, Is, G = d.H, d.E, d.I, d.Is, d.G
    shapes = dict(router_q=(E + 1, H), router_s=(E + 1, H // G), w13_q=(E, 2 * I, H // 2),
                  w13_s=(E, 2 * I, H // G), w2_q=(E, H, I // 2), w2_s=(E, H, I // G),
                  sh13_q=(2 * Is, H), sh13_s=(2 * Is, H // G), sh2_q=(H, Is), sh2_s=(H, Is // G))
    for name, a in W.items():
        assert a.shape == shapes[name], name
        assert a.flags.c_contiguous, name
        if name.endswith("_s"):
            assert a.dtype == np.uint16
            v = a.view(np.float16).astype(np.float64)
            assert np.all(np.isfinite(v)) and np.all(v >= 2.0 ** -14), name  # positive normal
    assert W.router_q.dtype == np.int8 and W.sh13_q.dtype == np.int8 and W.sh2_q.dtype == np.int8
    assert W.w13_q.dtype == np.uint8 and W.w2_q.dtype == np.uint8
    assert case.x.dtype == np.uint16 and case.x.shape == (case.T, H)
    assert np.all(np.isfinite(case.x.view(np.float16)))


def test_toy_config_format_and_determinism():
    a, b = gen.make_config(0), gen.make_config(0)
    _check_format(a)
    for (n, x), (_, y) in zip(a.weights.items(), b.weights.items()):
        assert np.array_equal(x, y), n
    assert np.array_equal(a.x, b.x)
    assert a.T == 1 and a.dims == gen.TOY


@pytest.mark.slow
@pytest.mark.parametrize("i,T", [(1, 1), (2, 32), (3, 128), (4, 512)])
def test_real_configs(i, T):
    c = gen.make_config(i)
    _check_format(c)
    assert c.T == T and c.dims == gen.REAL
    x = c.x.view(np.float16).astype(np.float64)
    assert abs(np.sqrt((x ** 2).mean()) - 1.0) < 0.05  # unit RMS rows
    r = ref.route(c.x, c.weights, c.dims)
    counts = np.bincount(r["ids"].ravel(), minlength=c.dims.E)
    lg = r["logits"][:, : c.dims.E]
    if i == 1:
        assert 0.7 < lg.std() < 1.3  # router logits scaled to std about 1
    if i == 2:
        assert 140 <= (counts > 0).sum() <= 190 and counts.max() <= 10  # near-uniform
    if i == 3:
        assert counts.max() >= 20  # moderate imbalance from the N(0, 0.5) bias
    if i == 4:
        assert (counts > 0).sum() <= 140 and counts.max() >= 300  # Zipf skew
        assert len(c.meta["near_tie_tokens"]) == 26


def test_real_weights_shared_across_configs():
    a, b = gen.make_config(1), gen.make_config(2)
    assert a.weights.w13_q is b.weights.w13_q  # one seeded expert set for configs 1-4
    assert not np.array_equal(a.weights.router_q, b.weights.router_q)
