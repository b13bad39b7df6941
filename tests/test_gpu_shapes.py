"""Parity at other admitted widths, exact router ties and the path boundary.

Same bar as test_gpu_parity: ids exact as sets off the near-tie rows, per-row
relative L2 <= 2e-3 against the float64 oracle.  The exact-tie tests add an
unexempted check: when two experts' router rows are identical, their logits
are bit-identical on both sides, and the lower expert index must win the
k-th place (the tie rule the oracle and the kernels share).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import w4a16_routed_experts_amd as m  # noqa: E402
from oracle import ref  # noqa: E402
from tests import _gpu  # noqa: E402
from workloads import gen  # noqa: E402
from workloads.gen import Case, Dims  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.lib()  # raises if the library is missing


# (H, E, k, I, Is): every width is 64 * 2^m or a multiple of 2048
SHAPES = [
    (512, 32, 4, 128, 256),
    (1024, 128, 6, 256, 1024),
    (4096, 64, 8, 1024, 128),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "H{}E{}k{}I{}Is{}".format(*s))
@pytest.mark.parametrize("T,flags", [(1, m.PATH_AUTO), (3, m.PATH_DECODE), (0, m.PATH_AUTO), (2, m.PATH_CHUNK)])
def test_other_widths(shape, T, flags):
    H, E, k, I, Is = shape
    if T == 0:  # a multi-token chunk, kept small where the float64 oracle is slow
        T = 10 if H >= 4096 else 24
    d = Dims(H=H, E=E, k=k, I=I, Is=Is)
    case = gen.make_case(d, T, seed=3000 + H + E + T)
    _gpu.log(f"shape {shape} T={T} flags={flags}")
    r = ref.forward(case.x, case.weights, d)
    g = _gpu.run_forward(case, flags=flags)
    _gpu.check_forward(case, r, g, f"{shape}-T{T}-f{flags}")


def _tie_case(base: Case, token: int = 0):
    """Give token `token`'s (k+1)-th expert the router row of its k-th expert,
    so the two boundary experts' logits tie exactly for every token."""
    d = base.dims
    r = ref.route(base.x, base.weights, d)
    order = np.lexsort((np.arange(d.E), -r["logits"][token, : d.E]))
    a, b = int(order[d.k - 1]), int(order[d.k])  # k-th and (k+1)-th
    rq = base.weights.router_q.copy()
    rs = base.weights.router_s.copy()
    rq[b] = rq[a]
    rs[b] = rs[a]
    W = dataclasses.replace(base.weights, router_q=rq, router_s=rs)
    return Case(name=base.name + "_tie", dims=d, weights=W, x=base.x, meta=dict(base.meta)), a, b


@pytest.mark.parametrize("T,flags", [(1, m.PATH_AUTO), (1, m.PATH_CHUNK), (40, m.PATH_AUTO)])
def test_exact_tie_takes_lower_index(T, flags):
    base = gen.make_case(gen.REAL, T, seed=4000 + T, real_experts=True)
    case, a, b = _tie_case(base)
    d = case.dims
    r = ref.forward(case.x, case.weights, d)
    lg = r["logits"][0, : d.E]
    assert lg[a] == lg[b], "the copied rows must tie exactly in float64"
    assert r["gap"][0] == 0.0
    winner, loser = min(a, b), max(a, b)
    assert winner in r["ids"][0] and loser not in r["ids"][0]
    _gpu.log(f"exact tie T={T} flags={flags}: experts {a} and {b}, lower index {winner} must be kept")
    g = _gpu.run_forward(case, flags=flags)
    assert set(g["ids"][0].tolist()) == set(r["ids"][0].tolist()), (sorted(g["ids"][0]), sorted(r["ids"][0]))
    _gpu.check_forward(case, r, g, f"tie-T{T}-f{flags}")
    # moe_route ranks the same way
    rr = _gpu.run_route(case, flags=flags)
    assert set(rr["ids"][0].tolist()) == set(r["ids"][0].tolist())


@pytest.mark.parametrize("T", [4, 5])
def test_path_boundary(T):
    """T = 4 is the last size the single-launch path takes on its own, T = 5 the first grouped-GEMM one."""
    case = gen.make_case(gen.REAL, T, seed=5000 + T, real_experts=True)
    r = ref.forward(case.x, case.weights, case.dims)
    g = _gpu.run_forward(case, flags=m.PATH_AUTO)
    _gpu.check_forward(case, r, g, f"boundary-T{T}")


def _near_max_case(T, seed):
    """Shared-expert down weights |code x scale| up to about 41600 (the largest
    binary16 is 65504) and outputs in the tens of thousands, with small
    activations: x divided by 11, and the router and routed gate/up scales
    multiplied by 11 so routing and the routed half are as in the unscaled case."""
    from dataclasses import replace
    case = gen.make_case(gen.REAL, T, seed=seed, real_experts=True)
    W = case.weights
    f = lambda b: b.view(np.float16).astype(np.float64)  # noqa: E731
    W2 = replace(W, router_s=gen.f16_bits(f(W.router_s) * 11), w13_s=gen.f16_bits(f(W.w13_s) * 11),
                 sh2_s=gen.f16_bits(f(W.sh2_s) * 2.0 ** 18))
    return replace(case, name=f"near_max_T{T}", weights=W2, x=gen.f16_bits(f(case.x) / 11))


@pytest.mark.parametrize("T,flags", [(3, m.PATH_DECODE), (40, m.PATH_CHUNK), (3, m.PATH_CHUNK)])
def test_weights_and_outputs_near_binary16_max(T, flags):
    case = _near_max_case(T, 9500 + T)
    r = ref.forward(case.x, case.weights, case.dims)
    sh2 = ref.dequant(case.weights.sh2_q, case.weights.sh2_s, case.dims.G)
    assert np.abs(sh2).max() > 30000.0 and 10000.0 < np.abs(r["out"]).max() < 65504.0
    g = _gpu.run_forward(case, flags=flags)
    _gpu.check_forward(case, r, g, f"near binary16 max T{T} f{flags}")


def _ids_with_counts(counts, T, k):
    """ids [T, k] in which expert e is listed by exactly counts[e] tokens (at
    most once per token): each expert's listings fill consecutive places of
    the column-major grid, so they fall on distinct tokens."""
    flat = np.repeat(np.arange(len(counts)), counts)
    assert flat.size == T * k and max(counts) <= T
    idx = np.arange(T * k)
    ids = np.empty((T, k), dtype=np.int64)
    ids[idx % T, idx // T] = flat
    return ids


def test_bucketing_tile_classes():
    """Caller routing that gives experts the row counts at every tile-class
    boundary of the grouped GEMMs: 1 and 16 (narrow), 17, 32, 33, 96, 97
    (the heaviest class as a last tile), 128 and 256 (full tiles with no last
    tile), 129 (a full tile and a one-row last tile) and 225 (a full tile and
    a 97-row last tile), among tiles of 100 rows.  Parity against the oracle,
    and two calls bit for bit (the pairs that fill an expert's last tile must
    be the same in every call)."""
    T, k = 260, 8
    case = gen.make_case(gen.REAL, T, seed=5300, real_experts=True)
    d = case.dims
    boundary = [256, 225, 129, 128, 97, 96, 33, 32, 17, 16, 1]
    rest = T * k - sum(boundary)
    counts = boundary + [100] * (rest // 100) + ([rest % 100] if rest % 100 else [])
    rng = np.random.default_rng(5301)
    perm = rng.permutation(d.E)[:len(counts)]
    ids = perm[_ids_with_counts(counts, T, k)]
    w = rng.uniform(0.05, 1.0, size=(T, k))
    _gpu.log(f"caller routing with tile-class boundary counts, T={T}, {len(counts)} experts")
    g1 = _gpu.run_experts(case, ids, w)
    g2 = _gpu.run_experts(case, ids, w)
    want = ref.experts(case.x, ids, w, case.weights, d)
    err = _gpu.row_rel_l2(g1, want)
    _gpu.log(f"  rel L2 max {err.max():.3e}")
    assert err.max() <= _gpu.ROW_TOL
    assert np.array_equal(g1, g2)
