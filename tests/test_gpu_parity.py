"""Parity of the HIP library (through the C ABI) with the float64 oracle."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import w4a16_routed_experts_amd as m  # noqa: E402
from oracle import ref  # noqa: E402
from tests import _fixtures, _gpu  # noqa: E402
from workloads import gen  # noqa: E402
from workloads.gen import Case  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.lib()  # raises if the library is missing


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_forward_configs(cfg):
    case = _gpu.config_case(cfg)
    _gpu.log(f"forward config {cfg} ({case.name}) T={case.T}")
    r = _gpu.config_oracle(cfg)
    g = _gpu.run_forward(case)
    _gpu.check_forward(case, r, g, f"cfg{cfg}")


@pytest.mark.parametrize("cfg", [0, 1])
def test_forward_configs_chunk_path(cfg):
    case = _gpu.config_case(cfg)
    _gpu.log(f"forward config {cfg} on the grouped-GEMM path")
    g = _gpu.run_forward(case, flags=m.PATH_CHUNK)
    _gpu.check_forward(case, _gpu.config_oracle(cfg), g, f"cfg{cfg}-chunk")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_route_configs(cfg):
    case = _gpu.config_case(cfg)
    _gpu.log(f"route config {cfg}")
    r = _gpu.config_oracle(cfg)
    g = _gpu.run_route(case)
    _gpu.check_routing(case, r, g, f"route cfg{cfg}")
    scale = np.abs(r["logits"]).max()
    assert np.abs(g["logits"] - r["logits"]).max() <= 1e-5 * max(1.0, scale)


@pytest.mark.parametrize("T", [2, 3, 4])
@pytest.mark.parametrize("flags", [m.PATH_DECODE, m.PATH_CHUNK])
def test_few_tokens_both_paths(T, flags):
    case = gen.make_case(gen.REAL, T, seed=2000 + T, real_experts=True)
    _gpu.log(f"few tokens T={T} flags={flags}")
    r = ref.forward(case.x, case.weights, case.dims)
    g = _gpu.run_forward(case, flags=flags)
    _gpu.check_forward(case, r, g, f"T{T}-f{flags}")


@pytest.mark.parametrize("T", [33, 70])
def test_ragged_chunks_real_width(T):
    case = gen.make_case(gen.REAL, T, seed=3000 + T, bias="normal0.5", c=8.0, real_experts=True)
    _gpu.log(f"ragged chunk T={T}")
    r = ref.forward(case.x, case.weights, case.dims)
    g = _gpu.run_forward(case)
    _gpu.check_forward(case, r, g, f"ragged T{T}")


@pytest.mark.parametrize("T,flags", [(1, m.PATH_DECODE), (3, m.PATH_DECODE), (45, m.PATH_AUTO), (1, m.PATH_CHUNK)])
def test_toy_widths(T, flags):
    case = gen.make_case(gen.TOY, T, seed=4000 + T)
    _gpu.log(f"toy widths T={T} flags={flags}")
    r = ref.forward(case.x, case.weights, case.dims)
    g = _gpu.run_forward(case, flags=flags)
    _gpu.check_forward(case, r, g, f"toy T{T}")


@pytest.mark.parametrize("flags", [m.PATH_DECODE, m.PATH_CHUNK])
def test_hand_derived_case(flags):
    dims, W, x, expect = _fixtures.load_hand_case()
    case = Case(name="hand", dims=dims, weights=W, x=x)
    g = _gpu.run_forward(case, flags=flags)
    for (t, i), v in expect["ids"].items():
        assert g["ids"][t, i] == int(v)
    for (t, i), v in expect["w"].items():
        assert abs(g["w"][t, i] - v) < 1e-6
    for (t,), v in expect["sigma"].items():
        assert abs(g["sigma"][t] - v) < 1e-6
    want = np.zeros_like(g["out"])
    for (t, n), v in expect["out"].items():
        want[t, n] = v
    assert np.abs(g["out"] - want).max() < 2e-3 * np.abs(want).max()


@pytest.mark.parametrize("T,flags", [(1, m.PATH_AUTO), (3, m.PATH_AUTO), (40, m.PATH_AUTO), (2, m.PATH_CHUNK)])
def test_experts_given_routing(T, flags):
    """Caller routing with repeated and out-of-range ids; those contribute nothing."""
    case = gen.make_case(gen.REAL, T, seed=5000 + T, real_experts=True)
    d = case.dims
    rng = np.random.default_rng(T)
    ids = rng.integers(0, d.E, size=(T, d.k))
    ids[0, 1] = ids[0, 0]  # an expert listed twice
    ids[-1, -1] = -1       # out of range: dropped
    ids[-1, -2] = d.E      # out of range: dropped
    w = rng.uniform(0.05, 1.0, size=(T, d.k))
    _gpu.log(f"experts with caller routing T={T} flags={flags}")
    g = _gpu.run_experts(case, ids, w, flags=flags)
    valid = (ids >= 0) & (ids < d.E)
    want = np.zeros((T, d.H))
    for t in range(T):
        for i in range(d.k):
            if valid[t, i]:
                want[t] += ref.experts(case.x[t:t + 1], ids[t:t + 1, i:i + 1], w[t:t + 1, i:i + 1],
                                       case.weights, d)[0]
    err = _gpu.row_rel_l2(g, want)
    _gpu.log(f"  rel L2 max {err.max():.3e}")
    assert err.max() <= _gpu.ROW_TOL


def test_zero_tokens_leaves_output_untouched():
    case = _gpu.config_case(1)
    d = case.dims
    dims = _gpu.dims_of(d)
    W = _gpu.device_weights(case)
    out = torch.full((1, d.H), 1234, dtype=torch.int16, device="cuda")
    assert m.moe_forward(dims, W.struct, _gpu.x_tensor(case), 0, out, ws=None) == 0
    torch.cuda.synchronize()
    assert bool((out == 1234).all())


@pytest.mark.parametrize("cfg", [1, 4])
def test_deterministic(cfg):
    case = _gpu.config_case(cfg)
    g = _gpu.run_forward(case, reps=3)
    for o in g["out_raw"][1:]:
        assert np.array_equal(o, g["out_raw"][0])


def test_workspace_reused_across_token_counts():
    """The counters a call leaves in the workspace let the next call run, on
    either path and at any token count."""
    case4 = gen.make_case(gen.REAL, 4, seed=6004, real_experts=True)
    case1 = gen.make_case(gen.REAL, 1, seed=6001, real_experts=True)
    case8 = gen.make_case(gen.REAL, 8, seed=6008, real_experts=True)  # the multi-token path
    d = case4.dims
    dims = _gpu.dims_of(d)
    W = _gpu.device_weights(_gpu.config_case(1))
    ws = torch.zeros(max(m.moe_workspace_bytes(dims, 4), m.moe_workspace_bytes(dims, 8)), dtype=torch.uint8,
                     device="cuda")
    seq = (case4, case1, case8, case1, case4)
    res = []
    for case in seq:
        out = torch.zeros((case.T, d.H), dtype=torch.int16, device="cuda")
        m.moe_forward(dims, W.struct, _gpu.x_tensor(case), case.T, out, ws=ws)
        torch.cuda.synchronize()
        res.append(_gpu.half_to_f64(out))
    W_host = _gpu.config_case(1).weights
    for case, o in zip(seq, res):
        want = ref.forward(case.x, W_host, d)["out"]
        assert _gpu.row_rel_l2(o, want).max() <= _gpu.ROW_TOL
    # The workspace's sync area: each of the 8 per-group call counters (64-bit,
    # one 128-byte line each) advanced by exactly 2^16 per few-token call (4 of
    # the 5 calls), the give-up word is zero, and every other word (arrival
    # counters, the multi-token path's counter) is back to zero.
    sync = ws[: 40 * 1024].cpu().numpy().view(np.uint32).copy()
    calls = sum(1 for c in seq if c.T <= 4)
    for g in range(8):
        lo, hi = sync[32 * g], sync[32 * g + 1]
        assert (int(hi) << 32 | int(lo)) == calls << 16, f"group {g} call counter"
        sync[32 * g] = sync[32 * g + 1] = 0
    assert int(sync.astype(np.int64).sum()) == 0


def test_max_token_count_sampled():
    """The largest admitted chunk (T = 65536 at real widths, iid routing, so
    every expert takes thousands of rows): ids valid and distinct on every row,
    every output finite, and sampled rows checked against the oracle computed
    for those tokens alone (routing and experts act on each token independently)."""
    T = 65536
    case = gen.make_case(gen.REAL, T, seed=6553, real_experts=True)
    _gpu.log(f"maximum chunk T={T}")
    g = _gpu.run_forward(case)
    d = case.dims
    ids = g["ids"]
    assert ids.min() >= 0 and ids.max() < d.E
    srt = np.sort(ids, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1]), "an expert listed twice for one token"
    assert np.all(np.isfinite(g["out"]))
    rng = np.random.default_rng(65)
    rows = np.sort(np.concatenate([[0, T - 1], rng.choice(T, 46, replace=False)]))
    sub = Case(name="max-sample", dims=d, weights=case.weights, x=case.x[rows], meta={})
    r = ref.forward(sub.x, sub.weights, d)
    gs = dict(out=g["out"][rows], ids=ids[rows], w=g["w"][rows], sigma=g["sigma"][rows])
    _gpu.check_forward(sub, r, gs, f"T{T}-sampled")


@pytest.mark.parametrize("T", [1, 40])
def test_hip_graph_replays_match_eager(T):
    """One call captured in a HIP graph and replayed several times, with eager
    calls on other inputs in between: every replay leaves exactly the eager
    output (the library records no memset and leaves its counters at zero)."""
    case = gen.make_case(gen.REAL, T, seed=6600 + T, real_experts=True)
    other = gen.make_case(gen.REAL, T, seed=6700 + T, real_experts=True)
    d = case.dims
    dims = _gpu.dims_of(d)
    W = _gpu.device_weights(_gpu.config_case(1))
    x, x2 = _gpu.x_tensor(case), _gpu.x_tensor(other)
    out = torch.zeros((T, d.H), dtype=torch.int16, device="cuda")
    out2 = torch.zeros((T, d.H), dtype=torch.int16, device="cuda")
    ws = m.workspace(dims, T)
    m.moe_forward(dims, W.struct, x, T, out, ws=ws)
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.moe_forward(dims, W.struct, x, T, out, ws=ws)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep} differs from eager"
        m.moe_forward(dims, W.struct, x2, T, out2, ws=ws)  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [0, 1])
def test_few_token_give_up_is_loud_and_recoverable(cfg):
    """A few-token call whose bounded waits give up (forced from the host with
    the MOE_DEBUG_WAIT_GIVE_UP flag, so every kernel still exits normally)
    writes NaN to every output and counts the give-ups in the workspace; the
    next call on the same workspace is correct again."""
    case = _gpu.config_case(cfg)
    d, T = case.dims, case.T
    W = _gpu.device_weights(case)
    x = _gpu.x_tensor(case)
    ws = m.workspace(_gpu.dims_of(d), T)
    word = m.GIVE_UP_WORD_OFFSET // 4
    before = int(ws.view(torch.int32)[word].item())
    for mode in ("forward", "experts"):
        out = torch.zeros((T, d.H), dtype=torch.int16, device="cuda")
        dims = _gpu.dims_of(d, m.PATH_DECODE | m.DEBUG_WAIT_GIVE_UP)
        if mode == "forward":
            m.moe_forward(dims, W.struct, x, T, out, ws=ws)
        else:
            ids = torch.zeros((T, d.k), dtype=torch.int32, device="cuda")
            w = torch.full((T, d.k), 0.5, dtype=torch.float32, device="cuda")
            m.moe_experts_w4a16(dims, W.struct, x, T, ids, w, out, ws=ws)
        torch.cuda.synchronize()
        got = _gpu.half_to_f64(out)
        assert np.isnan(got).all(), f"{mode}: {np.isfinite(got).sum()} finite outputs after a give-up"
    after = int(ws.view(torch.int32)[word].item())
    assert after - before >= 2 * 8, "the give-ups were not counted"
    _gpu.log(f"give-up word {before} -> {after}")
    # the workspace is consistent: a normal call right after is correct
    out = torch.full((T, d.H), 0x7E00, dtype=torch.int16, device="cuda")
    ids = torch.full((T, d.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, d.k), -1.0, dtype=torch.float32, device="cuda")
    sig = torch.full((T,), -1.0, dtype=torch.float32, device="cuda")
    m.moe_forward(_gpu.dims_of(d, m.PATH_DECODE), W.struct, x, T, out, ids, w, sig, ws)
    torch.cuda.synchronize()
    g = dict(out=_gpu.half_to_f64(out), ids=ids.cpu().numpy(), w=w.cpu().numpy().astype(np.float64),
             sigma=sig.cpu().numpy().astype(np.float64))
    _gpu.check_forward(case, _gpu.config_oracle(cfg), g, f"cfg{cfg} after give-up")


def test_grid_bucketing_zipf_2048():
    """Above 1024 tokens the top-k writes per-workgroup expert counts and the
    sort runs over the grid (count, scan, scatter launches).  2048 Zipf-skewed
    tokens give the popular experts full tiles and last tiles of every class:
    parity against the oracle on every row, and two calls bit for bit."""
    case = gen.make_case(gen.REAL, 2048, seed=2048, bias="zipf1.1", c=8.0, real_experts=True)
    _gpu.log("grid-wide bucketing T=2048 zipf")
    g = _gpu.run_forward(case, reps=2)
    assert np.array_equal(g["out_raw"][0], g["out_raw"][1])
    r = ref.forward(case.x, case.weights, case.dims)
    _gpu.check_forward(case, r, g, "T2048-zipf")


def test_route_many_tokens():
    """Above 4096 tokens the router GEMM runs one workgroup per 32 tokens over
    every block of router rows (4127 tokens: a ragged last block)."""
    case = gen.make_case(gen.REAL, 4127, seed=4127, bias="normal0.5", c=8.0, real_experts=True)
    _gpu.log("route T=4127")
    r = ref.route(case.x, case.weights, case.dims)
    g = _gpu.run_route(case)
    _gpu.check_routing(case, r, g, "route T4127")
    scale = np.abs(r["logits"]).max()
    assert np.abs(g["logits"] - r["logits"]).max() <= 1e-5 * max(1.0, scale)
