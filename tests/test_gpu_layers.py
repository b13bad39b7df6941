"""Several MoE sub-blocks per call (moe_layers_forward) on the GPU.

The Chimera notebook ("Pipeline") runs the decoder's layers in one kernel per
token, every layer's weights a fixed offset from the previous layer's.  The
few-token path does the same for L sub-blocks in one launch; larger T runs L
launches.  Checked: against the float64 oracle's chain of sub-blocks (binary16
between layers), bit for bit against L chained moe_block_forward calls, with
a zero stride (one layer L times), with affine experts, over repeated calls on
one workspace, and on the forced give-up path.
"""
from __future__ import annotations

import ctypes
import functools

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import w4a16_routed_experts_amd as m  # noqa: E402
from oracle import ref  # noqa: E402
from tests import _gpu  # noqa: E402
from workloads import gen  # noqa: E402
from workloads.gen import f16_bits  # noqa: E402

EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.lib()


@functools.lru_cache(maxsize=4)
def _layers(dims_name, L, seed, affine=False):
    """L layers of weights (router, experts and shared expert all drawn anew per layer) and gains."""
    dims = {"real": gen.REAL, "toy": gen.TOY}[dims_name]
    Ws, gains = [], []
    for l in range(L):
        W, _, rng = gen.make_weights(dims, seed + 13 * l, bias="normal0.5", c=4.0)
        if affine:
            W = gen.with_affine_offsets(W, seed + 13 * l + 5)
        Ws.append(W)
        gains.append(f16_bits(rng.uniform(0.5, 1.5, size=dims.H)))
    return dims, tuple(Ws), tuple(gains)


def _h(dims, T, seed):
    rng = np.random.default_rng(seed)
    return f16_bits(rng.standard_normal((T, dims.H)) * rng.uniform(0.5, 4.0, size=(T, 1)))


def _oracle_chain(h, gains, Ws, dims):
    """The oracle's chain, and the smallest k-th/(k+1)-th logit gap met on the way."""
    out = ref.layers_forward(h, gains, EPS, Ws, dims)
    gap, hb = np.inf, h
    for g, W in zip(gains, Ws):
        r = ref.block_forward(hb, g, EPS, W, dims)
        gap = min(gap, float(r["gap"].min()))
        hb = ref.f64_to_half_bits(r["out"])
    return out, gap


def _stack(dims_name, L, seed, affine=False):
    key = (dims_name, L, seed, affine)
    if key not in _stacks:
        dims, Ws, gains = _layers(dims_name, L, seed, affine)
        _stacks.clear()  # one stack on the device at a time (a real-width layer is ~430 MB)
        _stacks[key] = m.LayerStack(list(Ws), list(gains))
    return _stacks[key]


_stacks = {}


def _layer_struct(stack, l):
    base = stack.struct
    return m.MoeWeights(*[(getattr(base, f) + l * stack.stride) if getattr(base, f) else None
                          for f in m.binding.WEIGHT_FIELDS])


def _run_layers(dims, stack, h, L, flags, stride=None, ws=None):
    T = h.shape[0]
    d = _gpu.dims_of(dims, flags)
    ht = torch.from_numpy(h.view(np.int16)).cuda()
    out = torch.full((T, dims.H), 0x7E00, dtype=torch.int16, device="cuda")
    ws = ws if ws is not None else m.layers_workspace(d, T, L)
    m.moe_layers_forward(d, stack.struct, stack.gain, stack.stride if stride is None else stride, L, EPS, ht, T, out,
                         ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().copy()


def _run_chained_blocks(dims, stack, h, L, flags, stride=None):
    T = h.shape[0]
    d = _gpu.dims_of(dims, flags)
    s = stack.stride if stride is None else stride
    cur = torch.from_numpy(h.view(np.int16)).cuda()
    ws = m.workspace(d, T)
    for l in range(L):
        W = _layer_struct(stack, 0) if s == 0 else _layer_struct(stack, l)
        nxt = torch.empty_like(cur)
        m.moe_block_forward(d, W, cur, stack.gain + l * s, EPS, T, nxt, ws=ws)
        cur = nxt
    torch.cuda.synchronize()
    return cur.cpu().numpy().copy()


def _check_oracle(out_bits, want, gap, label):
    assert gap >= _gpu.GAP_EXEMPT, f"{label}: a near-tie row ({gap:.2e}); pick another seed"
    got = out_bits.view(np.float16).astype(np.float64)
    err = _gpu.row_rel_l2(got, want)
    elem = _gpu.elem_err(got, want)
    _gpu.log(f"{label}: per-row rel L2 max {err.max():.3e}, largest element error {elem.max():.3e} of the row RMS")
    assert np.all(np.isfinite(got))
    assert err.max() <= _gpu.ROW_TOL
    assert elem.max() <= _gpu.ELEM_TOL


@pytest.mark.parametrize("dims_name,T,L,flags", [
    ("real", 1, 3, m.PATH_AUTO), ("real", 4, 2, m.PATH_DECODE), ("toy", 2, 4, m.PATH_AUTO),
    ("real", 12, 2, m.PATH_AUTO), ("real", 2, 2, m.PATH_CHUNK)])
def test_layers_match_oracle_and_chained_calls(dims_name, T, L, flags):
    seed = 8100 + 7 * T + L
    dims, Ws, gains = _layers(dims_name, L, seed)
    stack = _stack(dims_name, L, seed)
    h = _h(dims, T, seed + 1)
    _gpu.log(f"layers {dims_name} T={T} L={L} flags={flags} (layer stride {stack.stride} bytes)")
    got = _run_layers(dims, stack, h, L, flags)
    chained = _run_chained_blocks(dims, stack, h, L, flags)
    assert np.array_equal(got, chained), "one launch differs from L chained sub-block calls"
    want, gap = _oracle_chain(h, list(gains), list(Ws), dims)
    _check_oracle(got, want, gap, f"layers {dims_name} T{T} L{L}")


def test_zero_stride_repeats_one_layer():
    dims_name, T, L = "real", 1, 5
    seed = 8200
    dims, Ws, gains = _layers(dims_name, 1, seed)
    stack = _stack(dims_name, 1, seed)
    h = _h(dims, T, seed + 1)
    got = _run_layers(dims, stack, h, L, m.PATH_AUTO, stride=0)
    assert np.array_equal(got, _run_chained_blocks(dims, stack, h, L, m.PATH_AUTO, stride=0))
    want, gap = _oracle_chain(h, [gains[0]] * L, [Ws[0]] * L, dims)
    _check_oracle(got, want, gap, "layers stride 0 L5")


def test_affine_layers():
    dims_name, T, L = "real", 1, 2
    seed = 8300
    dims, Ws, gains = _layers(dims_name, L, seed, affine=True)
    stack = _stack(dims_name, L, seed, affine=True)
    h = _h(dims, T, seed + 1)
    flags = m.PATH_AUTO | m.FMT_AFFINE4
    got = _run_layers(dims, stack, h, L, flags)
    assert np.array_equal(got, _run_chained_blocks(dims, stack, h, L, flags))
    want, gap = _oracle_chain(h, list(gains), list(Ws), dims)
    _check_oracle(got, want, gap, "affine layers T1 L2")


def test_repeated_calls_on_one_workspace_and_give_up():
    """Calls with several layers advance the tags like any other call: results
    repeat bit for bit on one workspace, a forced give-up writes NaN and is
    counted, and the next call is right again."""
    dims_name, T, L = "real", 1, 3
    seed = 8100 + 7 * T + L
    dims, Ws, gains = _layers(dims_name, L, seed)
    stack = _stack(dims_name, L, seed)
    h = _h(dims, T, seed + 1)
    d = _gpu.dims_of(dims, m.PATH_AUTO)
    ws = m.layers_workspace(d, T, L)
    first = _run_layers(dims, stack, h, L, m.PATH_AUTO, ws=ws)
    for _ in range(2):
        assert np.array_equal(_run_layers(dims, stack, h, L, m.PATH_AUTO, ws=ws), first)
    before = int(ws[m.GIVE_UP_WORD_OFFSET:m.GIVE_UP_WORD_OFFSET + 4].view(torch.int32).item())
    bad = _run_layers(dims, stack, h, L, m.PATH_AUTO | m.DEBUG_WAIT_GIVE_UP, ws=ws)
    assert np.all(np.isnan(bad.view(np.float16).astype(np.float32)))
    after = int(ws[m.GIVE_UP_WORD_OFFSET:m.GIVE_UP_WORD_OFFSET + 4].view(torch.int32).item())
    assert after > before
    assert np.array_equal(_run_layers(dims, stack, h, L, m.PATH_AUTO, ws=ws), first)
    # a single-layer call on the same workspace is unaffected by the layers calls
    W0 = _layer_struct(stack, 0)
    ht = torch.from_numpy(h.view(np.int16)).cuda()
    o1 = torch.empty_like(ht)
    m.moe_block_forward(d, W0, ht, stack.gain, EPS, T, o1, ws=ws)
    o2 = torch.empty_like(ht)
    m.moe_block_forward(d, W0, ht, stack.gain, EPS, T, o2, ws=m.workspace(d, T))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert ctypes.sizeof(W0) == ctypes.sizeof(m.MoeWeights)
