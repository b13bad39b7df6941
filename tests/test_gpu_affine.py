"""Affine int4 routed experts (w = q s + b, unsigned 4-bit codes) on the GPU.

The TensorFold PR runs a 4-bit affine checkpoint ("Receipts") and its review
thread speaks of affine gathers at the layer's widths; the pages give no
layout, so the format read here is the plain one: unsigned codes q in [0, 15],
a binary16 scale s and offset b per group of 64, w = q s + b.  The routed
experts are read that way with the flag MOE_FMT_AFFINE4 and two offset arrays
laid out like the scales.  The float64 oracle dequantises q s + b per group;
both paths are compared with it to the same bar as the symmetric format, and
two planted mistakes (the flag left off, so the codes are read as signed and
the offsets ignored; one offset of one down row doubled on the device) must
fail that bar.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import w4a16_routed_experts_amd as m  # noqa: E402
from oracle import ref  # noqa: E402
from tests import _gpu  # noqa: E402
from workloads import gen  # noqa: E402

AFF = m.FMT_AFFINE4


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.lib()


@functools.lru_cache(maxsize=8)
def _case(dims_name, T, seed):
    dims = {"real": gen.REAL, "toy": gen.TOY}[dims_name]
    return gen.make_affine_case(dims, T, seed, bias="normal0.5", c=4.0, real_experts=dims_name == "real")


@functools.lru_cache(maxsize=8)
def _oracle(dims_name, T, seed):
    c = _case(dims_name, T, seed)
    return ref.forward(c.x, c.weights, c.dims)


@pytest.mark.parametrize("dims_name,T,path", [
    ("real", 1, m.PATH_DECODE), ("real", 3, m.PATH_DECODE), ("real", 4, m.PATH_CHUNK),
    ("real", 70, m.PATH_AUTO), ("toy", 1, m.PATH_DECODE), ("toy", 45, m.PATH_AUTO)])
def test_affine_forward(dims_name, T, path):
    case = _case(dims_name, T, 7300 + T)
    _gpu.log(f"affine forward {dims_name} T={T} path={path}")
    g = _gpu.run_forward(case, flags=path | AFF)
    _gpu.check_forward(case, _oracle(dims_name, T, 7300 + T), g, f"affine {dims_name} T{T}")


@pytest.mark.parametrize("T,path,pool", [(1, m.PATH_AUTO, 0), (2, m.PATH_CHUNK, 0), (40, m.PATH_AUTO, 0),
                                         (40, m.PATH_AUTO, 3)])
def test_affine_experts_given_routing(T, path, pool):
    """pool > 0: every slot routed to one of `pool` experts, so their tiles take
    the 32-row-block grouped GEMM (more than 16 rows) rather than the narrow one."""
    case = _case("real", T, 7400 + T)
    d = case.dims
    rng = np.random.default_rng(74 + T + pool)
    ids = rng.integers(0, d.E, size=(T, d.k)) if pool == 0 else (rng.integers(0, pool, size=(T, d.k)) * 37) % d.E
    ids[-1, -1] = -1  # dropped
    w = rng.uniform(0.05, 1.0, size=(T, d.k))
    _gpu.log(f"affine experts with caller routing T={T} path={path} pool={pool}")
    g = _gpu.run_experts(case, ids, w, flags=path | AFF)
    want = np.zeros((T, d.H))
    for t in range(T):
        for i in range(d.k):
            if 0 <= ids[t, i] < d.E:
                want[t] += ref.experts(case.x[t:t + 1], ids[t:t + 1, i:i + 1], w[t:t + 1, i:i + 1],
                                       case.weights, d)[0]
    err = _gpu.row_rel_l2(g, want)
    elem = _gpu.elem_err(g, want)
    _gpu.log(f"  rel L2 max {err.max():.3e}, largest element error {elem.max():.3e} of the row RMS")
    assert err.max() <= _gpu.ROW_TOL
    assert elem.max() <= _gpu.ELEM_TOL


def _offset_doubled(case, e):
    d = case.dims
    W = _gpu.device_weights(case)
    t = {f: v.clone() for f, v in W.tensors.items()}
    b = t["w2_b"][e].view(torch.float16)
    b[d.H // 3, 0] *= 2
    return m.DeviceWeights(tensors=t)


def _run_with(case, W, flags):
    T, d = case.T, case.dims
    dims = _gpu.dims_of(d, flags)
    out = torch.full((T, d.H), 0x7E00, dtype=torch.int16, device="cuda")
    ids = torch.full((T, d.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, d.k), -1.0, dtype=torch.float32, device="cuda")
    sig = torch.full((T,), -1.0, dtype=torch.float32, device="cuda")
    m.moe_forward(dims, W.struct, _gpu.x_tensor(case), T, out, ids, w, sig, m.workspace(dims, T))
    torch.cuda.synchronize()
    return dict(out=_gpu.half_to_f64(out), ids=ids.cpu().numpy(), w=w.cpu().numpy().astype(np.float64),
                sigma=sig.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("T,path", [(1, m.PATH_DECODE), (32, m.PATH_CHUNK)])
@pytest.mark.parametrize("control", ["flag_off", "down_offset_doubled"])
def test_affine_controls_fail(T, path, control):
    case = _case("real", T, 7500 + T)
    r = _oracle("real", T, 7500 + T)
    if control == "flag_off":
        W, flags = _gpu.device_weights(case), path
    else:
        W, flags = _offset_doubled(case, int(r["ids"][0, 0])), path | AFF
    g = _run_with(case, W, flags)
    with pytest.raises(AssertionError):
        _gpu.check_forward(case, r, g, f"affine control {control} T{T}")
    _gpu.log(f"affine control {control} T={T} path={path}: red as planted")
