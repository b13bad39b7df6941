"""GPU parity of the MoE sub-block (post-attention RMSNorm -> block -> residual
add) against the float64 oracle's block_forward, on both paths."""
from __future__ import annotations

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
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.lib()


def _inputs(case, seed):
    """Residual rows at varied scales (the norm has work to do) and a gain vector."""
    rng = np.random.default_rng(seed)
    scale = rng.uniform(0.25, 4.0, size=(case.T, 1))
    h_bits = f16_bits(gen_x(case) * scale)
    gain_bits = f16_bits(rng.uniform(0.5, 1.5, size=case.dims.H))
    return h_bits, gain_bits


def gen_x(case):
    return ref.half_bits_to_f64(case.x)


def _run_block(case, h_bits, gain_bits, flags):
    T, d = case.T, case.dims
    dims = _gpu.dims_of(d, flags)
    W = _gpu.device_weights(case)
    h = torch.from_numpy(h_bits.view(np.int16)).cuda()
    g = torch.from_numpy(gain_bits.view(np.int16)).cuda()
    out = torch.full((T, d.H), 0x7E00, dtype=torch.int16, device="cuda")  # NaN fill
    ids = torch.full((T, d.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, d.k), -1.0, dtype=torch.float32, device="cuda")
    sig = torch.full((T,), -1.0, dtype=torch.float32, device="cuda")
    ws = m.workspace(dims, T)
    m.moe_block_forward(dims, W.struct, h, g, EPS, T, out, ids, w, sig, ws)
    torch.cuda.synchronize()
    assert torch.equal(h.cpu(), torch.from_numpy(h_bits.view(np.int16))), "the residual stream was modified"
    return dict(out=_gpu.half_to_f64(out), ids=ids.cpu().numpy(), w=w.cpu().numpy().astype(np.float64),
                sigma=sig.cpu().numpy().astype(np.float64))


def _check(case, h_bits, gain_bits, gpu, label, plus_one=False):
    d = case.dims
    r = ref.block_forward(h_bits, gain_bits, EPS, case.weights, d, plus_one=plus_one)
    differ = _gpu.check_routing(case, r, gpu, label, w_tol=_gpu.W_TOL_NORMED)
    want = r["out"].copy()
    lr = r["logits"][:, : d.E]
    for t in differ:  # near-tie rows the GPU routed otherwise: the oracle with the GPU's ids
        ids_g = gpu["ids"][t : t + 1].astype(np.int64)
        w_g = ref.softmax_renormalised(lr[t : t + 1], ids_g)
        routed = ref.experts(r["a_bits"][t : t + 1], ids_g, w_g, case.weights, d)
        want[t] = ref.half_bits_to_f64(h_bits[t]) + routed[0] + r["sigma"][t] * r["shared"][t]
    err = _gpu.row_rel_l2(gpu["out"], want)
    _gpu.log(f"{label}: per-row rel L2 max {err.max():.3e} median {np.median(err):.3e}")
    assert np.all(np.isfinite(gpu["out"])), f"{label}: non-finite output"
    assert err.max() <= _gpu.ROW_TOL, f"{label}: row {int(err.argmax())} rel L2 {err.max():.3e}"


@pytest.mark.parametrize("cfg,flags", [(0, m.PATH_AUTO), (1, m.PATH_AUTO), (2, m.PATH_AUTO), (3, m.PATH_AUTO),
                                       (4, m.PATH_AUTO), (0, m.PATH_CHUNK), (1, m.PATH_CHUNK)])
def test_block_configs(cfg, flags):
    case = _gpu.config_case(cfg)
    _gpu.log(f"sub-block config {cfg} ({case.name}) T={case.T} flags={flags}")
    h_bits, gain_bits = _inputs(case, 700 + cfg)
    gpu = _run_block(case, h_bits, gain_bits, flags)
    _check(case, h_bits, gain_bits, gpu, f"block-cfg{cfg}-f{flags}")


# 4127 tokens: the router runs one workgroup per 32 tokens over all row blocks
# (the norm computed once per token block; a ragged last block) and the sort
# runs over the grid
@pytest.mark.parametrize("T,flags", [(3, m.PATH_DECODE), (3, m.PATH_CHUNK), (70, m.PATH_AUTO), (4127, m.PATH_AUTO)])
def test_block_token_counts(T, flags):
    case = gen.make_case(gen.REAL, T, seed=7100 + T, real_experts=True)
    _gpu.log(f"sub-block T={T} flags={flags}")
    h_bits, gain_bits = _inputs(case, 7200 + T)
    gpu = _run_block(case, h_bits, gain_bits, flags)
    _check(case, h_bits, gain_bits, gpu, f"block-T{T}-f{flags}")


# other admitted widths: 512 (toy-sized rows), 4096 (the router takes two load
# batches per row, so the norm needs its own first pass over x)
@pytest.mark.parametrize("shape", [(512, 32, 4, 128, 256), (4096, 64, 8, 1024, 128)],
                         ids=lambda s: "H{}E{}k{}I{}Is{}".format(*s))
@pytest.mark.parametrize("T,flags", [(1, m.PATH_AUTO), (2, m.PATH_CHUNK), (10, m.PATH_AUTO)])
def test_block_other_widths(shape, T, flags):
    H, E, k, I, Is = shape
    d = gen.Dims(H=H, E=E, k=k, I=I, Is=Is)
    case = gen.make_case(d, T, seed=7300 + H + T)
    _gpu.log(f"sub-block shape {shape} T={T} flags={flags}")
    h_bits, gain_bits = _inputs(case, 7400 + H + T)
    gpu = _run_block(case, h_bits, gain_bits, flags)
    _check(case, h_bits, gain_bits, gpu, f"block-{shape}-T{T}-f{flags}")


@pytest.mark.parametrize("T", [40, 70])
def test_block_narrow_rows_chunk(T):
    """Hidden 256: four 64-groups, fewer than the router GEMM's eight waves, so
    half its waves have no group; they must still take part in the workgroup
    barriers of the norm (a wave that skipped them once left the partial sums
    of tokens 8..31 of every 32-token block unfinished when they were added)."""
    d = gen.Dims(H=256, E=8, k=2, I=64, Is=64)
    case = gen.make_case(d, T, seed=7600 + T)
    _gpu.log(f"sub-block hidden 256 T={T} (grouped-GEMM path)")
    h_bits, gain_bits = _inputs(case, 7700 + T)
    gpu = _run_block(case, h_bits, gain_bits, m.PATH_CHUNK)
    _check(case, h_bits, gain_bits, gpu, f"block-H256-T{T}")


@pytest.mark.parametrize("T,flags", [(3, m.PATH_DECODE), (40, m.PATH_CHUNK)])
def test_block_gain_plus_one(T, flags):
    """MOE_NORM_GAIN_PLUS_ONE: the gain array holds w and the norm multiplies by
    1 + w formed in fp32 (w here is small, so 1 + w would lose most of its bits
    if rounded to binary16 first)."""
    case = gen.make_case(gen.REAL, T, seed=9300 + T, real_experts=True)
    rng = np.random.default_rng(9301 + T)
    h_bits = f16_bits(gen_x(case) * rng.uniform(0.5, 3.0, size=(T, 1)))
    w_bits = f16_bits(rng.uniform(-0.02, 0.02, size=case.dims.H))
    gpu = _run_block(case, h_bits, w_bits, flags | m.NORM_GAIN_PLUS_ONE)
    _check(case, h_bits, w_bits, gpu, f"block (1 + w) T{T}", plus_one=True)
    # without the flag the same array is the gain itself: a different result
    other = _run_block(case, h_bits, w_bits, flags)
    assert _gpu.row_rel_l2(other["out"], gpu["out"]).max() > 0.1


@pytest.mark.parametrize("T,flags", [(3, m.PATH_DECODE), (40, m.PATH_CHUNK)])
def test_block_residual_in_the_thousands(T, flags):
    """A residual stream with elements in the thousands: the norm's sums of
    squares and the residual add stay exact enough on both paths."""
    case = gen.make_case(gen.REAL, T, seed=9400 + T, real_experts=True)
    rng = np.random.default_rng(9401 + T)
    h_bits = f16_bits(gen_x(case) * rng.uniform(256.0, 1024.0, size=(T, 1)))
    gain_bits = f16_bits(rng.uniform(0.5, 1.5, size=case.dims.H))
    assert np.abs(ref.half_bits_to_f64(h_bits)).max() > 1000.0
    gpu = _run_block(case, h_bits, gain_bits, flags)
    _check(case, h_bits, gain_bits, gpu, f"block large residual T{T}")
