"""moe_forward_noalloc (the entry point that allocates nothing) against
moe_forward on the same inputs, through the C ABI.

Two calls in a row share the library's static scratch: a 70-token chunk
(grouped-GEMM path) and then a single token (few-token path), so the second
call runs on scratch the first one used.  Each output must equal moe_forward's
bit for bit (the same kernels run on the same inputs; their results do not
depend on where the scratch lives) and meet the parity bar against the float64
oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import w4a16_routed_experts_amd as m  # noqa: E402
from oracle import ref  # noqa: E402
from tests import _gpu  # noqa: E402
from workloads import gen  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.lib()


def _run_noalloc(case):
    T, d = case.T, case.dims
    dims = _gpu.dims_of(d)
    W = _gpu.device_weights(case)
    x = _gpu.x_tensor(case)
    out = torch.full((T, d.H), 0x7E00, dtype=torch.int16, device="cuda")
    ids = torch.full((T, d.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, d.k), -1.0, dtype=torch.float32, device="cuda")
    sig = torch.full((T,), -1.0, dtype=torch.float32, device="cuda")
    m.moe_forward_noalloc(dims, W.struct, x, T, out, ids, w, sig)
    torch.cuda.synchronize()
    return dict(out=_gpu.half_to_f64(out), out_raw=[out.cpu().numpy()], ids=ids.cpu().numpy(),
                w=w.cpu().numpy().astype(np.float64), sigma=sig.cpu().numpy().astype(np.float64))


def test_noalloc_matches_forward_two_calls():
    big = gen.make_case(gen.REAL, 70, seed=7070, bias="normal0.5", c=8.0, real_experts=True)
    small = _gpu.config_case(1)
    for label, case in (("T=70 chunk", big), ("T=1 decode", small)):
        _gpu.log(f"noalloc {label}")
        got = _run_noalloc(case)
        want = _gpu.run_forward(case)
        assert np.array_equal(got["out_raw"][0], want["out_raw"][0]), f"{label}: differs from moe_forward"
        assert np.array_equal(got["ids"], want["ids"]), f"{label}: routing differs from moe_forward"
        r = ref.forward(case.x, case.weights, case.dims)
        _gpu.check_forward(case, r, got, f"noalloc {label}")


def test_noalloc_refuses_oversized_call():
    d = gen.REAL
    dims = _gpu.dims_of(d)
    T = next(t for t in range(1, 4097) if m.moe_workspace_bytes(dims, t) > m.NOALLOC_SCRATCH_BYTES)
    case = gen.make_case(gen.REAL, T, seed=7071, real_experts=True)
    W = _gpu.device_weights(case)
    x = _gpu.x_tensor(case)
    out = torch.zeros((T, d.H), dtype=torch.int16, device="cuda")
    st = m.moe_forward_noalloc(dims, W.struct, x, T, out, raise_on_error=False)
    assert st == -7
    torch.cuda.synchronize()
    assert int(out.abs().sum()) == 0  # nothing was enqueued
