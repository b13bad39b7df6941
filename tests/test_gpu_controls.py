"""Planted mistakes on the GPU side, and the pages' own gates.

Controls (the TensorFold PR, "Receipts": controls that must go red as
planted): the device copy of the weights is changed in ways a kernel mistake
could mimic, while the oracle keeps the true weights, and the comparator must
fail on every such call, on the few-token path (the single-token workload) and
on the grouped-GEMM path (the 32-token workload).  The changes: one routed
expert's gate and up halves swapped; the nibbles of 16 of its gate rows
swapped; one group scale of one of its down rows doubled; the shared expert's
down scales of one row doubled; two router rows exchanged.

Gates (the Chimera notebook, "Summary"): router exact top-k and score error
under 2e-3; routed half cosine >= 0.98 with norm ratio within 2%; complete
block cosine >= 0.999 with norm ratio within 2%, and the shared branch moving
the output at least half as far from the routed half as it does in the
reference.  They are computed for all five workloads and logged beside the
stricter per-row bar that the parity tests apply.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import w4a16_routed_experts_amd as m  # noqa: E402
from oracle import ref  # noqa: E402
from tests import _gpu  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.lib()


def _perturbed(case, control, e):
    """A private device copy of the case's weights with one planted change."""
    d = case.dims
    W = _gpu.device_weights(case)
    t = {f: v.clone() for f, v in W.tensors.items()}
    I = d.I
    if control == "gate_up_swapped":
        for f in ("w13_q", "w13_s"):
            a = t[f][e]
            a.copy_(torch.cat([a[I:].clone(), a[:I].clone()]))
    elif control == "nibbles_swapped":
        rows = t["w13_q"][e, 0:16]
        rows.copy_(((rows >> 4) | (rows << 4)) & 0xFF)
    elif control == "down_group_scale_doubled":
        s = t["w2_s"][e].view(torch.float16)
        s[d.H // 3, 0] *= 2
    elif control == "shared_down_row_scaled":
        s = t["sh2_s"].view(torch.float16)
        s[d.H // 2] *= 2
    elif control == "router_rows_exchanged":
        other = (e + d.E // 2) % d.E
        for f in ("router_q", "router_s"):
            a = t[f]
            tmp = a[e].clone()
            a[e].copy_(a[other])
            a[other].copy_(tmp)
    else:
        raise ValueError(control)
    return m.DeviceWeights(tensors=t)


def _run(case, W, flags):
    T, d = case.T, case.dims
    dims = _gpu.dims_of(d, flags)
    x = _gpu.x_tensor(case)
    out = torch.full((T, d.H), 0x7E00, dtype=torch.int16, device="cuda")
    ids = torch.full((T, d.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, d.k), -1.0, dtype=torch.float32, device="cuda")
    sig = torch.full((T,), -1.0, dtype=torch.float32, device="cuda")
    m.moe_forward(dims, W.struct, x, T, out, ids, w, sig, m.workspace(dims, T))
    torch.cuda.synchronize()
    return dict(out=_gpu.half_to_f64(out), ids=ids.cpu().numpy(), w=w.cpu().numpy().astype(np.float64),
                sigma=sig.cpu().numpy().astype(np.float64))


CONTROLS = ["gate_up_swapped", "nibbles_swapped", "down_group_scale_doubled", "shared_down_row_scaled",
            "router_rows_exchanged"]


@pytest.mark.parametrize("control", CONTROLS)
@pytest.mark.parametrize("cfg,flags", [(1, m.PATH_DECODE), (2, m.PATH_CHUNK)])
def test_planted_control_goes_red(cfg, flags, control):
    case = _gpu.config_case(cfg)
    r = _gpu.config_oracle(cfg)
    # the first token's top expert: routed in every workload
    e = int(r["ids"][0, 0])
    good = _run(case, _gpu.device_weights(case), flags)
    _gpu.check_forward(case, r, good, f"cfg{cfg} unperturbed")
    bad = _run(case, _perturbed(case, control, e), flags)
    with pytest.raises(AssertionError) as exc:
        _gpu.check_forward(case, r, bad, f"cfg{cfg} {control}")
    _gpu.log(f"control {control} on cfg{cfg} (flags {flags}) red as planted: {str(exc.value).splitlines()[0]}")


def _cos(a, b):
    return float((a * b).sum() / np.sqrt((a * a).sum() * (b * b).sum()))


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_pages_gates(cfg):
    case = _gpu.config_case(cfg)
    d, T = case.dims, case.T
    r = _gpu.config_oracle(cfg)
    g = _gpu.run_forward(case)
    _gpu.check_routing(case, r, g, f"gates cfg{cfg}")
    same = np.array([set(g["ids"][t]) == set(r["ids"][t]) for t in range(T)])
    score_err = 0.0
    for t in np.nonzero(same)[0]:
        ref_w = dict(zip(r["ids"][t].tolist(), r["w"][t].tolist()))
        score_err = max(score_err, max(abs(wv - ref_w[e]) for e, wv in zip(g["ids"][t].tolist(), g["w"][t].tolist())))
    # the routed half on the oracle's routing, through moe_experts_w4a16
    routed = _gpu.run_experts(case, r["ids"], r["w"])
    cos_routed, ratio_routed = _cos(routed, r["routed"]), float(np.linalg.norm(routed) / np.linalg.norm(r["routed"]))
    out = g["out"]
    cos_block, ratio_block = _cos(out, r["out"]), float(np.linalg.norm(out) / np.linalg.norm(r["out"]))
    delta_gpu = float(np.linalg.norm(out - routed) / np.linalg.norm(routed))
    delta_ref = float(np.linalg.norm(r["out"] - r["routed"]) / np.linalg.norm(r["routed"]))
    _gpu.log(f"gates cfg{cfg} ({case.name}): router same top-k on {int(same.sum())}/{T} rows "
             f"({int((r['gap'] < _gpu.GAP_EXEMPT).sum())} near-tie rows), score error {score_err:.2e}; "
             f"routed half cos {cos_routed:.7f} ratio {ratio_routed:.6f}; block cos {cos_block:.7f} "
             f"ratio {ratio_block:.6f}; shared-branch delta {100 * delta_gpu:.3f}% vs {100 * delta_ref:.3f}%")
    assert score_err < 2e-3
    assert cos_routed >= 0.98 and abs(ratio_routed - 1) <= 0.02
    assert cos_block >= 0.999 and abs(ratio_block - 1) <= 0.02
    assert delta_gpu >= 0.5 * delta_ref
