"""Pin of the float64 oracle against the published implementation.

The Chimera notebook ("Qwen3.6-35B-A3B Decode on Chimera GPNPU", section 5.2)
checks its own NumPy reference of the MoE block against transformers'
``Qwen3_5MoeSparseMoeBlock`` and reports a relative difference of a few 1e-8
against a 1e-6 gate.  The same check is made here, on the CPU: the oracle's
dequantised weights are loaded into transformers' block (in float64) and the
two outputs are compared per token.  The RMSNorm of the sub-block is checked
against ``Qwen3_5MoeRMSNorm`` the same way.

transformers' router takes the softmax in float32 (its ``dtype=torch.float``),
so its routing weights carry float32 rounding: the per-row gate of 1e-6 is the
notebook's and still leaves two orders of magnitude over that rounding.  Its
``torch.topk`` does not fix an order for exact ties, so ids are compared as
sets, on rows whose k-th/(k+1)-th logit gap is clear of float32 rounding.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
transformers = pytest.importorskip("transformers")

from oracle import ref  # noqa: E402
from workloads import gen  # noqa: E402

try:
    from transformers.models.qwen3_5_moe import modeling_qwen3_5_moe as qmoe
    from transformers.models.qwen3_5_moe.configuration_qwen3_5_moe import Qwen3_5MoeTextConfig
except ImportError:  # an older transformers without the Qwen3.5-MoE family
    pytest.skip("transformers has no Qwen3.5-MoE modules", allow_module_level=True)

ROW_GATE = 1e-6      # the notebook's gate for reference vs transformers
GAP_CLEAR = 1e-5     # k-th/(k+1)-th logit gaps below this are left out of the id check


def _hf_block(case, experts_needed):
    """transformers' sparse MoE block in float64, holding the oracle's
    dequantised weights.  Experts no token selects keep zero weights: the
    block's router reads only the router rows, so they never reach the output."""
    d, W = case.dims, case.weights
    cfg = Qwen3_5MoeTextConfig(hidden_size=d.H, num_experts=d.E, num_experts_per_tok=d.k,
                               moe_intermediate_size=d.I, shared_expert_intermediate_size=d.Is,
                               hidden_act="silu")
    blk = qmoe.Qwen3_5MoeSparseMoeBlock(cfg)
    with torch.no_grad():
        for p in blk.parameters():
            p.data = torch.zeros(p.shape, dtype=torch.float64)
        wr = ref.dequant(W.router_q, W.router_s, d.G)
        blk.gate.weight.data = torch.from_numpy(wr[: d.E].copy())
        blk.shared_expert_gate.weight.data = torch.from_numpy(wr[d.E : d.E + 1].copy())
        for e in experts_needed:
            w13, w2 = ref.routed_expert_weights(W, d, int(e))
            blk.experts.gate_up_proj.data[e] = torch.from_numpy(w13)
            blk.experts.down_proj.data[e] = torch.from_numpy(w2)
        s13 = ref.dequant(W.sh13_q, W.sh13_s, d.G)
        blk.shared_expert.gate_proj.weight.data = torch.from_numpy(s13[: d.Is].copy())
        blk.shared_expert.up_proj.weight.data = torch.from_numpy(s13[d.Is :].copy())
        blk.shared_expert.down_proj.weight.data = torch.from_numpy(ref.dequant(W.sh2_q, W.sh2_s, d.G))
    return blk


def _compare(case):
    d = case.dims
    r = ref.forward(case.x, case.weights, d)
    blk = _hf_block(case, np.unique(r["ids"]))
    X = torch.from_numpy(ref.half_bits_to_f64(case.x))
    with torch.no_grad():
        out = blk(X[None]).reshape(case.T, d.H).numpy()
        _, _, hf_ids = blk.gate(X)
    clear = r["gap"] >= GAP_CLEAR
    assert clear.sum() >= case.T - 1, "the seeded case should have clear routing on (almost) every row"
    for t in np.nonzero(clear)[0]:
        assert set(hf_ids[t].tolist()) == set(r["ids"][t].tolist()), f"token {t}: routing differs"
    num = np.sqrt(((out - r["out"]) ** 2).sum(axis=1))
    den = np.sqrt((r["out"] ** 2).sum(axis=1))
    rel = num[clear] / den[clear]
    assert rel.max() <= ROW_GATE, f"per-row relative difference {rel.max():.3e}"
    return rel


def test_block_matches_transformers_toy_widths():
    case = gen.make_case(gen.TOY, 16, seed=7100)
    rel = _compare(case)
    assert rel.max() > 0  # float32 routing weights: a difference exists, below the gate


@pytest.mark.slow
def test_block_matches_transformers_real_widths():
    # hidden 2048, 256 experts, top-8, intermediates 512, with the same expert
    # set as the real-width workloads; 8 tokens touch up to 64 experts
    case = gen.make_case(gen.REAL, 8, seed=7101, real_experts=True)
    _compare(case)


def test_block_matches_transformers_skewed_router():
    # the 128-token workload's recipe (per-expert logit bias, shared direction)
    # at toy widths, so tokens share experts
    case = gen.make_case(gen.TOY, 24, seed=7102, bias="normal0.5", c=8.0)
    _compare(case)


def test_affine_block_matches_transformers():
    """The affine int4 experts (w = q s + b), dequantised by the oracle and
    loaded into transformers' block, agree with the oracle's forward."""
    case = gen.make_affine_case(gen.TOY, 16, seed=7103)
    assert case.weights.affine
    _compare(case)


@pytest.mark.parametrize("H", [256, 2048])
def test_rmsnorm_matches_transformers(H):
    """Qwen3_5MoeRMSNorm multiplies by (1 + w) in float32 and rounds once to
    the input dtype; the oracle's norm with gain = 1 + w, rounded to binary16,
    agrees to within one binary16 ulp."""
    rng = np.random.default_rng(H)
    h_bits = gen.f16_bits(rng.normal(0.0, 3.0, size=(5, H)))
    gain_bits = gen.f16_bits(rng.uniform(0.25, 1.9, size=H))
    w = ref.half_bits_to_f64(gain_bits) - 1.0  # exact in float32 as well
    eps = 1e-6
    norm = qmoe.Qwen3_5MoeRMSNorm(H, eps=eps)
    with torch.no_grad():
        norm.weight.data = torch.from_numpy(w.astype(np.float32))
        hf = norm(torch.from_numpy(h_bits.view(np.float16))).numpy()
    ours = ref.f64_to_half_bits(ref.rmsnorm(h_bits, gain_bits, eps)).view(np.float16)
    a = hf.astype(np.float64)
    b = ours.astype(np.float64)
    ulp = np.spacing(np.abs(b).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(a - b) <= ulp), f"max |diff| / ulp {np.max(np.abs(a - b) / ulp):.2f}"
    assert np.mean(a == b) > 0.95  # almost every element rounds identically


@pytest.mark.parametrize("H", [256, 2048])
def test_rmsnorm_plus_one_matches_transformers(H):
    """The oracle's (1 + w) form takes w as stored (transformers' weight) and
    agrees with Qwen3_5MoeRMSNorm to within one binary16 ulp, also for small w
    whose 1 + w binary16 cannot hold."""
    rng = np.random.default_rng(H + 1)
    h_bits = gen.f16_bits(rng.normal(0.0, 3.0, size=(5, H)))
    w_bits = gen.f16_bits(rng.uniform(-0.02, 0.02, size=H))
    eps = 1e-6
    norm = qmoe.Qwen3_5MoeRMSNorm(H, eps=eps)
    with torch.no_grad():
        norm.weight.data = torch.from_numpy(ref.half_bits_to_f64(w_bits).astype(np.float32))
        hf = norm(torch.from_numpy(h_bits.view(np.float16))).numpy().astype(np.float64)
    ours = ref.f64_to_half_bits(ref.rmsnorm(h_bits, w_bits, eps, plus_one=True)).view(np.float16).astype(np.float64)
    ulp = np.spacing(np.abs(ours).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(hf - ours) <= ulp)
    # read as the gain itself, the same array gives another norm altogether
    plain = ref.rmsnorm(h_bits, w_bits, eps)
    assert np.abs(plain - ours).max() > 0.5


def test_control_swapped_gate_up_is_caught(monkeypatch):
    """A planted mistake in the oracle (gate and up halves swapped) turns this
    pin red: the comparison with transformers is not blind to it."""
    orig = ref.swiglu_ffn

    def swapped(X, w13, w2, inter):
        return orig(X, np.concatenate([w13[inter:], w13[:inter]]), w2, inter)

    case = gen.make_case(gen.TOY, 16, seed=7100)
    r_good = ref.forward(case.x, case.weights, case.dims)
    monkeypatch.setattr(ref, "swiglu_ffn", swapped)
    with pytest.raises(AssertionError):
        _compare(case)
    monkeypatch.setattr(ref, "swiglu_ffn", orig)
    assert np.allclose(ref.forward(case.x, case.weights, case.dims)["out"], r_good["out"])
