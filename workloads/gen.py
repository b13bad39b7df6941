"""Seeded generators for the five MoE-layer workloads and for ad-hoc test cases.

Storage format produced here (it is also what the C ABI consumes):

* activations ``x``: ``[T][H]`` IEEE binary16, kept as ``uint16`` bit patterns;
* router ``router_q``: ``[E+1][H]`` int8, row ``E`` is the shared-expert gate
  row stacked under the ``E`` router rows (the TensorFold PR, "Design": the
  router runs on stored 8-bit group-64 rows stacked with the shared gate);
* routed experts ``w13_q``: ``[E][2I][H/2]`` bytes of int4 codes (rows ``0..I-1``
  gate, ``I..2I-1`` up) and ``w2_q``: ``[E][H][I/2]`` (the Chimera notebook,
  pipeline intro: routed experts int4);
* shared expert ``sh13_q``: ``[2Is][H]`` int8 (gate rows, then up rows) and
  ``sh2_q``: ``[H][Is]`` int8 (same notebook: shared expert int8);
* every ``*_s`` array holds binary16 group scales ``[rows][K/G]``, one per run
  of ``G`` consecutive input (K) elements of a row.

An int4 code is a two's-complement nibble in ``[-8, 7]``; element ``2j`` of a
row sits in the low nibble of byte ``j``, element ``2j+1`` in the high nibble.
int8 codes are two's complement.

The five configurations follow the workloads the layer is specified on: a toy
layer (hidden 256, 8 experts, top-2, intermediates 64), single-token decode,
32-token batched decode, a 128-token prefill chunk with a N(0, 0.5) per-expert
logit bias, and a 512-token chunk with Zipf(1.1) expert popularity and about
5% near-tied rows.  Widths follow the Qwen3.6-35B-A3B geometry (the Chimera
notebook, pipeline intro: hidden 2048, 256 experts, top-8, shared intermediate
512; the TensorFold PR, "Design": 256 experts of 512).
"""
from __future__ import annotations

import functools
import os
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

NEAR_TIE_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "near_ties_cfg4.txt")

WEIGHT_SEED_REAL = 999


@dataclass(frozen=True)
class Dims:
    H: int      # hidden width
    E: int      # routed experts
    k: int      # experts selected per token
    I: int      # routed-expert intermediate width
    Is: int     # shared-expert intermediate width
    G: int = 64  # quantisation group along K


@dataclass
class Weights:
    """One layer's weights in the storage format (numpy, host memory)."""
    router_q: np.ndarray  # int8   [E+1][H]
    router_s: np.ndarray  # uint16 [E+1][H/G]
    w13_q: np.ndarray     # uint8  [E][2I][H/2]
    w13_s: np.ndarray     # uint16 [E][2I][H/G]
    w2_q: np.ndarray      # uint8  [E][H][I/2]
    w2_s: np.ndarray      # uint16 [E][H][I/G]
    sh13_q: np.ndarray    # int8   [2Is][H]
    sh13_s: np.ndarray    # uint16 [2Is][H/G]
    sh2_q: np.ndarray     # int8   [H][Is]
    sh2_s: np.ndarray     # uint16 [H][Is/G]
    # affine int4 routed experts: unsigned codes in w13_q / w2_q and one
    # binary16 offset per group; None for the symmetric (two's-complement) form
    w13_b: Optional[np.ndarray] = None  # uint16 [E][2I][H/G]
    w2_b: Optional[np.ndarray] = None   # uint16 [E][H][I/G]

    FIELDS = ("router_q", "router_s", "w13_q", "w13_s", "w2_q", "w2_s",
              "sh13_q", "sh13_s", "sh2_q", "sh2_s")
    AFFINE_FIELDS = ("w13_b", "w2_b")

    @property
    def affine(self) -> bool:
        return self.w13_b is not None

    def items(self):
        fields = self.FIELDS + (self.AFFINE_FIELDS if self.affine else ())
        return [(f, getattr(self, f)) for f in fields]

    def nbytes(self) -> int:
        return sum(a.nbytes for _, a in self.items())


@dataclass
class Case:
    """A full layer invocation: dims, weights and the activations."""
    name: str
    dims: Dims
    weights: Weights
    x: np.ndarray               # uint16 [T][H] binary16 bits
    meta: Dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.x.shape[0])


TOY = Dims(H=256, E=8, k=2, I=64, Is=64, G=64)
REAL = Dims(H=2048, E=256, k=8, I=512, Is=512, G=64)

# bias: how per-expert additive logit offsets are injected through the data
# c: weight of the shared unit direction u in every activation row
CONFIGS = {
    0: dict(name="toy", dims=TOY, T=1, bias="none", c=0.0, near_ties=0),
    1: dict(name="decode_t1", dims=REAL, T=1, bias="none", c=0.0, near_ties=0),
    2: dict(name="batched_decode_t32", dims=REAL, T=32, bias="none", c=0.0, near_ties=0),
    3: dict(name="prefill_t128", dims=REAL, T=128, bias="normal0.5", c=8.0, near_ties=0),
    4: dict(name="zipf_chunk_t512", dims=REAL, T=512, bias="zipf1.1", c=8.0, near_ties=26),
}


# ---------------------------------------------------------------------------
# format helpers
# ---------------------------------------------------------------------------

def f16_bits(a) -> np.ndarray:
    """Round to binary16 (round-to-nearest-even) and return the bit patterns."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Pack int4 codes (last axis even length, values in [-8, 7]) two per byte."""
    q = np.asarray(q)
    if q.shape[-1] % 2:
        raise ValueError("int4 rows need an even length")
    if q.min(initial=0) < -8 or q.max(initial=0) > 7:
        raise ValueError("int4 code out of [-8, 7]")
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def _scales_uniform(rng, shape, lo, hi) -> np.ndarray:
    return f16_bits(rng.uniform(lo, hi, size=shape))


def _quantise_rows_int8(r: np.ndarray, G: int):
    """Group-absmax int8 codes for freshly drawn float rows r [R][K]."""
    R, K = r.shape
    g = r.reshape(R, K // G, G)
    amax = np.abs(g).max(axis=-1)
    s_bits = f16_bits(amax / 127.0)
    s = s_bits.view(np.float16).astype(np.float64)
    if not np.all(s > 0):
        raise ValueError("degenerate all-zero group")
    q = np.clip(np.rint(g / s[..., None]), -127, 127).astype(np.int8).reshape(R, K)
    return q, s_bits


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------

def _uniform_bytes(rng, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def _expert_and_shared(dims: Dims, rng):
    H, E, I, Is, G = dims.H, dims.E, dims.I, dims.Is, dims.G
    # Uniform bytes are two independent uniform nibbles, i.e. int4 codes
    # uniform on [-8, 7].
    w13_q = _uniform_bytes(rng, (E, 2 * I, H // 2))
    w13_s = _scales_uniform(rng, (E, 2 * I, H // G), 0.005, 0.02)
    w2_q = _uniform_bytes(rng, (E, H, I // 2))
    w2_s = _scales_uniform(rng, (E, H, I // G), 0.005, 0.02)
    # int8 shared expert; the scale range is divided by 16 so its weights
    # have about the same spread as the routed int4 weights.
    sh13_q = rng.integers(-127, 128, size=(2 * Is, H), dtype=np.int8)
    sh13_s = _scales_uniform(rng, (2 * Is, H // G), 0.005 / 16, 0.02 / 16)
    sh2_q = rng.integers(-127, 128, size=(H, Is), dtype=np.int8)
    sh2_s = _scales_uniform(rng, (H, Is // G), 0.005 / 16, 0.02 / 16)
    return dict(w13_q=w13_q, w13_s=w13_s, w2_q=w2_q, w2_s=w2_s,
                sh13_q=sh13_q, sh13_s=sh13_s, sh2_q=sh2_q, sh2_s=sh2_s)


def _expert_bias(dims: Dims, bias: str, rng) -> np.ndarray:
    E = dims.E
    if bias == "none":
        return np.zeros(E)
    if bias == "normal0.5":
        return rng.normal(0.0, 0.5, size=E)
    if bias == "zipf1.1":
        rank = rng.permutation(E) + 1
        return -1.1 * np.log(rank.astype(np.float64))
    raise ValueError(bias)


def _unit_vector(H: int, rng) -> np.ndarray:
    u = rng.normal(size=H)
    return u / np.linalg.norm(u)


def _router(dims: Dims, bias: np.ndarray, u: np.ndarray, c: float, rng):
    """Router rows r_e ~ N(0, 1/H) plus (b_e / c) u, and a shared-gate row."""
    H, E = dims.H, dims.E
    r = rng.normal(0.0, 1.0 / np.sqrt(H), size=(E + 1, H))
    if c > 0:
        r[:E] += (bias / c)[:, None] * u[None, :]
    return _quantise_rows_int8(r, dims.G)


@functools.lru_cache(maxsize=4)
def _real_expert_set(dims: Dims, seed: int):
    return _expert_and_shared(dims, np.random.default_rng(seed))


def make_weights(dims: Dims, seed: int, bias: str = "none", c: float = 0.0,
                 expert_seed: Optional[int] = None):
    """Return (Weights, u): router from ``seed``, experts from ``expert_seed``."""
    rng = np.random.default_rng(seed)
    u = _unit_vector(dims.H, rng)
    b = _expert_bias(dims, bias, rng)
    router_q, router_s = _router(dims, b, u, c, rng)
    if expert_seed is None:
        ex = _expert_and_shared(dims, rng)
    else:
        ex = _real_expert_set(dims, expert_seed)
    return Weights(router_q=router_q, router_s=router_s, **ex), u, rng


def make_x(T: int, H: int, rng, c: float = 0.0, u: Optional[np.ndarray] = None) -> np.ndarray:
    """fp16 rows with unit RMS: sqrt(1 - c^2/H) n + c u, n ~ N(0, I)."""
    n = rng.normal(size=(T, H))
    if c > 0:
        x = np.sqrt(1.0 - c * c / H) * n + c * u[None, :]
    else:
        x = n
    return f16_bits(x)


# ---------------------------------------------------------------------------
# near-tie rows (512-token chunk)
# ---------------------------------------------------------------------------

def read_near_tie_edits(path: str = NEAR_TIE_FILE):
    """Parse ``token coord fp16_hex`` lines; '#' starts a comment."""
    edits = []
    if not os.path.exists(path):
        return edits
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            t, j, bits = line.split()
            edits.append((int(t), int(j), int(bits, 16)))
    return edits


def apply_edits(x: np.ndarray, edits) -> np.ndarray:
    x = x.copy()
    for t, j, bits in edits:
        x[t, j] = bits
    return x


# ---------------------------------------------------------------------------
# public entry points
# ---------------------------------------------------------------------------

def make_config(i: int, near_ties: bool = True) -> Case:
    """The seeded workload of configuration ``i`` (0..4)."""
    cfg = CONFIGS[i]
    dims = cfg["dims"]
    seed = 1000 + i
    expert_seed = None if i == 0 else WEIGHT_SEED_REAL
    W, u, rng = make_weights(dims, seed, cfg["bias"], cfg["c"], expert_seed)
    x = make_x(cfg["T"], dims.H, rng, cfg["c"], u)
    meta = dict(config=i, seed=seed, expert_seed=expert_seed, bias=cfg["bias"], c=cfg["c"])
    if near_ties and cfg["near_ties"]:
        edits = read_near_tie_edits()
        x = apply_edits(x, edits)
        meta["near_tie_tokens"] = sorted({t for t, _, _ in edits})
    return Case(name=cfg["name"], dims=dims, weights=W, x=x, meta=meta)


def make_case(dims: Dims, T: int, seed: int, bias: str = "none", c: float = 0.0,
              real_experts: bool = False) -> Case:
    """An ad-hoc seeded case (ragged sizes, edge cases) in the same recipe."""
    expert_seed = WEIGHT_SEED_REAL if real_experts else None
    if real_experts and dims != REAL:
        raise ValueError("the shared real-width expert set only exists at real widths")
    W, u, rng = make_weights(dims, seed, bias, c, expert_seed)
    x = make_x(T, dims.H, rng, c, u)
    return Case(name=f"case_T{T}_seed{seed}", dims=dims, weights=W, x=x,
                meta=dict(seed=seed, bias=bias, c=c, expert_seed=expert_seed))


def with_dims(d: Dims, **kw) -> Dims:
    return replace(d, **kw)


def pack_uint4(u: np.ndarray) -> np.ndarray:
    """Pack unsigned 4-bit codes (values in [0, 15]) two per byte, even element low."""
    u = np.asarray(u)
    if u.shape[-1] % 2:
        raise ValueError("int4 rows need an even length")
    if u.min(initial=0) < 0 or u.max(initial=0) > 15:
        raise ValueError("unsigned 4-bit code out of [0, 15]")
    u = u.astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def with_affine_offsets(W: Weights, seed: int) -> Weights:
    """The same routed-expert bytes and scales read as affine int4: each byte's
    nibbles become unsigned codes q in [0, 15] (uniform, as the bytes are), and
    every group gets a binary16 offset b = -s * u with u ~ U(7, 9), so that
    w = s q + b is centred near zero as in an affine 4-bit checkpoint."""
    rng = np.random.default_rng(seed)

    def offsets(s_bits):
        s = s_bits.view(np.float16).astype(np.float64)
        return f16_bits(-s * rng.uniform(7.0, 9.0, size=s.shape))

    return replace(W, w13_b=offsets(W.w13_s), w2_b=offsets(W.w2_s))


def make_affine_case(dims: Dims, T: int, seed: int, bias: str = "none", c: float = 0.0,
                     real_experts: bool = False) -> Case:
    """An ad-hoc case whose routed experts are affine int4."""
    case = make_case(dims, T, seed, bias=bias, c=c, real_experts=real_experts)
    return replace(case, name=case.name + "_affine", weights=with_affine_offsets(case.weights, seed + 77))
