"""Float64 CPU oracle of the routed Mixture-of-Experts FFN under W4A16.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
executes this module; only the tests, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP library.

What it computes (all in float64, no intermediate rounding):

* The block (the Chimera notebook, section 5 "Validate the MoE FFN block"):
  the output is the routed part plus sigmoid(x . W_sg) times a dense shared
  SwiGLU expert applied to every token.
* The router ordering (same notebook, section 5.2): softmax over the router
  logits, then top-k, then renormalise the k kept probabilities; SwiGLU
  experts; the sigmoid output gate.
* The MoE sub-block of a decoder layer (the Chimera notebook, sections 7 and
  10, the decoder-layer assemblies): post-attention RMSNorm, the MoE block on
  the normalised activations, then the residual add.
* Several sub-blocks in turn (the Chimera notebook, "Pipeline"), with each
  layer's output stored as binary16 before the next layer reads it.
* The router and the shared-gate row are stored 8-bit, group-64 rows, stacked
  (the TensorFold PR, "Design").  Routed experts int4, shared expert int8,
  activations fp16 (the Chimera notebook, pipeline intro and "Key takeaways").

Readings where the pages are silent (each is stated where it is used):
top-k ties go to the lower expert index; int4 codes are two's-complement
nibbles with the even element in the low nibble; a dequantised weight is
code x scale with one binary16 scale per 64 consecutive K elements of a row;
there is no router bias term and no zero point; the RMSNorm is
h / sqrt(mean(h^2) + eps) * gain with the gain vector as applied, and its output
is rounded to binary16 (the MoE input everywhere else) before the block.

Every function below is pinned by the ``-m "not gpu"`` tests (hand-derived
fixtures, brute force, closed forms and invariants), and the block and the
RMSNorm also against transformers' Qwen3.5-MoE modules (the published
implementation the Chimera notebook checks its reference against, section 5.2).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# storage format -> float64
# ---------------------------------------------------------------------------


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Bytes [..., K/2] -> int4 codes [..., K] in [-8, 7].

    Element 2j is the low nibble of byte j, element 2j+1 the high nibble;
    each nibble is a two's-complement value.
    """
    b = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int16)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = (b >> 4) & 0x0F
    out[out >= 8] -= 16
    return out


def unpack_uint4(packed: np.ndarray) -> np.ndarray:
    """Bytes [..., K/2] -> unsigned 4-bit codes [..., K] in [0, 15] (the affine
    int4 form): element 2j is the low nibble of byte j, element 2j+1 the high."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int16)
    out[..., 0::2] = b % 16
    out[..., 1::2] = b // 16
    return out


def half_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant(codes: np.ndarray, scale_bits: np.ndarray, G: int) -> np.ndarray:
    """code x scale, one scale per run of G consecutive elements of a row."""
    q = np.asarray(codes).astype(np.float64)
    s = half_bits_to_f64(scale_bits)
    if q.shape[-1] != s.shape[-1] * G:
        raise ValueError("scale count does not match K / G")
    return q * np.repeat(s, G, axis=-1)


def dequant_affine(codes: np.ndarray, scale_bits: np.ndarray, offset_bits: np.ndarray, G: int) -> np.ndarray:
    """Affine 4-bit dequantisation, per run of G consecutive elements of a row:
    w = q * s + b with an unsigned code q, the group's scale s and offset b.
    (The TensorFold PR runs a 4-bit affine checkpoint; the pages give no layout,
    so this reading keeps the symmetric form's layout and adds one binary16
    offset per group.)  Exact in float64."""
    q = np.asarray(codes).astype(np.float64)
    s = half_bits_to_f64(scale_bits)
    b = half_bits_to_f64(offset_bits)
    if q.shape[-1] != s.shape[-1] * G or s.shape != b.shape:
        raise ValueError("scale or offset count does not match K / G")
    return q * np.repeat(s, G, axis=-1) + np.repeat(b, G, axis=-1)


# ---------------------------------------------------------------------------
# elementwise pieces
# ---------------------------------------------------------------------------


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):  # exp overflow -> inf -> sigmoid 0, as intended
        return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    """SiLU(z) = z * sigmoid(z), the gate activation of SwiGLU."""
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------


def router_logits(x_bits, W, dims) -> np.ndarray:
    """[T, E+1] float64: columns 0..E-1 router logits, column E the shared-gate logit."""
    X = half_bits_to_f64(x_bits)
    Wr = dequant(W.router_q, W.router_s, dims.G)
    return X @ Wr.T


def topk_ids(lr: np.ndarray, k: int) -> np.ndarray:
    """Per row, the k experts of largest logit, descending; ties to the lower index."""
    T, E = lr.shape
    ids = np.empty((T, k), dtype=np.int64)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -lr[t]))  # primary key: -logit, then index
        ids[t] = order[:k]
    return ids


def softmax_renormalised(lr: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """softmax over all E logits, keep the selected k, divide by their sum."""
    m = lr.max(axis=1, keepdims=True)
    p = np.exp(lr - m)
    p /= p.sum(axis=1, keepdims=True)
    kept = np.take_along_axis(p, ids, axis=1)
    return kept / kept.sum(axis=1, keepdims=True)


def kth_gap(lr: np.ndarray, k: int) -> np.ndarray:
    """k-th largest minus (k+1)-th largest router logit per row (inf when k == E)."""
    T, E = lr.shape
    if k >= E:
        return np.full(T, np.inf)
    srt = -np.sort(-lr, axis=1)
    return srt[:, k - 1] - srt[:, k]


def route(x_bits, W, dims):
    """Routing of every token: dict(ids, w, sigma, logits, gap)."""
    lg = router_logits(x_bits, W, dims)
    lr = lg[:, : dims.E]
    ids = topk_ids(lr, dims.k)
    w = softmax_renormalised(lr, ids)
    return dict(ids=ids, w=w, sigma=sigmoid(lg[:, dims.E]), logits=lg, gap=kth_gap(lr, dims.k))


# ---------------------------------------------------------------------------
# experts
# ---------------------------------------------------------------------------


def routed_expert_weights(W, dims, e: int):
    """Dequantised (W13_e [2I][H], W2_e [H][I]) of routed expert e: symmetric
    int4 (code x scale), or affine int4 (code x scale + offset) when the
    weights carry offsets."""
    if getattr(W, "w13_b", None) is not None:
        w13 = dequant_affine(unpack_uint4(W.w13_q[e]), W.w13_s[e], W.w13_b[e], dims.G)
        w2 = dequant_affine(unpack_uint4(W.w2_q[e]), W.w2_s[e], W.w2_b[e], dims.G)
        return w13, w2
    w13 = dequant(unpack_int4(W.w13_q[e]), W.w13_s[e], dims.G)
    w2 = dequant(unpack_int4(W.w2_q[e]), W.w2_s[e], dims.G)
    return w13, w2


def swiglu_ffn(X: np.ndarray, w13: np.ndarray, w2: np.ndarray, inter: int) -> np.ndarray:
    """(silu(X W_gate^T) * (X W_up^T)) W_down^T; w13 rows are gate then up."""
    A = X @ w13.T
    Hh = silu(A[:, :inter]) * A[:, inter:]
    return Hh @ w2.T


def experts(x_bits, ids, w, W, dims) -> np.ndarray:
    """Routed half: out[t] = sum_i w[t,i] * FFN_{ids[t,i]}(x_t), float64 [T, H].

    Each selected expert is dequantised once and applied to its tokens.
    """
    X = half_bits_to_f64(x_bits)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    T = X.shape[0]
    out = np.zeros((T, dims.H))
    for e in np.unique(ids):
        tok, slot = np.nonzero(ids == e)
        w13, w2 = routed_expert_weights(W, dims, int(e))
        Y = swiglu_ffn(X[tok], w13, w2, dims.I)
        # a token could list an expert twice only through caller-supplied
        # routing; np.add.at accumulates every occurrence
        np.add.at(out, tok, w[tok, slot][:, None] * Y)
    return out


def shared_expert(x_bits, W, dims) -> np.ndarray:
    """Dense int8 SwiGLU expert applied to every token, float64 [T, H]."""
    X = half_bits_to_f64(x_bits)
    s13 = dequant(W.sh13_q, W.sh13_s, dims.G)
    s2 = dequant(W.sh2_q, W.sh2_s, dims.G)
    return swiglu_ffn(X, s13, s2, dims.Is)


def forward(x_bits, W, dims):
    """The complete block: dict(out, routed, shared, ids, w, sigma, logits, gap)."""
    r = route(x_bits, W, dims)
    routed = experts(x_bits, r["ids"], r["w"], W, dims)
    S = shared_expert(x_bits, W, dims)
    out = routed + r["sigma"][:, None] * S
    r.update(out=out, routed=routed, shared=S)
    return r


# ---------------------------------------------------------------------------
# a second formulation, used only to check the first
# ---------------------------------------------------------------------------


def forward_dense(x_bits, W, dims) -> np.ndarray:
    """Every expert on every token, masked by a dense [T, E] gate matrix."""
    X = half_bits_to_f64(x_bits)
    lg = router_logits(x_bits, W, dims)
    lr = lg[:, : dims.E]
    T = X.shape[0]
    ids = topk_ids(lr, dims.k)
    p = np.exp(lr - lr.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    mask = np.zeros_like(p)
    np.put_along_axis(mask, ids, 1.0, axis=1)
    gates = p * mask
    gates /= gates.sum(axis=1, keepdims=True)
    routed = np.zeros((T, dims.H))
    for e in range(dims.E):
        w13, w2 = routed_expert_weights(W, dims, e)
        routed += gates[:, e : e + 1] * swiglu_ffn(X, w13, w2, dims.I)
    return routed + sigmoid(lg[:, dims.E])[:, None] * shared_expert(x_bits, W, dims)


# ---------------------------------------------------------------------------
# the MoE sub-block of a decoder layer: RMSNorm -> MoE block -> residual add
# ---------------------------------------------------------------------------


def f64_to_half_bits(v) -> np.ndarray:
    """float64 -> binary16 bit patterns, rounded to nearest even."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def rmsnorm(h_bits, gain_bits, eps: float, plus_one: bool = False) -> np.ndarray:
    """Post-attention RMSNorm (the Chimera notebook, sections 7 and 10: the
    norm in front of the MoE FFN), float64 [T, H]: each token's row divided by
    the square root of (the mean of its squares + eps), times the gain vector.
    plus_one: the stored vector is w and the gain is 1 + w (the form of the
    published Qwen3.5-MoE norm)."""
    X = half_bits_to_f64(h_bits)
    g = half_bits_to_f64(gain_bits) + (1.0 if plus_one else 0.0)
    ms = np.mean(X * X, axis=1, keepdims=True)
    return X / np.sqrt(ms + eps) * g


def block_forward(h_bits, gain_bits, eps: float, W, dims, plus_one: bool = False):
    """The MoE sub-block (same sections: post-attn RMSNorm -> MoE FFN ->
    residual): a = binary16(rmsnorm(h)), out = h + forward(a)["out"].

    Returns forward's dict with out replaced by the sub-block's output, the
    block's own output as moe, and the normalised activations as a_bits.
    """
    a_bits = f64_to_half_bits(rmsnorm(h_bits, gain_bits, eps, plus_one))
    r = forward(a_bits, W, dims)
    r["moe"] = r["out"]
    r["out"] = half_bits_to_f64(h_bits) + r["moe"]
    r["a_bits"] = a_bits
    return r


def layers_forward(h_bits, gain_bits_per_layer, eps: float, W_per_layer, dims, plus_one: bool = False) -> np.ndarray:
    """Several MoE sub-blocks applied in turn (the Chimera notebook,
    "Pipeline": the decoder's layers run one after another inside one kernel
    per token).  Reading: each layer's output is stored as binary16 before the
    next layer reads it, as it would be between separate calls, so
    h_{l+1} = binary16(block_forward(h_l)["out"]).  Returns the last layer's
    output in float64 (before its own binary16 rounding)."""
    h = np.asarray(h_bits)
    out = None
    for gain_bits, W in zip(gain_bits_per_layer, W_per_layer):
        out = block_forward(h, gain_bits, eps, W, dims, plus_one)["out"]
        h = f64_to_half_bits(out)
    return out
