"""Write the near-tie activation edits of the 512-token Zipf chunk.

TEST INFRASTRUCTURE.  Run as ``python -m oracle.make_near_ties`` from the
repository root; it rewrites ``workloads/near_ties_cfg4.txt``.

The 512-token workload asks for about 5% of its rows to have a k-th / (k+1)-th
router-logit gap under 1e-3, so that the routing-tie accounting is exercised
(the TensorFold PR, "Receipts", shows bf16 routing flipping to another expert
where the float64 router gap is small).  Starting from the unedited seeded
activations, this script picks the ceil(0.05 T) rows whose float64 gap is the
smallest among those not already under 1e-3, and for each one moves a single
activation coordinate (the one where the two boundary experts' dequantised
router rows differ most) so that the float64 gap lands in [0, 1e-3).  The
moved value is a binary16 number; it is searched ulp by ulp near the linear
estimate.  Gaps are always measured with this oracle's router.
"""
from __future__ import annotations

import math
import sys

import numpy as np

from oracle import ref
from workloads import gen

TARGET = 2.5e-4
LIMIT = 1e-3


def _row_gap(x_row_bits, W, dims):
    lg = ref.router_logits(x_row_bits[None, :], W, dims)[:, : dims.E]
    return float(ref.kth_gap(lg, dims.k)[0])


def near_tie_edits(case, count):
    dims, W = case.dims, case.weights
    r = ref.route(case.x, W, dims)
    gap = r["gap"]
    lr = r["logits"][:, : dims.E]
    order = np.argsort(gap, kind="stable")
    wr = ref.dequant(W.router_q, W.router_s, dims.G)
    edits = []
    for t in order:
        if len(edits) == count:
            break
        if gap[t] < LIMIT:
            continue  # already a natural near-tie; it stays and is counted
        srt = np.lexsort((np.arange(dims.E), -lr[t]))
        a, b = int(srt[dims.k - 1]), int(srt[dims.k])
        d = wr[a] - wr[b]
        j = int(np.argmax(np.abs(d)))
        x_row = case.x[t].copy()
        x0 = float(x_row[j:j + 1].view(np.float16)[0])
        est = x0 - (gap[t] - TARGET) / d[j]
        if abs(est - x0) > 1.0:
            continue
        base = np.float16(est)
        found = None
        # walk outward from the estimate, one binary16 ulp at a time
        for m in range(0, 400):
            for sgn in ((1,) if m == 0 else (1, -1)):
                cand = base
                step = np.float16(np.inf) if sgn > 0 else np.float16(-np.inf)
                for _ in range(m):
                    cand = np.nextafter(cand, step)
                x_row[j] = np.array([cand], dtype=np.float16).view(np.uint16)[0]
                g = _row_gap(x_row, W, dims)
                if 0.0 <= g < LIMIT:
                    found = int(x_row[j])
                    break
            if found is not None:
                break
        if found is None:
            continue
        edits.append((int(t), j, found))
    if len(edits) != count:
        raise RuntimeError(f"only {len(edits)} of {count} near-tie rows could be placed")
    return sorted(edits)


def main(argv=None):
    cfg_index = 4
    case = gen.make_config(cfg_index, near_ties=False)
    count = math.ceil(0.05 * case.T)
    edits = near_tie_edits(case, count)
    lines = [
        "# Near-tie edits of the 512-token Zipf chunk, written by oracle/make_near_ties.py.",
        "# Each line replaces one activation: token coord binary16-bits (hex).",
        f"# {count} rows = ceil(0.05 * {case.T}); every edited row has a float64",
        "# k-th/(k+1)-th router-logit gap in [0, 1e-3).",
    ]
    lines += [f"{t} {j} {bits:04x}" for t, j, bits in edits]
    with open(gen.NEAR_TIE_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {len(edits)} edits to {gen.NEAR_TIE_FILE}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
