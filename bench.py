"""Throughput of the routed MoE layer (W4A16) on one MI355X.

One step = one call of the whole layer (router, top-k, experts, shared
expert, combine) on one batch of seeded synthetic input already resident in
HBM.  The headline workload is single-token decode at real widths (T=1,
H=2048, E=256, top-8, I=512, Is=512); the 512-token Zipf chunk and the other
three workloads (toy layer, 32-token batched decode, 128-token prefill) are
measured in the same run and reported beside it.

Cold-cache discipline: the weights are replicated R times at distinct device
addresses and step s (warm-up steps included) uses copy s mod R, so a copy's
touched bytes have been evicted from L2 and the 256 MB last-level cache before
it is used again.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, TFLOP/s
METRIC = "MoE-layer tokens/s at T=1 and T=512; achieved HBM GB/s and MFMA % of peak"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "decode_kernel_t1_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------- accounting

def algorithmic_bytes(d, T, distinct_experts):
    """Bytes a layer call must move at least once: router, shared expert, the
    distinct routed experts' weights (codes + scales), x and out."""
    H, E, I, Is, G = d.H, d.E, d.I, d.Is, d.G
    router = (E + 1) * H + (E + 1) * (H // G) * 2
    shared = 2 * Is * H + 2 * Is * (H // G) * 2 + H * Is + H * (Is // G) * 2
    expert = 2 * I * H // 2 + 2 * I * (H // G) * 2 + H * I // 2 + H * (I // G) * 2
    return router + shared + distinct_experts * expert + 2 * T * H * 2


def algorithmic_flops(d, T):
    return T * (2 * (d.E + 1) * d.H + d.k * 6 * d.I * d.H + 6 * d.Is * d.H)


# the sources the single-token kernel and its launch are built from: the
# decode kernel, the headers it includes, and the host code that sizes its grid
DECODE_SOURCES = ("api.hip", "common.hpp", "decode.hip", "decode.hpp", "gemv.hpp")


def _code_only(text):
    """C/C++ source without its comments and blank space, so that an edit of
    the comments leaves the digest alone (the sources hold no string literal
    with a comment marker in it)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4a16_routed_experts_amd", "csrc")
    paths = [(name, os.path.join(csrc, name)) for name in DECODE_SOURCES]
    paths.append(("moe_w4a16.h", os.path.join(ROOT, "include", "moe_w4a16.h")))
    for name, path in paths:
        with open(path, encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(expected_digest):
    """HBM bytes per launch from the committed counter summary, if it still
    describes the current kernels (same source digest)."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    vals = {}
    with open(PROFILE_TRAFFIC) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != expected_digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------- GPU leg

def build_if_missing():
    import w4a16_routed_experts_amd as m
    if not os.path.exists(m.library_path()):
        from w4a16_routed_experts_amd import build
        build.build()
    m.lib()


def make_copies(case, R, torch, m):
    """R device copies of the layer's weights at distinct addresses."""
    import numpy as np
    base = {}
    for f, a in case.weights.items():
        view = {"|i1": np.int8, "|u1": np.uint8, "<u2": np.int16}[a.dtype.str]
        base[f] = torch.from_numpy(a.view(view)).cuda()
    copies = [m.DeviceWeights(tensors=base)]
    for _ in range(R - 1):
        copies.append(m.DeviceWeights(tensors={f: t.clone() for f, t in base.items()}))
    torch.cuda.synchronize()
    return copies


def time_block(cfg, steps, warmup, R, torch, m, gen):
    """Per-call time of the MoE sub-block (RMSNorm -> block -> residual add)
    on the same workload, weights rotated the same way."""
    import ctypes
    import numpy as np
    case = gen.make_config(cfg)
    d, T = case.dims, case.T
    dims = m.make_dims(d.H, d.E, d.k, d.I, d.Is, d.G)
    copies = make_copies(case, R, torch, m)
    x = torch.from_numpy(case.x.view(np.int16)).cuda()
    gain = torch.from_numpy(np.ones(d.H, dtype=np.float16).view(np.int16)).cuda()
    out = torch.empty((T, d.H), dtype=torch.int16, device="cuda")
    ws = m.workspace(dims, T)
    stream = torch.cuda.current_stream()
    fn = m.lib().moe_block_forward
    args = [(ctypes.byref(dims), ctypes.byref(c.struct), x.data_ptr(), gain.data_ptr(), 1e-6, T, out.data_ptr(),
             None, None, None, ws.data_ptr(), ws.numel(), stream.cuda_stream) for c in copies]
    for s in range(warmup):
        st = fn(*args[s % R])
        if st != 0:
            raise RuntimeError(f"moe_block_forward: {m.moe_status_string(st)}")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(steps):  # the rotation continues past warm-up: no timed step reuses a warm copy
        fn(*args[(warmup + s) % R])
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    del copies
    torch.cuda.empty_cache()
    return us


def time_layers(L, steps, warmup, R, torch, m, gen):
    """Per-layer time of L MoE sub-blocks at T=1, real widths, each layer's
    weights drawn anew (the decode-token recipe: no router bias): one
    moe_layers_forward launch per step, against L moe_block_forward launches
    per step.  R device copies of the L-layer stack are rotated so no step
    finds its weights in the last-level cache."""
    import ctypes
    import numpy as np
    d = gen.REAL
    Ws, gains = [], []
    for l in range(L):
        W, _, rng = gen.make_weights(d, 4000 + l)
        Ws.append(W)
        gains.append(gen.f16_bits(rng.uniform(0.5, 1.5, size=d.H)))
    x = gen.make_x(1, d.H, np.random.default_rng(4999))
    stacks = [m.LayerStack(Ws, gains)]
    del Ws
    for _ in range(R - 1):
        s_ = object.__new__(m.LayerStack)
        s_.buffer = stacks[0].buffer.clone()
        off = s_.buffer.data_ptr() - stacks[0].buffer.data_ptr()
        s_.struct = m.MoeWeights(*[(getattr(stacks[0].struct, f) + off) if getattr(stacks[0].struct, f) else None
                                   for f in m.binding.WEIGHT_FIELDS])
        s_.gain, s_.stride, s_.L = stacks[0].gain + off, stacks[0].stride, L
        stacks.append(s_)
    dims = m.make_dims(d.H, d.E, d.k, d.I, d.Is, d.G)
    xt = torch.from_numpy(x.view(np.int16)).cuda()
    out = torch.empty_like(xt)
    tmp = [torch.empty_like(xt) for _ in range(2)]
    ws = m.layers_workspace(dims, 1, L)
    stream = torch.cuda.current_stream().cuda_stream
    lib = m.lib()

    def one_launch(st):
        return lib.moe_layers_forward(ctypes.byref(dims), ctypes.byref(st.struct), st.gain, st.stride, L, 1e-6,
                                      xt.data_ptr(), 1, out.data_ptr(), ws.data_ptr(), ws.numel(), stream)

    per_layer = []
    for st in stacks:
        row = []
        for l in range(L):
            row.append(m.MoeWeights(*[(getattr(st.struct, f) + l * st.stride) if getattr(st.struct, f) else None
                                      for f in m.binding.WEIGHT_FIELDS]))
        per_layer.append(row)

    def chained(i):
        cur = xt
        for l in range(L):
            dst = out if l == L - 1 else tmp[l % 2]
            r = lib.moe_block_forward(ctypes.byref(dims), ctypes.byref(per_layer[i][l]), cur.data_ptr(),
                                      stacks[i].gain + l * stacks[i].stride, 1e-6, 1, dst.data_ptr(), None, None,
                                      None, ws.data_ptr(), ws.numel(), stream)
            if r != 0:
                return r
            cur = dst
        return 0

    res = {}
    for name, fn in (("one_launch", lambda i: one_launch(stacks[i])), ("launch_per_layer", chained)):
        for s in range(warmup):
            st_ = fn(s % R)
            if st_ != 0:
                raise RuntimeError(f"{name}: {m.moe_status_string(st_)}")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(steps):
            fn((warmup + s) % R)
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / steps
    del stacks, per_layer
    torch.cuda.empty_cache()
    return res


def time_config(cfg, steps, warmup, R, torch, m, gen, per_launch_events):
    return time_case(gen.make_config(cfg), cfg, steps, warmup, R, torch, m, per_launch_events)


def time_case(case, cfg, steps, warmup, R, torch, m, per_launch_events):
    import ctypes
    import numpy as np
    d, T = case.dims, case.T
    dims = m.make_dims(d.H, d.E, d.k, d.I, d.Is, d.G)
    copies = make_copies(case, R, torch, m)
    x = torch.from_numpy(case.x.view(np.int16)).cuda()
    out = torch.empty((T, d.H), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, d.k), dtype=torch.int32, device="cuda")
    ws = m.workspace(dims, T)
    stream = torch.cuda.current_stream()
    L = m.lib()
    fwd = L.moe_forward
    # pre-marshalled arguments: the timed loop makes one ctypes call per step
    args = [(ctypes.byref(dims), ctypes.byref(c.struct), x.data_ptr(), T, out.data_ptr(), ids.data_ptr(), None,
             None, ws.data_ptr(), ws.numel(), stream.cuda_stream) for c in copies]
    for s in range(warmup):
        st = fwd(*args[s % R])
        if st != 0:
            raise RuntimeError(f"moe_forward: {m.moe_status_string(st)}")
    torch.cuda.synchronize()
    distinct = int(np.unique(ids.cpu().numpy()).size)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    t0 = time.perf_counter()
    for s in range(steps):  # the rotation continues past warm-up: no timed step reuses a warm copy
        fwd(*args[(warmup + s) % R])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1)
    res = dict(cfg=cfg, name=case.name, T=T, dims=d, steps=steps, ms_total=ms, wall_s=wall,
               us_per_step=ms * 1e3 / steps, distinct_experts=distinct)

    if per_launch_events:
        # the same steps with an event pair around every launch (one kernel per step)
        n = min(steps, 2000)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for s in range(n):
            ev[s][0].record(stream)
            fwd(*args[(warmup + steps + s) % R])
            ev[s][1].record(stream)
        torch.cuda.synchronize()
        durs = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
        res["us_per_launch"] = float(durs.mean())
        res["us_per_launch_median"] = float(np.median(durs))

        # the same steps replayed from one HIP graph (R steps captured, one per
        # weight copy); informational beside the plain-stream figure.  Every
        # replay ends with the same output as eager execution, which is checked.
        try:
            torch.cuda.synchronize()
            want = out.clone()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = torch.cuda.current_stream().cuda_stream
                for s in range(R):
                    fwd(*(args[s][:-1] + (cs,)))
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, n // R)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            res["us_per_step_graph"] = e0.elapsed_time(e1) * 1e3 / (reps * R)
            res["graph_matches_eager"] = bool(torch.equal(out, want))
        except Exception as ex:  # a runtime without graph capture: report, do not fail
            res["graph_error"] = repr(ex)
    del copies
    torch.cuda.empty_cache()
    return res


def workload_summary(r, copies, description):
    """tokens/s, HBM GB/s, MFMA % and roofline fraction of one timed workload."""
    d, T = r["dims"], r["T"]
    b = algorithmic_bytes(d, T, r["distinct_experts"])
    f = algorithmic_flops(d, T)
    t = r["us_per_step"] * 1e-6
    return {"workload": description, "tokens_per_s": round(T / t, 1), "us_per_step": round(r["us_per_step"], 3),
            "hbm_gbs": round(b / t / 1e9, 1), "hbm_frac": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_pct": round(100 * f / t / (MFMA_F16_PEAK_TFLOPS * 1e12), 3),
            "roofline_frac": round(max(b / (HBM_PEAK_GBS * 1e9), f / (MFMA_F16_PEAK_TFLOPS * 1e12)) / t, 4),
            "algorithmic_bytes": b, "flops": f, "distinct_experts": r["distinct_experts"],
            "weight_copies_rotated": copies, "steps": r["steps"]}


# a chunk large enough that the grouped GEMMs run many rounds (informational)
LARGE_T = 16384

# configurations besides the headline: (steps, warm-up, weight copies, description)
OTHER_WORKLOADS = {
    0: (2000, 100, 1, "toy layer: T=1, hidden 256, 8 experts, top-2, intermediates 64 (0.1 MB of weights: "
                      "one copy, cache-warm)"),
    2: (300, 20, 3, "batched decode: T=32 iid tokens, real widths (about 280 MB touched per call, "
                    "3 copies rotated)"),
    3: (300, 20, 3, "prefill chunk: T=128, per-expert logit bias N(0, 0.5), real widths (3 copies rotated)"),
}


# --------------------------------------------------------------- CPU leg

def cpu_baseline(gen, budget_s=12.0):
    """The float64 oracle on the host cores, on the single-token workload."""
    from oracle import ref
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    case = gen.make_config(1)
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s or n == 0:
        ref.forward(case.x, case.weights, case.dims)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(n * case.T / dt, 3), "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{n} calls of the float64 oracle forward on the T=1 decode input "
                      f"({dt:.1f} s; host has {len(os.sched_getaffinity(0))} cores available)"}


# --------------------------------------------------------------- counter runs

def profile_run(kind, steps, torch, m, gen):
    """Untimed steps of one workload plus a calibration copy, for rocprofv3
    counter passes: FETCH_SIZE / WRITE_SIZE of the layer's kernels are scaled by
    what the same counters read for the copy, whose bytes are known."""
    import ctypes
    import numpy as np
    cfg = 1 if kind == "decode" else 4
    case = gen.make_config(cfg)
    d, T = case.dims, case.T
    dims = m.make_dims(d.H, d.E, d.k, d.I, d.Is, d.G)
    R = 32 if cfg == 1 else 4
    copies = make_copies(case, R, torch, m)
    x = torch.from_numpy(case.x.view(np.int16)).cuda()
    out = torch.empty((T, d.H), dtype=torch.int16, device="cuda")
    ws = m.workspace(dims, T)
    stream = torch.cuda.current_stream()
    L = m.lib()
    for s in range(steps):
        st = L.moe_forward(ctypes.byref(dims), ctypes.byref(copies[s % R].struct), x.data_ptr(), T, out.data_ptr(),
                           None, None, None, ws.data_ptr(), ws.numel(), stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"moe_forward: {m.moe_status_string(st)}")
    torch.cuda.synchronize()
    log(f"{steps} {kind} steps done")
    # calibration: a plain device copy of 64 MiB (reads and writes 64 MiB each)
    src = torch.randint(0, 1 << 30, (16 << 20,), dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("calibration copy of 64 MiB x 5 done")
    print(json.dumps({"profile_run": kind, "steps": steps, "calibration_copy_bytes": src.numel() * 4}), flush=True)


# --------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--copies", type=int, default=32, help="weight copies rotated for cold-cache timing")
    ap.add_argument("--chunk-steps", type=int, default=300, help="steps of the 512-token workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-other-workloads", action="store_true", help="time only T=1 and T=512")
    ap.add_argument("--no-large", action="store_true", help="skip the 16384-token chunk")
    ap.add_argument("--no-sub-block", action="store_true",
                    help="skip the RMSNorm + residual sub-block timing (its launches share the block's kernel names)")
    ap.add_argument("--layers", type=int, default=8, help="sub-blocks per call in the multi-layer timing (0: skip)")
    ap.add_argument("--profile-run", choices=["decode", "chunk"], default=None,
                    help="untimed steps plus a calibration copy, for rocprofv3 counter passes (no JSON metric line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this layer runs and is measured on one GPU: the library has no multi-GPU path",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import w4a16_routed_experts_amd as m
    from workloads import gen
    build_if_missing()
    if args.profile_run:
        profile_run(args.profile_run, args.steps, torch, m, gen)
        return

    digest = source_digest()
    log("decode T=1 ...")
    r1 = time_config(1, args.steps, args.warmup, args.copies, torch, m, gen, per_launch_events=True)
    log(f"  {r1['us_per_step']:.3f} us/step, {r1['us_per_launch']:.3f} us/launch")
    log("chunk T=512 ...")
    r4 = time_config(4, args.chunk_steps, max(10, args.warmup // 10), max(4, args.copies // 8), torch, m, gen,
                     per_launch_events=False)
    log(f"  {r4['us_per_step']:.3f} us/step")

    others = {}
    if not args.no_other_workloads:
        for cfg, (steps, warm, R, desc) in OTHER_WORKLOADS.items():
            log(f"config {cfg} ...")
            r = time_config(cfg, steps, warm, R, torch, m, gen, per_launch_events=False)
            others[f"config{cfg}"] = workload_summary(r, R, desc)
            log(f"  {r['us_per_step']:.3f} us/step")

    large = None
    if not args.no_large:
        log(f"chunk T={LARGE_T} ...")
        case = gen.make_case(gen.REAL, LARGE_T, seed=LARGE_T, real_experts=True)
        large = time_case(case, "large", 20, 3, 1, torch, m, per_launch_events=False)
        log(f"  {large['us_per_step']:.3f} us/step")

    sb1 = sb4 = None
    if not args.no_sub_block:
        log("sub-block (RMSNorm -> block -> residual) T=1 and T=512 ...")
        sb1 = time_block(1, args.steps, args.warmup, args.copies, torch, m, gen)
        sb4 = time_block(4, args.chunk_steps, max(10, args.warmup // 10), max(4, args.copies // 8), torch, m, gen)
        log(f"  {sb1:.3f} / {sb4:.3f} us/step")

    lay = None
    if args.layers > 0:
        log(f"{args.layers} sub-blocks per step at T=1: one launch, and one launch per layer ...")
        lay = time_layers(args.layers, max(20, args.steps // 10), max(5, args.warmup // 10), 4, torch, m, gen)
        log(f"  {lay['one_launch']:.3f} / {lay['launch_per_layer']:.3f} us/step")

    d1 = r1["dims"]
    b1 = algorithmic_bytes(d1, 1, r1["distinct_experts"])
    f1 = algorithmic_flops(d1, 1)
    # one T=1 step is exactly one launch of the decode kernel, so the timed
    # region's average per step is that kernel's average launch duration
    us_launch = r1["us_per_step"]
    achieved_gbs = b1 / (us_launch * 1e-6) / 1e9
    traffic = read_traffic(digest)
    value = r1["T"] * r1["steps"] / (r1["ms_total"] * 1e-3)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r1["ms_total"] / r1["steps"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "single-token decode: T=1, hidden 2048, 256 experts, top-8, expert intermediate 512, "
                               "shared intermediate 512, int4 g64 experts, int8 g64 router and shared expert",
                   "weight_copies_rotated": args.copies, "distinct_experts": r1["distinct_experts"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode_kernel<0> (the whole layer in one launch)",
                     "algorithmic_bytes_per_launch": b1, "us_per_launch": round(us_launch, 3),
                     "us_per_launch_event_pairs": round(r1["us_per_launch"], 3),
                     "us_per_step_hip_graph": (round(r1["us_per_step_graph"], 3) if "us_per_step_graph" in r1
                                               else r1.get("graph_error")),
                     "hip_graph_matches_eager": r1.get("graph_matches_eager"),
                     "mfma_pct": round(100 * f1 / (us_launch * 1e-6) / (MFMA_F16_PEAK_TFLOPS * 1e12), 4)},
        "chunk_t512": workload_summary(r4, max(4, args.copies // 8),
                                       "512-token chunk, Zipf(1.1) expert popularity, same widths"),
        "source_digest": digest,
    }
    line.update(others)
    if large is not None:
        line["large_chunk"] = workload_summary(
            large, 1, f"{LARGE_T}-token chunk, iid routing (every expert), real widths; one weight copy "
                      "(272 MB of expert weights, above the 256 MB last-level cache)")
    if sb1 is not None:
        line["sub_block"] = {"workload": "post-attention RMSNorm -> the same block -> residual add, same inputs",
                             "t1_us_per_step": round(sb1, 3), "t512_us_per_step": round(sb4, 3),
                             "t1_tokens_per_s": round(1e6 / sb1, 1), "t512_tokens_per_s": round(512e6 / sb4, 1),
                             "t1_extra_us_vs_block": round(sb1 - r1["us_per_step"], 3),
                             "t512_extra_us_vs_block": round(sb4 - r4["us_per_step"], 3)}
    if lay is not None:
        L = args.layers
        line["layers"] = {"workload": f"{L} MoE sub-blocks in turn at T=1, real widths, weights drawn anew per layer, "
                                      "4 copies of the stack rotated",
                          "layers": L,
                          "one_launch_us_per_layer": round(lay["one_launch"] / L, 3),
                          "launch_per_layer_us_per_layer": round(lay["launch_per_layer"] / L, 3),
                          "one_launch_tokens_per_s": round(1e6 / lay["one_launch"], 1),
                          "speedup": round(lay["launch_per_layer"] / lay["one_launch"], 3)}
    if not args.no_cpu:
        log("cpu baseline ...")
        line["cpu_baseline"] = cpu_baseline(gen)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
