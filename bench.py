"""Benchmark of the routed int4 MoE layer on one MI355X.

Default workload (decode): one token through 40 distinct MoE layers (d=2048, 256 experts
top-8 + shared, I=512, int4 groups of 64), so the 18.2 GB of expert weights stream from HBM
rather than from the 256 MB cache. A step is one pass over the 40 layers, replayed as a HIP
graph; value = MoE-layer tokens per second.

Also reported, on the same stream with HIP events: each kernel's average duration, the
dominant kernel's algorithmic bytes (or flops) per launch and its roofline fraction, and the
CPU oracle timed on the host cores on a bounded sample of the same workload.

The same line also carries, under "workloads", the tiny, prefill (T=512), long (4 x 1024,
Zipf-skewed) and diffusion (T=256 x 30 layers) workloads, each with tokens/s, time per layer
call, the whole-layer roofline fraction (HBM and matrix-core), the dominant kernel's fraction,
per-stage times and the oracle timed beside it (--extra selects them; --workload picks the
headline).

Fail-closed: nothing is reported unless layer outputs match the CPU oracle and the graph
replays reproduce the eager results bit for bit.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402  (before the library: bind to torch's HIP runtime)

from bit_moe_expert_amd import moe  # noqa: E402
from workload import gen  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak

DESCR = {
    "tiny": "tiny: T=8, d=256, 16 experts top-4 + shared (I=I_s=128), int4 g64",
    "decode": "decode: T=1, d=2048, 256 experts top-8 + shared, I=I_s=512, int4 g64, 40 layers cycled",
    "prefill": "prefill: T=512, d=2048, 256 experts top-8 + shared, I=I_s=512, int4 g64, 4 layers cycled",
    "long": "long: T=4096 as 4 chunks of 1024 (one layer each), Zipf logit bias, d=2048, 256 experts top-8 + shared, I=512",
    "diffusion": "diffusion: T=256 canvas x 30 layers, d=2048, 128 experts top-8, I=768, no shared expert",
    "m2": "small-M: T=2, decode shapes, 40 layers cycled",
    "m4": "small-M: T=4, decode shapes, 40 layers cycled",
    "m8": "small-M: T=8, decode shapes, 40 layers cycled",
    "m16": "small-M: T=16, decode shapes, 40 layers cycled",
    "m32": "small-M: T=32, decode shapes, 40 layers cycled",
    "m64": "small-M: T=64, decode shapes, 40 layers cycled",
    "decode3": "decode with 3-bit expert codes: T=1, d=2048, 256 experts top-8 + shared, I=I_s=512, g64, 40 layers",
    "decode2": "decode with 2-bit expert codes: T=1, d=2048, 256 experts top-8 + shared, I=I_s=512, g64, 40 layers",
    "m32_3": "small-M with 3-bit expert codes: T=32, decode shapes, 40 layers cycled",
    "m32_2": "small-M with 2-bit expert codes: T=32, decode shapes, 40 layers cycled",
    "tiny3": "tiny with 3-bit expert codes: T=8, d=256, 16 experts top-4 + shared (I=I_s=128), g64",
    "tiny2": "tiny with 2-bit expert codes: T=8, d=256, 16 experts top-4 + shared (I=I_s=128), g64",
    "prefill3": "prefill with 3-bit expert codes: T=512, d=2048, 256 experts top-8 + shared, I=I_s=512, g64, 4 layers",
    "diffusion3": "diffusion with 3-bit expert codes: T=256 canvas x 30 layers, d=2048, 128 experts top-8, I=768",
    "diffusion2": "diffusion with 2-bit expert codes: T=256 canvas x 30 layers, d=2048, 128 experts top-8, I=768",
}
# layers held on the GPU and calls per step (a one-layer workload repeats its layer, so the graph's
# launch is spread over as many calls as the decode workload's)
PLAN = {"tiny": (1, 40), "decode": (40, 40), "prefill": (4, 4), "long": (4, 4), "diffusion": (30, 30),
        "m2": (40, 40), "m4": (40, 40), "m8": (40, 40), "m16": (40, 40), "m32": (40, 40), "m64": (40, 40),
        "decode3": (40, 40), "decode2": (40, 40), "m32_3": (40, 40), "m32_2": (40, 40), "tiny3": (1, 40), "tiny2": (1, 40),
        "prefill3": (4, 4), "diffusion3": (30, 30), "diffusion2": (30, 30)}
DOMINANT = {"tiny": "gemv_gateup_topk", "decode": "gemv_gateup_topk", "prefill": "gateup_gemm", "long": "gateup_gemm",
            "diffusion": "gateup_gemm", "m2": "gemv_gateup_topk", "m4": "gemv_gateup_topk",
            "m8": "gemv_gateup_topk", "m16": "gemv_gateup_topk", "m32": "gemv_gateup_topk",
            "m64": "gateup_gemm", "decode3": "gemv_gateup_topk", "decode2": "gemv_gateup_topk",
            "m32_3": "gemv_gateup_topk", "m32_2": "gemv_gateup_topk", "tiny3": "gemv_gateup_topk",
            "tiny2": "gemv_gateup_topk", "prefill3": "gateup_gemm", "diffusion3": "gateup_gemm",
            "diffusion2": "gateup_gemm"}
STAGE_SOURCE = {"router_decode": "gemv.hip", "router_prefill": "route.hip", "route_meta": "route.hip",
                "gemv_gateup": "gemv.hip", "gemv_gateup_topk": "gemv.hip", "decode_topk": "route.hip",
                "topk_prefill": "route.hip",
                "gemv_down_combine": "gemv.hip", "gateup_gemm": "gemm_impl.h",
                "down_gemm": "gemm_impl.h", "combine": "gemm.hip", "chunk_max": "vocab_topk.hip",
                "topk_rows": "vocab_topk.hip"}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def bf16_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)


def to_layer(L: dict, k: int, dev) -> moe.Layer:
    def proj(p):
        return moe.QProj(torch.from_numpy(p["codes"]).to(dev), bf16_dev(p["scales"], dev), bf16_dev(p["biases"], dev),
                         p.get("bits", 4))

    def ffn(f):
        return None if f is None else moe.QuantFFN(proj(f["gate"]), proj(f["up"]), proj(f["down"]))

    wr = torch.from_numpy(L["w_router"]).to(dev)
    bias = None if L["logit_bias"] is None else torch.from_numpy(L["logit_bias"]).to(dev)
    return moe.Layer(wr, ffn(L["routed"]), ffn(L["shared"]), k, bias)


def f32_of_bits(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------------- algorithmic work per launch
def stage_work(w: gen.Workload, name: str, counts: np.ndarray):
    """(bytes, flops) the method must move / do in one launch of a stage, from the routing of that
    call. Weight bytes count only experts with at least one row; activations are counted once."""
    d, E, k, I, Is, T = w.d, w.E, w.k, w.I, w.Is, w.chunk
    P = T * k
    act = int((counts > 0).sum())
    per_w = lambda out, inn: out * inn * w.bits // 8 + 2 * 2 * out * inn // 64  # noqa: E731  codes + scales + biases
    if name == "router_decode":  # router weights, x, chunk partials out (one plane per token)
        return 4 * d * E + 2 * T * d + 4 * T * (d // 64) * E, 2 * T * d * E
    if name == "router_prefill":  # router weights, x, logits out
        return 4 * d * E + 2 * T * d + 4 * T * E, 2 * T * d * E
    if name == "topk_prefill":
        return 4 * T * E + 8 * P, 0
    if name == "decode_topk":
        return 4 * T * (d // 64) * E + 8 * P, 0
    if name == "gemv_gateup_topk":  # reads the router partials; routed slots + the shared expert's rows
        return 2 * act * per_w(I, d) + 2 * T * d + 2 * P * I + 4 * T * (d // 64) * E + \
            (2 * per_w(Is, d) + 2 * T * Is if Is else 0), 4 * d * (P * I + T * Is)
    if name == "route_meta":  # routing arrays; the layer's launch also rewrites x in pair order
        return 4 * P * 3 + 4 * (2 * E + 1) + 2 * 2 * T * d, 0
    if name == "gemv_gateup":
        return 2 * (act * per_w(I, d) + (per_w(Is, d) if Is else 0)) + 2 * T * d + 2 * (P * I + T * Is), \
            4 * d * (P * I + T * Is)
    if name == "gemv_down_combine":
        return (act * per_w(d, I) + (per_w(d, Is) if Is else 0)) + 2 * (P * I + T * Is) + 2 * T * d, \
            2 * d * (P * I + T * Is)
    if name == "gateup_gemm":
        wb = 2 * (act * per_w(I, d) + (per_w(Is, d) if Is else 0))
        return wb + 2 * T * d + 2 * (P * I + T * Is), 4 * d * (P * I + T * Is)
    if name == "down_gemm":
        wb = act * per_w(d, I) + (per_w(d, Is) if Is else 0)
        return wb + 2 * (P * I + T * Is) + (2 * d + d // 32) * (P + (T if Is else 0)), 2 * d * (P * I + T * Is)
    if name == "combine":  # fp16 rows with one exponent byte per 32 values
        return (2 * d + d // 32) * (P + (T if Is else 0)) + 2 * T * d + 8 * P, 2 * P * d
    raise KeyError(name)


def source_sha(name: str) -> str:
    p = os.path.join(ROOT, "bit_moe_expert_amd", "csrc", STAGE_SOURCE[name])
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def traffic_from_profiles(workload: str, kernel: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None when absent or
    when the kernel's source changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(p):
        return None
    txt = open(p).read()
    m_sha = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", txt)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_sha or not m_b or m_sha.group(1) != source_sha(kernel):
        return None
    return float(m_b.group(1))


def calib_mfma(dev, n: int = 8192, reps: int = 20) -> dict:
    """A plain bf16 torch.matmul of n x n by n x n (contiguous operands, fp32 accumulate in the
    library): the dense matrix-core rate a library GEMM reaches on this machine, beside the nominal peak."""
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    tfs = 2.0 * n ** 3 / (us * 1e-6) / 1e12
    log(f"calibration: bf16 matmul {n}^3 in {us:.1f} us -> {tfs:.0f} TFLOP/s ({100 * tfs / MFMA_BF16_PEAK_TFS:.1f}% of "
        f"the {MFMA_BF16_PEAK_TFS:.0f} TFLOP/s dense peak)")
    return {"bf16_matmul_n": n, "us": round(us, 2), "TFLOPs": round(tfs, 1),
            "frac_of_peak": round(tfs / MFMA_BF16_PEAK_TFS, 4)}


# ------------------------------------------------------------------------- CPU oracle baseline
def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_cycle(w: gen.Workload, n_layers: int, seconds: float):
    """The oracle on the workload's own calls, layer after layer of its cycle (each layer regenerated
    on the host, outside the timed region). The first layer takes one call; every later layer takes as
    many calls (each on its own seeded tokens) as spread about `seconds` of oracle time over the cycle,
    and the cycle stops early once twice that has passed. Only the oracle calls are timed."""
    from oracle import oracle
    spent, tokens, calls, reps, layers = 0.0, 0, 0, 1, 0
    for li in range(n_layers):
        L = gen.layer(w, li)
        for c in range(reps):
            x = gen.tokens(w, li, (li if w.calls > 1 else 0) + c * n_layers)
            t0 = time.perf_counter()
            oracle.forward_layer(x, L["w_router"], L["routed"], L["shared"], w.k, L["logit_bias"])
            spent += time.perf_counter() - t0
            tokens += x.shape[0]
            calls += 1
        del L
        layers += 1
        if li == 0:
            reps = max(1, min(64, int(seconds / (n_layers * max(spent, 1e-6)))))
        if spent >= 2 * seconds:
            break
    return {"value": tokens / spent, "unit": "MoE-layer tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{calls} layer calls of {w.chunk} tokens over layers 0..{layers - 1} of the {n_layers}-layer "
                      f"cycle ({reps} per layer after the first), {spent:.1f} s of oracle time"}


# ------------------------------------------------------------------------- exact top-K of logit rows
def vocab_work(w: gen.VocabWorkload, stage: int):
    """(bytes) one launch of a top-K kernel must move: stage 0 reads every logit once and writes the
    chunk maxima; stage 1 reads the chunk maxima and the K chosen chunks and writes K ids and values."""
    C = 1024 if w.K <= 32 else 512 if w.K <= 64 else 256  # the library's chunk size for this K
    nch = (w.V + C - 1) // C
    if stage == 0:
        return 4 * w.R * w.V + 4 * w.R * nch
    return w.R * (4 * nch + 4 * min(w.K, nch) * C + 8 * w.K)


def main_vocab(args) -> int:
    dev = torch.device("cuda:0")
    w = gen.VOCAB_WORKLOADS[args.workload]
    t0 = time.perf_counter()
    host = [gen.vocab_logits(w, s) for s in range(w.steps)]
    xs = [torch.from_numpy(h).to(dev) for h in host]
    ws = torch.empty(moe.vocab_topk_workspace_bytes(w.R, w.V, w.K), dtype=torch.uint8, device=dev)
    ids = [torch.empty((w.R, w.K), dtype=torch.int32, device=dev) for _ in xs]
    vals = [torch.empty((w.R, w.K), dtype=torch.float32, device=dev) for _ in xs]
    torch.cuda.synchronize()
    log(f"{w.steps} logit matrices [{w.R}][{w.V}] resident in {time.perf_counter() - t0:.1f} s")
    # eager pass + parity gate (bit-exact on sampled rows of every matrix)
    for s in range(w.steps):
        moe.vocab_topk(xs[s], w.K, ws, ids[s], vals[s])
    torch.cuda.synchronize()
    eager = [(i.clone(), v.clone()) for i, v in zip(ids, vals)]
    from oracle import oracle
    rows = np.linspace(0, w.R - 1, min(w.R, 8)).astype(np.int64)
    for s in range(w.steps):
        ri, rv = oracle.vocab_topk(host[s][rows], w.K)
        gi, gv = ids[s].cpu().numpy()[rows], vals[s].cpu().numpy()[rows]
        if not ((gi == ri).all() and (gv.view(np.uint32) == rv.view(np.uint32)).all()):
            log(f"PARITY FAILED on matrix {s}; no throughput reported")
            return 1
    log("parity vs oracle ok (bit-exact ids and values on sampled rows)")
    # one step = the top-K of every matrix, captured as a HIP graph
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(w.steps):
            moe.vocab_topk(xs[s], w.K, ws, ids[s], vals[s])
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    for s in range(w.steps):
        if not (torch.equal(ids[s], eager[s][0]) and torch.equal(vals[s].view(torch.int32), eager[s][1].view(torch.int32))):
            log(f"graph replay differs from eager on matrix {s}; no throughput reported")
            return 1
    rows_per_step = w.steps * w.R
    value = rows_per_step / (ms_step / 1e3)
    log(f"step {ms_step * 1e3:.1f} us for {w.steps} matrices of {w.R} rows -> {value:,.0f} rows/s")
    # each kernel alone: graphs of back-to-back launches cycling the matrices
    stages = {}
    for st, name in ((0, "chunk_max"), (1, "topk_rows")):
        gs = torch.cuda.CUDAGraph()
        per = 4 * w.steps
        with torch.cuda.graph(gs):
            for i in range(per):
                moe.vocab_topk(xs[i % w.steps], w.K, ws, ids[i % w.steps], vals[i % w.steps], stage=st)
        gs.replay()
        torch.cuda.synchronize()
        reps = max(1, args.stage_reps // per)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            gs.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (reps * per)
        wb = vocab_work(w, st)
        stages[name] = {"us": round(us, 3), "bytes": int(wb), "flops": 0, "GBps": round(wb / us / 1e3, 1), "TFLOPs": 0.0}
        log(f"  {name:18s} {us:8.2f} us  {wb / 1e6:9.3f} MB  {wb / us / 1e3:8.1f} GB/s")
        del gs
    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
    st = stages["chunk_max"]
    roof = {"bound": "hbm", "achieved": st["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(st["GBps"] / HBM_PEAK_GBS, 4), "kernel": "chunk_max", "bytes_per_launch": st["bytes"],
            "flops_per_launch": 0, "avg_us": st["us"], "traffic": traffic_from_profiles(args.workload, "chunk_max")}
    out = {
        "metric": "top-K rows/s", "value": round(value, 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded generator)",
        "config": {"workload": f"exact top-{w.K} of {w.R} rows x {w.V} fp32 logits (softcapped normal), "
                               f"{w.steps} matrices cycled", "parallelism": "single GPU"},
        "roofline": roof, "stages": stages,
    }
    if not args.no_cpu:
        n, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < args.cpu_seconds:
            oracle.vocab_topk(host[0][n % w.R:n % w.R + 1], w.K)
            n += 1
        el = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": n / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} rows of the first matrix, one full sort each, {el:.1f} s"}
        log(f"cpu oracle: {n / el:.1f} rows/s")
    print(json.dumps(out), flush=True)
    return 0


# ------------------------------------------------------------------------- one workload
def layer_work(w: gen.Workload, counts: np.ndarray):
    """(bytes, expert flops) the method itself must move / do in one layer call: the packed weights
    of the experts with at least one row and of the shared expert, the router matrix, x and y; the
    flops of the expert products (2 per weight per row, no padding)."""
    d, E, k, I, Is, T = w.d, w.E, w.k, w.I, w.Is, w.chunk
    per_w = lambda out, inn: out * inn * w.bits // 8 + 2 * 2 * out * inn // 64  # noqa: E731
    act = int((counts > 0).sum())
    wb = act * 3 * per_w(I, d) + (3 * per_w(Is, d) if Is else 0)
    return wb + 4 * d * E + 2 * 2 * T * d, 2 * 3 * d * (T * k * I + T * Is)


def run_workload(name: str, args, dev, cpu_seconds: float, headline: bool) -> dict:
    """Parity gate, a HIP graph of one step timed with events, per-stage times, whole-layer and
    dominant-kernel roofline fractions and the oracle beside it, for one workload."""
    w = gen.WORKLOADS[name]
    n_layers, calls = PLAN[name]
    T = w.chunk

    # ---- inputs (seeded, synthetic), resident in HBM before timing
    t0 = time.perf_counter()
    layers, xs = [], []
    for li in range(n_layers):
        L = gen.layer(w, li)
        layers.append(to_layer(L, w.k, dev))
        xs.append(bf16_dev(gen.tokens(w, li, li if w.calls > 1 else 0), dev))
        del L
    ys = [torch.empty_like(x) for x in xs]
    wss = [lay.workspace(T) for lay in layers]
    torch.cuda.synchronize()
    log(f"{name}: {n_layers} layers resident in {time.perf_counter() - t0:.1f} s "
        f"({torch.cuda.memory_allocated(dev) / 1e9:.2f} GB)")
    order = [(i % n_layers) for i in range(calls)]

    # ---- eager pass + parity gate against the oracle on whole calls (fail-closed); the oracle's
    # time on these calls is the CPU baseline of the non-headline workloads
    for li in order:
        layers[li].forward(xs[li], wss[li], ys[li])
    torch.cuda.synchronize()
    eager = [ys[li].clone() for li in range(n_layers)]
    from oracle import oracle
    worst, o_time, o_tok, o_calls = 0.0, 0.0, 0, 0
    for li in range(min(2, n_layers)):
        L = gen.layer(w, li)
        x = gen.tokens(w, li, li if w.calls > 1 else 0)
        t1 = time.perf_counter()
        ref = oracle.forward_layer(x, L["w_router"], L["routed"], L["shared"], w.k, L["logit_bias"])["y"]
        o_time += time.perf_counter() - t1
        o_tok += x.shape[0]
        o_calls += 1
        r, g = f32_of_bits(ref), f32_of_bits(bits_of(eager[li]))
        tol = 1e-2 * np.abs(r).max() + 1e-3
        err = float(np.abs(g - r).max())
        worst = max(worst, err / tol)
        if not err <= tol:
            raise RuntimeError(f"{name}: PARITY FAILED on layer {li}: max err {err} > {tol}; no throughput reported")
        del L
    log(f"{name}: parity vs oracle ok on {o_calls} whole calls (worst error {worst:.3f} of the allowance)")

    # ---- HIP graph of one step
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(device=dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cap):
        for li in order:  # warm the capture stream once eagerly
            layers[li].forward(xs[li], wss[li], ys[li])
    torch.cuda.current_stream(dev).wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for li in order:
            layers[li].forward(xs[li], wss[li], ys[li])
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    for li in range(n_layers):  # replays must reproduce the eager results
        if not torch.equal(ys[li].view(torch.int16), eager[li].view(torch.int16)):
            raise RuntimeError(f"{name}: graph replay differs from eager on layer {li}; no throughput reported")
    del g
    tokens_per_step = calls * T
    value = tokens_per_step / (ms_step / 1e3)
    us_call = ms_step * 1e3 / calls
    log(f"{name}: step {ms_step * 1e3:.1f} us for {calls} layer calls ({us_call:.2f} us each) -> "
        f"{value:,.0f} MoE-layer tokens/s")

    # ---- per-kernel durations: each stage alone, captured as a HIP graph of back-to-back launches
    # that cycle the layers (so weights stream from HBM), timed with events on the launch stream
    names = layers[0].stages(T)
    counts = []
    for li in range(n_layers):
        r = moe.route(xs[li], layers[li].w_router, w.k, w.I, w.Is, layers[li].logit_bias)
        counts.append(r["counts"].cpu().numpy())
    per_graph = n_layers * max(1, 40 // n_layers)
    launch_layers = [i % n_layers for i in range(per_graph)]
    reps = max(1, args.stage_reps // per_graph)
    stages = {}
    for s, sname in enumerate(names):
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs):
            for li in launch_layers:
                layers[li].launch_stage(s, xs[li], ys[li], wss[li])
        gs.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            gs.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (reps * per_graph)
        wb = float(np.mean([stage_work(w, sname, counts[li])[0] for li in launch_layers]))
        wf = float(np.mean([stage_work(w, sname, counts[li])[1] for li in launch_layers]))
        stages[sname] = {"us": round(us, 3), "bytes": int(wb), "flops": int(wf),
                         "GBps": round(wb / us / 1e3, 1), "TFLOPs": round(wf / us / 1e6, 2)}
        log(f"  {sname:18s} {us:8.2f} us  {wb / 1e6:9.3f} MB  {wb / us / 1e3:8.1f} GB/s  {wf / us / 1e6:7.2f} TFLOP/s")
        del gs
    for li in range(n_layers):  # the stage loop leaves every layer's outputs as the eager pass did
        if not torch.equal(ys[li].view(torch.int16), eager[li].view(torch.int16)):
            raise RuntimeError(f"{name}: stage launches changed layer {li}'s output")

    # ---- whole-layer roofline: algorithmic bytes and expert flops per call against the call time
    lw = [layer_work(w, counts[li]) for li in order]
    lb = float(np.mean([b for b, _ in lw]))
    lf = float(np.mean([f for _, f in lw]))
    t_hbm = lb / (HBM_PEAK_GBS * 1e9)
    t_mfma = lf / (MFMA_BF16_PEAK_TFS * 1e12)
    layer = {"bytes_per_call": int(lb), "expert_flops_per_call": int(lf), "us_per_call": round(us_call, 3),
             "hbm_frac": round(lb / (us_call * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
             "mfma_frac": round(lf / (us_call * 1e-6) / (MFMA_BF16_PEAK_TFS * 1e12), 4),
             "bound": "hbm" if t_hbm >= t_mfma else "mfma",
             "floor_us": round(max(t_hbm, t_mfma) * 1e6, 3),
             "roofline_frac": round(max(t_hbm, t_mfma) * 1e6 / us_call, 4)}

    # ---- roofline of the dominant kernel (the gate/up stage of the path this call takes)
    dom = next((s for s in (DOMINANT[name], "gemv_gateup_topk", "gateup_gemm") if s in stages), None)
    if dom is None:
        raise RuntimeError(f"{name}: no gate/up stage on this call's path; stages: {list(stages)}")
    st = stages[dom]
    k_hbm = st["bytes"] / (HBM_PEAK_GBS * 1e9)
    k_mfma = st["flops"] / (MFMA_BF16_PEAK_TFS * 1e12)
    if k_hbm >= k_mfma:
        roof = {"bound": "hbm", "achieved": st["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(st["GBps"] / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": st["TFLOPs"], "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(st["TFLOPs"] / MFMA_BF16_PEAK_TFS, 4)}
    roof.update(kernel=dom, bytes_per_launch=st["bytes"], flops_per_launch=st["flops"], avg_us=st["us"],
                hbm_frac=round(st["GBps"] / HBM_PEAK_GBS, 4), mfma_frac=round(st["TFLOPs"] / MFMA_BF16_PEAK_TFS, 4),
                traffic=traffic_from_profiles(name, dom))

    res = {"workload": DESCR[name], "tokens_per_s": round(value, 1), "ms_per_step": round(ms_step, 6),
           "tokens_per_call": T, "layer_calls_per_step": calls, "parity_worst_of_allowance": round(worst, 4),
           "layer": layer, "roofline": roof, "stages": stages}
    # ---- the oracle beside it: the headline cycles its layers; the others report the oracle's
    # time on the parity calls above (whole calls of the same workload)
    if not args.no_cpu:
        if headline:
            res["cpu_baseline"] = cpu_baseline_cycle(w, n_layers, cpu_seconds)
        else:
            res["cpu_baseline"] = {"value": o_tok / o_time, "unit": "MoE-layer tokens/s", "cores": oracle.num_threads(),
                                   "kind": "oracle", "cpu": cpu_model(),
                                   "sample": f"{o_calls} whole layer calls of {T} tokens (the parity calls), "
                                             f"{o_time:.1f} s of oracle time"}
        log(f"{name}: cpu oracle {res['cpu_baseline']['value']:.2f} tokens/s on {res['cpu_baseline']['cores']} threads")
    del layers, xs, ys, wss, eager
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------- main
EXTRA_DEFAULT = "tiny,prefill,long,diffusion,diffusion2"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=sorted(PLAN) + sorted(gen.VOCAB_WORKLOADS))
    ap.add_argument("--extra", default=EXTRA_DEFAULT,
                    help="comma-separated workloads measured after the headline one and reported under "
                         "'workloads' in the same JSON line ('' for none)")
    ap.add_argument("--stage-reps", type=int, default=200, help="timed launches per stage")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib-copy", action="store_true", help="also run a plain 256 MiB device copy (counter scale)")
    ap.add_argument("--calib-mfma", action="store_true",
                    help="also time a large bf16 torch.matmul (8192^3): the matrix-core rate a library GEMM reaches")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        return 2
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.workload in gen.VOCAB_WORKLOADS:
        return main_vocab(args)
    dev = torch.device("cuda:0")
    log(f"device {torch.cuda.get_device_name(dev)}; host {cpu_model()}")
    try:
        head = run_workload(args.workload, args, dev, args.cpu_seconds, headline=True)
        extras = {}
        for name in [n for n in args.extra.split(",") if n and n != args.workload]:
            extras[name] = run_workload(name, args, dev, args.cpu_seconds, headline=False)
    except RuntimeError as e:
        log(str(e))
        return 1

    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
    calib = calib_mfma(dev) if args.calib_mfma else None

    w = gen.WORKLOADS[args.workload]
    out = {
        "metric": "MoE-layer tokens/s", "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded generator)",
        "config": {"workload": DESCR[args.workload], "tokens_per_call": w.chunk,
                   "layer_calls_per_step": head["layer_calls_per_step"], "parallelism": "single GPU"},
        "roofline": head["roofline"], "layer": head["layer"], "stages": head["stages"],
        "parity_worst_of_allowance": head["parity_worst_of_allowance"],
    }
    if calib is not None:
        out["calibration"] = calib
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head["cpu_baseline"]
    if extras:
        out["workloads"] = extras
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
