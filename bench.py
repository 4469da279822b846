#!/usr/bin/env python3
"""Benchmark of the 3-bit FP8-codebook decode linear layer on one MI355X.

Headline (the JSON line's `value`): packed-weight GB/s of the M=1 decode GEMV
on the 4096 x 4096 layer shape (K = N = 4096, M = 1), streamed over a stack of
128 distinct packed copies of that layer (872 MB, more than three times the
256 MB last-level cache) so every launch reads cold weights from HBM.  One *step*
is one pass over the stack: one launch per layer, back to back on one stream,
replayed from a HIP graph.  value = payload bytes per step / step time, where
payload = N*K*13/32 bytes per layer (3-bit codes + one 8-bit scale per 32
weights, 3.25 bits/weight).

The same line carries:
  roofline      the dominant kernel's algorithmic bytes per launch over its
                average launch duration (HIP events on the launch stream),
                against the 8 TB/s HBM peak; traffic from rocprofv3 counters
                when the committed counter file matches the current sources.
  cpu_baseline  the CPU oracle (numpy fp64) on a bounded sample of the same
                layer, on this host's cores.
  points        per-kernel throughput at M = 1/4/8 (4096 x 4096), M = 16
                (K=8192, N=28672), M = 64 (K=4096, N=151936), the
                expert-grouped MoE verify round and the two-bit draft head
                (2-bit shortlist of 16 over N=151936, MXFP8 rescore), each on
                cold rotating copies; the quantizer and the per-row codebook
                fit on the K=8192 N=28672 matrix.

Inputs are synthetic and seeded (codes uniform 0..7, per-row codebooks of
N(0,1) draws rounded to E4M3, power-of-two group scales 2^-10..2^-4, bf16
N(0,1) activations); no dataset or trained weight is involved.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from bench_traffic import source_hash  # noqa: E402  (hash of the library sources the counters were taken on)

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
LLC_BYTES = 256 << 20
METRIC = "packed-weight HBM GB/s and % of MI355X peak at M=1/8/64; oracle-exact"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
MOE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_moe_round.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


# The sustained M=1 weight stream of the headline: 128 distinct 4096x4096 layers
# back to back (872 MB of packed weights, over 3x the last-level cache).
HEADLINE_LAYERS = 128


def copies_for(nbytes: int, minimum: int = 2) -> int:
    """Distinct copies so that one cycle through them is >= 2x the LLC."""
    return max(minimum, -(-2 * LLC_BYTES // max(nbytes, 1)))


GRAPH_LAUNCHES = 64


def cycles_for(copies: int) -> int:
    """Passes over the copies captured in one graph: at least GRAPH_LAUNCHES
    launches per replay, so the gap between two replays is spread over as many
    back-to-back launches as a layer stream has (a graph of 3 launches of the
    151936-row matrix would add that gap to every third launch).  Each copy is
    still read cold: the other copies pass through the cache in between."""
    return max(1, -(-GRAPH_LAUNCHES // copies))


class Timer:
    """HIP events recorded on the stream the kernels are launched on."""

    def __init__(self, stream):
        import torch
        self.stream = stream
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.a.record(self.stream)
        return self

    def __exit__(self, *exc):
        self.b.record(self.stream)
        self.b.synchronize()
        self.ms = self.a.elapsed_time(self.b)


def capture(fn, stream):
    """Capture fn() (a sequence of library launches on `stream`) into a graph."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn()                       # warm: loads code objects, sets attributes
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            fn()
    torch.cuda.synchronize()
    return g


TRIALS = 5
REPS = 0          # --reps: replays per trial for every point (0: each point's own default)


def time_graph(g, stream, reps: int, warmup: int, trials: int = None):
    """Median over `trials` timings of `reps` back-to-back replays (ms per
    replay), and every trial's figure."""
    import torch
    trials = TRIALS if trials is None else trials
    reps = REPS or reps
    per = []
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        for _ in range(trials):
            with Timer(stream) as t:
                for _ in range(reps):
                    g.replay()
            per.append(t.ms / reps)
    s = sorted(per)
    return s[len(s) // 2], per


def algorithmic_bytes(n, k, m):
    """Payload (codes + scales) + codebook + bf16 activations + fp32 outputs."""
    return n * k * 13 // 32 + 8 * n + 2 * m * k + 4 * m * n


# ------------------------------------------------------------------ points

def linear_point(q3, synth, n, k, m, kernel, reps=20, warmup=3, name=""):
    import torch
    layer, x = synth.make_linear(n, k, m, seed=0)
    w0 = q3.q3_pack(to_dev(layer.codes), to_dev(layer.scales), to_dev(layer.codebook))
    del layer
    ncopy = copies_for(w0.payload_bytes)
    ws = [w0] + [w0.clone() for _ in range(ncopy - 1)]
    xd = to_dev(x)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    if kernel == "mfma_ws":
        # one caller-owned workspace serves every launch (they run in order on one stream)
        wsb = torch.empty(max(16, q3.q3_gemm_small_m_workspace_bytes(n, k, m)), dtype=torch.uint8, device="cuda")
        fn = lambda w_, x_, y_: q3.q3_gemm_small_m_ws(w_, x_, y_, wsb)  # noqa: E731
    else:
        fn = q3.q3_gemv if kernel == "gemv" else q3.q3_gemm_small_m
    stream = torch.cuda.Stream()
    cyc = cycles_for(len(ws))
    g = capture(lambda: [fn(w, xd, y) for _ in range(cyc) for w in ws], stream)
    ms, trials = time_graph(g, stream, reps, warmup)
    us = ms * 1e3 / (cyc * len(ws))
    payload = n * k * 13 // 32
    flops = 2.0 * m * n * k
    pt = dict(name=name, n=n, k=k, m=m, kernel=kernel, copies=len(ws), us_per_launch=round(us, 2),
              trials_us=[round(t * 1e3 / (cyc * len(ws)), 2) for t in trials],
              payload_GBps=round(payload / us / 1e3, 1),
              pct_of_8TBps=round(100 * payload / us / 1e3 / HBM_PEAK_GBPS, 1),
              algorithmic_GBps=round(algorithmic_bytes(n, k, m) / us / 1e3, 1),
              tokens_per_s=round(m / (us * 1e-6), 1),
              mfma_pct_of_bf16_peak=round(100 * flops / (us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 2)
              if kernel != "gemv" else None)
    if kernel == "mfma_ws":
        pt["k_splits"] = max(1, q3.q3_gemm_small_m_workspace_bytes(n, k, m) // (4 * m * n))
    del ws, w0, g
    torch.cuda.empty_cache()
    return pt


def moe_point(q3, synth, budget=None, fused=False, reps=20, warmup=3):
    """Config 2: 64 experts (gate/up 2048->1536, down 768->2048), 8 drafted
    tokens, top-8 routing; one round = router + grouped gate/up + grouped down.
    With a budget the router keeps the `budget` experts of largest routing mass
    and routes each token's top-8 inside them.  Fused: the round is the router
    and the fused expert MLP (SwiGLU between the products, outputs combined by
    routing weight into one row per token)."""
    import numpy as np
    import torch
    moe = synth.make_moe(seed=0)
    E = len(moe.experts_gu)

    def stack(layers):
        L = layers[0]
        st = q3.empty_stack(E, L.n, L.k, "cuda")
        for e, layer in enumerate(layers):
            q3.q3_pack(to_dev(layer.codes), to_dev(layer.scales), to_dev(layer.codebook), out=st.expert(e))
        return st

    st_gu0, st_dn0 = stack(moe.experts_gu), stack(moe.experts_dn)
    per_expert = st_gu0.payload_bytes_per_expert + st_dn0.payload_bytes_per_expert
    ncopy = copies_for(E * per_expert)
    stacks = [(st_gu0, st_dn0)]
    for _ in range(ncopy - 1):
        a, b = st_gu0, st_dn0
        stacks.append((q3.ExpertStack(E, a.n, a.k, a.code_plane.clone(), a.scale_plane.clone(), a.codebook.clone()),
                       q3.ExpertStack(E, b.n, b.k, b.code_plane.clone(), b.scale_plane.clone(), b.codebook.clone())))
    logits = to_dev(moe.logits)
    x = to_dev(moe.x)
    x_dn = to_dev(np.ascontiguousarray(moe.x_dn).reshape(-1, moe.x_dn.shape[-1]))
    t, topk = moe.logits.shape[0], 8
    ids = torch.empty((t, topk), dtype=torch.int32, device="cuda")
    y_gu = torch.empty((t * topk, st_gu0.n), dtype=torch.float32, device="cuda")
    y_dn = torch.empty((t * topk, st_dn0.n), dtype=torch.float32, device="cuda")
    kept = torch.empty(budget or 1, dtype=torch.int32, device="cuda")
    ws = q3.moe_mlp_workspace(st_gu0, st_dn0, t, topk, "cuda") if fused else None
    out = torch.empty((t, st_dn0.n), dtype=torch.float32, device="cuda")

    cyc = cycles_for(len(stacks))

    def round_all():
        for gu, dn in [st for _ in range(cyc) for st in stacks]:
            if budget is None:
                q3.q3_moe_topk(logits, topk, ids)
            else:
                q3.q3_moe_budget_topk(logits, topk, budget, ids, kept)
            if fused:
                q3.q3_moe_mlp(gu, dn, x, ids, logits, ws, out)
            else:
                q3.q3_grouped_expert_gemv(gu, x, ids, False, y_gu)
                q3.q3_grouped_expert_gemv(dn, x_dn, ids, True, y_dn)

    stream = torch.cuda.Stream()
    g = capture(round_all, stream)
    ms, trials = time_graph(g, stream, reps, warmup)
    us = ms * 1e3 / (cyc * len(stacks))
    union = int(np.unique(ids.cpu().numpy()).size)
    payload = union * per_expert
    # share of the round's routing mass on the experts read (plain softmax of the logits)
    z = np.exp(moe.logits.astype(np.float64) - moe.logits.max(axis=1, keepdims=True))
    mass = (z / z.sum(axis=1, keepdims=True)).sum(axis=0)
    read_mass = float(mass[np.unique(ids.cpu().numpy())].sum() / mass.sum())
    name = ("moe_mlp_round" if fused else "moe_verify_round") + ("" if budget is None else f"_budget{budget}")
    pt = dict(name=name, experts=E, tokens=t, topk=topk, budget=budget, experts_read=union,
              routing_mass_read=round(read_mass, 4),
              copies=len(stacks), us_per_round=round(us, 2),
              trials_us=[round(t_ * 1e3 / (cyc * len(stacks)), 2) for t_ in trials],
              union_payload_bytes=payload,
              payload_GBps=round(payload / us / 1e3, 1),
              pct_of_8TBps=round(100 * payload / us / 1e3 / HBM_PEAK_GBPS, 1),
              tokens_per_s=round(t / (us * 1e-6), 1),
              kernel=("router + fused SwiGLU gate/up + down with combine" if fused
                      else "mfma grouped + top-k router"))
    if budget is None and not fused:
        # Union pin: a round's two expert passes read |U| experts' planes and
        # codebooks once (HBM counters of the same sources, when committed).
        pt["union_bytes_with_codebooks"] = union * (per_expert + 8 * (st_gu0.n + st_dn0.n))
        tr = moe_traffic()
        if tr is not None:
            pt["hbm_read_bytes_per_round"] = tr["read_bytes_per_round"]
            pt["hbm_read_over_union_bytes"] = round(tr["read_bytes_per_round"] / pt["union_bytes_with_codebooks"], 4)
    del stacks, g
    torch.cuda.empty_cache()
    return pt


def quantize_point(q3, synth, n=28672, k=8192, reps=10, warmup=2):
    """Quantizer on the K=8192 N=28672 matrix: fp32 weights (N(0,1) times a
    power of two per group, drawn on the GPU from a fixed seed) and E4M3FN
    codebooks -> codes and scale bytes, one launch.  Algorithmic bytes: 4 per
    weight read, 1 + 1/32 written, 8 per row of codebook."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(0)
    w = torch.randn((n, k), generator=gen, device="cuda", dtype=torch.float32)
    u = torch.randint(-12, 4, (n, k // 32), generator=gen, device="cuda").to(torch.float32)
    w *= torch.exp2(u).repeat_interleave(32, dim=1)
    del u
    cb = (torch.randn((n, 8), generator=gen, device="cuda")).to(torch.float8_e4m3fn).view(torch.uint8)
    codes = torch.empty((n, k), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, k // 32), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            q3.q3_quantize(w, cb, codes, scales)
        stream.synchronize()
        with Timer(stream) as t:
            for _ in range(reps):
                q3.q3_quantize(w, cb, codes, scales)
    us = t.ms * 1e3 / reps
    alg = n * k * 4 + n * k + n * k // 32 + n * 8
    pt = dict(name=f"quantize K={k} N={n} (fp32 -> codes + scales)", n=n, k=k, us_per_launch=round(us, 1),
              algorithmic_bytes=alg, GBps=round(alg / us / 1e3, 1),
              pct_of_8TBps=round(100 * alg / us / 1e3 / HBM_PEAK_GBPS, 1), kernel="quantize_kernel")
    del w, codes, scales, cb
    torch.cuda.empty_cache()
    return pt


def fit_point(q3, n=28672, k=8192, reps=5, warmup=1):
    """Per-row codebook fitting on the K=8192 N=28672 matrix: fp32 weights
    (N(0,1) drawn on the GPU from a fixed seed) -> one 8-entry E4M3FN codebook
    per row, one launch.  Algorithmic bytes: 4 per weight read, 8 per row written."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(0)
    w = torch.randn((n, k), generator=gen, device="cuda", dtype=torch.float32)
    cb = torch.empty((n, 8), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    per = []
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            q3.q3_fit_codebook(w, cb)
        stream.synchronize()
        for _ in range(TRIALS):
            with Timer(stream) as t:
                for _ in range(reps):
                    q3.q3_fit_codebook(w, cb)
            per.append(t.ms * 1e3 / reps)
    us = sorted(per)[len(per) // 2]
    alg = n * k * 4 + n * 8
    pt = dict(name=f"codebook fit K={k} N={n} (fp32 -> per-row E4M3FN codebooks)", n=n, k=k,
              us_per_launch=round(us, 1), trials_us=[round(v, 1) for v in per], algorithmic_bytes=alg,
              GBps=round(alg / us / 1e3, 1), pct_of_8TBps=round(100 * alg / us / 1e3 / HBM_PEAK_GBPS, 1),
              rows_per_s=round(n / (us * 1e-6), 1), kernel="fit_kernel")
    del w, cb
    torch.cuda.empty_cache()
    return pt


def draft_head_point(q3, synth, n=151936, k=4096, m=1, size=16, reps=10, warmup=2):
    """Two-bit draft head on a vocabulary-sized head: 2-bit scores of every row,
    shortlist of 16, MXFP8 rescoring of the 16 and the decision (four launches),
    on cold copies of the 2-bit head."""
    import torch
    head, x = synth.make_head(n, k, m, seed=0)
    w0 = q3.q3_pack2(to_dev(head.codes), to_dev(head.scales), to_dev(head.codebook))
    h8 = q3.Mxfp8Head(n, k, to_dev(head.e8), to_dev(head.s8))
    del head
    ncopy = copies_for(w0.payload_bytes)
    ws = [w0] + [q3.PackedHead2(n, k, w0.code_plane.clone(), w0.scale_plane.clone(), w0.codebook.clone())
                 for _ in range(ncopy - 1)]
    xd = to_dev(x)
    work = q3.draft_head_workspace(m, n, "cuda")
    stream = torch.cuda.Stream()
    cyc = cycles_for(len(ws))
    g = capture(lambda: [q3.q3_draft_head(w, h8, xd, size, work) for _ in range(cyc) for w in ws], stream)
    ms, trials = time_graph(g, stream, reps, warmup)
    us = ms * 1e3 / (cyc * len(ws))
    payload = w0.payload_bytes + m * size * (k + k // 32)     # 2-bit head + the listed MXFP8 rows
    pt = dict(name="draft head K=4096 N=151936 M=1 (2-bit shortlist of 16, MXFP8 rescore)", n=n, k=k, m=m,
              shortlist=size, copies=len(ws), us_per_decision=round(us, 2),
              trials_us=[round(t * 1e3 / (cyc * len(ws)), 2) for t in trials], payload_bytes=payload,
              payload_GBps=round(payload / us / 1e3, 1),
              pct_of_8TBps=round(100 * payload / us / 1e3 / HBM_PEAK_GBPS, 1),
              decisions_per_s=round(m / (us * 1e-6), 1),
              kernel="2-bit matrix-core scores + two-pass shortlist + MXFP8 rescore")
    del ws, w0, h8, g, work
    torch.cuda.empty_cache()
    return pt


# ------------------------------------------------------------ read ceilings

def read_ceiling(nbytes: int, configs, reps: int = 10, warmup: int = 2, name: str = "", copies: int = 0):
    """The best a launch that only streams `nbytes` achieves on this GPU, timed
    like the products: graph-replayed back-to-back launches over distinct
    copies (one cycle >= 2x the last-level cache), median of 5 trials, over a
    sweep of (blocks, loads in flight per thread).  Also the cost of one
    dependent launch of an empty kernel (the per-launch floor)."""
    import torch
    import bench_ceiling
    copies = copies or copies_for(nbytes)
    bufs = [torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    sp = stream.cuda_stream
    cyc = cycles_for(copies)
    launches = cyc * copies
    sweep = []
    for blocks, unroll in configs:
        g = capture(lambda: [bench_ceiling.read(b, blocks, unroll, sink, sp) for _ in range(cyc) for b in bufs],
                    stream)
        ms, _ = time_graph(g, stream, reps, warmup)
        sweep.append((round(ms * 1e3 / launches, 3), blocks, unroll))
        del g
    g = capture(lambda: [bench_ceiling.empty(256, sp) for _ in range(launches)], stream)
    empty_us = time_graph(g, stream, reps, warmup)[0] * 1e3 / launches
    del g, bufs
    torch.cuda.empty_cache()
    us, blocks, unroll = min(sweep)
    return dict(name=name, bytes=nbytes, copies=copies, launches_per_graph=launches, us_per_launch=us,
                GBps=round(nbytes / us / 1e3, 1), pct_of_8TBps=round(100 * nbytes / us / 1e3 / HBM_PEAK_GBPS, 1),
                best_blocks=blocks, best_loads_in_flight_per_thread=unroll,
                empty_kernel_us_per_launch=round(empty_us, 3),
                sweep_us=[[u, b, r] for u, b, r in sweep])


# Launch shapes swept per size: (blocks of 256 threads, 16-byte loads in flight per thread).
CEILING_SWEEPS = {
    "layer_4096x4096": (4096 * 4096 * 13 // 32,
                        [(b, u) for b in (256, 512, 1024, 1664, 2048) for u in (1, 2, 4, 8)]),
    "layer_K8192_N28672": (28672 * 8192 * 13 // 32,
                           [(b, u) for b in (1024, 2048, 4096, 8192) for u in (2, 4, 8, 16)]),
    "layer_K4096_N151936": (151936 * 4096 * 13 // 32, [(b, u) for b in (2048, 8192) for u in (4, 8)]),
}


def eager_us_per_call(fn, ws, xd, y, stream, rounds: int = 3):
    """Per-call time of back-to-back calls issued from Python (no graph),
    median of 5 trials of `rounds` passes over the copies: includes the host's
    launch cost, which bounds it when a launch is short."""
    import torch
    per = []
    with torch.cuda.stream(stream):
        for w in ws:
            fn(w, xd, y)
        torch.cuda.synchronize()
        for _ in range(TRIALS):
            with Timer(stream) as t:
                for _ in range(rounds):
                    for w in ws:
                        fn(w, xd, y)
            per.append(t.ms * 1e3 / (rounds * len(ws)))
    return round(sorted(per)[len(per) // 2], 3)


# -------------------------------------------------------------- cpu baseline

def cpu_baseline(synth, budget_s=12.0):
    """The CPU oracle on the 4096 x 4096, M = 1 layer: unpack from the packed
    planes, fp64 dequantisation and products, as the tests use it.  A bounded
    sample: passes until about budget_s seconds (at most 200)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    cores = len(os.sched_getaffinity(0))
    layer, x = synth.make_linear(4096, 4096, 1, seed=0)
    cp, sp = oracle.pack(layer.codes, layer.scales)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.linear(cp, sp, layer.codebook, 4096, 4096, x)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 200:
            break
    per = el / reps
    payload = 4096 * 4096 * 13 // 32
    # The same oracle with BLAS held to one thread, on a shorter bounded sample.
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            reps1, t1 = 0, time.perf_counter()
            while True:
                oracle.linear(cp, sp, layer.codebook, 4096, 4096, x)
                reps1 += 1
                el1 = time.perf_counter() - t1
                if el1 >= budget_s / 2 or reps1 >= 50:
                    break
        single = dict(value=round(payload / (el1 / reps1) / 1e9, 4), unit="GB/s", cores=1,
                      seconds_per_layer=round(el1 / reps1, 3), passes=reps1)
    except ImportError:
        pass
    return dict(value=round(payload / per / 1e9, 4), unit="GB/s", cores=int(min(threads, cores)),
                kind="oracle", seconds_per_layer=round(per, 3), host_cores=cores,
                sample=f"{reps} oracle passes over one 4096x4096 layer at M=1 "
                       "(unpack from packed planes, fp64 dequant and product; BLAS may use every "
                       "core, the numpy unpacking and dequantisation run on one)",
                single_thread=single)


def _traffic_file(path=None):
    try:
        with open(path or TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("source_hash") == source_hash() else None


def _kernel_args(name: str, family: str):
    if not (name.startswith(family + "<") and name.endswith(">")):
        return None
    return [a.strip() for a in name[len(family) + 1:-1].split(",")]


def read_traffic(dot: bool):
    """(kernel name, per-launch HBM bytes) of the M=1 kernel of the measured
    layer from the committed counter file, or (family name, None) when that
    file was taken on other sources.  Kernels are named by their template
    arguments."""
    family = "splitk_kernel (vector-ALU, M=1)" if dot else "splitk_kernel (matrix-core, M=1)"
    t = _traffic_file()
    if t is None:
        return family, None

    def dense_m1(k):
        # The 4096 x 4096 layer at one token runs the split-K kernel: 16 waves,
        # one half-step each, one token (template <waves, half-steps, vector-ALU, tokens>).
        args = _kernel_args(k, "splitk_kernel")
        return args == ["16", "1", "true" if dot else "false", "1"]
    cands = [(v.get("dispatches", 0), k, v) for k, v in t.get("kernels", {}).items() if dense_m1(k)]
    if not cands:
        return family, None
    _, name, v = max(cands)
    return name, v


def moe_traffic():
    """HBM bytes the two grouped products of one plain verify round read, from
    the committed counter file (None when absent or taken on other sources):
    the expert passes are one kernel instance (grouping 1) dispatched once for
    gate/up and once for down per round, so a round reads twice its average
    (counters of a run that times only the plain round)."""
    t = _traffic_file(MOE_TRAFFIC_FILE)
    if t is None:
        return None
    cands = []
    for k, v in t.get("kernels", {}).items():
        args = _kernel_args(k, "linear_kernel")
        if args is not None and len(args) == 7 and args[3] == "1" and args[6] == "3" and v.get("read_bytes"):
            cands.append((v.get("dispatches", 0), k, v))
    if not cands:
        return None
    _, k, v = max(cands)
    return dict(kernel=k, read_bytes_per_round=2 * v["read_bytes"], dispatches=v.get("dispatches"))


# --------------------------------------------------------------------- main

def main():
    global REPS, TRIALS
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=HEADLINE_LAYERS, help="distinct layers per step (default 128)")
    ap.add_argument("--kernel", choices=["auto", "gemv", "mfma"], default="auto")
    ap.add_argument("--no-points", action="store_true", help="skip the per-config points")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the read-ceiling probes")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB device copy first (scale reference for counter runs)")
    ap.add_argument("--only-vocab", action="store_true",
                    help="time only the K=4096 N=151936 M=64 point (for counter runs of its kernel) and print it")
    ap.add_argument("--only-moe", action="store_true",
                    help="time only the plain MoE verify round (for counter runs of the expert passes) and print it")
    ap.add_argument("--only-layer", action="store_true",
                    help="time only the 4096x4096 M=1 layer on the matrix cores (counter runs) and print it")
    ap.add_argument("--only-stream", action="store_true",
                    help="time only the K=8192 N=28672 M=1 stream on the matrix cores (counter runs) and print it")
    ap.add_argument("--reps", type=int, default=0, help="graph replays per trial for every point (profiler runs)")
    ap.add_argument("--trials", type=int, default=TRIALS, help="trials per point (median reported)")
    args = ap.parse_args()
    REPS, TRIALS = args.reps, max(1, args.trials)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: the decode linear layer is benchmarked on a single "
                  "MI355X (multi-GPU sharding is a design note, not a measured path); run with --gpus 1.",
                  file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_fp8_codebook_amd as q3
    import synth
    q3.lib()
    torch.cuda.init()

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.only_vocab:
        print(json.dumps(linear_point(q3, synth, 151936, 4096, 64, "mfma", reps=args.steps, warmup=args.warmup,
                                      name="K=4096 N=151936 M=64")), flush=True)
        return
    if args.only_moe:
        print(json.dumps(moe_point(q3, synth, reps=args.steps, warmup=args.warmup)), flush=True)
        return
    if args.only_layer or args.only_stream:
        n_, k_ = (4096, 4096) if args.only_layer else (28672, 8192)
        print(json.dumps(linear_point(q3, synth, n_, k_, 1, "mfma", reps=args.steps, warmup=args.warmup,
                                      name=f"K={k_} N={n_} M=1")), flush=True)
        return

    n = k = 4096
    m = 1
    layer, x = synth.make_linear(n, k, m, seed=0)
    w0 = q3.q3_pack(to_dev(layer.codes), to_dev(layer.scales), to_dev(layer.codebook))
    xd = to_dev(x)

    # Parity of the measured layer against the oracle (the metric is oracle-exact).
    import oracle
    cp, sp = oracle.pack(layer.codes, layer.scales)
    y_ref, bound = oracle.linear(cp, sp, layer.codebook, n, k, x)
    parity = {}
    for name, fn in (("gemv", q3.q3_gemv), ("mfma", q3.q3_gemm_small_m)):
        ok, ratio = oracle.within_tolerance(fn(w0, xd).cpu().numpy(), y_ref, bound)
        parity[name] = dict(ok=ok, max_err_over_bound=ratio)
        if not ok:
            log(f"parity FAILED for {name}: {ratio:.3e}")
            sys.exit(1)
    log(f"parity of the measured layer: {parity}")

    layers = args.layers if args.layers > 0 else HEADLINE_LAYERS
    ws = [w0] + [w0.clone() for _ in range(layers - 1)]
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    kernels = {"gemv": q3.q3_gemv, "mfma": q3.q3_gemm_small_m}

    # Pick the faster M=1 kernel on this stack (both are reported in points).
    probe = {}
    for name, fn in kernels.items():
        g = capture(lambda fn=fn: [fn(w, xd, y) for w in ws], stream)
        probe[name] = time_graph(g, stream, 5, 2, trials=1)[0]
        del g
    chosen = min(probe, key=probe.get) if args.kernel == "auto" else args.kernel
    fn = kernels[chosen]
    g = capture(lambda: [fn(w, xd, y) for w in ws], stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            g.replay()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    with torch.cuda.stream(stream):
        with Timer(stream) as t:
            for _ in range(args.steps):
                g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = t.ms / args.steps
    # The same graph over 5 further trials of the same length, for the spread.
    _, spread = time_graph(g, stream, args.steps, 1)
    del g
    eager = eager_us_per_call(fn, ws, xd, y, stream)
    log(f"headline: {ms_step * 1e3 / layers:.3f} us per launch ({chosen}), eager {eager} us per call")
    payload = w0.payload_bytes
    value = layers * payload / (ms_step * 1e-3) / 1e9
    launch_us = ms_step * 1e3 / layers
    alg = algorithmic_bytes(n, k, m)
    achieved = alg / (launch_us * 1e-6) / 1e9
    kname, counted = read_traffic(dot=(chosen == "gemv"))
    # traffic: HBM bytes per launch (read + written, copy-calibrated counters);
    # the two directions and the dispatch count beside it.
    traffic = None
    if counted is not None and counted.get("read_bytes") is not None and counted.get("write_bytes") is not None:
        traffic = int(counted["read_bytes"]) + int(counted["write_bytes"])
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=traffic,
                    traffic_read_bytes=None if traffic is None else int(counted["read_bytes"]),
                    traffic_write_bytes=None if traffic is None else int(counted["write_bytes"]),
                    traffic_counted_dispatches=None if traffic is None else counted.get("dispatches"),
                    kernel=kname, algorithmic_bytes_per_launch=alg, avg_launch_us=round(launch_us, 3),
                    trials_us_per_launch=[round(v * 1e3 / layers, 3) for v in spread],
                    eager_us_per_call=eager)

    ceilings = {}
    if not args.no_ceiling:
        for cname, (nbytes, cfgs) in CEILING_SWEEPS.items():
            ceilings[cname] = read_ceiling(nbytes, cfgs, name=cname,
                                           copies=layers if cname == "layer_4096x4096" else 0)
            log(cname, {k_: v_ for k_, v_ in ceilings[cname].items() if k_ != "sweep_us"})
        c = ceilings["layer_4096x4096"]
        roofline["read_ceiling_us_per_launch"] = c["us_per_launch"]
        roofline["pct_of_read_ceiling"] = round(100 * c["us_per_launch"] / launch_us, 1)

    def with_ceiling(pt, cname):
        if cname in ceilings:
            pt["read_ceiling_us"] = ceilings[cname]["us_per_launch"]
            pt["pct_of_read_ceiling"] = round(100 * ceilings[cname]["us_per_launch"] / pt["us_per_launch"], 1)
        return pt

    points = []
    if not args.no_points:
        for kn in ("gemv", "mfma"):
            for mm in (1, 4, 8):
                points.append(linear_point(q3, synth, 4096, 4096, mm, kn, name=f"4096x4096 M={mm}"))
                log(points[-1])
        for kn in ("gemv", "mfma"):
            points.append(with_ceiling(linear_point(q3, synth, 28672, 8192, 1, kn, name="K=8192 N=28672 M=1"),
                                       "layer_K8192_N28672"))
            log(points[-1])
        points.append(with_ceiling(linear_point(q3, synth, 28672, 8192, 16, "mfma", name="K=8192 N=28672 M=16"),
                                   "layer_K8192_N28672"))
        log(points[-1])
        points.append(with_ceiling(linear_point(q3, synth, 151936, 4096, 64, "mfma", reps=5,
                                                name="K=4096 N=151936 M=64"), "layer_K4096_N151936"))
        log(points[-1])
        # Verify batches on matrices with few row tiles: one pass, and K split
        # over blocks through a workspace (q3_gemm_small_m_ws).
        for nn, kk, mm in ((4096, 4096, 16), (4096, 4096, 64), (8192, 28672, 16)):
            for kn in ("mfma", "mfma_ws"):
                points.append(linear_point(q3, synth, nn, kk, mm, kn, name=f"K={kk} N={nn} M={mm}"))
                log(points[-1])
        for fused in (False, True):
            for budget in (None, 16):
                points.append(moe_point(q3, synth, budget=budget, fused=fused))
                log(points[-1])
        points.append(draft_head_point(q3, synth))
        log(points[-1])
        points.append(quantize_point(q3, synth))
        log(points[-1])
        points.append(fit_point(q3))
        log(points[-1])
        points.append(linear_point(q3, synth, 1024, 1024, 1, chosen, name="1024x1024 M=1"))
        log(points[-1])

    cpu = None if args.no_cpu_baseline else cpu_baseline(synth)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded codes, E4M3 codebooks, E8M0 scales, bf16 N(0,1) activations)",
        "config": {"workload": f"decode GEMV, K=4096 N=4096 M=1, a sustained stream of {layers} distinct layers per step",
                   "K": k, "N": n, "M": m, "layers_per_step": layers, "kernel": chosen,
                   "pct_of_8TBps": round(100 * value / HBM_PEAK_GBPS, 2),
                   "tokens_per_s_per_layer": round(m / (launch_us * 1e-6), 1),
                   "wall_s_timed_region": round(wall, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "kernel_choice_ms_per_step": {k_: round(v_, 4) for k_, v_ in probe.items()},
        "read_ceilings": ceilings,
        "points": points,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
