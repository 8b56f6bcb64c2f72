#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet token mixer on one MI355X.

One step = the hot path over one batch of synthetic input:
  prefill layer on the Qwen3.5-9B shape, T = 4096 tokens, bf16 io:
      gdn_conv_chunk_prefill (conv + chunked core in one call) -> gdn_gated_rmsnorm
  decode step on the Qwen3.5-9B shape, 256 sequences, bf16 io, fp32 state:
      gdn_recurrent_step (conv + state updated in place) -> gdn_gated_rmsnorm
  and, timed beside the step, the same step with the conv and the chunked core as two
  calls (prefill_unfused, with the chunked core's own roofline), the decode step on a
  bf16-stored state
  (gdn_recurrent_step_bf16_state, roofline_decode_bf16_state) and the prompt -> decode
  replay (one sequence: 1024-token prompt, then 256 decode steps eager and as one HIP
  graph; "replay"), and the chunked core and fused prefill layer on the 397B T=32768 and
  9B 64-sequence varlen workloads ("prefill_configs").

Reported ("value"): layer prefill tokens/s = 4096 / (conv+chunk call + norm time),
with the core's algorithmic flops over that call's time against the bf16 dense MFMA peak
(roofline) and the decode
step's algorithmic bytes against the HBM peak (roofline_decode).  Kernel times come
from HIP events recorded on the stream the kernels run on (torch's current stream).
Inputs are resident in HBM before timing starts.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --calib-copy MIB   (one plain copy, for PMC byte scaling)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

D = 128
CHUNK = 64
PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12       # MI355X HBM3E
FLUSH_BYTES = 512 << 20       # overwritten before each timed prefill (last-level cache 256 MB)


CSRC = os.path.join(ROOT, "hybrid_linear_attention_causal_amd", "csrc")
KERNEL_SOURCES = {"gdn_chunk_prefill": ("gdn_chunk.hip", "gdn_common.hpp", "gdn_launch.hpp"),
                  "gdn_conv_chunk_prefill": ("gdn_chunk.hip", "gdn_conv1d.hip", "gdn_common.hpp",
                                             "gdn_launch.hpp"),
                  "gdn_recurrent_step": ("gdn_step.hip", "gdn_common.hpp", "gdn_launch.hpp"),
                  "gdn_recurrent_step_bf16_state": ("gdn_step.hip", "gdn_common.hpp",
                                                    "gdn_launch.hpp")}
# HBM bytes per launch from rocprofv3 PMC FETCH_SIZE and WRITE_SIZE, each scaled by what
# the counter reads for a plain 256 MiB copy (the summaries with the commands are
# profiles/pmc_bench_qwen35_9b_prefill_T4096_decode_B256.txt and profiles/pmc_prefill_*.txt,
# those of the segment_scan leg in profiles/pmc_prefill_segment_scan_*.txt):
# key -> (call whose sources the figure belongs to, their digest, bytes).  A figure is not
# reported once those sources change.
MEASURED_TRAFFIC = {
    "gdn_chunk_prefill": ("gdn_chunk_prefill", "6d1b9ac6e5ec6db2", 248.6e6),
    "gdn_conv_chunk_prefill": ("gdn_conv_chunk_prefill", "224f272e80008db9", 355.8e6),
    "gdn_recurrent_step": ("gdn_recurrent_step", "d9d1bfb2ad95a136", 1105.8e6),
    "gdn_recurrent_step_bf16_state": ("gdn_recurrent_step_bf16_state", "d9d1bfb2ad95a136", 568.8e6),
    # the chunk call on the prefill_configs workloads
    "gdn_chunk_prefill@l0_qwen3.5-0.8b_T256_fp32": ("gdn_chunk_prefill", "6d1b9ac6e5ec6db2", 24.3e6),
    "gdn_chunk_prefill@l3_qwen3.5-397b_T32768_bf16": ("gdn_chunk_prefill", "6d1b9ac6e5ec6db2", 3461.9e6),
    "gdn_chunk_prefill@l4_qwen3.5-9b_varlen64_bf16": ("gdn_chunk_prefill", "6d1b9ac6e5ec6db2", 3970.7e6),
    # and on the segment_scan workloads
    "gdn_chunk_prefill@qwen3.5-9b_shard8_T32768_bf16": ("gdn_chunk_prefill", "6d1b9ac6e5ec6db2", 335.6e6),
    "gdn_chunk_prefill@qwen3.5-0.8b_T32768_bf16": ("gdn_chunk_prefill", "6d1b9ac6e5ec6db2", 1701.3e6),
}


def source_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    if key not in MEASURED_TRAFFIC:
        return None
    kernel, digest, nbytes = MEASURED_TRAFFIC[key]
    return nbytes if source_digest(kernel) == digest else None


def chunk_core_flops(n_tokens: int, hk: int, hv: int, seqlens=None) -> float:
    """Algorithmic flops of the chunked core (triangles at their triangle, Gram
    products once per key head), summed per chunk with partial chunks at their length:
      per token  Hk (2 C d) + Hv (3 C d + C^2/3 + 6 d^2)."""
    seqlens = seqlens or [n_tokens]
    tot = 0.0
    for L in seqlens:
        full, tail = divmod(L, CHUNK)
        for c, cnt in ((CHUNK, full), (tail, 1 if tail else 0)):
            per_tok = hk * (2 * c * D) + hv * (3 * c * D + c * c / 3.0 + 6 * D * D)
            tot += cnt * c * per_tok
    return tot


def decode_bytes(B: int, hk: int, hv: int, io_bytes: int = 2, state_bytes: int = 4) -> float:
    """Compulsory HBM bytes of one decode step: state read + write (fp32, or bf16 for a
    bf16-stored state), conv state read + write, x, a, b, conv weight, o."""
    cq = 2 * hk * D + hv * D
    state = 2.0 * B * hv * D * D * state_bytes
    conv_state = 2.0 * B * 3 * cq * io_bytes
    x = B * cq * io_bytes
    ab = 2.0 * B * hv * io_bytes
    w = cq * 4 * 4 + 2 * hv * 4
    o = B * hv * D * io_bytes
    return state + conv_state + x + ab + w + o


def _cpu_chain(task):
    """Oracle work for one value head of the prefill layer (runs in a worker process)."""
    import numpy as np
    from oracle import gdn_oracle as G
    x, w, a, b, A_log, dt_bias, z, norm_w, io = task
    y, _ = G.conv1d_fwd(x, w)
    y = G.to_io(y, io)
    q, k, v = y[:, :D], y[:, D:2 * D], y[:, 2 * D:]
    g, beta = G.gates(a[:, None], b[:, None], np.array([A_log]), np.array([dt_bias]))
    o, S = G.delta_rule(G.l2_normalize(q), G.l2_normalize(k), v, g[:, 0], beta[:, 0],
                        np.zeros((D, D)), 1.0 / np.sqrt(D))
    o = G.to_io(o, io)
    return G.to_io(G.gated_rmsnorm(o, z, norm_w), io).shape[0]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def pool_procs(n_tasks: int):
    """Worker processes for the CPU legs: the host cores this process may run on, at most
    16 (the host's CPU share for one GPU); returns (procs, cores in the affinity mask)."""
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    return max(1, min(16, ncpu, n_tasks)), ncpu


def _cpu_decode(task):
    """Oracle decode step for a block of sequences (runs in a worker process)."""
    from oracle import gdn_oracle as G
    x, w, cs, a, b, A_log, dt_bias, st, hk, hv, io = task
    o, _, _ = G.recurrent_step(x, w, cs, a, b, A_log, dt_bias, st, hk, hv, D, D, io=io)
    return o.shape[0]


def _single_threaded_blas():
    keep = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                           "MKL_NUM_THREADS")}
    for k in keep:
        os.environ[k] = "1"
    return keep


def _restore_env(keep):
    for k, v in keep.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


def cpu_baseline_decode(dec, reps=2):
    """Time the fp64 oracle's decode step on the whole decode workload (all sequences, all
    value heads), in a process pool over blocks of sequences, reps times over."""
    import multiprocessing as mp

    B = dec["N"]
    procs, ncpu = pool_procs(B)
    blocks = [list(range(i, B, procs)) for i in range(procs)]
    tasks = [(dec["x"][bl], dec["conv_w"], dec["conv_state_in"][bl], dec["a"][bl], dec["b"][bl],
              dec["A_log"], dec["dt_bias"], dec["state_in"][bl], dec["Hk"], dec["Hv"], dec["io"])
             for bl in blocks]
    keep = _single_threaded_blas()
    try:
        with mp.get_context("spawn").Pool(procs) as pool:
            pool.map(_cpu_decode, [(t[0][:1], t[1], t[2][:1], t[3][:1], t[4][:1], t[5], t[6],
                                    t[7][:1], t[8], t[9], t[10]) for t in tasks])   # warm
            t0 = time.perf_counter()
            done = sum(pool.map(_cpu_decode, tasks * reps, chunksize=1))
            wall = time.perf_counter() - t0
    finally:
        _restore_env(keep)
    assert done == reps * B
    return {"value": reps * B / wall, "unit": "sequence-steps/s", "cores": procs,
            "kind": "oracle", "wall_s": wall, "cpu_model": cpu_model(), "affinity_cores": ncpu,
            "sample": (f"fp64 NumPy oracle decode step of the Qwen3.5-9B layer, all {B} "
                       f"sequences x {dec['Hv']} value heads (conv + recurrence), run {reps} "
                       f"times, {procs} worker processes")}


def cpu_baseline(inp, budget_heads=None, reps=2):
    """Time the fp64 oracle on the prefill layer workload in a process pool over value
    heads (one BLAS thread per worker), the head list run reps times over (about 6 s of
    CPU time per pass on 16 cores).  Returns the cpu_baseline object."""
    import multiprocessing as mp

    import numpy as np
    hk, hv, N = inp["Hk"], inp["Hv"], inp["N"]
    r = hv // hk
    heads = list(range(hv)) if budget_heads is None else list(range(budget_heads))
    tasks = []
    for h in heads:
        kh = h // r
        chans = np.concatenate([np.arange(kh * D, kh * D + D),
                                hk * D + np.arange(kh * D, kh * D + D),
                                2 * hk * D + np.arange(h * D, h * D + D)])
        tasks.append((inp["x"][:, chans], inp["conv_w"][chans], inp["a"][:, h], inp["b"][:, h],
                      float(inp["A_log"][h]), float(inp["dt_bias"][h]),
                      inp["z"][:, h * D:(h + 1) * D], inp["norm_w"], inp["io"]))
    procs, ncpu = pool_procs(len(tasks))
    keep = _single_threaded_blas()
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(procs) as pool:
            pool.map(_cpu_chain, tasks[:procs])          # warm the workers (imports)
            t0 = time.perf_counter()
            pool.map(_cpu_chain, tasks * reps, chunksize=1)
            wall = time.perf_counter() - t0
    finally:
        _restore_env(keep)
    tokens_per_s = reps * N * (len(heads) / hv) / wall
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": procs, "kind": "oracle",
            "wall_s": wall, "cpu_model": cpu_model(), "affinity_cores": ncpu,
            "sample": (f"fp64 NumPy oracle (token-by-token recurrence) of the Qwen3.5-9B prefill "
                       f"layer, T={N}, {len(heads)} of {hv} value heads (conv+core+norm per head) "
                       f"run {reps} times, {procs} worker processes; tokens/s scaled by heads/{hv}")}


def replay_leg(reps: int, warmup: int) -> dict:
    """Beside the step: the prompt -> decode replay on one 9B-shaped layer, B=1: the
    1024-token prompt through the prefill layer, then 256 decode steps (recurrent step +
    gated norm in one launch) on the carried state, eagerly and as one captured HIP graph;
    also the graph of the unfused steps (two launches per token)."""
    import numpy as np
    import torch

    import hybrid_linear_attention_causal_amd as gdn
    from hybrid_linear_attention_causal_amd import synth

    inp = synth.make(synth.replay_workload())
    T, T1, hk, hv = inp["N"], synth.REPLAY_PROMPT, inp["Hk"], inp["Hv"]
    n = T - T1

    def dev(a, f32=False):
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return (t if f32 else t.to(torch.bfloat16)).cuda()

    x, a, b, z = (dev(inp[k]) for k in ("x", "a", "b", "z"))
    z = z.view(T, hv, D)
    w, A_log, dt, nw = (dev(inp[k], True) for k in ("conv_w", "A_log", "dt_bias", "norm_w"))
    bufs = {}
    prefill = lambda: gdn.prefill_layer(x[:T1], w, a[:T1], b[:T1], A_log, dt, z[:T1], nw, hk,
                                        hv, bufs=bufs)
    out = prefill()
    for k in ("y_conv", "o", "y", "conv_state_out", "state_out"):
        bufs[k] = out[k]
    cs, st = out["conv_state_out"], out["state_out"]
    xs = x[T1:].reshape(n, 1, -1).clone()
    As, Bs = a[T1:].reshape(n, 1, hv).clone(), b[T1:].reshape(n, 1, hv).clone()
    zs = z[T1:].reshape(n, 1, hv, D).clone()
    dbufs = {"o": torch.empty((1, hv, D), dtype=torch.bfloat16, device="cuda"),
             "y": torch.empty((1, hv, D), dtype=torch.bfloat16, device="cuda")}

    def decode_eager():
        for t in range(n):
            gdn.decode_step(xs[t], w, cs, As[t], Bs[t], A_log, dt, st, zs[t], nw, hk, hv,
                            bufs=dbufs)

    graph = gdn.DecodeGraph(xs, w, cs, As, Bs, A_log, dt, st, zs, nw, hk, hv)
    graph2 = gdn.DecodeGraph(xs, w, cs, As, Bs, A_log, dt, st, zs, nw, hk, hv, fused=False)

    def timed(fn, k):
        for _ in range(warmup):
            fn()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        e[0].record()
        for _ in range(k):
            fn()
        e[1].record()
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / k

    pre_ms = timed(prefill, reps)
    eager_ms = timed(decode_eager, max(2, reps // 4))
    graph_ms = timed(graph.replay, reps)
    graph2_ms = timed(graph2.replay, reps)
    state_bytes = 2.0 * hv * D * D * 4
    return {"workload": f"Qwen3.5-9B GDN layer, one sequence: {T1}-token prompt then {n} "
                        "decode steps (bf16 io, fp32 state)",
            "prompt_tokens": T1, "decode_steps": n,
            "prefill_layer_ms": pre_ms,
            "decode_eager_us_per_token": eager_ms * 1e3 / n,
            "decode_graph_us_per_token": graph_ms * 1e3 / n,
            "decode_graph_unfused_us_per_token": graph2_ms * 1e3 / n,
            "decode_graph_tokens_per_s": n / (graph_ms * 1e-3),
            "decode_graph_state_GBps": state_bytes * n / (graph_ms * 1e-3) / 1e9}


def segment_scan_leg(reps: int) -> dict:
    """Beside the step: the chunked core where it runs the intra-sequence scan (bf16 io, few
    long chains whose row-split launch would fill at most half the compute units): one
    sequence of 32768 tokens at the 9B layer's share under 8-way head sharding (2 key, 4
    value heads) and at the 0.8B shape (16 and 16).  Timed as in the prefill_configs leg
    (median of `reps` HIP-event timings, each after a 512 MiB overwrite), on device-drawn
    inputs with the recipe's distributions."""
    import math
    import statistics

    import torch

    import hybrid_linear_attention_causal_amd as gdn
    from hybrid_linear_attention_causal_amd.mixer import qkv_views

    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    out = {}
    for name, hk, hv, N in (("qwen3.5-9b_shard8_T32768_bf16", 2, 4, 32768),
                            ("qwen3.5-0.8b_T32768_bf16", 16, 16, 32768)):
        g = torch.Generator(device="cuda").manual_seed(9)
        cq = (2 * hk + hv) * D
        y = torch.randn(N, cq, device="cuda", generator=g).to(torch.bfloat16)
        a = torch.randn(N, hv, device="cuda", generator=g).to(torch.bfloat16)
        b = torch.randn(N, hv, device="cuda", generator=g).to(torch.bfloat16)
        A_log = torch.rand(hv, device="cuda", generator=g) * math.log(16.0)
        dt = torch.log(torch.expm1(1e-3 + 0.099 * torch.rand(hv, device="cuda", generator=g)))
        s_in = 0.02 * torch.randn(1, hv, D, D, device="cuda", generator=g)
        o = torch.empty(N, hv, D, dtype=torch.bfloat16, device="cuda")
        s_out = torch.empty_like(s_in)
        ws = torch.empty(gdn.gdn_chunk_prefill_workspace_size(N, 1, hk, hv, io=torch.bfloat16),
                         dtype=torch.uint8, device="cuda")
        q, k, v = qkv_views(y, hk, hv)

        def call():
            gdn.gdn_chunk_prefill(q, k, v, a, b, A_log, dt, o, hk, hv, None, s_in, s_out,
                                  workspace=ws)

        call()
        ts = []
        for _ in range(reps):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = statistics.median(ts)
        flops = chunk_core_flops(N, hk, hv)
        out[name] = {"Hk": hk, "Hv": hv, "tokens": N, "chunk_prefill_ms": ms,
                     "tokens_per_s": N / (ms * 1e-3),
                     "core_TFLOPs": flops / (ms * 1e-3) / 1e12,
                     "frac_bf16_peak": flops / (ms * 1e-3) / PEAK_BF16_FLOPS,
                     "traffic": measured_traffic(f"gdn_chunk_prefill@{name}")}
        del y, a, b, o, ws, s_in, s_out, q, k, v
        torch.cuda.empty_cache()
    return out


def prefill_configs_leg(reps: int) -> dict:
    """Beside the step: the chunked core (gdn_chunk_prefill) and the prefill layer in one call
    (gdn_prefill_layer), in two (gdn_conv_chunk_prefill -> gdn_gated_rmsnorm) and in three
    (gdn_conv1d_fwd -> gdn_chunk_prefill -> gdn_gated_rmsnorm) on the three other prefill
    workloads: the
    0.8B shape at T=256 with fp32 io, the 397B-A17B shape at T=32768 (one sequence) and the
    9B shape over 64 packed sequences of seeded lengths in [16, 2048] with carried recurrent
    and conv states.  Each call is timed
    with HIP events after a 512 MiB overwrite (inputs of these sizes would otherwise sit in
    the 256 MB last-level cache from the previous call); the median of `reps` is reported.
    The inputs are drawn on the device (torch's seeded Philox generator) with the
    distributions of the recipe: the values steer no kernel's control flow, and NumPy draws
    of these sizes would take longer than the timing."""
    import math
    import statistics

    import numpy as np
    import torch

    import hybrid_linear_attention_causal_amd as gdn
    from hybrid_linear_attention_causal_amd import synth
    from hybrid_linear_attention_causal_amd._lib import (gdn_chunk_prefill, gdn_conv1d_fwd,
                                                         gdn_conv_chunk_prefill,
                                                         gdn_gated_rmsnorm, gdn_prefill_layer)
    from hybrid_linear_attention_causal_amd.mixer import qkv_views

    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    out = {}
    for idx in (0, 3, 4):
        wl = synth.workload(idx)
        sh = wl.shape
        seqlens = (synth.draw_lengths(np.random.default_rng(wl.seed)) if wl.lengths_from_rng
                   else list(wl.seqlens))
        N, Ns, hk, hv, cq = sum(seqlens), len(seqlens), sh.hk, sh.hv, sh.cq
        g = torch.Generator(device="cuda").manual_seed(wl.seed)
        iodt = torch.float32 if wl.io == "f32" else torch.bfloat16
        bf = lambda *shape, s=1.0, o=0.0: (o + s * torch.randn(*shape, device="cuda", generator=g)
                                           ).to(iodt)
        x = bf(N, cq)
        w = 0.25 * torch.randn(cq, 4, device="cuda", generator=g)
        a, b = bf(N, hv), bf(N, hv)
        A_log = torch.rand(hv, device="cuda", generator=g) * math.log(16.0)
        dt = torch.log(torch.expm1(1e-3 + (0.1 - 1e-3) * torch.rand(hv, device="cuda", generator=g)))
        z = bf(N, hv, D)
        nw = 1.0 + 0.1 * torch.randn(D, device="cuda", generator=g)
        cu = s_in = cs_in = None
        if Ns > 1:
            cu = torch.tensor(np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32),
                              device="cuda")
        if wl.init_state:
            s_in = 0.02 * torch.randn(Ns, hv, D, D, device="cuda", generator=g)
            cs_in = bf(Ns, 3, cq)
        y = torch.empty_like(x)
        o = torch.empty(N, hv, D, dtype=iodt, device="cuda")
        yn = torch.empty_like(o)
        s_out = torch.empty(Ns, hv, D, D, device="cuda")
        cs_out = torch.empty(Ns, 3, cq, dtype=iodt, device="cuda")
        ws = torch.empty(gdn.gdn_chunk_prefill_workspace_size(N, Ns, hk, hv, io=iodt),
                         dtype=torch.uint8, device="cuda")
        q, k, v = qkv_views(y, hk, hv)

        def fused():
            gdn_conv_chunk_prefill(x, w, y, a, b, A_log, dt, o, hk, hv, cu, cs_in, cs_out, s_in,
                                   s_out, workspace=ws)

        def chunk():
            gdn_chunk_prefill(q, k, v, a, b, A_log, dt, o, hk, hv, cu, s_in, s_out, workspace=ws)

        def layer():
            gdn_prefill_layer(x, w, y, a, b, A_log, dt, o, z, nw, yn, hk, hv, cu, cs_in, cs_out,
                              s_in, s_out, workspace=ws)

        def norm():
            gdn_gated_rmsnorm(o, z, nw, yn)

        def conv():
            gdn_conv1d_fwd(x, w, y, cu, cs_in, cs_out)

        def med(fn):
            fn()
            ts = []
            for _ in range(reps):
                flush.fill_(1)
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record()
                fn()
                e[1].record()
                torch.cuda.synchronize()
                ts.append(e[0].elapsed_time(e[1]))
            return statistics.median(ts)

        fused_ms, norm_ms, conv_ms, chunk_ms = med(fused), med(norm), med(conv), med(chunk)
        layer_ms = med(layer)
        flops = chunk_core_flops(N, hk, hv, seqlens)
        tf = flops / (chunk_ms * 1e-3) / 1e12
        name = {0: "Qwen3.5-0.8B GDN layer prefill T=256 (B=1), fp32 io",
                3: "Qwen3.5-397B-A17B GDN layer prefill T=32768 (B=1)",
                4: f"Qwen3.5-9B GDN layer prefill, {Ns} sequences, {N} tokens, carried states"}[idx]
        out[wl.name] = {
            "workload": name, "tokens": N, "sequences": Ns, "Hk": hk, "Hv": hv, "io": wl.io,
            "chunk_prefill_ms": chunk_ms, "chunk_prefill_tokens_per_s": N / (chunk_ms * 1e-3),
            "roofline_chunk_prefill": {"kernel": "gdn_chunk_prefill", "bound": "mfma",
                                       "achieved": tf, "peak": PEAK_BF16_FLOPS / 1e12,
                                       "unit": "TFLOP/s", "frac": tf * 1e12 / PEAK_BF16_FLOPS,
                                       "traffic": measured_traffic(f"gdn_chunk_prefill@{wl.name}"),
                                       "algorithmic_per_launch": flops},
            "conv_chunk_prefill_ms": fused_ms, "prefill_norm_ms": norm_ms,
            "prefill_layer_ms": layer_ms,
            "layer_tokens_per_s": N / (layer_ms * 1e-3),
            "layer_two_calls_tokens_per_s": N / ((fused_ms + norm_ms) * 1e-3),
            "conv1d_ms": conv_ms,
            "layer_unfused_tokens_per_s": N / ((conv_ms + chunk_ms + norm_ms) * 1e-3)}
        del x, y, z, o, yn, ws, s_out, cs_out, s_in, cs_in, q, k, v
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="only run one device-to-device copy of MIB MiB and exit: the "
                         "reference kernel that scales PMC byte counters to bytes")
    ap.add_argument("--cpu-heads", type=int, default=None,
                    help="value heads in the CPU-oracle sample (default: all)")
    ap.add_argument("--cpu-reps", type=int, default=2,
                    help="passes over the CPU-oracle sample (default 2)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(the mixer would shard by head groups or sequences with no exchange; "
              "see the design notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calib_copy:
        nbytes = args.calib_copy << 20
        torch.cuda.set_device(0)
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": nbytes}), flush=True)
        return

    import hybrid_linear_attention_causal_amd as gdn
    from hybrid_linear_attention_causal_amd import synth
    from hybrid_linear_attention_causal_amd._lib import (gdn_chunk_prefill, gdn_conv1d_fwd,
                                                         gdn_conv_chunk_prefill,
                                                         gdn_gated_rmsnorm, gdn_recurrent_step)
    from hybrid_linear_attention_causal_amd.mixer import qkv_views

    torch.cuda.set_device(0)
    wl_p, wl_d = synth.workload(1), synth.workload(2)
    pre = synth.make(wl_p)
    dec = synth.make(wl_d)

    def dev(a, f32=False):
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return (t if f32 else t.to(torch.bfloat16)).cuda()

    hk, hv, N = pre["Hk"], pre["Hv"], pre["N"]
    cq = pre["Cq"]
    P = {name: dev(pre[name]) for name in ("x", "a", "b", "z")}
    for name in ("conv_w", "A_log", "dt_bias", "norm_w"):
        P[name] = dev(pre[name], True)
    P["y"] = torch.empty_like(P["x"])
    P["cs_out"] = torch.empty((1, 3, cq), dtype=torch.bfloat16, device="cuda")
    P["o"] = torch.empty((N, hv, D), dtype=torch.bfloat16, device="cuda")
    P["s_out"] = torch.empty((1, hv, D, D), dtype=torch.float32, device="cuda")
    P["yn"] = torch.empty_like(P["o"])
    P["ws"] = torch.empty(gdn.gdn_chunk_prefill_workspace_size(N, 1, hk, hv, io=torch.bfloat16), dtype=torch.uint8,
                          device="cuda")
    q, k, v = qkv_views(P["y"], hk, hv)
    zv = P["z"].view(N, hv, D)

    B = dec["N"]
    Dd = {name: dev(dec[name]) for name in ("x", "a", "b", "z", "conv_state_in")}
    for name in ("conv_w", "A_log", "dt_bias", "norm_w", "state_in"):
        Dd[name] = dev(dec[name], True)
    Dd["o"] = torch.empty((B, hv, D), dtype=torch.bfloat16, device="cuda")
    Dd["yn"] = torch.empty_like(Dd["o"])
    Dd["state_bf16"] = Dd["state_in"].to(torch.bfloat16)
    zd = Dd["z"].view(B, hv, D)
    torch.cuda.synchronize()

    def decode(ev, i):
        gdn_recurrent_step(Dd["x"], Dd["conv_w"], Dd["conv_state_in"], Dd["a"], Dd["b"],
                           Dd["A_log"], Dd["dt_bias"], Dd["state_in"], Dd["o"], hk, hv)
        if ev:
            ev[i].record()
        gdn_gated_rmsnorm(Dd["o"], zd, Dd["norm_w"], Dd["yn"])
        if ev:
            ev[i + 1].record()

    def step(ev=None):
        # prefill layer: conv + chunked core in one call, then the gated norm; then decode
        if ev:
            ev[0].record()
        gdn_conv_chunk_prefill(P["x"], P["conv_w"], P["y"], P["a"], P["b"], P["A_log"],
                               P["dt_bias"], P["o"], hk, hv, None, None, P["cs_out"], None,
                               P["s_out"], workspace=P["ws"])
        if ev:
            ev[1].record()
        gdn_gated_rmsnorm(P["o"], zv, P["norm_w"], P["yn"])
        if ev:
            ev[2].record()
        decode(ev, 3)

    def step_unfused(ev=None):
        # the same step with the conv and the chunked core as two calls
        if ev:
            ev[0].record()
        gdn_conv1d_fwd(P["x"], P["conv_w"], P["y"], None, None, P["cs_out"])
        if ev:
            ev[1].record()
        gdn_chunk_prefill(q, k, v, P["a"], P["b"], P["A_log"], P["dt_bias"], P["o"], hk, hv,
                          None, None, P["s_out"], workspace=P["ws"])
        if ev:
            ev[2].record()
        gdn_gated_rmsnorm(P["o"], zv, P["norm_w"], P["yn"])
        if ev:
            ev[3].record()
        decode(ev, 4)

    # Before each step's prefill a 512 MiB overwrite evicts the 256 MB last-level cache,
    # outside the kernel events (the 67 MB x and the workspace records would otherwise be
    # read from it on the next step); the wall clock of the K steps includes it.
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        flush.fill_(1)
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush.fill_(1)
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ["conv_chunk_prefill", "prefill_norm", "recurrent_step", "decode_norm"]
    ms = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(names)}

    # Beside the step: the same step with the conv and the chunked core as two calls.
    for _ in range(args.warmup):
        flush.fill_(1)
        step_unfused()
    evu = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for i in range(args.steps):
        flush.fill_(1)
        step_unfused(evu[i])
    torch.cuda.synchronize()
    names_u = ["conv1d", "chunk_prefill", "prefill_norm", "recurrent_step", "decode_norm"]
    ms_u = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evu]))
            for j, n in enumerate(names_u)}

    # Beside the step: the same decode step on a bf16-stored recurrent state.
    def step_bf16_state():
        gdn_recurrent_step(Dd["x"], Dd["conv_w"], Dd["conv_state_in"], Dd["a"], Dd["b"],
                           Dd["A_log"], Dd["dt_bias"], Dd["state_bf16"], Dd["o"], hk, hv)

    for _ in range(args.warmup):
        step_bf16_state()
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    for i in range(args.steps):
        ev_b[2 * i].record()
        step_bf16_state()
        ev_b[2 * i + 1].record()
    torch.cuda.synchronize()
    ms_bf16_state = float(np.mean([ev_b[2 * i].elapsed_time(ev_b[2 * i + 1])
                                   for i in range(args.steps)]))
    replay = replay_leg(args.steps, args.warmup)
    configs = prefill_configs_leg(args.steps)
    segscan = segment_scan_leg(args.steps)
    prefill_ms = ms["conv_chunk_prefill"] + ms["prefill_norm"]
    tokens_per_s = N / (prefill_ms * 1e-3)
    prefill_u_ms = ms_u["conv1d"] + ms_u["chunk_prefill"] + ms_u["prefill_norm"]

    # the chunked core's algorithmic flops (the conv adds 8 flops per channel and token,
    # under 2% of them, and is not counted)
    flops = chunk_core_flops(N, hk, hv)
    chunk_tflops = flops / (ms["conv_chunk_prefill"] * 1e-3) / 1e12
    chunk_only_tflops = flops / (ms_u["chunk_prefill"] * 1e-3) / 1e12
    dbytes = decode_bytes(B, hk, hv)
    step_gbs = dbytes / (ms["recurrent_step"] * 1e-3) / 1e9
    dbytes_bf = decode_bytes(B, hk, hv, state_bytes=2)

    res = {
        "metric": "GDN layer prefill tokens/s (%MFMA peak) + decode step state GB/s (%HBM peak)",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Qwen3.5-9B linear-attention layer shapes, random parameters)",
        "config": {"workload": "Qwen3.5-9B GDN layer prefill T=4096 (B=1) + decode step B=256",
                   "prefill_tokens": N, "decode_batch": B, "Hk": hk, "Hv": hv, "d": D,
                   "conv_channels": cq, "chunk": CHUNK, "io": "bf16", "state": "fp32"},
        "kernel_ms": ms,
        "roofline": {"kernel": "gdn_conv_chunk_prefill", "bound": "mfma",
                     "achieved": chunk_tflops, "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": chunk_tflops * 1e12 / PEAK_BF16_FLOPS,
                     "traffic": measured_traffic("gdn_conv_chunk_prefill"),
                     "algorithmic_per_launch": flops},
        "prefill_unfused": {
            "calls": "gdn_conv1d_fwd -> gdn_chunk_prefill -> gdn_gated_rmsnorm",
            "kernel_ms": {n: ms_u[n] for n in ("conv1d", "chunk_prefill", "prefill_norm")},
            "tokens_per_s": N / (prefill_u_ms * 1e-3),
            "roofline_chunk_prefill": {
                "kernel": "gdn_chunk_prefill", "bound": "mfma", "achieved": chunk_only_tflops,
                "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                "frac": chunk_only_tflops * 1e12 / PEAK_BF16_FLOPS,
                "traffic": measured_traffic("gdn_chunk_prefill"),
                "algorithmic_per_launch": flops}},
        "roofline_decode": {"kernel": "gdn_recurrent_step", "bound": "hbm", "achieved": step_gbs,
                            "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                            "frac": step_gbs * 1e9 / PEAK_HBM_BYTES,
                            "traffic": measured_traffic("gdn_recurrent_step"),
                            "algorithmic_per_launch": dbytes},
        "roofline_decode_bf16_state": {
            "kernel": "gdn_recurrent_step_bf16_state", "bound": "hbm", "ms": ms_bf16_state,
            "achieved": dbytes_bf / (ms_bf16_state * 1e-3) / 1e9, "peak": PEAK_HBM_BYTES / 1e9,
            "unit": "GB/s", "frac": dbytes_bf / (ms_bf16_state * 1e-3) / PEAK_HBM_BYTES,
            "traffic": measured_traffic("gdn_recurrent_step_bf16_state"),
            "algorithmic_per_launch": dbytes_bf},
        "replay": replay,
        "prefill_configs": configs,
        "segment_scan": segscan,
        "cpu_baseline": None,
        "cpu_baseline_decode": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(pre, args.cpu_heads, args.cpu_reps)
        res["cpu_baseline_decode"] = cpu_baseline_decode(dec, args.cpu_reps)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
