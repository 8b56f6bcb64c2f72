"""Whole-tensor parity at full workload sizes: the fp64 oracle over every (sequence,
value head) chain of a prefill layer, in a pool of worker processes, each chain compared
with the GPU's result as soon as it is computed.

Test infrastructure only (it runs the oracle).  The workers import NumPy, the oracle and
the error measures of `parity`, never torch or the HIP library.  Every chain carries its
own inputs and the GPU's outputs for it; a worker returns only error measures, which the
caller combines into the whole-tensor checks of `parity` (the bf16 bound uses the RMS of
the whole reference tensor, so the sums of squares travel with the maxima).

bf16 tensors travel as their upper 16 bits (uint16), which halves what is pickled.
"""
from __future__ import annotations

import os

import numpy as np

D = 128
MAX_PROCS = 16   # the GPU machine's CPU share for one GPU


def pack(a, io):
    """A float32 array of io-dtype values, ready to send (bf16: the upper 16 bits)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16) if io == "bf16" else a


def unpack(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def chain_task(task):
    """Oracle of one (sequence, value head) chain of the prefill layer and its error
    measures against the GPU's outputs for the same chain, two ways:

    * per call: each call's output against the oracle's evaluation of that call on the
      GPU's own inputs to it -- the conv on x, the delta-rule core on the GPU's conv
      output, the gated norm on the GPU's core output -- each compared before the
      oracle's rounding, with the slack of the GPU's own bf16 store (parity: s = 2^-8);
    * through the layer: the oracle's whole pipeline from x, rounding at each call
      boundary, against the GPU's o and norm output; there each bf16 call output upstream
      can sit one ulp from the GPU's (parity: s = 2^-8 (1 + 2 upstream)).
    """
    from oracle import gdn_oracle as G
    from parity import excess_stats

    io = task["io"]
    scale = 1.0 / np.sqrt(D)
    x = unpack(task["x"])
    cs_in = None if task["cs_in"] is None else unpack(task["cs_in"])[None]
    y_exact, cs_out = G.conv1d_fwd(x, task["conv_w"], None, cs_in)
    g, beta = G.gates(task["a"][:, None], task["b"][:, None], np.array([task["A_log"]]),
                      np.array([task["dt_bias"]]))
    S0 = np.zeros((D, D)) if task["S0"] is None else task["S0"]
    z = unpack(task["z"])

    def core(y):
        return G.delta_rule(G.l2_normalize(y[:, :D]), G.l2_normalize(y[:, D:2 * D]),
                            y[:, 2 * D:], g[:, 0], beta[:, 0], S0, scale)

    gpu_yc = unpack(task["gpu_yc"])
    gpu_o = unpack(task["gpu_o"])
    gpu_y = unpack(task["gpu_y"])
    # per call: the core on the GPU's conv output, the norm on the GPU's core output
    o_call, S_call = core(gpu_yc)
    yn_call = G.gated_rmsnorm(gpu_o, z, task["norm_w"])
    # through the layer: the oracle's own pipeline, rounded at each call boundary
    o_layer, S_layer = core(G.to_io(y_exact, io))
    yn_layer = G.gated_rmsnorm(G.to_io(o_layer, io), z, task["norm_w"])
    # the q and k channels are shared by the r value heads of a key head: the first of
    # them carries their conv check
    yc_cols = slice(0, 3 * D) if task["check_qk"] else slice(2 * D, 3 * D)
    gS = task["gpu_S"].astype(np.float64)
    return {
        "s": task["s"], "h": task["h"],
        "yc": excess_stats(gpu_yc[:, yc_cols], y_exact[:, yc_cols], io, 0),
        "o": excess_stats(gpu_o, o_call, io, 0),
        "o_diag": _diag(gpu_o, o_call),
        "y": excess_stats(gpu_y, yn_call, io, 0),
        "o_layer": excess_stats(gpu_o, o_layer, io, 1),
        "y_layer": excess_stats(gpu_y, yn_layer, io, 2),
        "dS2": float(np.sum((gS - S_call) ** 2)), "S2": float(np.sum(S_call ** 2)),
        "dS2_layer": float(np.sum((gS - S_layer) ** 2)), "S2_layer": float(np.sum(S_layer ** 2)),
        "S_finite": bool(np.all(np.isfinite(task["gpu_S"]))),
        "cs_equal": bool(np.array_equal(unpack(task["gpu_cs"]), cs_out[0])),
    }


def _diag(gpu, ref):
    """Where a chain's output is worst: (largest |delta|, |ref| there, the chain's RMS,
    token of it)."""
    d = np.abs(gpu - ref)
    if d.size == 0:
        return (0.0, 0.0, 0.0, -1)
    i = int(np.argmax(d))
    t = i // ref.shape[-1]
    return (float(d.flat[i]), float(abs(ref.flat[i])), float(np.sqrt(np.mean(ref * ref))), t)


def procs_for(n_tasks):
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    return max(1, min(MAX_PROCS, ncpu, n_tasks))


def run(tasks, n_tasks):
    """Map chain_task over an iterable of tasks in a spawn pool (one BLAS thread per
    worker); yields the results in completion order."""
    import multiprocessing as mp

    keep = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                           "MKL_NUM_THREADS")}
    for k in keep:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(procs_for(n_tasks)) as pool:
            for res in pool.imap_unordered(chain_task, tasks, chunksize=1):
                yield res
    finally:
        for k, v in keep.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


class Combined:
    """Whole-tensor checks from the per-chain measures."""

    def __init__(self, io, ns):
        self.io = io
        self.parts = {k: [0.0, 0.0, 0] for k in ("yc", "o", "y", "o_layer", "y_layer")}
        self.dS2 = {k: np.zeros(ns) for k in ("", "_layer")}
        self.S2 = {k: np.zeros(ns) for k in ("", "_layer")}
        self.chains = 0
        self.bad = []
        self.worst = []     # (o excess, sequence, head, diagnostics) of the worst chains

    def add(self, res):
        self.chains += 1
        for key, (ex, ss, n) in ((k, res[k]) for k in self.parts):
            p = self.parts[key]
            p[0] = max(p[0], ex)
            p[1] += ss
            p[2] += n
        self.worst.append((res["o"][0], res["s"], res["h"], res.get("o_diag")))
        self.worst = sorted(self.worst, key=lambda w: -w[0])[:6]
        for k in self.dS2:
            self.dS2[k][res["s"]] += res["dS2" + k]
            self.S2[k][res["s"]] += res["S2" + k]
        if not res["S_finite"]:
            self.bad.append(f"non-finite final state at sequence {res['s']} head {res['h']}")
        if not res["cs_equal"]:
            self.bad.append(f"conv state differs at sequence {res['s']} head {res['h']}")

    def summary(self):
        return "worst o chains, per call (excess, seq, head, (|d|, |ref| there, chain rms, token)): " + \
            "; ".join(f"{e:.2e} s{s} h{h} {d}" for e, s, h, d in self.worst)

    def check(self, what, report_only=()):
        """Assert every measure against its bound, except the keys in report_only, which
        are printed only."""
        from parity import STATE_REL_TOL, bound_of
        print(f"{what}: {self.summary()}", flush=True)
        assert not self.bad, f"{what}: " + "; ".join(self.bad[:5])
        report = {}
        for key, (ex, ss, n) in self.parts.items():
            report[key] = (ex, bound_of(self.io, ss, n))
        print(f"{what}: " + ", ".join(f"{k} {e:.2e}/{b:.2e}" for k, (e, b) in report.items()),
              flush=True)
        for key, (ex, bound) in report.items():
            if key not in report_only:
                assert ex <= bound, f"{what} {key}: error {ex:.3e} > bound {bound:.3e} ({self.io})"
        for k in self.dS2:
            rel = np.sqrt(self.dS2[k]) / np.where(self.S2[k] > 0, np.sqrt(self.S2[k]), 1.0)
            worst = float(rel.max(initial=0.0))
            report["state" + k] = (worst, STATE_REL_TOL)
            assert worst <= STATE_REL_TOL, f"{what}: state{k} rel err {worst:.3e} > {STATE_REL_TOL}"
        return report
