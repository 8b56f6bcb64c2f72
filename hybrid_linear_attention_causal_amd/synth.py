"""Seeded synthetic inputs for the Gated DeltaNet token mixer.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic. Both the HIP path (through the Python binding) and the
CPU oracle are fed from the arrays produced here, so the two see identical
inputs.

Shapes follow the linear-attention layers of three Qwen3.5 family members
(all with key/value head width 128 and a width-4 causal conv):

* 0.8B  -- 16 key heads, 16 value heads, 6144 conv channels
  (Qwen3.5 KerasFormers page, "API", Qwen3_5Model defaults table).
* 9B    -- 16 key heads, 32 value heads, 8192 conv channels
  (llm-arch-viz Qwen3.5-9B page, module tree of Qwen3_5GatedDeltaNet;
  16 key heads follows from 8192 = 2*16*128 + 32*128).
* 397B-A17B -- 16 key heads, 64 value heads, 12288 conv channels
  (llm-architectures-explained Qwen3.5 397B-A17B page,
  "Every architecture field" table, mixers.linear.*).

Recipe (all draws fp64 from ``numpy.random.default_rng(seed)`` (PCG64), in the
order listed, then cast fp64 -> fp32, and for bf16 inputs fp32 -> bf16 with
round-to-nearest-even):

* varlen lengths (workload 4 only) ~ uniform integers in [16, 2048]
* mixed_qkv ~ N(0, 1)
* conv weight ~ 0.25 * N(0, 1)                          (fp32 parameter)
* a ~ N(0, 1), b ~ N(0, 1)
* A_log ~ U(0, ln 16)                                   (fp32 parameter)
* dt_bias = log(expm1(U(1e-3, 0.1)))  (inverse softplus) (fp32 parameter)
* z ~ N(0, 1)
* norm weight = 1 + 0.1 * N(0, 1)                       (fp32 parameter)
* initial recurrent state ~ 0.02 * N(0, 1)              (fp32, when present)
* initial conv state ~ N(0, 1)                          (io dtype, when present)

bf16 tensors are returned as float32 numpy arrays whose values are exactly
representable in bf16, together with the dtype tag ``io`` ("f32" or "bf16").
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

D_HEAD = 128
CONV_K = 4
RMS_EPS = 1e-6


@dataclasses.dataclass
class Shape:
    name: str
    hk: int
    hv: int
    dk: int = D_HEAD
    dv: int = D_HEAD

    @property
    def cq(self) -> int:
        return 2 * self.hk * self.dk + self.hv * self.dv


QWEN35_08B = Shape("qwen3.5-0.8b", hk=16, hv=16)
QWEN35_9B = Shape("qwen3.5-9b", hk=16, hv=32)
QWEN35_397B = Shape("qwen3.5-397b-a17b", hk=16, hv=64)


@dataclasses.dataclass
class Workload:
    """One seeded workload: packed prefill (kind='prefill') or decode (kind='decode')."""
    name: str
    kind: str
    shape: Shape
    io: str
    seed: int
    seqlens: Optional[list] = None    # prefill: per-sequence token counts
    batch: int = 0                    # decode: number of sequences
    init_state: bool = False          # nonzero initial recurrent + conv state
    lengths_from_rng: bool = False    # varlen lengths drawn first from the rng

    @property
    def n_tokens(self) -> int:
        return int(sum(self.seqlens)) if self.kind == "prefill" else self.batch


def workload(idx: int) -> Workload:
    """The five standard workloads (0: 0.8B fp32 layer, 1: 9B prefill, 2: 9B decode,
    3: 397B long prefill, 4: 9B varlen prefill with carried state)."""
    if idx == 0:
        return Workload("l0_qwen3.5-0.8b_T256_fp32", "prefill", QWEN35_08B, "f32", 0, [256])
    if idx == 1:
        return Workload("l1_qwen3.5-9b_T4096_bf16", "prefill", QWEN35_9B, "bf16", 1, [4096])
    if idx == 2:
        return Workload("l2_qwen3.5-9b_decode_B256_bf16", "decode", QWEN35_9B, "bf16", 2,
                        batch=256, init_state=True)
    if idx == 3:
        return Workload("l3_qwen3.5-397b_T32768_bf16", "prefill", QWEN35_397B, "bf16", 3,
                        [32768])
    if idx == 4:
        return Workload("l4_qwen3.5-9b_varlen64_bf16", "prefill", QWEN35_9B, "bf16", 4,
                        None, init_state=True, lengths_from_rng=True)
    raise ValueError(f"no workload {idx}")


# the prompt -> decode replay: one sequence, a 1024-token prompt then 256 decode tokens
# (HF transformers docs, Qwen3.5 page, "Usage tips and notes": its one measured generation
# has a 1024-token prompt and 256 greedily decoded tokens; that measurement is of a whole
# 27B model, here it is one linear-attention layer of the 9B shape)
REPLAY_PROMPT, REPLAY_STEPS = 1024, 256


def replay_workload(shape: Shape = QWEN35_9B, prompt: int = REPLAY_PROMPT,
                    steps: int = REPLAY_STEPS, seed: int = 5) -> Workload:
    """All prompt + steps tokens of the replay as one sequence; the first `prompt` go to
    the chunked prefill and the rest to decode steps on the carried state."""
    return Workload(f"replay_{shape.name}_p{prompt}_d{steps}_bf16", "prefill", shape, "bf16",
                    seed, [prompt + steps])


def custom(shape: Shape, io: str, seed: int, seqlens=None, batch: int = 0,
           init_state: bool = False, kind: str = "prefill") -> Workload:
    return Workload(f"custom_{shape.name}_{io}_s{seed}", kind, shape, io, seed,
                    list(seqlens) if seqlens is not None else None, batch, init_state)


def round_io(x32: np.ndarray, io: str) -> np.ndarray:
    """Cast an fp32 array to the io dtype (values kept in a float32 container)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if io == "f32":
        return x32
    if io != "bf16":
        raise ValueError(io)
    import torch  # torch's fp32 -> bf16 cast rounds to nearest even
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy()


def draw_lengths(rng) -> list:
    """The varlen workload's 64 sequence lengths, uniform integers in [16, 2048] (the
    first draw of its generator)."""
    return [int(v) for v in rng.integers(16, 2049, size=64)]


def _normal(rng, shape, scale=1.0, offset=0.0):
    return (offset + scale * rng.standard_normal(shape)).astype(np.float32)


def make(wl: Workload) -> dict:
    """Draw every input of the workload.  Returns a dict of numpy arrays plus metadata."""
    sh = wl.shape
    rng = np.random.default_rng(wl.seed)
    seqlens = wl.seqlens
    if wl.lengths_from_rng:
        seqlens = draw_lengths(rng)
        wl.seqlens = seqlens
    if wl.kind == "prefill":
        ns = len(seqlens)
        n = int(sum(seqlens))
        cu = np.zeros(ns + 1, dtype=np.int32)
        cu[1:] = np.cumsum(np.asarray(seqlens, dtype=np.int64))
    else:
        ns = n = wl.batch
        cu = None
    out = {"workload": wl, "io": wl.io, "Ns": ns, "N": n, "cu_seqlens": cu,
           "Hk": sh.hk, "Hv": sh.hv, "dk": sh.dk, "dv": sh.dv, "Cq": sh.cq, "K": CONV_K}
    out["x"] = round_io(_normal(rng, (n, sh.cq)), wl.io)
    out["conv_w"] = _normal(rng, (sh.cq, CONV_K), 0.25)
    out["a"] = round_io(_normal(rng, (n, sh.hv)), wl.io)
    out["b"] = round_io(_normal(rng, (n, sh.hv)), wl.io)
    out["A_log"] = rng.uniform(0.0, math.log(16.0), size=sh.hv).astype(np.float32)
    dt = rng.uniform(1e-3, 0.1, size=sh.hv)
    out["dt_bias"] = np.log(np.expm1(dt)).astype(np.float32)
    out["z"] = round_io(_normal(rng, (n, sh.hv * sh.dv)), wl.io)
    out["norm_w"] = _normal(rng, (sh.dv,), 0.1, 1.0)
    if wl.init_state:
        out["state_in"] = _normal(rng, (ns, sh.hv, sh.dk, sh.dv), 0.02)
        out["conv_state_in"] = round_io(_normal(rng, (ns, CONV_K - 1, sh.cq)), wl.io)
    else:
        out["state_in"] = None
        out["conv_state_in"] = None
    return out

