"""Gated DeltaNet token mixer -- plain fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg
do.  It shares no code with the HIP library.

What it computes (the linear-attention layer that fills three of every four
Qwen3.5 decoder blocks -- HF transformers Qwen3.5 docs page, introduction;
"conv1d + delta rule", KerasFormers Qwen page, "Architecture notes" table):

1. causal depthwise conv1d of width 4 over the packed q|k|v channels, no bias
   (llm-arch-viz Qwen3.5-9B page, module tree: conv1d 8192x1x4), then SiLU;
   conv state = the last 3 raw input rows of each sequence
   (KerasFormers Qwen page, "Generation": per-layer conv state);
2. split into q, k, v; L2-normalise q and k per head; value head h reads
   key/query head h // (Hv / Hk);
3. gates g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b), per token
   and value head (a and b have one column per value head and the module owns
   two length-Hv vectors: llm-arch-viz Qwen3.5-9B page, module tree);
4. the gated delta rule on an fp32 (here fp64) state S of shape dk x dv:
       S_t = exp(g_t) S_{t-1} + beta_t k_t (v_t - (exp(g_t) S_{t-1})^T k_t)^T
       o_t = S_t^T q_t / sqrt(dk)
   run token by token; states carried across calls
   (KerasFormers Qwen page, "Generation": delta-rule recurrent state);
5. z-gated RMSNorm over each value head's dv outputs with a shared [dv]
   weight (llm-arch-viz Qwen3.5-9B page: norm Qwen3_5RMSNormGated, 128) and
   eps 1e-6 (KerasFormers Qwen3.5 page, "API" table, norm_eps).

Readings taken where the pages are silent (each is listed in the design notes):
conv tap w[c, 3] multiplies the current token; conv state holds raw pre-conv
rows oldest first; qkv channels are q | k | v, head-major; value head h uses
key head h // r; L2 norm is x / sqrt(sum x^2 + 1e-6); the norm weight is applied
directly (not 1 + w) and the gate is silu(z) applied after normalisation;
rounding to the io dtype happens only at call boundaries (round-to-nearest-even
fp64 -> fp32 -> bf16).
"""
from __future__ import annotations

import numpy as np

L2_EPS = 1e-6
RMS_EPS = 1e-6


# --------------------------------------------------------------------------
# dtype handling at call boundaries
# --------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round to bf16 (round-to-nearest-even) via fp32; returned as float64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def to_io(x, io: str) -> np.ndarray:
    """Round an fp64 result to the io dtype at a call boundary."""
    if io == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if io == "bf16":
        return bf16_round(x)
    raise ValueError(io)


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


# --------------------------------------------------------------------------
# step 1: causal depthwise conv1d + SiLU, with conv state
# --------------------------------------------------------------------------
def _seq_bounds(n_tokens, cu_seqlens):
    if cu_seqlens is None:
        return [(0, int(n_tokens))]
    cu = [int(c) for c in cu_seqlens]
    return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def conv1d_fwd(x, w, cu_seqlens=None, conv_state_in=None):
    """y[t, c] = silu(sum_j w[c, j] * xpad[t + j, c]) per sequence.

    x: [N, C]; w: [C, K]; conv_state_in: [Ns, K-1, C] (oldest row first) or None
    for zeros.  Returns (y [N, C], conv_state_out [Ns, K-1, C]), fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    n, c = x.shape
    kw = w.shape[1]
    bounds = _seq_bounds(n, cu_seqlens)
    y = np.zeros((n, c))
    state_out = np.zeros((len(bounds), kw - 1, c))
    for s, (b0, b1) in enumerate(bounds):
        if conv_state_in is None:
            hist = np.zeros((kw - 1, c))
        else:
            hist = np.asarray(conv_state_in[s], dtype=np.float64)
        xpad = np.concatenate([hist, x[b0:b1]], axis=0)      # [(K-1) + L, C]
        length = b1 - b0
        acc = np.zeros((length, c))
        for j in range(kw):
            acc += w[:, j][None, :] * xpad[j: j + length]
        y[b0:b1] = silu(acc)
        state_out[s] = xpad[xpad.shape[0] - (kw - 1):]
    return y, state_out


# --------------------------------------------------------------------------
# steps 2 and 3: L2 norm, head mapping, gates
# --------------------------------------------------------------------------
def l2_normalize(x, eps=L2_EPS):
    """x / sqrt(sum(x^2) + eps) along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def softplus(x):
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def gates(a, b, A_log, dt_bias):
    """g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b); arrays [N, Hv]."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    g = -np.exp(A_log)[None, :] * softplus(a + dt_bias[None, :])
    beta = sigmoid(b)
    return g, beta


def head_slice(x, h, d):
    return np.asarray(x[:, h * d:(h + 1) * d], dtype=np.float64)


# --------------------------------------------------------------------------
# step 4: the gated delta rule, token by token
# --------------------------------------------------------------------------
def delta_rule(q, k, v, g, beta, S0, scale):
    """One (sequence, value-head) chain.

    q, k: [L, dk] (already normalised if the caller wants that); v: [L, dv];
    g, beta: [L]; S0: [dk, dv].  Returns (o [L, dv], S_L [dk, dv]).
    """
    S = np.array(S0, dtype=np.float64, copy=True)
    L = q.shape[0]
    o = np.zeros((L, v.shape[1]))
    for t in range(L):
        S = np.exp(g[t]) * S                     # decayed state
        u = beta[t] * (v[t] - S.T @ k[t])        # delta-rule correction
        S = S + np.outer(k[t], u)
        o[t] = scale * (S.T @ q[t])
    return o, S


def prefill(q, k, v, a, b, A_log, dt_bias, Hk, Hv, dk, dv, state_in=None,
            cu_seqlens=None, scale=None, use_qk_l2norm=True, g=None, beta=None,
            pairs=None):
    """The delta-rule core over packed sequences.

    q, k: [N, Hk*dk]; v: [N, Hv*dv]; a, b: [N, Hv]; state_in: [Ns, Hv, dk, dv]
    or None (zeros).  g / beta: optional [N, Hv] arrays that replace the gate
    formula.  pairs: optional list of (sequence, value head) chains to compute
    (others are left as NaN) -- every chosen chain runs its full length.
    Returns (o [N, Hv, dv], state_out [Ns, Hv, dk, dv]), fp64.
    """
    n = q.shape[0]
    bounds = _seq_bounds(n, cu_seqlens)
    ns = len(bounds)
    r = Hv // Hk
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(dk)
    if g is None or beta is None:
        g_f, beta_f = gates(a, b, A_log, dt_bias)
        g = g_f if g is None else np.asarray(g, dtype=np.float64)
        beta = beta_f if beta is None else np.asarray(beta, dtype=np.float64)
    else:
        g = np.asarray(g, dtype=np.float64)
        beta = np.asarray(beta, dtype=np.float64)
    o = np.full((n, Hv, dv), np.nan)
    state_out = np.full((ns, Hv, dk, dv), np.nan)
    if pairs is None:
        pairs = [(s, h) for s in range(ns) for h in range(Hv)]
    for s, h in pairs:
        b0, b1 = bounds[s]
        kh = h // r
        qh = head_slice(q[b0:b1], kh, dk)
        kk = head_slice(k[b0:b1], kh, dk)
        if use_qk_l2norm:
            qh = l2_normalize(qh)
            kk = l2_normalize(kk)
        vh = head_slice(v[b0:b1], h, dv)
        S0 = np.zeros((dk, dv)) if state_in is None else state_in[s, h]
        oh, S = delta_rule(qh, kk, vh, g[b0:b1, h], beta[b0:b1, h], S0, scale)
        o[b0:b1, h] = oh
        state_out[s, h] = S
    return o, state_out


# --------------------------------------------------------------------------
# step 5: z-gated RMSNorm
# --------------------------------------------------------------------------
def gated_rmsnorm(o, z, w, eps=RMS_EPS):
    """y = w * o / sqrt(mean(o^2) + eps) * silu(z), over the last axis of size dv.

    o, z: [..., dv] (z reshaped by the caller to match); w: [dv].
    """
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    inv_rms = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return w * (o * inv_rms) * silu(z)


# --------------------------------------------------------------------------
# decode: one token per sequence on carried conv and recurrent state
# --------------------------------------------------------------------------
def recurrent_step(x, conv_w, conv_state, a, b, A_log, dt_bias, state, Hk, Hv, dk, dv,
                   scale=None, use_qk_l2norm=True, g=None, beta=None, io="bf16",
                   pairs=None, state_io="f64"):
    """x: [B, Cq]; conv_state: [B, K-1, Cq]; state: [B, Hv, dk, dv].

    Returns (o [B, Hv, dv] fp64, conv_state_new [B, K-1, Cq], state_new).  The
    conv output is rounded to io before the core, as at the prefill boundary.
    state_io="bf16" is the bf16-stored state (llm-architectures-explained, Qwen3.5
    397B-A17B page, "Modelled costs": the state kept in BF16): the step runs on the
    stored values and only the state written back is rounded to bf16; o comes from the
    updated state before that rounding.
    """
    bsz = x.shape[0]
    cu = np.arange(bsz + 1)
    y, conv_state_new = conv1d_fwd(x, conv_w, cu, conv_state)
    y = to_io(y, io)
    q = y[:, : Hk * dk]
    k = y[:, Hk * dk: 2 * Hk * dk]
    v = y[:, 2 * Hk * dk:]
    if pairs is None:
        pairs = [(s, h) for s in range(bsz) for h in range(Hv)]
    o, state_new = prefill(q, k, v, a, b, A_log, dt_bias, Hk, Hv, dk, dv, state, cu, scale,
                           use_qk_l2norm, g, beta, pairs=pairs)
    if state_io == "bf16":
        state_new = to_io(state_new, "bf16")
    return o, conv_state_new, state_new


def recurrent_step_slots(x, conv_w, conv_pool, a, b, A_log, dt_bias, state_pool, slots, Hk, Hv,
                         dk, dv, io="bf16", state_io="f64", **kw):
    """The step for a batch whose states are entries of pools (KerasFormers Qwen page,
    "Generation": each sequence carries its own conv and recurrent state; here they
    are picked from a pool by index).  Row i uses entry slots[i]; a negative or
    out-of-range slot is a padding row: its o is zero and no entry changes.

    Returns (o [B, Hv, dv], conv_pool_new, state_pool_new) as new arrays.
    """
    slots = np.asarray(slots)
    n = state_pool.shape[0]
    live = [i for i, s in enumerate(slots) if 0 <= s < n]
    o = np.zeros((x.shape[0], Hv, dv))
    conv_new = np.array(conv_pool, dtype=np.float64, copy=True)
    state_new = np.array(state_pool, dtype=np.float64, copy=True)
    if live:
        idx = slots[live]
        assert len(set(idx.tolist())) == len(idx), "two rows share a slot"
        g = None if kw.get("g") is None else kw.pop("g")[live]
        beta = None if kw.get("beta") is None else kw.pop("beta")[live]
        o_l, cs_l, st_l = recurrent_step(x[live], conv_w, conv_pool[idx], a[live], b[live], A_log,
                                         dt_bias, state_pool[idx], Hk, Hv, dk, dv, io=io,
                                         state_io=state_io, g=g, beta=beta, **kw)
        o[live] = o_l
        conv_new[idx] = cs_l
        state_new[idx] = st_l
    return o, conv_new, state_new


# --------------------------------------------------------------------------
# the whole mixer, rounding to io at each call boundary
# --------------------------------------------------------------------------
def layer(inp, pairs=None):
    """Run conv -> core -> gated norm on a dict of inputs (see the input generator).

    Returns dict with y_conv, conv_state_out, o, state_out, y (all fp64 holding
    io-rounded values where they cross a call boundary), and y_conv_exact, o_exact,
    y_exact: the same three call outputs before their own rounding (each computed from
    the rounded outputs of the calls before it, as the next call receives them).
    """
    io = inp["io"]
    Hk, Hv, dk, dv = inp["Hk"], inp["Hv"], inp["dk"], inp["dv"]
    y_exact, cs_out = conv1d_fwd(inp["x"], inp["conv_w"], inp["cu_seqlens"], inp["conv_state_in"])
    y = to_io(y_exact, io)
    q = y[:, : Hk * dk]
    k = y[:, Hk * dk: 2 * Hk * dk]
    v = y[:, 2 * Hk * dk:]
    o_exact, s_out = prefill(q, k, v, inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], Hk, Hv,
                             dk, dv, inp["state_in"], inp["cu_seqlens"], pairs=pairs)
    o = to_io(o_exact, io)
    z = np.asarray(inp["z"], dtype=np.float64).reshape(o.shape)
    yn_exact = gated_rmsnorm(o, z, inp["norm_w"])
    return {"y_conv": y, "conv_state_out": cs_out, "o": o, "state_out": s_out,
            "y": to_io(yn_exact, io), "y_conv_exact": y_exact, "o_exact": o_exact,
            "y_exact": yn_exact}
