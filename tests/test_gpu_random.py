"""Seeded random shapes through the whole layer against the fp64 oracle.

Each case draws its own key-head count (1, 2, 4), value heads per key head (1..8), io
dtype, sequence lengths (empty, short, several chunks with a ragged tail), whether the
states are carried in, and fused or separate calls.  The chain counts these give fall
on every sweep the chunked core has (row-split, column-chain, 4-wave, 8-wave), and the
per-key-head ratios on every gate batch the prep stages.  Decode cases draw the batch,
the heads, the io and state dtypes and fused or separate step + norm.
"""
import numpy as np
import pytest
import torch

import hybrid_linear_attention_causal_amd as gdn
from hybrid_linear_attention_causal_amd import synth
from hybrid_linear_attention_causal_amd.mixer import decode_step, prefill_layer
from oracle import gdn_oracle as G

from parity import assert_bf16_state, assert_out, assert_state, f32_dev, host, to_dev

pytestmark = pytest.mark.gpu

D = 128
TOKEN_HEADS = 24000      # bound on tokens x value heads, so the oracle takes about a second


def _prefill_case(seed):
    rng = np.random.default_rng(5000 + seed)
    hk = int(rng.choice([1, 2, 4]))
    hv = hk * int(rng.integers(1, 9))
    io = str(rng.choice(["bf16", "bf16", "f32"]))
    while True:
        ns = int(rng.integers(1, 17))
        lens = [0 if rng.random() < 0.15 else int(rng.integers(1, 301)) for _ in range(ns)]
        if sum(lens) * hv <= TOKEN_HEADS:
            break
    return dict(hk=hk, hv=hv, io=io, lens=lens, init_state=bool(rng.random() < 0.7),
                fused=bool(rng.random() < 0.6))


def _decode_case(seed):
    rng = np.random.default_rng(6000 + seed)
    hk = int(rng.choice([1, 2, 4]))
    return dict(hk=hk, hv=hk * int(rng.integers(1, 9)), io=str(rng.choice(["bf16", "f32"])),
                state_io=str(rng.choice(["f32", "bf16"])), B=int(rng.integers(1, 41)),
                fused=bool(rng.random() < 0.6))


PREFILL = [_prefill_case(s) for s in range(24)] + [
    # inputs of at most one row built from NumPy (an empty array has strides (0, 0)) through
    # the separate calls, whose binding passes the q, k, v row strides
    dict(hk=2, hv=14, io="bf16", lens=[0], init_state=False, fused=False),
    dict(hk=2, hv=4, io="bf16", lens=[0, 0], init_state=True, fused=False),
    dict(hk=1, hv=2, io="f32", lens=[1], init_state=True, fused=False),
]
DECODE = [_decode_case(s) for s in range(16)]


def _id(c):
    return "-".join(f"{k}{v}" if not isinstance(v, list) else f"ns{len(v)}n{sum(v)}"
                    for k, v in c.items())


@pytest.mark.parametrize("c", PREFILL, ids=[_id(c) for c in PREFILL])
def test_random_prefill_layer(c):
    hk, hv, io = c["hk"], c["hv"], c["io"]
    sh = synth.Shape(f"h{hk}x{hv}", hk=hk, hv=hv)
    inp = synth.make(synth.custom(sh, io, 5000 + sum(c["lens"]), seqlens=c["lens"],
                                  init_state=c["init_state"]))
    N = inp["N"]
    cu = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).cuda()
    cs_in = to_dev(inp["conv_state_in"], io) if c["init_state"] else None
    s_in = f32_dev(inp["state_in"]) if c["init_state"] else None
    out = prefill_layer(to_dev(inp["x"], io), f32_dev(inp["conv_w"]), to_dev(inp["a"], io),
                        to_dev(inp["b"], io), f32_dev(inp["A_log"]), f32_dev(inp["dt_bias"]),
                        to_dev(inp["z"], io).view(N, hv, D), f32_dev(inp["norm_w"]), hk, hv,
                        cu, cs_in, s_in, fused=c["fused"])
    torch.cuda.synchronize()
    ref = G.layer(inp)
    assert_out(host(out["y_conv"]), ref["y_conv_exact"], io, "conv y")
    np.testing.assert_array_equal(host(out["conv_state_out"]), ref["conv_state_out"])
    assert_out(host(out["o"]), ref["o_exact"], io, "core o", upstream_bf16=1)
    assert_out(host(out["y"]), ref["y_exact"], io, "norm y", upstream_bf16=2)
    assert_state(host(out["state_out"]), ref["state_out"], "final state")


@pytest.mark.parametrize("c", DECODE, ids=[_id(c) for c in DECODE])
def test_random_decode_step(c):
    hk, hv, io, st_io, B = c["hk"], c["hv"], c["io"], c["state_io"], c["B"]
    sh = synth.Shape(f"h{hk}x{hv}", hk=hk, hv=hv)
    inp = synth.make(synth.custom(sh, io, 6000 + B, batch=B, init_state=True, kind="decode"))
    rng = np.random.default_rng(6000 + B)
    z = G.to_io(rng.standard_normal((B, hv, D)), io)
    nw = 1.0 + 0.1 * rng.standard_normal(D)
    s0 = G.to_io(inp["state_in"], st_io)
    cs = to_dev(inp["conv_state_in"], io)
    st = to_dev(s0, "bf16") if st_io == "bf16" else f32_dev(s0)
    out = decode_step(to_dev(inp["x"], io), f32_dev(inp["conv_w"]), cs, to_dev(inp["a"], io),
                      to_dev(inp["b"], io), f32_dev(inp["A_log"]), f32_dev(inp["dt_bias"]), st,
                      to_dev(z, io), f32_dev(nw), hk, hv, fused=c["fused"])
    torch.cuda.synchronize()
    o_ref, cs_ref, st_ref = G.recurrent_step(
        inp["x"], inp["conv_w"], inp["conv_state_in"], inp["a"], inp["b"], inp["A_log"],
        inp["dt_bias"], s0, hk, hv, D, D, io=io, state_io="bf16" if st_io == "bf16" else "f64")
    y_ref = G.gated_rmsnorm(G.to_io(o_ref, io), z, nw)
    assert_out(host(out["o"]), o_ref, io, "step o", upstream_bf16=1)
    assert_out(host(out["y"]), y_ref, io, "step y", upstream_bf16=2)
    np.testing.assert_array_equal(host(cs), cs_ref)
    if st_io == "bf16":
        assert_bf16_state(host(st), st_ref, "bf16 state", upstream_bf16=1)
    else:
        assert_state(host(st), st_ref, "state")


def _chunk_case(seed):
    rng = np.random.default_rng(7000 + seed)
    hk = int(rng.choice([1, 2, 4]))
    hv = hk * int(rng.integers(1, 9))
    while True:
        ns = int(rng.integers(1, 13))
        lens = [0 if rng.random() < 0.15 else int(rng.integers(1, 301)) for _ in range(ns)]
        if sum(lens) * hv <= TOKEN_HEADS:
            break
    return dict(hk=hk, hv=hv, io=str(rng.choice(["bf16", "bf16", "f32"])), lens=lens,
                gates=bool(rng.random() < 0.4), l2=bool(rng.random() < 0.7),
                scale=float(rng.choice([0.0, round(float(rng.uniform(0.05, 0.5)), 3)])),
                init_state=bool(rng.random() < 0.7))


CHUNK = [_chunk_case(s) for s in range(16)]


@pytest.mark.parametrize("c", CHUNK, ids=[_id(c) for c in CHUNK])
def test_random_chunk_prefill(c):
    """The chunked core alone on q, k, v in separate buffers with padded rows, with given
    gates or the gate formula, the L2 norm on or off and a given or default output scale;
    the no-allocation entry point equals it bit for bit."""
    hk, hv, io = c["hk"], c["hv"], c["io"]
    sh = synth.Shape(f"h{hk}x{hv}", hk=hk, hv=hv)
    inp = synth.make(synth.custom(sh, io, 7000 + sum(c["lens"]), seqlens=c["lens"],
                                  init_state=c["init_state"]))
    N = inp["N"]
    rng = np.random.default_rng(7100 + N)
    # unnormalised keys of norm ~1 keep beta |k|^2 < 2, so the recurrence stays bounded
    ks = 1.0 if c["l2"] else 0.09
    q = G.to_io(rng.standard_normal((N, hk * D)), io)
    k = G.to_io(ks * rng.standard_normal((N, hk * D)), io)
    v = G.to_io(rng.standard_normal((N, hv * D)), io)
    g = beta = None
    if c["gates"]:
        g = -rng.uniform(0.0, 0.5, (N, hv))
        beta = rng.uniform(0.0, 1.0, (N, hv))
    padded = []
    for arr, pad in ((q, 16), (k, 40), (v, 8)):
        buf = torch.full((N, arr.shape[1] + pad), float("nan"), device="cuda",
                         dtype=torch.bfloat16 if io == "bf16" else torch.float32)
        buf[:, : arr.shape[1]] = to_dev(arr, io)
        padded.append(buf[:, : arr.shape[1]])
    cu = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).cuda()
    s_in = f32_dev(inp["state_in"]) if c["init_state"] else None
    gate_args = [to_dev(inp["a"], io), to_dev(inp["b"], io), f32_dev(inp["A_log"]),
                 f32_dev(inp["dt_bias"])]
    kw = dict(g_opt=f32_dev(g), beta_opt=f32_dev(beta), scale=c["scale"],
              use_qk_l2norm=c["l2"])
    Ns = len(c["lens"])
    outs = []
    for fn in (gdn.gdn_chunk_prefill, gdn.gdn_chunk_prefill_noalloc):
        o = torch.empty((N, hv, D), dtype=padded[0].dtype, device="cuda")
        s_out = torch.empty((Ns, hv, D, D), device="cuda")
        fn(*padded, *gate_args, o, hk, hv, cu, s_in, s_out, **kw)
        outs.append((o, s_out))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]), "no-allocation o"
    assert torch.equal(outs[0][1], outs[1][1]), "no-allocation state"
    o_ref, s_ref = G.prefill(q, k, v, inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], hk, hv,
                             D, D, inp["state_in"], inp["cu_seqlens"], scale=c["scale"],
                             use_qk_l2norm=c["l2"], g=g, beta=beta)
    assert_out(host(outs[0][0]), o_ref, io, "chunk o")
    assert_state(host(outs[0][1]), s_ref, "chunk state")
