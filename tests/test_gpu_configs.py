"""GPU parity at the five standard workload sizes, through the same layer calls the
benchmark times.  The whole layer runs on the GPU; the oracle recomputes sampled
(sequence, value head) chains over their full length, plus the conv channels
they read, and the comparison covers every token of those chains.

Workloads (seeded, see the input generator):
0  Qwen3.5-0.8B shape, fp32, T=256 (checked in full)
1  Qwen3.5-9B shape, bf16, T=4096
2  Qwen3.5-9B decode, B=256, nonzero states (checked in full)
3  Qwen3.5-397B-A17B shape, bf16, T=32768
4  Qwen3.5-9B varlen, 64 sequences with lengths in [16, 2048], carried states
"""
import numpy as np
import pytest
import torch

import hybrid_linear_attention_causal_amd as gdn
from hybrid_linear_attention_causal_amd import synth
from oracle import gdn_oracle as G

from parity import assert_out, assert_state, f32_dev, host, to_dev

pytestmark = pytest.mark.gpu

D = 128


def _upload(inp):
    io = inp["io"]
    d = {k: to_dev(inp[k], io) for k in ("x", "a", "b", "z", "conv_state_in")}
    for k in ("conv_w", "A_log", "dt_bias", "norm_w", "state_in"):
        d[k] = f32_dev(inp[k])
    cu = inp["cu_seqlens"]
    d["cu"] = None if cu is None else torch.from_numpy(cu.astype(np.int32)).cuda()
    return d


def _oracle_chain(inp, s, h):
    """Full-length oracle for one (sequence, value head): conv of the channels it reads,
    L2 norm, gates, recurrence and gated norm, rounding at the call boundaries."""
    io, hk, hv = inp["io"], inp["Hk"], inp["Hv"]
    kh = h // (hv // hk)
    cu = inp["cu_seqlens"]
    b0, b1 = (0, inp["N"]) if cu is None else (int(cu[s]), int(cu[s + 1]))
    chans = np.concatenate([np.arange(kh * D, kh * D + D),
                            hk * D + np.arange(kh * D, kh * D + D),
                            2 * hk * D + np.arange(h * D, h * D + D)])
    cs_in = None if inp["conv_state_in"] is None else inp["conv_state_in"][s:s + 1][:, :, chans]
    y, cs_out = G.conv1d_fwd(inp["x"][b0:b1, chans], inp["conv_w"][chans], None, cs_in)
    y = G.to_io(y, io)
    q, k, v = y[:, :D], y[:, D:2 * D], y[:, 2 * D:]
    g, beta = G.gates(inp["a"][b0:b1, h:h + 1], inp["b"][b0:b1, h:h + 1],
                      inp["A_log"][h:h + 1], inp["dt_bias"][h:h + 1])
    S0 = np.zeros((D, D)) if inp["state_in"] is None else inp["state_in"][s, h]
    o, S = G.delta_rule(G.l2_normalize(q), G.l2_normalize(k), v, g[:, 0], beta[:, 0], S0,
                        1.0 / np.sqrt(D))
    o = G.to_io(o, io)
    z = inp["z"][b0:b1, h * D:(h + 1) * D]
    yn = G.to_io(G.gated_rmsnorm(o, z, inp["norm_w"]), io)
    return {"chans": chans, "b0": b0, "b1": b1, "y_conv": y, "o": o, "y": yn, "S": S,
            "cs_out": cs_out[0]}


def _check_prefill(widx, pairs):
    inp = synth.make(synth.workload(widx))
    io, hk, hv = inp["io"], inp["Hk"], inp["Hv"]
    d = _upload(inp)
    N = inp["N"]
    out = gdn.prefill_layer(d["x"], d["conv_w"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                            d["z"].view(N, hv, D), d["norm_w"], hk, hv, d["cu"],
                            d["conv_state_in"], d["state_in"])
    torch.cuda.synchronize()
    if pairs is None:
        pairs = [(s, h) for s in range(inp["Ns"]) for h in range(hv)]
    o_all, y_all, yc_all, s_all = [], [], [], []
    o_ref, y_ref, yc_ref, s_ref = [], [], [], []
    for s, h in pairs:
        r = _oracle_chain(inp, s, h)
        b0, b1 = r["b0"], r["b1"]
        chans = torch.from_numpy(r["chans"]).cuda()
        yc_all.append(host(out["y_conv"][b0:b1].index_select(1, chans)))
        yc_ref.append(r["y_conv"])
        o_all.append(host(out["o"][b0:b1, h]))
        o_ref.append(r["o"])
        y_all.append(host(out["y"][b0:b1, h]))
        y_ref.append(r["y"])
        s_all.append(host(out["state_out"][s, h])[None])
        s_ref.append(r["S"][None])
        np.testing.assert_array_equal(host(out["conv_state_out"][s].index_select(1, chans)),
                                      r["cs_out"])
    assert_out(np.concatenate(yc_all), np.concatenate(yc_ref), io, f"w{widx} conv y")
    assert_out(np.concatenate(o_all), np.concatenate(o_ref), io, f"w{widx} o")
    assert_out(np.concatenate(y_all), np.concatenate(y_ref), io, f"w{widx} y", upstream_bf16=1)
    assert_state(np.concatenate(s_all), np.concatenate(s_ref), f"w{widx} state")


def test_workload0_qwen35_08b_fp32_full():
    _check_prefill(0, None)


def test_workload1_qwen35_9b_prefill_sampled():
    _check_prefill(1, [(0, 0), (0, 13), (0, 31)])


def test_workload3_qwen35_397b_long_prefill_sampled():
    _check_prefill(3, [(0, 5), (0, 62)])


def test_workload4_varlen_carried_state_sampled():
    _check_prefill(4, [(0, 0), (17, 9), (40, 30), (63, 17)])


def test_workload2_qwen35_9b_decode_full():
    inp = synth.make(synth.workload(2))
    io, hk, hv, B = inp["io"], inp["Hk"], inp["Hv"], inp["N"]
    d = _upload(inp)
    out = gdn.decode_step(d["x"], d["conv_w"], d["conv_state_in"], d["a"], d["b"], d["A_log"],
                          d["dt_bias"], d["state_in"], d["z"].view(B, hv, D), d["norm_w"], hk, hv)
    torch.cuda.synchronize()
    o_ref, cs_ref, st_ref = G.recurrent_step(inp["x"], inp["conv_w"], inp["conv_state_in"],
                                             inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                                             inp["state_in"], hk, hv, D, D, io=io)
    o_ref = G.to_io(o_ref, io)
    y_ref = G.to_io(G.gated_rmsnorm(o_ref, inp["z"].reshape(B, hv, D), inp["norm_w"]), io)
    assert_out(host(out["o"]), o_ref, io, "decode o")
    assert_out(host(out["y"]), y_ref, io, "decode y", upstream_bf16=1)
    np.testing.assert_array_equal(host(d["conv_state_in"]), cs_ref)
    assert_state(host(d["state_in"]), st_ref, "decode state")
