"""Prompt -> decode replay on one layer of the 9B shape: a 1024-token prompt through the
chunked prefill, then 256 decode steps on the carried conv and recurrent state (the
generation shape of the HF transformers Qwen3.5 page, "Usage tips and notes"), checked
against the oracle run over all 1280 tokens as one sequence on sampled value heads.
The 256 steps also run as one captured HIP graph, replayed several times with eager work
in between, every replay bit-identical to the eager steps.
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
HEADS = [0, 9, 17, 31]    # value heads of key heads 0, 4, 8 and 15


@pytest.fixture(scope="module")
def replay():
    wl = synth.replay_workload()
    inp = synth.make(wl)
    T, T1 = inp["N"], synth.REPLAY_PROMPT
    hk, hv = inp["Hk"], inp["Hv"]
    d = {k: to_dev(inp[k], "bf16") for k in ("x", "a", "b", "z")}
    for k in ("conv_w", "A_log", "dt_bias", "norm_w"):
        d[k] = f32_dev(inp[k])
    d["z"] = d["z"].view(T, hv, D)
    return inp, d, T, T1, hk, hv


def _prefill(d, T1, hk, hv):
    return gdn.prefill_layer(d["x"][:T1], d["conv_w"], d["a"][:T1], d["b"][:T1], d["A_log"],
                             d["dt_bias"], d["z"][:T1], d["norm_w"], hk, hv)


@pytest.mark.parametrize("fused", [True, False])
def test_replay_eager_matches_oracle(replay, fused):
    inp, d, T, T1, hk, hv = replay
    out = _prefill(d, T1, hk, hv)
    cs, st = out["conv_state_out"], out["state_out"]
    ys = [out["y"]]
    for t in range(T1, T):
        r = gdn.decode_step(d["x"][t:t + 1], d["conv_w"], cs, d["a"][t:t + 1], d["b"][t:t + 1],
                            d["A_log"], d["dt_bias"], st, d["z"][t:t + 1], d["norm_w"], hk, hv,
                            fused=fused)
        ys.append(r["y"])
    y = torch.cat(ys)
    torch.cuda.synchronize()
    ref = G.layer(inp, pairs=[(0, h) for h in HEADS])
    yg = host(y)
    assert_out(yg[:T1][:, HEADS], ref["y_exact"][:T1][:, HEADS], "bf16", "prompt y", upstream_bf16=2)
    assert_out(yg[T1:][:, HEADS], ref["y_exact"][T1:][:, HEADS], "bf16", "decoded y", upstream_bf16=2)
    assert_state(host(st)[0, HEADS][None], ref["state_out"][0, HEADS][None], "final state")
    np.testing.assert_array_equal(host(cs), ref["conv_state_out"])


def test_replay_graph_equals_eager(replay):
    inp, d, T, T1, hk, hv = replay
    n = T - T1
    out = _prefill(d, T1, hk, hv)
    torch.cuda.synchronize()
    cs0, st0 = out["conv_state_out"].clone(), out["state_out"].clone()
    # eager reference of the 256 steps
    cs, st = cs0.clone(), st0.clone()
    ys = []
    for t in range(T1, T):
        r = gdn.decode_step(d["x"][t:t + 1], d["conv_w"], cs, d["a"][t:t + 1], d["b"][t:t + 1],
                            d["A_log"], d["dt_bias"], st, d["z"][t:t + 1], d["norm_w"], hk, hv)
        ys.append(r["y"])
    y_eager = torch.stack(ys)
    cs_eager, st_eager = cs.clone(), st.clone()
    # the same steps as one graph over static input buffers
    xs = d["x"][T1:].reshape(n, 1, -1).clone()
    As = d["a"][T1:].reshape(n, 1, hv).clone()
    Bs = d["b"][T1:].reshape(n, 1, hv).clone()
    zs = d["z"][T1:].reshape(n, 1, hv, D).clone()
    gcs, gst = cs0.clone(), st0.clone()
    graph = gdn.DecodeGraph(xs, d["conv_w"], gcs, As, Bs, d["A_log"], d["dt_bias"], gst, zs,
                            d["norm_w"], hk, hv)
    for rep in range(3):
        gcs.copy_(cs0)
        gst.copy_(st0)
        torch.cuda.synchronize()
        y = graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {rep}: y differs from the eager steps"
        assert torch.equal(gst, st_eager), f"replay {rep}: state differs"
        assert torch.equal(gcs, cs_eager), f"replay {rep}: conv state differs"
        # eager work between replays
        scratch = torch.randn(1 << 20, device="cuda")
        (scratch * 2).sum().item()
