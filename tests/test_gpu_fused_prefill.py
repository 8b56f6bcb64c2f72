"""gdn_conv_chunk_prefill (conv + chunked core in one call) against the two calls it
replaces: y, o, the final recurrent state and the final conv state bit for bit, in every
launch shape of the chunked core (row-split sweep; 4-wave and 8-wave sweeps), with
carried states, ragged and empty sequences, in-place conv state and both io dtypes; and
the fused layer against the oracle."""
import numpy as np
import pytest
import torch

import hybrid_linear_attention_causal_amd as gdn
from hybrid_linear_attention_causal_amd import synth
from hybrid_linear_attention_causal_amd.mixer import qkv_views
from oracle import gdn_oracle as G

from parity import assert_out, assert_state, f32_dev, host, to_dev

pytestmark = pytest.mark.gpu

D = 128
LENS = [1, 17, 63, 64, 65, 130, 0, 200, 5, 64, 129, 33]


def _inputs(hk, hv, io, seed, lens):
    sh = synth.Shape(f"h{hk}x{hv}", hk=hk, hv=hv)
    inp = synth.make(synth.custom(sh, io, seed, seqlens=lens, init_state=True))
    d = {k: to_dev(inp[k], io) for k in ("x", "a", "b", "conv_state_in")}
    for k in ("conv_w", "A_log", "dt_bias", "state_in"):
        d[k] = f32_dev(inp[k])
    d["cu"] = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).cuda()
    return inp, d


def _both(d, hk, hv, in_place=False):
    x = d["x"]
    N, Cq = x.shape
    Ns = d["cu"].numel() - 1
    res = []
    for fused in (True, False):
        y = torch.empty_like(x)
        o = torch.empty((N, hv, D), dtype=x.dtype, device="cuda")
        s_out = torch.empty((Ns, hv, D, D), device="cuda")
        cs_in = d["conv_state_in"].clone()
        cs_out = cs_in if in_place else torch.empty_like(cs_in)
        if fused:
            gdn.gdn_conv_chunk_prefill(x, d["conv_w"], y, d["a"], d["b"], d["A_log"],
                                       d["dt_bias"], o, hk, hv, d["cu"], cs_in, cs_out,
                                       d["state_in"], s_out)
        else:
            gdn.gdn_conv1d_fwd(x, d["conv_w"], y, d["cu"], cs_in, cs_out)
            q, k, v = qkv_views(y, hk, hv)
            gdn.gdn_chunk_prefill(q, k, v, d["a"], d["b"], d["A_log"], d["dt_bias"], o, hk, hv,
                                  d["cu"], d["state_in"], s_out)
        res.append((y, o, s_out, cs_out))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("io,hk,hv,lens,in_place", [
    ("bf16", 2, 4, LENS, False),            # 48 chains: row-split sweep, two rounds
    ("bf16", 1, 3, LENS[:7], True),         # 21 chains, three value heads per key head
    ("bf16", 4, 4, [2, 130, 64, 0, 65], False),   # 20 chains, one value head per key head
    ("bf16", 2, 4, LENS * 2, False),        # 96 chains: 4-wave sweep
    ("bf16", 2, 4, LENS * 4, True),         # 192 chains: 8-wave sweep
    ("f32", 2, 4, LENS, False),             # fp32 io: conv then the chunk call
    ("bf16", 16, 32, [4096], False),        # 1024 prep workgroups, one round: conv in the prep
    # more prep workgroups than fit on the chip at once: the conv kernel runs ahead of
    # the prep inside the fused call
    ("bf16", 16, 32, [8192], False),        # 2064 prep workgroups, row-split sweep
    ("bf16", 4, 8, LENS * 24, True),        # 288 sequences, 8-wave sweep
    ("bf16", 1, 2, [16500], False),         # 2 long chains: the intra-sequence scan
    # more than four value heads per key head: the prep stages gates in batches of four,
    # and the fused conv takes two (112 channel groups) or three (160) passes
    ("bf16", 1, 5, LENS[:7], False),        # 35 chains: row-split sweep, a partial batch
    ("bf16", 2, 16, LENS * 4, True),        # 768 chains: 8-wave sweep, two full batches
])
def test_fused_equals_two_calls(io, hk, hv, lens, in_place):
    inp, d = _inputs(hk, hv, io, 70 + len(lens), lens)
    (y1, o1, s1, c1), (y2, o2, s2, c2) = _both(d, hk, hv, in_place)
    assert torch.equal(y1, y2), "conv output"
    assert torch.equal(c1, c2), "final conv state"
    assert torch.equal(o1, o2), "core output"
    assert torch.equal(s1, s2), "final recurrent state"


def test_fused_layer_against_oracle():
    io, hk, hv = "bf16", 2, 4
    inp, d = _inputs(hk, hv, io, 91, LENS)
    N = inp["N"]
    z = to_dev(inp["z"], io).view(N, hv, D)
    out = gdn.prefill_layer(d["x"], d["conv_w"], d["a"], d["b"], d["A_log"], d["dt_bias"], z,
                            f32_dev(inp["norm_w"]), hk, hv, d["cu"], d["conv_state_in"],
                            d["state_in"], fused=True)
    torch.cuda.synchronize()
    ref = G.layer(inp)
    assert_out(host(out["y_conv"]), ref["y_conv_exact"], io, "fused conv y")
    np.testing.assert_array_equal(host(out["conv_state_out"]), ref["conv_state_out"])
    assert_out(host(out["o"]), ref["o_exact"], io, "fused o", upstream_bf16=1)
    assert_out(host(out["y"]), ref["y_exact"], io, "fused y", upstream_bf16=2)
    assert_state(host(out["state_out"]), ref["state_out"], "fused state")


def test_fused_equals_two_calls_with_given_gates_and_no_l2norm():
    """Precomputed g / beta and use_qk_l2norm=False take the same paths in both forms."""
    io, hk, hv = "bf16", 2, 4
    inp, d = _inputs(hk, hv, io, 93, LENS)
    N = inp["N"]
    rng = np.random.default_rng(93)
    g = f32_dev(-rng.uniform(0.0, 0.5, (N, hv)))
    # unnormalised keys have |k|^2 ~ 10 here: beta |k|^2 < 2 keeps the recurrence stable
    beta = f32_dev(rng.uniform(0.0, 0.1, (N, hv)))
    x = d["x"]
    Ns = d["cu"].numel() - 1
    outs = []
    for fused in (True, False):
        y = torch.empty_like(x)
        o = torch.empty((N, hv, D), dtype=x.dtype, device="cuda")
        s_out = torch.empty((Ns, hv, D, D), device="cuda")
        cs_out = torch.empty_like(d["conv_state_in"])
        if fused:
            gdn.gdn_conv_chunk_prefill(x, d["conv_w"], y, None, None, None, None, o, hk, hv,
                                       d["cu"], d["conv_state_in"], cs_out, d["state_in"], s_out,
                                       g_opt=g, beta_opt=beta, use_qk_l2norm=False)
        else:
            gdn.gdn_conv1d_fwd(x, d["conv_w"], y, d["cu"], d["conv_state_in"], cs_out)
            q, k, v = qkv_views(y, hk, hv)
            gdn.gdn_chunk_prefill(q, k, v, None, None, None, None, o, hk, hv, d["cu"],
                                  d["state_in"], s_out, g_opt=g, beta_opt=beta,
                                  use_qk_l2norm=False)
        outs.append((y, o, s_out, cs_out))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    assert torch.isfinite(outs[0][1].float()).all()


@pytest.mark.parametrize("T", [1, 2, 3, 5, 64, 130])
@pytest.mark.parametrize("with_state", [False, True])
def test_fused_single_sequence_final_conv_state(T, with_state):
    """One sequence: the prep writes the final conv state itself (rows from x, or from the
    conv state before a sequence shorter than 3); equal to the two calls bit for bit."""
    io, hk, hv = "bf16", 1, 2
    sh = synth.Shape("h1x2", hk=hk, hv=hv)
    inp = synth.make(synth.custom(sh, io, 94 + T, seqlens=[T], init_state=with_state))
    x = to_dev(inp["x"], io)
    w = f32_dev(inp["conv_w"])
    a, b = to_dev(inp["a"], io), to_dev(inp["b"], io)
    A_log, dt = f32_dev(inp["A_log"]), f32_dev(inp["dt_bias"])
    cs_in = to_dev(inp["conv_state_in"], io) if with_state else None
    s_in = f32_dev(inp["state_in"]) if with_state else None
    outs = []
    for fused in (True, False):
        y = torch.empty_like(x)
        o = torch.empty((T, hv, D), dtype=x.dtype, device="cuda")
        s_out = torch.empty((1, hv, D, D), device="cuda")
        cs_out = torch.full((1, 3, x.shape[1]), 7.0, dtype=x.dtype, device="cuda")
        if fused:
            gdn.gdn_conv_chunk_prefill(x, w, y, a, b, A_log, dt, o, hk, hv, None, cs_in, cs_out,
                                       s_in, s_out)
        else:
            gdn.gdn_conv1d_fwd(x, w, y, None, cs_in, cs_out)
            q, k, v = qkv_views(y, hk, hv)
            gdn.gdn_chunk_prefill(q, k, v, a, b, A_log, dt, o, hk, hv, None, s_in, s_out)
        outs.append((y, o, s_out, cs_out))
    torch.cuda.synchronize()
    for name, u, v in zip(("y", "o", "state", "conv state"), *outs):
        assert torch.equal(u, v), name
    ref = G.layer(inp)
    np.testing.assert_array_equal(host(outs[0][3]), ref["conv_state_out"])


def test_fused_empty_sequence_passes_states_through():
    """One sequence given by cu_seqlens = {0, 0} over a non-empty x: no token belongs to it,
    so its final conv state is its initial conv state and its final recurrent state is its
    initial state (the prep, which writes the conv state for one sequence without
    cu_seqlens, has no chunk to do it from here)."""
    io, hk, hv = "bf16", 1, 2
    sh = synth.Shape("h1x2", hk=hk, hv=hv)
    inp = synth.make(synth.custom(sh, io, 97, seqlens=[8], init_state=True))
    x = to_dev(inp["x"], io)
    w = f32_dev(inp["conv_w"])
    a, b = to_dev(inp["a"], io), to_dev(inp["b"], io)
    A_log, dt = f32_dev(inp["A_log"]), f32_dev(inp["dt_bias"])
    cs_in = to_dev(inp["conv_state_in"], io)
    s_in = f32_dev(inp["state_in"])
    cu = torch.tensor([0, 0], dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    o = torch.empty((8, hv, D), dtype=x.dtype, device="cuda")
    s_out = torch.full((1, hv, D, D), 3.0, device="cuda")
    cs_out = torch.full((1, 3, x.shape[1]), 7.0, dtype=x.dtype, device="cuda")
    gdn.gdn_conv_chunk_prefill(x, w, y, a, b, A_log, dt, o, hk, hv, cu, cs_in, cs_out, s_in,
                               s_out)
    torch.cuda.synchronize()
    assert torch.equal(cs_out, cs_in)
    assert torch.equal(s_out, s_in)


@pytest.mark.parametrize("hk,hv,lens", [
    (2, 4, LENS),            # row-split sweep
    (2, 4, LENS * 2),        # 4-wave sweep
    (2, 4, LENS * 4),        # 8-wave sweep
    (4, 8, LENS * 24),       # 288 sequences, 8-wave sweep
])
def test_prefill_layer_equals_conv_chunk_then_norm(hk, hv, lens):
    """gdn_prefill_layer (conv + chunked core + gated norm in one call) against
    gdn_conv_chunk_prefill followed by gdn_gated_rmsnorm: every output bit for bit, on each
    sweep shape."""
    io = "bf16"
    inp, d = _inputs(hk, hv, io, 80 + len(lens), lens)
    x = d["x"]
    N = x.shape[0]
    Ns = d["cu"].numel() - 1
    z = to_dev(inp["z"], io).view(N, hv, D)
    nw = f32_dev(inp["norm_w"])
    outs = []
    for one_call in (True, False):
        y = torch.empty_like(x)
        o = torch.empty((N, hv, D), dtype=x.dtype, device="cuda")
        yn = torch.full_like(o, 3.0)
        s_out = torch.empty((Ns, hv, D, D), device="cuda")
        cs_out = torch.empty_like(d["conv_state_in"])
        if one_call:
            gdn.gdn_prefill_layer(x, d["conv_w"], y, d["a"], d["b"], d["A_log"], d["dt_bias"], o,
                                  z, nw, yn, hk, hv, d["cu"], d["conv_state_in"], cs_out,
                                  d["state_in"], s_out)
        else:
            gdn.gdn_conv_chunk_prefill(x, d["conv_w"], y, d["a"], d["b"], d["A_log"],
                                       d["dt_bias"], o, hk, hv, d["cu"], d["conv_state_in"],
                                       cs_out, d["state_in"], s_out)
            gdn.gdn_gated_rmsnorm(o, z, nw, yn)
        outs.append((y, o, yn, s_out, cs_out))
    torch.cuda.synchronize()
    for name, u, v in zip(("conv y", "o", "norm y", "state", "conv state"), *outs):
        assert torch.equal(u, v), name
    ref = G.layer(inp)
    assert_out(host(outs[0][2]), ref["y_exact"], io, "layer y", upstream_bf16=2)


@pytest.mark.parametrize("io,hk,hv,lens", [
    ("bf16", 2, 4, LENS),          # row-split sweep, two column tiles per workgroup
    ("bf16", 2, 4, LENS * 2),      # 4-wave sweep
    ("bf16", 2, 4, LENS * 4),      # 8-wave sweep
    ("f32", 2, 4, LENS),           # fp32 io
    ("bf16", 1, 2, [16500]),       # the intra-sequence scan
])
def test_chunk_prefill_row_strides_and_no_state_out(io, hk, hv, lens):
    """q, k and v in three separate buffers with padded rows (their own row strides, not
    views into one conv output) give the same o and final state bit for bit; and a call
    without state_out gives the same o."""
    inp, d = _inputs(hk, hv, io, 110 + len(lens), lens)
    x = d["x"]
    N = x.shape[0]
    Ns = d["cu"].numel() - 1
    y = torch.empty_like(x)
    gdn.gdn_conv1d_fwd(x, d["conv_w"], y, d["cu"], d["conv_state_in"], None)
    q, k, v = qkv_views(y, hk, hv)
    padded = []
    for t, pad in ((q, 24), (k, 8), (v, 40)):
        buf = torch.full((N, t.shape[1] + pad), float("nan"), dtype=t.dtype, device="cuda")
        buf[:, : t.shape[1]] = t
        padded.append(buf[:, : t.shape[1]])
    outs = []
    for qq, kk, vv, with_state in ((q, k, v, True), (*padded, True), (q, k, v, False)):
        o = torch.empty((N, hv, D), dtype=x.dtype, device="cuda")
        s_out = torch.empty((Ns, hv, D, D), device="cuda") if with_state else None
        gdn.gdn_chunk_prefill(qq, kk, vv, d["a"], d["b"], d["A_log"], d["dt_bias"], o, hk, hv,
                              d["cu"], d["state_in"], s_out)
        outs.append((o, s_out))
    torch.cuda.synchronize()
    assert padded[0].stride(0) != q.stride(0)
    assert torch.equal(outs[0][0], outs[1][0]), "o with padded rows"
    assert torch.equal(outs[0][1], outs[1][1]), "state with padded rows"
    assert torch.equal(outs[0][0], outs[2][0]), "o without state_out"
    assert torch.isfinite(outs[0][0].float()).all()
