"""GPU parity: every libgdn call against the fp64 oracle on identical seeded inputs.

Small cases span several 64-token chunks, ragged tails, empty and 1-token
sequences, Hv/Hk in {1, 2, 4}, both io dtypes and carried states.  The
tolerances are stated in tests/parity.py.
"""
import numpy as np
import pytest
import torch

import hybrid_linear_attention_causal_amd as gdn
from hybrid_linear_attention_causal_amd import synth
from hybrid_linear_attention_causal_amd.mixer import qkv_views
from oracle import gdn_oracle as G

from parity import assert_bf16_state, assert_out, assert_state, f32_dev, host, to_dev

pytestmark = pytest.mark.gpu

D = 128


def _case(hk, hv, io, seed, seqlens=None, batch=0, init_state=True, kind="prefill"):
    sh = synth.Shape(f"h{hk}x{hv}", hk=hk, hv=hv)
    wl = synth.custom(sh, io, seed, seqlens=seqlens, batch=batch, init_state=init_state, kind=kind)
    return synth.make(wl)


def _cu_dev(inp):
    cu = inp["cu_seqlens"]
    return None if cu is None else torch.from_numpy(cu.astype(np.int32)).cuda()


# (A decode step rounds its conv output to the io dtype inside the call, as the prefill
# layer does at the conv call's boundary, so its o has one bf16 value upstream; see parity.)

# ------------------------------------------------------------------------- conv
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("init_state", [False, True])
def test_conv1d_parity(io, init_state):
    inp = _case(2, 4, io, 11, seqlens=[1, 2, 3, 5, 0, 64, 100, 37], init_state=init_state)
    N, Cq = inp["x"].shape
    x = to_dev(inp["x"], io)
    w = f32_dev(inp["conv_w"])
    y = torch.empty_like(x)
    cs_in = to_dev(inp["conv_state_in"], io)
    cs_out = torch.empty((inp["Ns"], 3, Cq), dtype=x.dtype, device="cuda")
    gdn.gdn_conv1d_fwd(x, w, y, _cu_dev(inp), cs_in, cs_out)
    torch.cuda.synchronize()
    y_ref, cs_ref = G.conv1d_fwd(inp["x"], inp["conv_w"], inp["cu_seqlens"], inp["conv_state_in"])
    assert_out(host(y), y_ref, io, "conv y")
    np.testing.assert_array_equal(host(cs_out), cs_ref)   # raw rows: bit-exact


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_conv1d_state_in_place(io):
    inp = _case(1, 1, io, 12, seqlens=[2, 7, 1, 40])
    x = to_dev(inp["x"], io)
    w = f32_dev(inp["conv_w"])
    y = torch.empty_like(x)
    cs = to_dev(inp["conv_state_in"], io)
    gdn.gdn_conv1d_fwd(x, w, y, _cu_dev(inp), cs, cs)       # in == out
    torch.cuda.synchronize()
    y_ref, cs_ref = G.conv1d_fwd(inp["x"], inp["conv_w"], inp["cu_seqlens"], inp["conv_state_in"])
    assert_out(host(y), y_ref, io, "conv y")
    np.testing.assert_array_equal(host(cs), cs_ref)


# ------------------------------------------------------------------------- norm
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_gated_rmsnorm_parity(io):
    rng = np.random.default_rng(13)
    rows = 1003
    o = synth.round_io((rng.standard_normal((rows, D)) * rng.uniform(1e-3, 3, (rows, 1))).astype(np.float32), io)
    z = synth.round_io(rng.standard_normal((rows, D)).astype(np.float32), io)
    w = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    og, zg = to_dev(o, io), to_dev(z, io)
    y = torch.empty_like(og)
    gdn.gdn_gated_rmsnorm(og, zg, f32_dev(w), y)
    torch.cuda.synchronize()
    assert_out(host(y), G.gated_rmsnorm(o, z, w), io, "norm y")
    gdn.gdn_gated_rmsnorm(og, zg, f32_dev(w), og)             # in place
    torch.cuda.synchronize()
    assert_out(host(og), G.gated_rmsnorm(o, z, w), io, "norm y in place")


# ------------------------------------------------------------------------- prefill core
def _run_prefill(inp, io, use_l2=True, g=None, beta=None, with_state=True):
    """Conv on the oracle (so the core sees oracle-made q/k/v), then the GPU core."""
    y_ref, _ = G.conv1d_fwd(inp["x"], inp["conv_w"], inp["cu_seqlens"], inp["conv_state_in"])
    y_io = G.to_io(y_ref, io).astype(np.float32)
    hk, hv = inp["Hk"], inp["Hv"]
    yd = to_dev(y_io, io)
    q, k, v = qkv_views(yd, hk, hv)
    N = inp["N"]
    o = torch.empty((N, hv, D), dtype=yd.dtype, device="cuda")
    s_out = torch.full((inp["Ns"], hv, D, D), float("nan"), device="cuda")
    gdn.gdn_chunk_prefill(q, k, v, to_dev(inp["a"], io), to_dev(inp["b"], io),
                          f32_dev(inp["A_log"]), f32_dev(inp["dt_bias"]), o, hk, hv,
                          _cu_dev(inp), f32_dev(inp["state_in"]) if with_state else None, s_out,
                          g_opt=f32_dev(g), beta_opt=f32_dev(beta), use_qk_l2norm=use_l2)
    torch.cuda.synchronize()
    return y_io.astype(np.float64), host(o), host(s_out)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("hk,hv", [(2, 2), (1, 2), (1, 4), (1, 5), (1, 8)])
def test_chunk_prefill_parity_small(io, hk, hv):
    """Ragged, empty and multi-chunk sequences with carried state; for bf16 the 16-64
    chains' row-split workgroups fit the chip at once (the chain/output sweep).  More than
    four value heads per key head take the prep's gates in batches of four: 5 ends on a
    partial batch, 8 is two full ones."""
    lens = [1, 63, 64, 65, 200, 0, 3, 130]
    inp = _case(hk, hv, io, 20 + hv, seqlens=lens, init_state=True)
    y, o, s = _run_prefill(inp, io)
    q = y[:, : hk * D]
    k = y[:, hk * D: 2 * hk * D]
    v = y[:, 2 * hk * D:]
    o_ref, s_ref = G.prefill(q, k, v, inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], hk, hv,
                             D, D, inp["state_in"], inp["cu_seqlens"])
    assert_out(o, o_ref, io, "prefill o")
    assert_state(s, s_ref, "prefill state")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_chunk_prefill_parity_many_chains(io):
    """More (sequence, head) chains than twice the compute units (40 x 4 x 2 > 256):
    the sweep runs as one 8-wave workgroup per chain instead of two 4-wave ones."""
    hk, hv = 2, 4
    lens = [1, 17, 63, 64, 65, 100, 0, 130] * 5
    inp = _case(hk, hv, io, 41, seqlens=lens, init_state=True)
    assert inp["Ns"] * hv * 2 > torch.cuda.get_device_properties(0).multi_processor_count
    y, o, s = _run_prefill(inp, io)
    o_ref, s_ref = G.prefill(y[:, :hk * D], y[:, hk * D:2 * hk * D], y[:, 2 * hk * D:],
                             inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], hk, hv, D, D,
                             inp["state_in"], inp["cu_seqlens"])
    assert_out(o, o_ref, io, "prefill o")
    assert_state(s, s_ref, "prefill state")


def test_chunk_prefill_parity_rowsplit_two_rounds():
    """bf16 with 48 (sequence, head) chains: the row-split sweep's 384 workgroups are more
    than one per compute unit, so two share a CU (ragged, full and empty sequences)."""
    io, hk, hv = "bf16", 2, 4
    lens = [1, 17, 63, 64, 65, 130, 0, 200, 5, 64, 129, 33]
    inp = _case(hk, hv, io, 61, seqlens=lens, init_state=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert cus < inp["Ns"] * hv * 8 <= 2 * cus
    y, o, s = _run_prefill(inp, io)
    o_ref, s_ref = G.prefill(y[:, :hk * D], y[:, hk * D:2 * hk * D], y[:, 2 * hk * D:],
                             inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], hk, hv, D, D,
                             inp["state_in"], inp["cu_seqlens"])
    assert_out(o, o_ref, io, "prefill o")
    assert_state(s, s_ref, "prefill state")


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("lens", [[1600], [1500, 37, 2000, 0]], ids=["one", "varlen"])
def test_chunk_prefill_parity_segmented(io, lens):
    """Few chains and long sequences.  fp32: each chain splits into segments (6 for one
    1600-token sequence at 2 heads, 3 for the varlen case, where the 37-token and the
    empty sequence leave segments without chunks) that run in parallel from transition
    matrices formed by a first pass.  bf16: the row-split sweep walks the long chains
    (25 and 32 chunks) with eight workgroups each."""
    hk, hv = 1, 2
    inp = _case(hk, hv, io, 51 + len(lens), seqlens=lens, init_state=True)
    y, o, s = _run_prefill(inp, io)
    o_ref, s_ref = G.prefill(y[:, :hk * D], y[:, hk * D:2 * hk * D], y[:, 2 * hk * D:],
                             inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], hk, hv, D, D,
                             inp["state_in"], inp["cu_seqlens"])
    assert_out(o, o_ref, io, "prefill o")
    assert_state(s, s_ref, "prefill state")


@pytest.mark.parametrize("lens", [[16500], [20000, 17000]], ids=["one", "varlen"])
def test_chunk_prefill_parity_segmented_bf16(lens):
    """bf16 with few, long chains: the intra-sequence scan instead of the row-split sweep
    (2 or 4 chains, whose row-split launch would fill at most half the compute units, of
    258 chunks with a ragged last one, or two sequences averaging 289 chunks), eight
    segments per sequence, with carried states."""
    io, hk, hv = "bf16", 1, 2
    inp = _case(hk, hv, io, 71 + len(lens), seqlens=lens, init_state=True)
    N, Ns = inp["N"], inp["Ns"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert 2 * Ns * hv * 8 <= cus and -(-N // 64) // Ns >= 256   # the scan's launch shape
    # the workspace holds the scan's segment pairs
    ws = gdn.gdn_chunk_prefill_workspace_size(N, Ns, hk, hv, io=torch.bfloat16)
    assert ws >= 7 * Ns * hv * 131072
    y, o, s = _run_prefill(inp, io)
    o_ref, s_ref = G.prefill(y[:, :hk * D], y[:, hk * D:2 * hk * D], y[:, 2 * hk * D:],
                             inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], hk, hv, D, D,
                             inp["state_in"], inp["cu_seqlens"])
    assert_out(o, o_ref, io, "prefill o")
    assert_state(s, s_ref, "prefill state")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_chunk_prefill_zero_state_single_sequence(io):
    inp = _case(2, 4, io, 31, seqlens=[257], init_state=False)
    y, o, s = _run_prefill(inp, io, with_state=False)
    hk, hv = 2, 4
    o_ref, s_ref = G.prefill(y[:, :hk * D], y[:, hk * D:2 * hk * D], y[:, 2 * hk * D:],
                             inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], hk, hv, D, D)
    assert_out(o, o_ref, io, "prefill o")
    assert_state(s, s_ref, "prefill state")


def test_chunk_prefill_no_write_no_decay():
    """beta = 0 and g = 0: the state passes through and o_t = scale S0^T q^_t."""
    io = "f32"
    inp = _case(1, 2, io, 32, seqlens=[70, 5])
    N = inp["N"]
    zeros = np.zeros((N, 2), np.float32)
    y, o, s = _run_prefill(inp, io, g=zeros, beta=zeros)
    np.testing.assert_allclose(s, inp["state_in"], rtol=0, atol=0)
    qn = G.l2_normalize(y[:, :D])
    cu = inp["cu_seqlens"]
    for si in range(2):
        for h in range(2):
            ref = qn[cu[si]:cu[si + 1]] @ inp["state_in"][si, h] / np.sqrt(D)
            np.testing.assert_allclose(o[cu[si]:cu[si + 1], h], ref, atol=2e-5)


def test_chunk_prefill_orthonormal_recall():
    """beta = 1, g = 0, orthonormal keys, no L2 norm: S^T k_i = v_i for every written key."""
    rng = np.random.default_rng(33)
    T = 100
    Qm, _ = np.linalg.qr(rng.standard_normal((D, D)))
    keys = Qm[:, :T].T.astype(np.float32)
    vals = rng.standard_normal((T, D)).astype(np.float32)
    x = np.concatenate([keys, keys, vals], axis=1)           # q | k | v, Hk = Hv = 1
    xd = f32_dev(x)
    q, k, v = qkv_views(xd, 1, 1)
    o = torch.empty((T, 1, D), device="cuda")
    s_out = torch.empty((1, 1, D, D), device="cuda")
    s_in = f32_dev(rng.standard_normal((1, 1, D, D)))
    gdn.gdn_chunk_prefill(q, k, v, None, None, None, None, o, 1, 1, None, s_in, s_out,
                          g_opt=f32_dev(np.zeros((T, 1))), beta_opt=f32_dev(np.ones((T, 1))),
                          use_qk_l2norm=False)
    torch.cuda.synchronize()
    S = host(s_out)[0, 0]
    np.testing.assert_allclose(keys.astype(np.float64) @ S, vals, atol=2e-4)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_explicit_output_scale(io):
    """A caller-given output scale (0.3, not 1/sqrt(dk)) in the chunked core, on the
    row-split sweep (bf16) and the 4-wave sweep (fp32), and in the decode step."""
    hk, hv, scale = 1, 2, 0.3
    inp = _case(hk, hv, io, 31, seqlens=[70, 5, 130], init_state=True)
    y_ref, _ = G.conv1d_fwd(inp["x"], inp["conv_w"], inp["cu_seqlens"], inp["conv_state_in"])
    y_io = G.to_io(y_ref, io).astype(np.float32)
    yd = to_dev(y_io, io)
    q, k, v = qkv_views(yd, hk, hv)
    N = inp["N"]
    o = torch.empty((N, hv, D), dtype=yd.dtype, device="cuda")
    s_out = torch.empty((inp["Ns"], hv, D, D), device="cuda")
    gdn.gdn_chunk_prefill(q, k, v, to_dev(inp["a"], io), to_dev(inp["b"], io),
                          f32_dev(inp["A_log"]), f32_dev(inp["dt_bias"]), o, hk, hv, _cu_dev(inp),
                          f32_dev(inp["state_in"]), s_out, scale=scale)
    torch.cuda.synchronize()
    y64 = y_io.astype(np.float64)
    o_ref, s_ref = G.prefill(y64[:, : hk * D], y64[:, hk * D: 2 * hk * D], y64[:, 2 * hk * D:],
                             inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], hk, hv, D, D,
                             inp["state_in"], inp["cu_seqlens"], scale=scale)
    assert_out(host(o), o_ref, io, "prefill o, scale 0.3")
    assert_state(host(s_out), s_ref, "prefill state, scale 0.3")

    dec = _case(hk, hv, io, 32, batch=5, init_state=True, kind="decode")
    x = to_dev(dec["x"], io)
    cs = to_dev(dec["conv_state_in"], io)
    st = f32_dev(dec["state_in"])
    od = torch.empty((5, hv, D), dtype=x.dtype, device="cuda")
    gdn.gdn_recurrent_step(x, f32_dev(dec["conv_w"]), cs, to_dev(dec["a"], io),
                           to_dev(dec["b"], io), f32_dev(dec["A_log"]), f32_dev(dec["dt_bias"]),
                           st, od, hk, hv, scale=scale)
    torch.cuda.synchronize()
    od_ref, _, st_ref = G.recurrent_step(dec["x"], dec["conv_w"], dec["conv_state_in"], dec["a"],
                                         dec["b"], dec["A_log"], dec["dt_bias"], dec["state_in"],
                                         hk, hv, D, D, scale=scale, io=io)
    assert_out(host(od), od_ref, io, "step o, scale 0.3", upstream_bf16=1)
    assert_state(host(st), st_ref, "step state, scale 0.3")


# ------------------------------------------------------------------------- decode step
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("hk,hv", [(2, 4), (2, 2), (1, 4), (1, 3)])
def test_recurrent_step_parity(io, hk, hv):
    inp = _case(hk, hv, io, 40 + hv, batch=7, init_state=True, kind="decode")
    B = 7
    x = to_dev(inp["x"], io)
    cs = to_dev(inp["conv_state_in"], io)
    st = f32_dev(inp["state_in"])
    o = torch.empty((B, hv, D), dtype=x.dtype, device="cuda")
    gdn.gdn_recurrent_step(x, f32_dev(inp["conv_w"]), cs, to_dev(inp["a"], io),
                           to_dev(inp["b"], io), f32_dev(inp["A_log"]), f32_dev(inp["dt_bias"]),
                           st, o, hk, hv)
    torch.cuda.synchronize()
    o_ref, cs_ref, st_ref = G.recurrent_step(inp["x"], inp["conv_w"], inp["conv_state_in"],
                                             inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                                             inp["state_in"], hk, hv, D, D, io=io)
    assert_out(host(o), o_ref, io, "step o", upstream_bf16=1)
    np.testing.assert_array_equal(host(cs), cs_ref)
    assert_state(host(st), st_ref, "step state")


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("hk,hv", [(2, 4), (1, 3)])
def test_recurrent_step_bf16_state_parity(io, hk, hv):
    """The step on a bf16-stored state: o as from the stored values, state rounded back."""
    inp = _case(hk, hv, io, 60 + hv, batch=5, init_state=True, kind="decode")
    B = 5
    s_bf = G.to_io(inp["state_in"], "bf16")
    x = to_dev(inp["x"], io)
    cs = to_dev(inp["conv_state_in"], io)
    st = to_dev(s_bf, "bf16")
    o = torch.empty((B, hv, D), dtype=x.dtype, device="cuda")
    gdn.gdn_recurrent_step(x, f32_dev(inp["conv_w"]), cs, to_dev(inp["a"], io),
                           to_dev(inp["b"], io), f32_dev(inp["A_log"]), f32_dev(inp["dt_bias"]),
                           st, o, hk, hv)
    torch.cuda.synchronize()
    assert st.dtype == torch.bfloat16
    o_ref, cs_ref, st_ref = G.recurrent_step(inp["x"], inp["conv_w"], inp["conv_state_in"],
                                             inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                                             s_bf, hk, hv, D, D, io=io, state_io="bf16")
    assert_out(host(o), o_ref, io, "bf16-state step o", upstream_bf16=1)
    np.testing.assert_array_equal(host(cs), cs_ref)
    assert_bf16_state(host(st), st_ref, "bf16-state step state", upstream_bf16=1)


def test_recurrent_step_bf16_state_many_steps():
    """24 steps on one bf16 state buffer against the oracle stepping a bf16 state."""
    io, hk, hv, B, n = "bf16", 2, 4, 3, 24
    rng = np.random.default_rng(71)
    inp = _case(hk, hv, io, 71, batch=B, init_state=True, kind="decode")
    C = (2 * hk + hv) * D
    xs = G.to_io(rng.standard_normal((n, B, C)), io)
    as_ = G.to_io(rng.standard_normal((n, B, hv)), io)
    bs = G.to_io(rng.standard_normal((n, B, hv)), io)
    w, A_log, dt = inp["conv_w"], inp["A_log"], inp["dt_bias"]
    s_ref = G.to_io(inp["state_in"], "bf16")
    cs_ref = inp["conv_state_in"]
    st = to_dev(s_ref, "bf16")
    cs = to_dev(cs_ref, io)
    wd, Ad, dd = f32_dev(w), f32_dev(A_log), f32_dev(dt)
    os_gpu, os_ref = [], []
    for t in range(n):
        o = torch.empty((B, hv, D), dtype=torch.bfloat16, device="cuda")
        gdn.gdn_recurrent_step(to_dev(xs[t], io), wd, cs, to_dev(as_[t], io), to_dev(bs[t], io),
                               Ad, dd, st, o, hk, hv)
        os_gpu.append(o)
        o_r, cs_ref, s_ref = G.recurrent_step(xs[t], w, cs_ref, as_[t], bs[t], A_log, dt, s_ref,
                                              hk, hv, D, D, io=io, state_io="bf16")
        os_ref.append(o_r)
    torch.cuda.synchronize()
    assert_out(np.stack([host(o) for o in os_gpu]), np.stack(os_ref), io, "bf16-state steps o", upstream_bf16=1)
    np.testing.assert_array_equal(host(cs), cs_ref)
    # One-ulp neighbours at one step carry into the next, so over many steps only the
    # Frobenius bound holds element-blind.
    assert_state(host(st), s_ref, "bf16-state steps state")


@pytest.mark.parametrize("state_io", ["f32", "bf16"])
def test_recurrent_step_slots_parity(state_io):
    """Slot-indexed decode: rows pick pool entries; padding rows touch nothing, o = 0."""
    io, hk, hv, B, n = "bf16", 2, 4, 5, 9
    rng = np.random.default_rng(90)
    inp = _case(hk, hv, io, 90, batch=B, init_state=True, kind="decode")
    C = (2 * hk + hv) * D
    conv_pool = G.to_io(rng.standard_normal((n, 3, C)), io)
    pool = G.to_io(0.02 * rng.standard_normal((n, hv, D, D)), state_io)
    slots = np.array([7, -1, 2, 12, 4], dtype=np.int32)
    cp = to_dev(conv_pool, io)
    sp = to_dev(pool, "bf16") if state_io == "bf16" else f32_dev(pool)
    o = torch.full((B, hv, D), 3.0, dtype=torch.bfloat16, device="cuda")
    gdn.gdn_recurrent_step_slots(to_dev(inp["x"], io), f32_dev(inp["conv_w"]), cp,
                                 to_dev(inp["a"], io), to_dev(inp["b"], io),
                                 f32_dev(inp["A_log"]), f32_dev(inp["dt_bias"]), sp,
                                 torch.from_numpy(slots).cuda(), o, hk, hv)
    torch.cuda.synchronize()
    o_ref, cp_ref, sp_ref = G.recurrent_step_slots(
        inp["x"], inp["conv_w"], conv_pool, inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
        pool, slots, hk, hv, D, D, io=io, state_io="bf16" if state_io == "bf16" else "f64")
    og = host(o)
    assert np.all(og[[1, 3]] == 0.0)
    assert_out(og, o_ref, io, "slot step o", upstream_bf16=1)
    np.testing.assert_array_equal(host(cp), cp_ref)
    spg = host(sp)
    live = [7, 2, 4]
    for s in sorted(set(range(n)) - set(live)):
        np.testing.assert_array_equal(spg[s], pool[s])
    if state_io == "bf16":
        assert_bf16_state(spg[live], sp_ref[live], "slot step bf16 state", upstream_bf16=1)
    else:
        assert_state(spg[live], sp_ref[live], "slot step state")


@pytest.mark.parametrize("io,state_io,hk,hv", [("bf16", "f32", 2, 4), ("bf16", "bf16", 2, 4),
                                              ("f32", "f32", 2, 4), ("bf16", "f32", 1, 3),
                                              ("f32", "bf16", 1, 3),
                                              # more value heads per key head than one z
                                              # row per thread: one head per pass (9) and
                                              # two per pass (18)
                                              ("bf16", "f32", 1, 9), ("f32", "f32", 1, 18)])
def test_recurrent_step_norm_parity(io, state_io, hk, hv):
    """The fused step + gated norm: y against the oracle's step -> norm, and o and the state
    bit for bit equal to the unfused step's (value heads two per pass, or one)."""
    B = 6
    inp = _case(hk, hv, io, 95, batch=B, init_state=True, kind="decode")
    rng = np.random.default_rng(95)
    z = G.to_io(rng.standard_normal((B, hv, D)), io)
    nw = 1.0 + 0.1 * rng.standard_normal(D)
    s0 = G.to_io(inp["state_in"], state_io)
    args = [f32_dev(inp["conv_w"]), None, to_dev(inp["a"], io), to_dev(inp["b"], io),
            f32_dev(inp["A_log"]), f32_dev(inp["dt_bias"])]
    x = to_dev(inp["x"], io)
    sdev = lambda: to_dev(s0, "bf16") if state_io == "bf16" else f32_dev(s0)
    # fused
    cs1, st1 = to_dev(inp["conv_state_in"], io), sdev()
    o1 = torch.empty((B, hv, D), dtype=x.dtype, device="cuda")
    y1 = torch.empty_like(o1)
    a1 = list(args)
    a1[1] = cs1
    gdn.gdn_recurrent_step_norm(x, *a1, st1, to_dev(z, io), f32_dev(nw), y1, hk, hv, o=o1)
    # unfused
    cs2, st2 = to_dev(inp["conv_state_in"], io), sdev()
    o2 = torch.empty_like(o1)
    a2 = list(args)
    a2[1] = cs2
    gdn.gdn_recurrent_step(x, *a2, st2, o2, hk, hv)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(st1, st2)
    assert torch.equal(cs1, cs2)
    o_ref, _, _ = G.recurrent_step(inp["x"], inp["conv_w"], inp["conv_state_in"], inp["a"],
                                   inp["b"], inp["A_log"], inp["dt_bias"], s0, hk, hv, D, D,
                                   io=io, state_io="bf16" if state_io == "bf16" else "f64")
    y_ref = G.gated_rmsnorm(G.to_io(o_ref, io), z, nw)
    assert_out(host(o1), o_ref, io, "fused step o", upstream_bf16=1)
    assert_out(host(y1), y_ref, io, "fused step y", upstream_bf16=2)


def test_step_entry_points_accept_an_empty_batch():
    """B = 0: every decode entry point returns without launching anything."""
    hk, hv = 2, 4
    C = (2 * hk + hv) * D
    e = torch.empty((0, C), dtype=torch.bfloat16, device="cuda")
    eh = torch.empty((0, hv), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((C, 4), device="cuda")
    hv_f = torch.zeros(hv, device="cuda")
    cs = torch.empty((1, 3, C), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros((1, hv, D, D), device="cuda")
    o = torch.empty((0, hv, D), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_recurrent_step(e, w, cs, eh, eh, hv_f, hv_f, st, o, hk, hv)
    gdn.gdn_recurrent_step_slots(e, w, cs, eh, eh, hv_f, hv_f, st,
                                 torch.empty(0, dtype=torch.int32, device="cuda"), o, hk, hv)
    gdn.gdn_recurrent_step_norm(e, w, cs, eh, eh, hv_f, hv_f, st, o, torch.ones(D, device="cuda"),
                                torch.empty_like(o), hk, hv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(st) == 0


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("ns", [1, 3])
def test_prefill_entry_points_accept_zero_tokens(io, ns):
    """N = 0: every sequence is empty, so the final recurrent and conv states equal the
    initial ones and nothing else is written (Ns = 1 without cu_seqlens, Ns = 3 with all
    offsets zero)."""
    hk, hv = 2, 4
    C = (2 * hk + hv) * D
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.empty((0, C), dtype=dt, device="cuda")
    y = torch.empty_like(x)
    ab = torch.empty((0, hv), dtype=dt, device="cuda")
    o = torch.empty((0, hv, D), dtype=dt, device="cuda")
    z = torch.empty_like(o)
    yn = torch.empty_like(o)
    w = torch.randn(C, 4, device="cuda", generator=g)
    hvf = torch.rand(hv, device="cuda", generator=g)
    nw = torch.ones(D, device="cuda")
    cu = None if ns == 1 else torch.zeros(ns + 1, dtype=torch.int32, device="cuda")
    s_in = torch.randn(ns, hv, D, D, device="cuda", generator=g)
    cs_in = torch.randn(ns, 3, C, device="cuda", generator=g).to(dt)
    q, k, v = qkv_views(y, hk, hv)
    calls = {
        "conv": lambda so, co: gdn.gdn_conv1d_fwd(x, w, y, cu, cs_in, co),
        "chunk": lambda so, co: gdn.gdn_chunk_prefill(q, k, v, ab, ab, hvf, hvf, o, hk, hv, cu,
                                                      s_in, so),
        "chunk_noalloc": lambda so, co: gdn.gdn_chunk_prefill_noalloc(
            q, k, v, ab, ab, hvf, hvf, o, hk, hv, cu, s_in, so),
        "conv_chunk": lambda so, co: gdn.gdn_conv_chunk_prefill(
            x, w, y, ab, ab, hvf, hvf, o, hk, hv, cu, cs_in, co, s_in, so),
        "layer": lambda so, co: gdn.gdn_prefill_layer(
            x, w, y, ab, ab, hvf, hvf, o, z, nw, yn, hk, hv, cu, cs_in, co, s_in, so),
    }
    for name, call in calls.items():
        s_out = torch.full_like(s_in, 7.0)
        cs_out = torch.full_like(cs_in, 7.0)
        call(s_out, cs_out)
        torch.cuda.synchronize()
        if name != "conv":
            assert torch.equal(s_out, s_in), f"{name}: recurrent state"
        if name not in ("chunk", "chunk_noalloc"):
            assert torch.equal(cs_out, cs_in), f"{name}: conv state"
    gdn.gdn_gated_rmsnorm(o, z, nw, yn)
    torch.cuda.synchronize()


def test_prefill_then_steps_equals_prefill():
    """Prefill of T1 tokens then T - T1 decode steps on carried state == prefill of T."""
    io = "bf16"
    hk, hv, T, T1 = 1, 2, 80, 70
    inp = _case(hk, hv, io, 50, seqlens=[T], init_state=False)
    ref = G.layer(inp)
    x = to_dev(inp["x"], io)
    w = f32_dev(inp["conv_w"])
    a, b = to_dev(inp["a"], io), to_dev(inp["b"], io)
    A_log, dt = f32_dev(inp["A_log"]), f32_dev(inp["dt_bias"])
    z = to_dev(inp["z"], io).view(T, hv, D)
    nw = f32_dev(inp["norm_w"])
    out = gdn.prefill_layer(x[:T1], w, a[:T1], b[:T1], A_log, dt, z[:T1], nw, hk, hv)
    cs, st = out["conv_state_out"], out["state_out"]
    ys = [host(out["y"])]
    for t in range(T1, T):
        r = gdn.decode_step(x[t:t + 1], w, cs, a[t:t + 1], b[t:t + 1], A_log, dt, st,
                            z[t:t + 1], nw, hk, hv)
        ys.append(host(r["y"]))
    torch.cuda.synchronize()
    assert_out(np.concatenate(ys), ref["y_exact"], io, "layer y", upstream_bf16=2)
    assert_state(host(st), ref["state_out"], "final state")
    np.testing.assert_array_equal(host(cs), ref["conv_state_out"])
