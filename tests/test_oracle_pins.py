"""Pins for the fp64 oracle, checked against things other than the oracle itself:
hand-worked examples, library routines, closed forms and invariants.
CPU only."""
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import checkers
from oracle import gdn_oracle as G

HERE = os.path.dirname(os.path.abspath(__file__))


def _rng(seed):
    return np.random.default_rng(seed)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------- golden hand examples
def _load_delta_fixture():
    rows, S = [], []
    with open(os.path.join(HERE, "golden", "delta_rule_hand_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("S "):
                S.append([float(t) for t in line.split()[1:]])
                continue
            lhs, rhs = line.split("|")
            rows.append(([float(t) for t in lhs.split()], [float(t) for t in rhs.split()]))
    return rows, np.array(S)


def test_delta_rule_hand_example():
    rows, S_ref = _load_delta_fixture()
    k = np.array([r[0][1:3] for r in rows])
    v = np.array([r[0][3:6] for r in rows])
    beta = np.array([r[0][6] for r in rows])
    g = np.log(np.array([r[0][7] for r in rows]))
    q = np.array([r[0][8:10] for r in rows])
    o_ref = np.array([r[1] for r in rows])
    o, S = G.delta_rule(q, k, v, g, beta, np.zeros((2, 3)), 1.0)
    np.testing.assert_allclose(o, o_ref, atol=1e-14)
    np.testing.assert_allclose(S, S_ref, atol=1e-14)
    # the same chain through the packed entry point with the default scale 1/sqrt(dk)
    o2, S2 = G.prefill(q, k, v, None, None, None, None, 1, 1, 2, 3, use_qk_l2norm=False,
                       g=g[:, None], beta=beta[:, None])
    np.testing.assert_allclose(o2[:, 0], o_ref / np.sqrt(2.0), atol=1e-14)
    np.testing.assert_allclose(S2[0, 0], S_ref, atol=1e-14)


def _load_conv_fixture():
    d = {}
    with open(os.path.join(HERE, "golden", "conv_hand_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lab, vals = line.split("|")
            d[lab.strip()] = np.array([float(t) for t in vals.split()])
    return d


def test_conv_hand_example():
    d = _load_conv_fixture()
    w = d["w"][None, :]
    x = d["x"][:, None]
    y, st = G.conv1d_fwd(x, w)
    np.testing.assert_allclose(y[:, 0], scipy.special.expit(d["p_zero"]) * d["p_zero"], rtol=1e-15)
    np.testing.assert_allclose(st[0, :, 0], d["state_out"])
    y, st = G.conv1d_fwd(x, w, None, d["state_in"][None, :, None])
    np.testing.assert_allclose(y[:, 0], scipy.special.expit(d["p_state"]) * d["p_state"], rtol=1e-15)
    np.testing.assert_allclose(st[0, :, 0], d["state_out"])


# ---------------------------------------------------------------- conv vs library routine
def test_conv_matches_np_convolve():
    rng = _rng(1)
    L, C = 23, 7
    x = rng.standard_normal((L, C))
    w = rng.standard_normal((C, 4))
    hist = rng.standard_normal((1, 3, C))
    y, st = G.conv1d_fwd(x, w, None, hist)
    for c in range(C):
        xpad = np.concatenate([hist[0, :, c], x[:, c]])
        pre = np.convolve(xpad, w[c, ::-1], mode="valid")     # convolution = flipped correlation
        np.testing.assert_allclose(y[:, c], pre * scipy.special.expit(pre), rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(st[0], x[-3:])


def test_conv_one_hot_taps():
    rng = _rng(2)
    x = rng.standard_normal((10, 5))
    w = np.zeros((5, 4))
    w[:, 3] = 1.0
    y, _ = G.conv1d_fwd(x, w)
    np.testing.assert_allclose(y, x * scipy.special.expit(x), rtol=1e-15)
    w = np.zeros((5, 4))
    w[:, 0] = 1.0                       # three-token delay
    y, _ = G.conv1d_fwd(x, w)
    np.testing.assert_array_equal(y[:3], 0.0)
    np.testing.assert_allclose(y[3:], x[:-3] * scipy.special.expit(x[:-3]), rtol=1e-15)


def test_conv_short_sequence_state():
    # a 1-token sequence: the new state keeps two rows of the old state
    rng = _rng(3)
    x = rng.standard_normal((1, 4))
    hist = rng.standard_normal((1, 3, 4))
    _, st = G.conv1d_fwd(x, rng.standard_normal((4, 4)), None, hist)
    np.testing.assert_array_equal(st[0, :2], hist[0, 1:])
    np.testing.assert_array_equal(st[0, 2], x[0])


def test_conv_varlen_and_split_invariance():
    rng = _rng(4)
    lens = [5, 1, 17, 2, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    C = 6
    x = rng.standard_normal((cu[-1], C))
    w = rng.standard_normal((C, 4))
    hist = rng.standard_normal((len(lens), 3, C))
    y, st = G.conv1d_fwd(x, w, cu, hist)
    for s in range(len(lens)):
        ys, sts = G.conv1d_fwd(x[cu[s]:cu[s + 1]], w, None, hist[s:s + 1])
        np.testing.assert_array_equal(y[cu[s]:cu[s + 1]], ys)
        np.testing.assert_array_equal(st[s], sts[0])
    # a sequence cut in two with the conv state carried gives the same outputs
    xs = x[cu[2]:cu[3]]
    y1, s1 = G.conv1d_fwd(xs[:7], w, None, hist[2:3])
    y2, s2 = G.conv1d_fwd(xs[7:], w, None, s1)
    np.testing.assert_allclose(np.concatenate([y1, y2]), y[cu[2]:cu[3]], rtol=1e-15)
    np.testing.assert_array_equal(s2[0], st[2])


# ---------------------------------------------------------------- gates, norms, rounding
def test_gates_vs_library():
    rng = _rng(5)
    a = rng.standard_normal((50, 8)) * 10
    b = rng.standard_normal((50, 8)) * 10
    A_log = rng.uniform(0, np.log(16), 8)
    dt_bias = np.log(np.expm1(rng.uniform(1e-3, 0.1, 8)))
    g, beta = G.gates(a, b, A_log, dt_bias)
    sp = -scipy.special.log_expit(-(a + dt_bias))          # softplus
    np.testing.assert_allclose(g, -np.exp(A_log) * sp, rtol=1e-13)
    np.testing.assert_allclose(beta, scipy.special.expit(b), rtol=1e-14)
    assert np.all(g <= 0) and np.all((beta > 0) & (beta < 1))


def test_l2_norm_invariant():
    rng = _rng(6)
    x = rng.standard_normal((40, 128)) * rng.uniform(0.01, 10, (40, 1))
    xn = G.l2_normalize(x)
    s = np.sum(x * x, axis=1)
    np.testing.assert_allclose(np.sum(xn * xn, axis=1), s / (s + 1e-6), rtol=1e-13)
    # direction preserved: equals torch's normalize up to the eps factor
    tn = torch.nn.functional.normalize(torch.from_numpy(x), dim=-1).numpy()
    np.testing.assert_allclose(xn * np.sqrt((s + 1e-6) / s)[:, None], tn, rtol=1e-12)


def test_bf16_round_matches_torch():
    rng = _rng(7)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # exact ties: bf16 value plus half an ulp
    base = torch.from_numpy(x[:1000]).to(torch.bfloat16).float().numpy()
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(G.bf16_round(x), ref)


def test_gated_rmsnorm_vs_torch_rms_norm():
    rng = _rng(8)
    o = rng.standard_normal((33, 128)) * 3
    z = rng.standard_normal((33, 128))
    w = 1 + 0.1 * rng.standard_normal(128)
    y = G.gated_rmsnorm(o, z, w)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (128,), torch.from_numpy(w), eps=1e-6)
    gate = z * scipy.special.expit(z)
    np.testing.assert_allclose(y, ref.numpy() * gate, rtol=1e-12, atol=1e-14)
    # invariant: removing weight and gate leaves unit mean square up to eps
    ms = np.mean(o * o, axis=1)
    np.testing.assert_allclose(np.mean((y / (w * gate)) ** 2, axis=1), ms / (ms + 1e-6), rtol=1e-11)


# ---------------------------------------------------------------- the recurrence
def _random_chain(seed, L, dk, dv, strong_decay=False):
    rng = _rng(seed)
    q = _unit_rows(rng.standard_normal((L, dk)))
    k = _unit_rows(rng.standard_normal((L, dk)))
    v = rng.standard_normal((L, dv))
    if strong_decay:
        g = -rng.exponential(3.0, L)
        g[rng.integers(0, L, max(1, L // 10))] = -25.0
    else:
        g = -rng.uniform(0, 0.5, L)
    beta = rng.uniform(0.05, 0.95, L)
    S0 = 0.3 * rng.standard_normal((dk, dv))
    return q, k, v, g, beta, S0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_recurrent_vs_closed_form(seed):
    q, k, v, g, beta, S0 = _random_chain(seed, 12, 3, 5)
    o, S = G.delta_rule(q, k, v, g, beta, S0, 0.7)
    o2, S2 = checkers.closed_form(q, k, v, g, beta, S0, 0.7)
    np.testing.assert_allclose(o, o2, atol=1e-12)
    np.testing.assert_allclose(S, S2, atol=1e-12)


@pytest.mark.parametrize("strong", [False, True])
@pytest.mark.parametrize("chunk", [64, 16])
def test_chunked_ut_vs_recurrent(strong, chunk):
    q, k, v, g, beta, S0 = _random_chain(10 + chunk, 200, 16, 24, strong)
    o, S = G.delta_rule(q, k, v, g, beta, S0, 0.25)
    o2, S2 = checkers.chunked_ut(q, k, v, g, beta, S0, 0.25, chunk)
    assert np.all(np.isfinite(o2))
    np.testing.assert_allclose(o2, o, atol=1e-11 * np.abs(o).max())
    np.testing.assert_allclose(S2, S, atol=1e-11 * np.abs(S).max())


def test_invariant_no_write_no_decay():
    q, k, v, g, beta, S0 = _random_chain(20, 30, 8, 6)
    o, S = G.delta_rule(q, k, v, np.zeros(30), np.zeros(30), S0, 0.5)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, 0.5 * q @ S0, rtol=1e-14)


def test_invariant_decay_only():
    q, k, v, g, beta, S0 = _random_chain(21, 30, 8, 6)
    _, S = G.delta_rule(q, k, v, g, np.zeros(30), S0, 0.5)
    np.testing.assert_allclose(S, np.exp(np.sum(g)) * S0, rtol=1e-13)


@pytest.mark.parametrize("zero_start", [True, False])
def test_invariant_orthonormal_recall(zero_start):
    rng = _rng(22)
    dk, dv, L = 16, 10, 16
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, :L].T                        # orthonormal rows
    v = rng.standard_normal((L, dv))
    S0 = np.zeros((dk, dv)) if zero_start else rng.standard_normal((dk, dv))
    _, S = G.delta_rule(k, k, v, np.zeros(L), np.ones(L), S0, 1.0)
    np.testing.assert_allclose(k @ S, v, atol=1e-13)


def test_head_mapping_is_grouped():
    # Hk = 2, Hv = 4: value heads 0,1 read key head 0 and heads 2,3 read key head 1.
    rng = _rng(23)
    L, d = 9, 4
    q = rng.standard_normal((L, 2 * d))
    k = rng.standard_normal((L, 2 * d))
    k[:, d:] = 0.0                         # key head 1 never writes
    v = rng.standard_normal((L, 4 * d))
    o, S = G.prefill(q, k, v, rng.standard_normal((L, 4)), rng.standard_normal((L, 4)),
                     np.zeros(4), np.zeros(4), 2, 4, d, d)
    assert np.all(np.abs(o[:, 0:2]).max(axis=(1, 2))[1:] > 0)
    np.testing.assert_array_equal(o[:, 2:4], 0.0)
    np.testing.assert_array_equal(S[0, 2:4], 0.0)


def test_qkv_channel_slots():
    # zeroing q, k or v channels of the packed input pins which slot each one reads
    rng = _rng(24)
    L, hk, hv, d = 12, 1, 2, 4
    x = rng.standard_normal((L, 2 * hk * d + hv * d))
    w = rng.standard_normal((x.shape[1], 4))
    base = dict(io="f32", Hk=hk, Hv=hv, dk=d, dv=d, conv_w=w, cu_seqlens=None,
                conv_state_in=None, state_in=None, a=rng.standard_normal((L, hv)),
                b=rng.standard_normal((L, hv)), A_log=np.zeros(hv), dt_bias=np.zeros(hv),
                z=rng.standard_normal((L, hv * d)), norm_w=np.ones(d))
    full = G.layer(dict(base, x=x))
    assert np.abs(full["o"]).max() > 0 and np.abs(full["state_out"]).max() > 0
    xq = x.copy()
    xq[:, :hk * d] = 0
    r = G.layer(dict(base, x=xq))
    np.testing.assert_array_equal(r["o"], 0.0)
    np.testing.assert_allclose(r["state_out"], full["state_out"], rtol=1e-15)
    xk = x.copy()
    xk[:, hk * d:2 * hk * d] = 0
    r = G.layer(dict(base, x=xk))
    np.testing.assert_array_equal(r["state_out"], 0.0)
    xv = x.copy()
    xv[:, 2 * hk * d:] = 0
    r = G.layer(dict(base, x=xv))
    np.testing.assert_array_equal(r["state_out"], 0.0)
    np.testing.assert_array_equal(r["o"], 0.0)


def test_prefill_varlen_and_split_invariance():
    rng = _rng(25)
    lens = [3, 70, 1, 130]
    cu = np.concatenate([[0], np.cumsum(lens)])
    n, hk, hv, d = cu[-1], 1, 2, 8
    q = rng.standard_normal((n, hk * d))
    k = rng.standard_normal((n, hk * d))
    v = rng.standard_normal((n, hv * d))
    a = rng.standard_normal((n, hv))
    b = rng.standard_normal((n, hv))
    A_log = rng.uniform(0, np.log(16), hv)
    dt = np.log(np.expm1(rng.uniform(1e-3, 0.1, hv)))
    S0 = 0.1 * rng.standard_normal((len(lens), hv, d, d))
    o, S = G.prefill(q, k, v, a, b, A_log, dt, hk, hv, d, d, S0, cu)
    for s in range(len(lens)):
        sl = slice(cu[s], cu[s + 1])
        os_, Ss = G.prefill(q[sl], k[sl], v[sl], a[sl], b[sl], A_log, dt, hk, hv, d, d,
                            S0[s:s + 1])
        np.testing.assert_array_equal(o[sl], os_)
        np.testing.assert_array_equal(S[s], Ss[0])
    # cut sequence 3 at token 50 and carry the state
    sl = slice(cu[3], cu[4])
    qa, ka, va, aa, ba = q[sl], k[sl], v[sl], a[sl], b[sl]
    o1, S1 = G.prefill(qa[:50], ka[:50], va[:50], aa[:50], ba[:50], A_log, dt, hk, hv, d, d,
                       S0[3:4])
    o2, S2 = G.prefill(qa[50:], ka[50:], va[50:], aa[50:], ba[50:], A_log, dt, hk, hv, d, d, S1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o[sl], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S2[0], S[3], rtol=1e-12, atol=1e-14)


def test_decode_steps_equal_prefill():
    # prefill of T tokens == prefill of T1 tokens, then T - T1 single-token steps
    rng = _rng(26)
    T, T1, hk, hv, d = 11, 6, 1, 2, 4
    cq = 2 * hk * d + hv * d
    x = rng.standard_normal((T, cq))
    w = 0.25 * rng.standard_normal((cq, 4))
    a = rng.standard_normal((T, hv))
    b = rng.standard_normal((T, hv))
    A_log = rng.uniform(0, np.log(16), hv)
    dt = np.log(np.expm1(rng.uniform(1e-3, 0.1, hv)))
    z = rng.standard_normal((T, hv * d))
    base = dict(io="f32", Hk=hk, Hv=hv, dk=d, dv=d, conv_w=w, cu_seqlens=None,
                A_log=A_log, dt_bias=dt, norm_w=np.ones(d))
    full = G.layer(dict(base, x=x, a=a, b=b, z=z, conv_state_in=None, state_in=None))
    part = G.layer(dict(base, x=x[:T1], a=a[:T1], b=b[:T1], z=z[:T1], conv_state_in=None,
                        state_in=None))
    cs, st = part["conv_state_out"], part["state_out"]
    for t in range(T1, T):
        o, cs, st = G.recurrent_step(x[t:t + 1], w, cs, a[t:t + 1], b[t:t + 1], A_log, dt, st,
                                     hk, hv, d, d, io="f32")
        np.testing.assert_allclose(G.to_io(o[0], "f32"), full["o"][t], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(st, full["state_out"], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(cs, full["conv_state_out"])


def _step_inputs(rng, hk, hv, d, bsz):
    cq = 2 * hk * d + hv * d
    return dict(x=rng.standard_normal((bsz, cq)), w=0.25 * rng.standard_normal((cq, 4)),
                cs=rng.standard_normal((bsz, 3, cq)), a=rng.standard_normal((bsz, hv)),
                b=rng.standard_normal((bsz, hv)), A_log=rng.uniform(0, np.log(16), hv),
                dt=np.log(np.expm1(rng.uniform(1e-3, 0.1, hv))))


def test_bf16_state_step_pass_through():
    # beta = 0, g = 0: the bf16-stored state comes back bit for bit (a bf16 value rounds to
    # itself) and o = scale S0^T q^ reads the stored values
    rng = _rng(27)
    hk, hv, d, bsz = 1, 2, 8, 3
    p = _step_inputs(rng, hk, hv, d, bsz)
    S0 = G.to_io(0.02 * rng.standard_normal((bsz, hv, d, d)), "bf16")
    zeros = np.zeros((bsz, hv))
    o, _, S1 = G.recurrent_step(p["x"], p["w"], p["cs"], p["a"], p["b"], p["A_log"], p["dt"], S0,
                                hk, hv, d, d, io="f32", g=zeros, beta=zeros, state_io="bf16")
    np.testing.assert_array_equal(S1, S0)
    y, _ = G.conv1d_fwd(p["x"], p["w"], np.arange(bsz + 1), p["cs"])
    q = G.l2_normalize(G.to_io(y, "f32")[:, :d])
    for s in range(bsz):
        for h in range(hv):
            np.testing.assert_allclose(o[s, h], S0[s, h].T @ q[s] / np.sqrt(d), rtol=1e-12,
                                       atol=1e-15)


def test_bf16_state_step_is_the_step_rounded():
    # the bf16-state step: o equal to the full-precision step's from the same stored state,
    # and the written state within half a bf16 ulp of the full-precision one (RNE)
    rng = _rng(28)
    hk, hv, d, bsz = 2, 4, 8, 2
    p = _step_inputs(rng, hk, hv, d, bsz)
    S0 = G.to_io(0.02 * rng.standard_normal((bsz, hv, d, d)), "bf16")
    args = (p["x"], p["w"], p["cs"], p["a"], p["b"], p["A_log"], p["dt"], S0, hk, hv, d, d)
    o_f, cs_f, S_f = G.recurrent_step(*args, io="bf16")
    o_b, cs_b, S_b = G.recurrent_step(*args, io="bf16", state_io="bf16")
    np.testing.assert_array_equal(o_b, o_f)
    np.testing.assert_array_equal(cs_b, cs_f)
    assert np.all(np.abs(S_b - S_f) <= 2.0 ** -8 * np.abs(S_f) * (1 + 2.0 ** -15))
    assert np.array_equal(G.to_io(S_b, "bf16"), S_b)          # representable in bf16
    assert not np.array_equal(S_b, S_f)                          # and actually rounded


def test_slot_step_picks_pool_entries():
    # Row i of a slot-indexed batch is the single-sequence step of pool entry slots[i];
    # a padding row (negative or out-of-range slot) yields o = 0; untouched entries and
    # padding leave the pools bit for bit as they were.
    rng = _rng(31)
    hk, hv, d, bsz, n = 1, 2, 8, 4, 6
    p = _step_inputs(rng, hk, hv, d, bsz)
    cq = 2 * hk * d + hv * d
    conv_pool = rng.standard_normal((n, 3, cq))
    pool = 0.05 * rng.standard_normal((n, hv, d, d))
    slots = np.array([4, -1, 0, 9])
    o, cp, sp = G.recurrent_step_slots(p["x"], p["w"], conv_pool, p["a"], p["b"], p["A_log"],
                                       p["dt"], pool, slots, hk, hv, d, d, io="f32")
    for i, s in enumerate(slots):
        if not 0 <= s < n:
            assert np.all(o[i] == 0.0)
            continue
        o1, c1, s1 = G.recurrent_step(p["x"][i:i + 1], p["w"], conv_pool[s:s + 1],
                                      p["a"][i:i + 1], p["b"][i:i + 1], p["A_log"], p["dt"],
                                      pool[s:s + 1], hk, hv, d, d, io="f32")
        np.testing.assert_array_equal(o[i], o1[0])
        np.testing.assert_array_equal(cp[s], c1[0])
        np.testing.assert_array_equal(sp[s], s1[0])
    for s in sorted(set(range(n)) - {4, 0}):
        np.testing.assert_array_equal(cp[s], conv_pool[s])
        np.testing.assert_array_equal(sp[s], pool[s])
    # the pools themselves are not modified
    assert not np.shares_memory(sp, pool)
    # a slot-indexed step changes its entries: the pin would catch a no-op gather
    assert np.abs(sp[4] - pool[4]).max() > 1e-3
