"""CPU check of the bf16 tolerance reasoning in tests/parity.py, using the oracle only:
a value computed from a bf16 call output (the gated norm of o) moves by more than its
own half-ulp when o itself differs by one bf16 ulp -- which independent fp32 and fp64
evaluations of o produce wherever o straddles a rounding boundary -- and stays within
the 3 * 2^-8 slack used for such downstream values; and a decode step's bf16 state,
whose k and v are rounded inside the call, needs the same allowance on a few elements."""
import numpy as np
import pytest

from hybrid_linear_attention_causal_amd import synth
from oracle import gdn_oracle as G
from parity import assert_bf16_state, out_error


def test_one_ulp_input_flips_need_the_downstream_slack():
    rng = np.random.default_rng(0)
    rows, D = 20000, 128
    o = G.bf16_round(rng.standard_normal((rows, D)) * np.exp(rng.uniform(-3, 1, (rows, 1))) * 0.01)
    z = G.bf16_round(rng.standard_normal((rows, D)))
    w = 1 + 0.1 * rng.standard_normal(D)
    y_ref = G.to_io(G.gated_rmsnorm(o, z, w), "bf16")
    bits = o.astype(np.float32).view(np.uint32).copy()
    flip = rng.random(bits.shape) < 0.01
    step = np.where(rng.random(int(flip.sum())) < 0.5, 1, -1).astype(np.int64) << 16
    bits[flip] = (bits[flip].astype(np.int64) + step).astype(np.uint32)
    y_flip = G.to_io(G.gated_rmsnorm(bits.view(np.float32).astype(np.float64), z, w), "bf16")
    err0, bound = out_error(y_flip, y_ref, "bf16", upstream_bf16=0)
    err1, _ = out_error(y_flip, y_ref, "bf16", upstream_bf16=1)
    assert err0 > bound          # a single-rounding slack would reject a correct kernel
    assert err1 < 0.5 * bound    # the downstream slack absorbs one-ulp input flips


def test_a_call_output_is_compared_before_the_oracles_rounding():
    """A GPU output is its fp32 value rounded once to bf16.  Against the oracle's fp64
    value before rounding, that store moves it by at most half an ulp, inside the 2^-8
    slack; against the oracle's value after its own rounding, values whose fp32 and fp64
    forms straddle a rounding midpoint sit one full ulp apart, which exceeds the bound at
    values of about ten times the RMS (the reading of the 2^-8 term: it is the GPU's store,
    which the fp64 reference does not have)."""
    rng = np.random.default_rng(1)
    o64 = rng.standard_normal(200000) * 3e-3
    # fp32 arithmetic: relative errors of a few ulp of fp32
    o32 = o64 * (1 + 3e-7 * rng.standard_normal(o64.size))
    # twenty values just above 2^-5 (about ten times the RMS), each next to a bf16 rounding
    # midpoint, the fp64 value a few fp32 ulp (3.7e-9 here) below it and the fp32 value as
    # far above
    mid = 2.0 ** -5 * (1 + (np.arange(20) + 1.5) * 2.0 ** -7)
    o64[:20] = mid - 1e-8
    o32[:20] = mid + 1e-8
    gpu = G.bf16_round(o32)
    err_exact, bound = out_error(gpu, o64, "bf16")
    err_rounded, _ = out_error(gpu, G.bf16_round(o64), "bf16")
    assert err_exact < 0.05 * bound
    assert err_rounded > bound


def test_a_conv_output_flip_moves_a_bf16_state_column():
    """A decode step rounds its conv output to bf16 inside the call.  One v value one ulp
    off there (fp32 and fp64 conv values on either side of a rounding boundary) moves
    column j of the updated state by beta k_i times that ulp: past the state's own
    rounding bound on some elements, which a correct kernel must still pass, and within the
    io outputs' 3e-2 RMS bound that the step's bf16 state is held to on those few elements.
    A wrong element of 5e-2 RMS still fails it."""
    hk, hv, B, D = 1, 2, 3, 128
    inp = synth.make(synth.custom(synth.Shape("h1x2", hk=hk, hv=hv), "bf16", 7, batch=B,
                                  init_state=True, kind="decode"))
    s0 = G.to_io(inp["state_in"], "bf16")
    y, _ = G.conv1d_fwd(inp["x"], inp["conv_w"], np.arange(B + 1), inp["conv_state_in"])
    y = G.to_io(y, "bf16")

    def step(yv):
        q, k, v = yv[:, :hk * D], yv[:, hk * D:2 * hk * D], yv[:, 2 * hk * D:]
        _, s = G.prefill(q, k, v, inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], hk, hv,
                         D, D, s0, np.arange(B + 1))
        return G.to_io(s, "bf16")

    ref = step(y)
    # the largest v value of sequence 1, one bf16 ulp up
    c = 2 * hk * D + int(np.argmax(np.abs(y[1, 2 * hk * D:])))
    yf = y.copy()
    bits = np.array([yf[1, c]], dtype=np.float32).view(np.uint32)
    yf[1, c] = float((bits + np.uint32(1 << 16)).view(np.float32)[0])
    flipped = step(yf)
    with pytest.raises(AssertionError, match="exceeds the rounding bound"):
        assert_bf16_state(flipped, ref, "strict")
    assert_bf16_state(flipped, ref, "upstream", upstream_bf16=1)
    rms = float(np.sqrt(np.mean(ref * ref)))
    wrong = flipped.copy()
    wrong[0, 0, 5, 7] += 5e-2 * rms
    with pytest.raises(AssertionError, match="RMS"):
        assert_bf16_state(wrong, ref, "planted", upstream_bf16=1)
