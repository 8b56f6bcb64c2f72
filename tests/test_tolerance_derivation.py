"""CPU check of the bf16 tolerance reasoning in tests/parity.py, using the oracle only:
a value computed from a bf16 call output (the gated norm of o) moves by more than its
own half-ulp when o itself differs by one bf16 ulp -- which independent fp32 and fp64
evaluations of o produce wherever o straddles a rounding boundary -- and stays within
the 3 * 2^-8 slack used for such downstream values."""
import numpy as np

from oracle import gdn_oracle as G
from parity import out_error


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
