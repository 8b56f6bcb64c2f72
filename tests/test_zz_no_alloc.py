"""gdn_chunk_prefill_noalloc (the chunked prefill on the library's fixed device workspace,
for callers that cannot allocate) against gdn_chunk_prefill with a caller workspace: o
and the final recurrent state bit for bit (the same kernels run), on calls in a row with
the later ones smaller (the fixed workspace keeps each call's contents for the next)."""
import numpy as np
import pytest
import torch

import hybrid_linear_attention_causal_amd as gdn
from hybrid_linear_attention_causal_amd import synth
from hybrid_linear_attention_causal_amd._lib import GdnError
from hybrid_linear_attention_causal_amd.mixer import qkv_views

from parity import f32_dev, to_dev

pytestmark = pytest.mark.gpu

D = 128
LENS = [1, 17, 63, 64, 65, 130, 0, 200, 5, 64, 129, 33]


def _case(hk, hv, io, seed, lens, init_state):
    sh = synth.Shape(f"h{hk}x{hv}", hk=hk, hv=hv)
    inp = synth.make(synth.custom(sh, io, seed, seqlens=lens, init_state=init_state))
    d = {"x": to_dev(inp["x"], io), "a": to_dev(inp["a"], io), "b": to_dev(inp["b"], io),
         "A_log": f32_dev(inp["A_log"]), "dt_bias": f32_dev(inp["dt_bias"]),
         "state_in": f32_dev(inp["state_in"]),
         "cu": None if len(lens) == 1 else
         torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).cuda()}
    return inp, d


def _both(hk, hv, d):
    """The no-alloc call first, then the workspace call, on the same inputs."""
    q, k, v = qkv_views(d["x"], hk, hv)      # raw rows serve as q, k, v
    N = d["x"].shape[0]
    Ns = 1 if d["cu"] is None else d["cu"].numel() - 1
    outs = []
    for noalloc in (True, False):
        o = torch.full((N, hv, D), 5.0, dtype=d["x"].dtype, device="cuda")
        s_out = torch.full((Ns, hv, D, D), 5.0, device="cuda")
        fn = gdn.gdn_chunk_prefill_noalloc if noalloc else gdn.gdn_chunk_prefill
        fn(q, k, v, d["a"], d["b"], d["A_log"], d["dt_bias"], o, hk, hv, d["cu"], d["state_in"],
           s_out)
        outs.append((o, s_out))
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_noalloc_equals_workspace_call_twice(io):
    # a large call (9B shape, T=2048: row-split sweep for bf16), then a smaller packed one
    # with ragged and empty sequences and carried states
    for hk, hv, lens, init in ((16, 32, [2048], False), (2, 4, LENS, True)):
        inp, d = _case(hk, hv, io, 60 + hk, lens, init)
        (o1, s1), (o2, s2) = _both(hk, hv, d)
        assert torch.equal(o1, o2), f"o ({hk}x{hv}, {len(lens)} sequences)"
        assert torch.equal(s1, s2), f"state ({hk}x{hv}, {len(lens)} sequences)"
        assert torch.isfinite(o1.float()).all()


def test_noalloc_rejects_sizes_beyond_its_workspace():
    hk, hv, N = 16, 32, 8192
    need = gdn.gdn_chunk_prefill_workspace_size(N, 1, hk, hv, io=torch.bfloat16)
    assert need > (128 << 20)
    x = torch.zeros((N, (2 * hk + hv) * D), dtype=torch.bfloat16, device="cuda")
    q, k, v = qkv_views(x, hk, hv)
    a = torch.zeros((N, hv), dtype=torch.bfloat16, device="cuda")
    p = torch.zeros(hv, device="cuda")
    o = torch.empty((N, hv, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(GdnError, match="workspace"):
        gdn.gdn_chunk_prefill_noalloc(q, k, v, a, a, p, p, o, hk, hv)
