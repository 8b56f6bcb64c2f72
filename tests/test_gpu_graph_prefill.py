"""The prefill calls under HIP graph capture: gdn_prefill_layer (conv, chunked core and
gated norm in one call) and gdn_chunk_prefill_noalloc (the chunked core on the library's
fixed workspace, for callers that cannot allocate) captured once, with every buffer
allocated beforehand, then replayed several times with eager library calls, torch work
and synchronizations between the replays.  Every replay must equal the eager calls bit for
bit, also after the static inputs are overwritten with another input set (the graph reads
its buffers when it replays, not when it was captured)."""
import numpy as np
import pytest
import torch

import hybrid_linear_attention_causal_amd as gdn
from hybrid_linear_attention_causal_amd import synth
from hybrid_linear_attention_causal_amd.mixer import qkv_views

from parity import f32_dev, to_dev

pytestmark = pytest.mark.gpu

D = 128
HK, HV, IO = 2, 4, "bf16"
LENS = [1, 17, 63, 64, 65, 130, 0, 200, 5, 64, 129, 33]


def _inputs(seed):
    sh = synth.Shape(f"h{HK}x{HV}", hk=HK, hv=HV)
    inp = synth.make(synth.custom(sh, IO, seed, seqlens=LENS, init_state=True))
    d = {k: to_dev(inp[k], IO) for k in ("x", "a", "b", "conv_state_in", "z")}
    for k in ("conv_w", "A_log", "dt_bias", "state_in", "norm_w"):
        d[k] = f32_dev(inp[k])
    d["z"] = d["z"].view(inp["N"], HV, D)
    d["cu"] = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).cuda()
    return d


class Calls:
    """Static inputs and outputs of the two calls, and one pass of them on the current
    stream."""

    def __init__(self, d):
        self.inp = {k: v.clone() for k, v in d.items()}
        x = self.inp["x"]
        N, Ns = x.shape[0], self.inp["cu"].numel() - 1
        self.out = {
            "y_conv": torch.empty_like(x),
            "conv_state_out": torch.empty_like(self.inp["conv_state_in"]),
            "o": torch.empty((N, HV, D), dtype=x.dtype, device="cuda"),
            "y": torch.empty((N, HV, D), dtype=x.dtype, device="cuda"),
            "state_out": torch.empty((Ns, HV, D, D), device="cuda"),
            "o_na": torch.empty((N, HV, D), dtype=x.dtype, device="cuda"),
            "state_na": torch.empty((Ns, HV, D, D), device="cuda"),
        }
        self.ws = torch.empty(gdn.gdn_chunk_prefill_workspace_size(N, Ns, HK, HV, io=x.dtype),
                              dtype=torch.uint8, device="cuda")

    def load(self, d):
        for k, v in d.items():
            self.inp[k].copy_(v)

    def run(self):
        i, o = self.inp, self.out
        gdn.gdn_prefill_layer(i["x"], i["conv_w"], o["y_conv"], i["a"], i["b"], i["A_log"],
                              i["dt_bias"], o["o"], i["z"], i["norm_w"], o["y"], HK, HV, i["cu"],
                              i["conv_state_in"], o["conv_state_out"], i["state_in"],
                              o["state_out"], workspace=self.ws)
        # the chunked core again on the raw rows, on the fixed workspace
        q, k, v = qkv_views(i["x"], HK, HV)
        gdn.gdn_chunk_prefill_noalloc(q, k, v, i["a"], i["b"], i["A_log"], i["dt_bias"],
                                      o["o_na"], HK, HV, i["cu"], i["state_in"], o["state_na"])

    def snapshot(self):
        return {k: v.clone() for k, v in self.out.items()}


def test_prefill_graph_replays_equal_eager():
    d1, d2 = _inputs(120), _inputs(121)
    calls = Calls(d1)
    eager = []
    for d in (d1, d2):
        calls.load(d)
        calls.run()
        torch.cuda.synchronize()
        eager.append(calls.snapshot())
    assert not torch.equal(eager[0]["o"], eager[1]["o"])

    calls.load(d1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls.run()
    torch.cuda.synchronize()

    other = Calls(d2)      # eager calls between the replays, on buffers of their own
    for rep, which in enumerate((0, 0, 1, 0)):
        calls.load((d1, d2)[which])
        for v in calls.out.values():
            v.fill_(7.0)           # every output is rewritten by the replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, ref in eager[which].items():
            assert torch.equal(calls.out[k], ref), f"replay {rep} (input set {which}): {k}"
        # eager library work between replays, including the no-allocation call that shares
        # the fixed workspace with the graph
        other.run()
        torch.cuda.synchronize()
        for k, ref in eager[1].items():
            assert torch.equal(other.out[k], ref), f"eager call after replay {rep}: {k}"
