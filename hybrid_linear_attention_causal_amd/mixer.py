"""Thin helpers that allocate outputs with torch and chain the libgdn calls.

prefill_layer:  conv1d+SiLU -> chunked delta rule -> z-gated RMSNorm (one call by default)
decode_step:    recurrent step (conv + delta rule, in place) + z-gated RMSNorm, fused in one
                launch by default
DecodeGraph:    n decode steps captured once as a HIP graph, replayed as one launch
"""
from __future__ import annotations

import torch

from ._lib import (gdn_chunk_prefill, gdn_chunk_prefill_workspace_size, gdn_conv1d_fwd,
                   gdn_gated_rmsnorm, gdn_prefill_layer, gdn_recurrent_step,
                   gdn_recurrent_step_norm)

D = 128


def qkv_views(y: torch.Tensor, Hk: int, Hv: int):
    """Row views of the packed conv output: q | k | v, head-major inside each."""
    return y[:, : Hk * D], y[:, Hk * D: 2 * Hk * D], y[:, 2 * Hk * D: 2 * Hk * D + Hv * D]


def prefill_layer(x, conv_w, a, b, A_log, dt_bias, z, norm_w, Hk, Hv, cu_seqlens=None,
                  conv_state_in=None, state_in=None, eps=1e-6, want_states=True, bufs=None,
                  stream=None, fused=True):
    """x [N, Cq] io; z [N, Hv*128] io.  Returns a dict of device tensors.  fused: the conv,
    the chunked core and the gated norm in one call (gdn_prefill_layer), else three calls."""
    N, Cq = x.shape
    Ns = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    dev, dt = x.device, x.dtype
    bufs = {} if bufs is None else bufs
    y = bufs.get("y_conv")
    if y is None:
        y = torch.empty_like(x)
    cs_out = bufs.get("conv_state_out")
    if cs_out is None and want_states:
        cs_out = torch.empty((Ns, 3, Cq), dtype=dt, device=dev)
    q, k, v = qkv_views(y, Hk, Hv)
    o = bufs.get("o")
    if o is None:
        o = torch.empty((N, Hv, D), dtype=dt, device=dev)
    s_out = bufs.get("state_out")
    if s_out is None and want_states:
        s_out = torch.empty((Ns, Hv, D, D), dtype=torch.float32, device=dev)
    ws = bufs.get("workspace")
    need = gdn_chunk_prefill_workspace_size(N, Ns, Hk, Hv, io=dt)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        bufs["workspace"] = ws
    yn = bufs.get("y")
    if yn is None:
        yn = torch.empty_like(o)
    if fused:
        gdn_prefill_layer(x, conv_w, y, a, b, A_log, dt_bias, o, z, norm_w, yn, Hk, Hv,
                          cu_seqlens, conv_state_in, cs_out, state_in, s_out, eps=eps,
                          workspace=ws, stream=stream)
    else:
        gdn_conv1d_fwd(x, conv_w, y, cu_seqlens, conv_state_in, cs_out, stream=stream)
        gdn_chunk_prefill(q, k, v, a, b, A_log, dt_bias, o, Hk, Hv, cu_seqlens, state_in, s_out,
                          workspace=ws, stream=stream)
        gdn_gated_rmsnorm(o, z, norm_w, yn, eps, stream=stream)
    return {"y_conv": y, "o": o, "y": yn, "conv_state_out": cs_out, "state_out": s_out}


def decode_step(x, conv_w, conv_state, a, b, A_log, dt_bias, state, z, norm_w, Hk, Hv,
                eps=1e-6, bufs=None, stream=None, fused=True):
    """One token per sequence.  conv_state [B,3,Cq] and state [B,Hv,128,128] update in place;
    the state may be float32 or bfloat16 (stored bf16, stepped in fp32).  fused: the step
    and the gated norm in one launch (gdn_recurrent_step_norm), else two calls."""
    B = x.shape[0]
    bufs = {} if bufs is None else bufs
    o = bufs.get("o")
    if o is None:
        o = torch.empty((B, Hv, D), dtype=x.dtype, device=x.device)
    yn = bufs.get("y")
    if yn is None:
        yn = torch.empty_like(o)
    if fused:
        gdn_recurrent_step_norm(x, conv_w, conv_state, a, b, A_log, dt_bias, state, z, norm_w,
                                yn, Hk, Hv, o=o, eps=eps, stream=stream)
    else:
        gdn_recurrent_step(x, conv_w, conv_state, a, b, A_log, dt_bias, state, o, Hk, Hv,
                           stream=stream)
        gdn_gated_rmsnorm(o, z, norm_w, yn, eps, stream=stream)
    return {"o": o, "y": yn}


class DecodeGraph:
    """n consecutive decode steps (one gdn_recurrent_step_norm per step, or with
    fused=False gdn_recurrent_step -> gdn_gated_rmsnorm) of one layer, captured once as a
    HIP graph and replayed with one launch.

    The graph reads x[t], a[t], b[t], z[t] from the static buffers given here
    (x [n, B, Cq], a and b [n, B, Hv], z [n, B, Hv, 128]) and writes o[t] and y[t] of its
    own buffers; conv_state and state are updated in place by every replay, as n calls
    of decode_step would.  Write the next inputs into the same buffers and replay.
    The calls enqueue no memset and allocate nothing, so they capture as plain kernel
    nodes.
    """

    def __init__(self, x, conv_w, conv_state, a, b, A_log, dt_bias, state, z, norm_w, Hk, Hv,
                 eps=1e-6, fused=True):
        n, B = x.shape[0], x.shape[1]
        self.o = torch.empty((n, B, Hv, D), dtype=x.dtype, device=x.device)
        self.y = torch.empty_like(self.o)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for t in range(n):
                if fused:
                    gdn_recurrent_step_norm(x[t], conv_w, conv_state, a[t], b[t], A_log, dt_bias,
                                            state, z[t], norm_w, self.y[t], Hk, Hv, o=self.o[t],
                                            eps=eps)
                else:
                    gdn_recurrent_step(x[t], conv_w, conv_state, a[t], b[t], A_log, dt_bias,
                                       state, self.o[t], Hk, Hv)
                    gdn_gated_rmsnorm(self.o[t], z[t], norm_w, self.y[t], eps)

    def replay(self):
        self.graph.replay()
        return self.y
