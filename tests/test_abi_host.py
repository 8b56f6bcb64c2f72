"""Host-side checks of the C ABI: the library loads without a GPU, exports every
function include/gdn.h declares, and rejects bad arguments before any launch."""
import ctypes
import os

import pytest

from hybrid_linear_attention_causal_amd import _lib

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libgdn.so not built (run __graft_entry__.build())")

EXPECTED = {"gdn_last_error", "gdn_version", "gdn_conv1d_fwd", "gdn_chunk_prefill_workspace_size",
            "gdn_chunk_prefill", "gdn_chunk_prefill_noalloc", "gdn_conv_chunk_prefill",
            "gdn_prefill_layer",
            "gdn_recurrent_step", "gdn_recurrent_step_bf16_state", "gdn_recurrent_step_slots",
            "gdn_recurrent_step_norm", "gdn_gated_rmsnorm"}


def test_header_declares_the_calls():
    assert set(_lib.declared_symbols()) == EXPECTED


def test_library_exports_every_declared_symbol():
    handle = ctypes.CDLL(_lib.LIB_PATH)
    for name in _lib.declared_symbols():
        assert hasattr(handle, name), name
    assert _lib.version() == "0.1.0"


def test_no_unexpected_exports():
    # dynamic symbol table: the C ABI plus nothing named gdn_* that the header omits
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True).stdout
    names = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    assert {n for n in names if n.startswith("gdn_")} == EXPECTED


L = None


def _L():
    global L
    if L is None:
        L = _lib.lib()
    return L


def _msg():
    return _L().gdn_last_error().decode()


P = ctypes.c_void_p(16)   # a non-null, aligned dummy address: never dereferenced on these paths


def test_conv_rejects():
    L = _L()
    assert L.gdn_conv1d_fwd(P, P, P, None, 1, 10, 8, 3, None, None, 1, None) == _lib.GDN_ERR_UNSUPPORTED
    assert "width" in _msg()
    assert L.gdn_conv1d_fwd(None, P, P, None, 1, 10, 8, 4, None, None, 1, None) == _lib.GDN_ERR_INVALID_ARG
    assert L.gdn_conv1d_fwd(P, P, P, None, 1, 10, 12, 4, None, None, 1, None) == _lib.GDN_ERR_INVALID_ARG
    assert L.gdn_conv1d_fwd(P, P, P, None, 2, 10, 8, 4, None, None, 1, None) == _lib.GDN_ERR_INVALID_ARG
    assert "cu_seqlens" in _msg()
    assert L.gdn_conv1d_fwd(P, P, P, None, 1, -1, 8, 4, None, None, 1, None) == _lib.GDN_ERR_INVALID_ARG
    assert L.gdn_conv1d_fwd(P, P, P, None, 1, 10, 8, 4, None, None, 7, None) == _lib.GDN_ERR_INVALID_ARG
    assert L.gdn_conv1d_fwd(P, P, ctypes.c_void_p(18), None, 1, 10, 8, 4, None, None, 1, None) == _lib.GDN_ERR_INVALID_ARG
    assert "aligned" in _msg()
    assert L.gdn_conv1d_fwd(P, P, P, None, 1, 10, 8, 4, None, None, 1, None) == _lib.GDN_ERR_INVALID_ARG
    assert "alias" in _msg()


def _prefill(**kw):
    args = dict(q=P, k=P, v=P, sq=4096, sk=4096, sv=4096, a=P, b=P, A_log=P, dt_bias=P, g=None,
                beta=None, s_in=None, s_out=None, o=P, cu=None, Ns=1, N=64, Hk=16, Hv=32, dk=128,
                dv=128, scale=0.0, l2=1, ws=None, ws_bytes=0, io=1)
    args.update(kw)
    return _L().gdn_chunk_prefill(*args.values(), None)


def test_prefill_rejects():
    assert _prefill(dk=64) == _lib.GDN_ERR_UNSUPPORTED
    assert _prefill(Hv=24) == _lib.GDN_ERR_INVALID_ARG
    assert _prefill(Hk=0) == _lib.GDN_ERR_INVALID_ARG
    assert _prefill(Ns=3) == _lib.GDN_ERR_INVALID_ARG
    assert _prefill(sq=100) == _lib.GDN_ERR_INVALID_ARG
    assert _prefill(sv=4100) == _lib.GDN_ERR_INVALID_ARG
    assert _prefill(sk=(1 << 20) + 8) == _lib.GDN_ERR_INVALID_ARG
    assert _prefill(g=P) == _lib.GDN_ERR_INVALID_ARG
    assert "both" in _msg()
    assert _prefill(o=None) == _lib.GDN_ERR_INVALID_ARG
    assert _prefill(a=None) == _lib.GDN_ERR_INVALID_ARG
    assert _prefill(io=5) == _lib.GDN_ERR_INVALID_ARG
    assert _prefill(ws=P, ws_bytes=1024) == _lib.GDN_ERR_INVALID_ARG
    assert "workspace" in _msg()
    # chunk offsets (int32 [Ns + 1]) and chunk table (int4 [cmax]), each padded to 256 B,
    # then cmax = ceil(N/64) + Ns chunks x (Hv x 38912 B + Hk x K record), K record 0 B
    # (bf16 io: K and Q are staged from the inputs) or 69632 B (fp32 io), then for at
    # most 64 (sequence, head) chains 7 segment-transition pairs of 128 KB per chain (fp32
    # io; bf16 io only for at most 16 chains averaging at least 256 chunks)
    ws = _lib.lib().gdn_chunk_prefill_workspace_size
    assert ws(4096, 1, 16, 32, 128, 1) == 256 + 1280 + 65 * (32 * 38912)
    assert ws(4096, 3, 16, 32, 128, 1) == 256 + 1280 + 67 * (32 * 38912)
    assert ws(100, 3, 1, 2, 128, 0) == 256 + 256 + 5 * (2 * 38912 + 1 * 69632) + 7 * 6 * 131072
    # bf16: 256 chunks of one sequence at 2 heads reserve the scan's pairs, 255 do not,
    # nor do 32 chains
    assert ws(16384, 1, 1, 2, 128, 1) == 256 + 4352 + 257 * (2 * 38912) + 7 * 2 * 131072
    assert ws(16320, 1, 1, 2, 128, 1) == 256 + 4096 + 256 * (2 * 38912)
    assert ws(32768, 1, 16, 32, 128, 1) == 256 + 8448 + 513 * (32 * 38912)
    assert ws(-1, 1, 16, 32, 128, 1) == 0
    assert ws(64, 1, 16, 32, 64, 1) == 0
    assert ws(64, 1, 16, 24, 128, 1) == 0            # Hv not a multiple of Hk
    # sizes beyond what the calls accept, or whose byte count would pass 2^62: 0, not a
    # wrapped-around 64-bit product
    assert ws(1 << 50, 1, 16, 64, 128, 1) == 0       # more than 2^31 chunks
    assert ws(1 << 36, 1, 1, 1 << 20, 128, 1) == 0   # 2^30 chunks x 2^20 heads
    assert ws((1 << 36) - 64, 1, 16, 64, 128, 1) > 0
    # and a call with such sizes is refused before the workspace is compared or a device used
    assert _prefill(N=1 << 50, ws=P, ws_bytes=1024) == _lib.GDN_ERR_INVALID_ARG
    assert "chunks" in _msg()
    # (row strides of at most 2^20 elements cap Hv at 8192, so through the call the size
    # stays below the bound, and is compared unwrapped with the workspace given)
    assert _prefill(N=1 << 36, Hk=1, Hv=8192, sv=1 << 20, ws=P, ws_bytes=1024) == \
        _lib.GDN_ERR_INVALID_ARG
    assert "workspace" in _msg()


def _step(fn="gdn_recurrent_step", **kw):
    args = dict(x=P, w=P, cs=P, a=P, b=P, A_log=P, dt_bias=P, g=None, beta=None, st=P, o=P,
                B=4, Hk=16, Hv=32, dk=128, dv=128, K=4, scale=0.0, l2=1, io=1)
    args.update(kw)
    return getattr(_L(), fn)(*args.values(), None)


def test_step_rejects():
    assert _step(K=2) == _lib.GDN_ERR_UNSUPPORTED
    assert _step(dv=64) == _lib.GDN_ERR_UNSUPPORTED
    assert _step(Hv=20) == _lib.GDN_ERR_INVALID_ARG
    assert _step(B=-1) == _lib.GDN_ERR_INVALID_ARG
    assert _step(st=None) == _lib.GDN_ERR_INVALID_ARG
    assert _step(beta=P) == _lib.GDN_ERR_INVALID_ARG
    assert _step(st=ctypes.c_void_p(20)) == _lib.GDN_ERR_INVALID_ARG


def test_step_bf16_state_rejects():
    fn = "gdn_recurrent_step_bf16_state"
    assert _step(fn, K=2) == _lib.GDN_ERR_UNSUPPORTED
    assert "recurrent_step_bf16_state" in _msg()
    assert _step(fn, dk=64) == _lib.GDN_ERR_UNSUPPORTED
    assert _step(fn, Hv=20) == _lib.GDN_ERR_INVALID_ARG
    assert _step(fn, st=None) == _lib.GDN_ERR_INVALID_ARG
    assert _step(fn, g=P) == _lib.GDN_ERR_INVALID_ARG
    assert _step(fn, st=ctypes.c_void_p(24)) == _lib.GDN_ERR_INVALID_ARG
    assert _step(fn, io=7) != 0


def test_norm_rejects():
    L = _L()
    assert L.gdn_gated_rmsnorm(P, P, P, P, 10, 64, 1e-6, 1, None) == _lib.GDN_ERR_UNSUPPORTED
    assert L.gdn_gated_rmsnorm(P, P, P, P, -1, 128, 1e-6, 1, None) == _lib.GDN_ERR_INVALID_ARG
    assert L.gdn_gated_rmsnorm(P, None, P, P, 10, 128, 1e-6, 1, None) == _lib.GDN_ERR_INVALID_ARG
    assert L.gdn_gated_rmsnorm(P, P, P, P, 10, 128, -1.0, 1, None) == _lib.GDN_ERR_INVALID_ARG
    # more rows than 2^31 - 1 blocks of 16 hold: refused, not a truncated grid
    assert L.gdn_gated_rmsnorm(P, P, P, P, (1 << 36) + 16, 128, 1e-6, 1, None) == \
        _lib.GDN_ERR_INVALID_ARG
    assert "rows" in _msg()


def _slots(**kw):
    args = dict(x=P, w=P, cs=P, a=P, b=P, A_log=P, dt_bias=P, g=None, beta=None, st=P,
                sdt=_lib.GDN_F32, slots=P, n_slots=8, o=P, B=4, Hk=16, Hv=32, dk=128, dv=128,
                K=4, scale=0.0, l2=1, io=1)
    args.update(kw)
    return _L().gdn_recurrent_step_slots(*args.values(), None)


def test_step_slots_rejects():
    assert _slots(sdt=5) == _lib.GDN_ERR_INVALID_ARG
    assert "state dtype" in _msg()
    assert _slots(n_slots=0) == _lib.GDN_ERR_INVALID_ARG
    assert _slots(slots=None) == _lib.GDN_ERR_INVALID_ARG
    assert _slots(slots=ctypes.c_void_p(18)) == _lib.GDN_ERR_INVALID_ARG
    assert _slots(K=3) == _lib.GDN_ERR_UNSUPPORTED
    assert "recurrent_step_slots" in _msg()
    assert _slots(Hv=20) == _lib.GDN_ERR_INVALID_ARG
    assert _slots(st=None) == _lib.GDN_ERR_INVALID_ARG


def _stepnorm(**kw):
    args = dict(x=P, w=P, cs=P, a=P, b=P, A_log=P, dt_bias=P, g=None, beta=None, st=P,
                sdt=_lib.GDN_F32, z=P, nw=P, eps=1e-6, o=None, y=P, B=4, Hk=16, Hv=32, dk=128,
                dv=128, K=4, scale=0.0, l2=1, io=1)
    args.update(kw)
    return _L().gdn_recurrent_step_norm(*args.values(), None)


def test_step_norm_rejects():
    assert _stepnorm(sdt=9) == _lib.GDN_ERR_INVALID_ARG
    assert _stepnorm(eps=-1.0) == _lib.GDN_ERR_INVALID_ARG
    assert _stepnorm(y=None) == _lib.GDN_ERR_INVALID_ARG
    assert _stepnorm(z=None) == _lib.GDN_ERR_INVALID_ARG
    assert "recurrent_step_norm" in _msg()
    assert _stepnorm(nw=None) == _lib.GDN_ERR_INVALID_ARG
    assert _stepnorm(nw=ctypes.c_void_p(24)) == _lib.GDN_ERR_INVALID_ARG
    assert _stepnorm(y=ctypes.c_void_p(20)) == _lib.GDN_ERR_INVALID_ARG
    assert _stepnorm(dv=64) == _lib.GDN_ERR_UNSUPPORTED


def _fused(**kw):
    args = dict(x=P, w=P, csi=None, cso=None, y=ctypes.c_void_p(4096), a=P, b=P, A_log=P,
                dt_bias=P, g=None, beta=None, si=None, so=None, o=P, cu=None, Ns=1, N=100, Hk=2,
                Hv=4, dk=128, dv=128, K=4, scale=0.0, l2=1, ws=P, ws_bytes=1 << 30, io=1)
    args.update(kw)
    return _L().gdn_conv_chunk_prefill(*args.values(), None)


def test_conv_chunk_prefill_rejects():
    assert _fused(K=3) == _lib.GDN_ERR_UNSUPPORTED
    assert "conv_chunk_prefill" in _msg()
    assert _fused(dk=64) == _lib.GDN_ERR_UNSUPPORTED
    assert _fused(io=5) == _lib.GDN_ERR_INVALID_ARG
    assert _fused(x=None) == _lib.GDN_ERR_INVALID_ARG
    assert _fused(y=None) == _lib.GDN_ERR_INVALID_ARG
    assert _fused(y=P) == _lib.GDN_ERR_INVALID_ARG          # aliases x
    assert "alias" in _msg()
    assert _fused(csi=ctypes.c_void_p(40)) == _lib.GDN_ERR_INVALID_ARG
    assert _fused(Hv=3) == _lib.GDN_ERR_INVALID_ARG          # not a multiple of Hk
    assert _fused(Ns=2) == _lib.GDN_ERR_INVALID_ARG          # cu_seqlens NULL
    assert _fused(ws=None) == _lib.GDN_ERR_INVALID_ARG
    assert _fused(g=P) == _lib.GDN_ERR_INVALID_ARG           # g without beta


def test_noalloc_rejects_a_workspace_beyond_its_array_before_any_launch():
    # 9B shape, 8192 tokens of one sequence: a 161 MB workspace against the fixed 128 MiB
    L = _L()
    args = [P, P, P, 4096, 4096, 4096, P, P, P, P, None, None, None, None, P, None, 1, 8192,
            16, 32, 128, 128, 0.0, 1, 1, None]
    assert L.gdn_chunk_prefill_noalloc(*args) == _lib.GDN_ERR_INVALID_ARG
    assert "workspace" in _msg()


def _layer(**kw):
    args = dict(x=P, w=P, cs_in=None, cs_out=None, y=ctypes.c_void_p(32), a=P, b=P, A_log=P,
                dt_bias=P, g=None, beta=None, s_in=None, s_out=None, o=ctypes.c_void_p(48),
                z=P, nw=P, eps=1e-6, yn=ctypes.c_void_p(64), cu=None, Ns=1, N=64, Hk=16, Hv=32,
                dk=128, dv=128, K=4, scale=0.0, l2=1, ws=None, ws_bytes=0, io=1)
    args.update(kw)
    return _L().gdn_prefill_layer(*args.values(), None)


def test_prefill_layer_rejects():
    assert _layer(yn=None) == _lib.GDN_ERR_INVALID_ARG
    assert "norm output" in _msg()
    assert _layer(z=None) == _lib.GDN_ERR_INVALID_ARG
    assert "z or norm_w" in _msg()
    assert _layer(eps=-1.0) == _lib.GDN_ERR_INVALID_ARG
    assert _layer(yn=ctypes.c_void_p(24)) == _lib.GDN_ERR_INVALID_ARG
    assert "aligned" in _msg()
    assert _layer(K=3) == _lib.GDN_ERR_UNSUPPORTED
    assert _layer() == _lib.GDN_ERR_INVALID_ARG     # no workspace
    assert "workspace" in _msg()


def test_binding_row_strides():
    """The binding passes q, k, v row strides: a view's stride(0) when it has rows to step
    over, its width when it has at most one (torch reports arbitrary strides for those: an
    empty array from NumPy has strides (0, 0)), and it refuses rows that are not contiguous."""
    import numpy as np
    import torch

    y = torch.zeros(5, 1536)
    assert _lib._row_stride(y[:, 256:512]) == 1536
    empty = torch.from_numpy(np.zeros((0, 1536), dtype=np.float32))
    assert empty.stride() == (0, 0)
    assert _lib._row_stride(empty[:, :256]) == 256
    one = torch.zeros(1, 1536).as_strided((1, 256), (1, 1))
    assert _lib._row_stride(one) == 256
    with pytest.raises(ValueError):
        _lib._row_stride(y.t()[:, :3])
    with pytest.raises(ValueError):
        _lib._row_stride(torch.zeros(1, 512)[:, ::2])
