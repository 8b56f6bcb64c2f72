"""CPU check of the whole-tensor comparison harness used at full workload sizes: fed the
oracle's own layer outputs as the "GPU" outputs it passes with zero error, and a single
wrong element of o, of the norm output, of the conv output or of a final state fails it.
(The harness recomputes every chain in worker processes, with its own per-chain oracle
calls; G.layer computes the same values in one process.)"""
import numpy as np
import pytest

from hybrid_linear_attention_causal_amd import synth
from oracle import gdn_oracle as G

import oracle_pool

D = 128


def _tasks(inp, ref, io):
    hk, hv, Ns, N = inp["Hk"], inp["Hv"], inp["Ns"], inp["N"]
    r = hv // hk
    cu = inp["cu_seqlens"]
    x_p, z_p = oracle_pool.pack(inp["x"], io), oracle_pool.pack(inp["z"], io)
    g = {k: oracle_pool.pack(ref[k], io) for k in ("y_conv", "o", "y", "conv_state_out")}
    out = []
    for s in range(Ns):
        b0, b1 = (0, N) if cu is None else (int(cu[s]), int(cu[s + 1]))
        for h in range(hv):
            kh = h // r
            blocks = (slice(kh * D, kh * D + D), slice((hk + kh) * D, (hk + kh + 1) * D),
                      slice(2 * hk * D + h * D, 2 * hk * D + (h + 1) * D))
            cols = lambda a: np.concatenate([a[..., c] for c in blocks], axis=-1)
            out.append({"s": s, "h": h, "io": io, "check_qk": h % r == 0,
                        "x": cols(x_p[b0:b1]), "conv_w": cols(inp["conv_w"].T).T.copy(),
                        "cs_in": None if inp["conv_state_in"] is None else
                        cols(oracle_pool.pack(inp["conv_state_in"][s], io)),
                        "a": inp["a"][b0:b1, h].astype(np.float64),
                        "b": inp["b"][b0:b1, h].astype(np.float64),
                        "A_log": float(inp["A_log"][h]), "dt_bias": float(inp["dt_bias"][h]),
                        "S0": None if inp["state_in"] is None else inp["state_in"][s, h],
                        "z": z_p[b0:b1, h * D:(h + 1) * D], "norm_w": inp["norm_w"],
                        "gpu_yc": cols(g["y_conv"][b0:b1]),
                        "gpu_o": g["o"].reshape(N, hv, D)[b0:b1, h],
                        "gpu_y": g["y"].reshape(N, hv, D)[b0:b1, h],
                        "gpu_S": ref["state_out"][s, h].astype(np.float32),
                        "gpu_cs": cols(g["conv_state_out"][s])})
    return out


def _run(tasks, io, ns):
    comb = oracle_pool.Combined(io, ns)
    for res in map(oracle_pool.chain_task, tasks):    # in process: the measures, not the pool
        comb.add(res)
    return comb.check("pool")


@pytest.fixture(scope="module")
def case():
    sh = synth.Shape("h2x4", hk=2, hv=4)
    inp = synth.make(synth.custom(sh, "bf16", 31, seqlens=[70, 5, 0, 40], init_state=True))
    return inp, G.layer(inp)


def test_pool_passes_on_the_oracles_own_outputs(case):
    inp, ref = case
    rep = _run(_tasks(inp, ref, "bf16"), "bf16", inp["Ns"])
    assert rep["o"][0] == 0 and rep["y"][0] == 0 and rep["yc"][0] == 0
    assert rep["state"][0] < 1e-6     # the final state travels as fp32


@pytest.mark.parametrize("part", ["gpu_o", "gpu_y", "gpu_yc", "gpu_S", "gpu_cs"])
def test_pool_catches_one_wrong_element(case, part):
    inp, ref = case
    tasks = _tasks(inp, ref, "bf16")
    t = tasks[5]
    arr = np.array(oracle_pool.unpack(t[part]) if part != "gpu_S" else t[part], dtype=np.float64)
    idx = tuple(s // 2 for s in arr.shape)
    if part == "gpu_yc":
        idx = (idx[0], 2 * D + 5)     # a v channel: this chain's own conv check
    arr[idx] = arr[idx] * 1.5 + 1.0
    t[part] = arr.astype(np.float32) if part == "gpu_S" else oracle_pool.pack(arr, "bf16")
    with pytest.raises(AssertionError):
        _run(tasks, "bf16", inp["Ns"])


def test_pool_runs_in_worker_processes(case):
    inp, ref = case
    tasks = _tasks(inp, ref, "bf16")
    comb = oracle_pool.Combined("bf16", inp["Ns"])
    for res in oracle_pool.run(iter(tasks), len(tasks)):
        comb.add(res)
    assert comb.chains == len(tasks)
    comb.check("pool")
