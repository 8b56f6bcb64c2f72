"""CPU checks of bench.py's host arithmetic: the decode step's compulsory bytes against an
enumeration of the tensors it moves, the chunked core's algorithmic flops against
properties any size must keep (additive over sequences, a partial chunk counted at its
length, linear in the heads), the measured-traffic table's source check, and the one-GPU
guard."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
D, C = 128, 64


def test_decode_bytes_enumerates_the_step_tensors():
    B, hk, hv = 256, 16, 32
    cq = (2 * hk + hv) * D                    # conv channels: q | k | v
    tensors = {
        "state read": B * hv * D * D * 4,
        "state write": B * hv * D * D * 4,
        "conv state read": B * 3 * cq * 2,
        "conv state write": B * 3 * cq * 2,
        "x": B * cq * 2,
        "a": B * hv * 2,
        "b": B * hv * 2,
        "conv weight (fp32)": cq * 4 * 4,
        "A_log, dt_bias (fp32)": 2 * hv * 4,
        "o": B * hv * D * 2,
    }
    assert bench.decode_bytes(B, hk, hv) == sum(tensors.values()) == 1_105_363_200
    # a bf16-stored state moves half the state bytes and the same rest
    half = tensors["state read"]
    assert bench.decode_bytes(B, hk, hv, state_bytes=2) == sum(tensors.values()) - half


def test_chunk_flops_are_per_chunk_at_its_length():
    f = bench.chunk_core_flops
    # additive over packed sequences, chunks restarting at each sequence
    assert f(0, 16, 32, [100, 37, 64]) == pytest.approx(
        f(100, 16, 32) + f(37, 16, 32) + f(64, 16, 32))
    # a sequence of 65 tokens is one full chunk and one chunk of a single token
    one_tok = 16 * (2 * 1 * D) + 32 * (3 * 1 * D + 1 / 3 + 6 * D * D)
    assert f(65, 16, 32) == pytest.approx(f(64, 16, 32) + one_tok)
    # full chunks only: linear in the token count
    assert f(4096, 16, 32) == pytest.approx(64 * f(64, 16, 32))
    # the per-token terms: key heads carry the Gram products, value heads the rest
    assert f(64, 2, 4) == pytest.approx(2 * f(64, 1, 0) + 4 * f(64, 0, 1))
    assert f(64, 1, 0) == pytest.approx(C * 2 * C * D)
    # the 9B T=4096 call the headline roofline prices
    assert f(4096, 16, 32) == pytest.approx(17_358_826_154.67, rel=1e-12)


def test_measured_traffic_needs_matching_sources(monkeypatch):
    key = "gdn_recurrent_step"
    kernel, digest, nbytes = bench.MEASURED_TRAFFIC[key]
    assert bench.measured_traffic(key) == (nbytes if bench.source_digest(kernel) == digest else None)
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, key, (kernel, "0" * 16, nbytes))
    assert bench.measured_traffic(key) is None
    assert bench.measured_traffic("no such call") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""
