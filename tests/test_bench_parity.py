"""The benchmark's parity record (CPU): the oracle leg compares the GPU step's
outputs for its sample rows with the oracle's own.  Here the "GPU" outputs are
the oracle's, so the record must say exact; one flipped code byte, scale byte
or C value must show up."""
import numpy as np
import pytest

import bench


@pytest.fixture(scope="module")
def small_sample(oracle):
    from microscaling_block_scaled_amd.synth import make
    ra, rw = 32, 16
    d = make("mxfp4_mlp", {"A": (ra, bench.K), "W": (rw, bench.K)})
    qa = oracle.quantize(d["A"], oracle.E2M1, 1, oracle.SR, oracle.FLAG_HADAMARD32, 42)
    qw = oracle.quantize(d["W"], oracle.E2M1, 1, oracle.RNE, oracle.FLAG_HADAMARD32)
    c, _ = oracle.gemm_f64(qa["q_row"], qa["s_row"], 4, qw["q_row"], qw["s_row"], 4, ra, rw, bench.K)
    gpu = {"qa": qa["q_row"], "sa": qa["s_row"], "qw": qw["q_row"], "sw": qw["s_row"],
           "c": c.astype(np.float32)}
    return ra, rw, {"A": d["A"], "W": d["W"], "gpu": gpu}


def run(monkeypatch, ra, rw, sample):
    monkeypatch.setattr(bench, "SAMPLE_A", ra)
    monkeypatch.setattr(bench, "SAMPLE_W", rw)
    return bench.cpu_baseline(sample)


def test_exact_outputs_report_exact(monkeypatch, small_sample):
    ra, rw, sample = small_sample
    base, parity = run(monkeypatch, ra, rw, sample)
    assert base["kind"] == "oracle" and base["value"] > 0
    assert parity["quant_a_bit_exact"] and parity["quant_w_bit_exact"]
    assert parity["gemm_elements_over_bound"] == 0


@pytest.mark.parametrize("what", ["qa", "sa", "qw", "sw", "c"])
def test_a_wrong_output_is_reported(monkeypatch, small_sample, what):
    ra, rw, sample = small_sample
    gpu = dict(sample["gpu"])
    x = gpu[what].copy()
    if what == "c":
        x[3, 5] = x[3, 5] * 1.001 + 1.0
    else:
        x[2, 1] ^= 0x10
    gpu[what] = x
    _, parity = run(monkeypatch, ra, rw, {**sample, "gpu": gpu})
    if what in ("qa", "sa"):
        assert not parity["quant_a_bit_exact"] and parity["quant_w_bit_exact"]
    elif what in ("qw", "sw"):
        assert parity["quant_a_bit_exact"] and not parity["quant_w_bit_exact"]
    else:
        assert parity["gemm_elements_over_bound"] == 1
