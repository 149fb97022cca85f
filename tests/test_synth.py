"""The shared input generator: deterministic, right shapes and statistics,
and bfloat16 rounding identical to torch's round-to-nearest-even."""

import numpy as np
import pytest

from transformer_head_scaled_amd import synth


def test_deterministic_and_distinct():
    a = synth.sdpa_inputs(5, 1, 2, 64, 64, 64)
    b = synth.sdpa_inputs(5, 1, 2, 64, 64, 64)
    for k in "QKV":
        assert np.array_equal(a[k][0], b[k][0])
    assert not np.array_equal(a["Q"][1], a["K"][1])
    c = synth.sdpa_inputs(3, 1, 2, 64, 64, 64)
    assert not np.array_equal(a["Q"][1], c["Q"][1])


def test_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rs = np.random.default_rng(0)
    x = np.concatenate([rs.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, 3.0e38, 65504.0,
                                  1.00390625, 1.01171875], dtype=np.float32)])
    bits, vals = synth.round_to(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    assert np.array_equal(vals, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    nb, _ = synth.round_to(np.array([np.nan], dtype=np.float32), "bf16")
    assert np.isnan(synth.bf16_to_f32(nb)[0])


def test_workload_shapes_and_lengths():
    ins, lens = synth.workload_inputs(2)
    w = synth.WORKLOADS[2]
    assert ins["x_q"][0].shape == (32, 64, 512) and ins["x_q"][0].dtype == np.uint16
    assert "x_kv" not in ins
    assert ins["Wq"][0].shape == (512, 512)
    assert lens.dtype == np.int32 and lens.min() >= 16 and lens.max() <= 64
    assert abs(ins["Wq"][1].std() * np.sqrt(512) - 1) < 0.02
    ins4, _ = synth.workload_inputs(4)
    assert ins4["x_kv"][0].shape == (8, 512, 1024)
    ins1, _ = synth.workload_inputs(1)
    assert ins1["Q"][0].dtype == np.float32 and ins1["Q"][0].shape == (1, 1, 16, 64)
    assert w["h"] == 8
