"""Input generator checks (no GPU): bf16 rounding and workload shapes."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    # exact ties and the largest finite values
    x[:4] = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.0e38], np.float32)
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_shapes():
    w = synth.WORKLOADS
    assert len(w["gpt2_small"].matrices) == 72
    assert len(w["gpt2_xl_1p5b"].matrices) == 288
    assert len(w["moe_share"].matrices) == 136
    assert w["gpt2_xl_1p5b"].n_params == 48 * (4 * 1600 * 1600 + 2 * 1600 * 6400)
    assert w["moe_share"].g_dtype == "bf16"


def test_numpy_matrix_is_seeded():
    w = synth.WORKLOADS["single256"]
    a = synth.numpy_matrix(w, 0, 0)
    b = synth.numpy_matrix(w, 0, 0)
    assert np.array_equal(a["G"], b["G"]) and np.array_equal(a["W0"], b["W0"])
    c = synth.numpy_matrix(synth.WORKLOADS["gpt2s_fc_10step"], 0, 1)
    d = synth.numpy_matrix(synth.WORKLOADS["gpt2s_fc_10step"], 0, 2)
    assert not np.array_equal(c["G"], d["G"])
    assert np.array_equal(c["W0"], d["W0"])
