"""The seeded input generators: determinism, the stated distributions, and
bf16 rounding checked against torch's conversion."""
import numpy as np
import torch

import synth
from synth.workloads import WORKLOADS, bias_for


def test_deterministic_and_streams_independent():
    a = synth.x_bf16(0, 4, 256)
    np.testing.assert_array_equal(a, synth.x_bf16(0, 4, 256))
    assert not np.array_equal(a, synth.x_bf16(1, 4, 256))
    # token offset t0 selects later tokens of the same stream
    np.testing.assert_array_equal(synth.x_bf16(0, 2, 256, t0=2), a[2:])
    w0 = synth.expert_f32(0, 0, 0, 8, 32, nthreads=1)
    np.testing.assert_array_equal(w0, synth.expert_f32(0, 0, 0, 8, 32, nthreads=4))
    assert not np.array_equal(w0, synth.expert_f32(0, 0, 1, 8, 32))


def test_normal_moments():
    z = synth.normals_f32(0, 99, 0, 2_000_000).astype(np.float64)
    assert abs(z.mean()) < 3e-3
    assert abs(z.var() - 1.0) < 3e-3
    assert abs(np.mean(z ** 4) - 2.9) < 0.02  # Irwin-Hall(12) kurtosis is 3 - 0.1
    assert np.abs(z).max() <= 6.0
    assert np.all(z * 65536 == np.round(z * 65536))  # exact multiples of 2^-16


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    f = np.concatenate([rng.normal(size=100000), rng.normal(size=1000) * 1e-30, [0.0, -0.0, 1.0]]).astype(np.float32)
    ref = torch.tensor(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.round_bf16(f), ref)


def test_weight_scales():
    wr = synth.bf16_to_f32(synth.router_bf16(0, 512, 896))
    assert abs(wr.std() - 0.02) < 2e-4
    w = synth.expert_f32(0, 1, 2, 512, 256)
    assert abs(w.std() - 0.02) < 2e-4


def test_zipf_bias_is_a_power_law_in_rank():
    pi = synth.popularity_perm(0, 896)
    assert sorted(pi) == list(range(896))
    b = synth.zipf_bias(0, 896, 0.5, 1.1)
    np.testing.assert_allclose(b, -0.5 * 1.1 * np.log1p(pi), rtol=1e-6)
    assert bias_for(WORKLOADS["tiny"]) is None
    assert bias_for(WORKLOADS["verify_256"]).shape == (896,)
