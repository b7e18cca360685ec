"""The seeded input generator: host (numpy) and device (torch) twins agree bit for bit."""
import numpy as np
import torch

from speculative_decoding_step_amd import synth


def test_normal_host_device_agree_bf16_and_f32():
    for dtype in ("bf16", "f32"):
        a = synth.normal_np(7, "w", (300, 17), 0.02, dtype)
        b = synth.normal_t(7, "w", (300, 17), "cpu", 0.02, dtype, chunk=1000).float().numpy()
        assert np.array_equal(a, b)
    assert abs(a.std() - 0.02) < 0.002 and abs(a.mean()) < 0.002


def test_tokens_and_uniforms_agree():
    assert np.array_equal(synth.tokens_np(3, "p", 999, 32000), synth.tokens_t(3, "p", 999, 32000, "cpu").numpy())
    u = synth.uniform24_np(5, "u", 1000)
    assert np.array_equal(u, synth.uniform24_t(5, "u", 1000, "cpu").numpy())
    assert u.min() >= 0 and u.max() < 1 and np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))


def test_streams_differ_by_name_and_seed():
    a = synth.tokens_np(3, "p", 64, 1000)
    assert not np.array_equal(a, synth.tokens_np(4, "p", 64, 1000))
    assert not np.array_equal(a, synth.tokens_np(3, "q", 64, 1000))
