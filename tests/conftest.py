import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def oracle_shape(ms):
    """oracle.llama.Shape from a configs.ModelShape."""
    from oracle.llama import Shape

    return Shape(ms.n_layers, ms.d, ms.n_heads, ms.n_kv_heads, ms.head_dim, ms.ffn, ms.vocab,
                 ms.rope_theta, ms.eps, ms.dtype, tuple(ms.taps))


@pytest.fixture
def toy_model():
    """A small bf16 model with weights wide enough (sigma 0.4) to be context-dependent."""
    from speculative_decoding_step_amd import configs

    def make(dtype="bf16", vocab=16, seed=11, sigma=0.4, layers=2, d=64, heads=4, kv=2, hd=16, ffn=96,
             taps=(0, 1, 1)):
        ms = configs.ModelShape(layers, d, heads, kv, hd, ffn, vocab, 1e4, taps, dtype=dtype)
        W, H = configs.weights_np(ms, seed, seed + 1, sigma=sigma)
        return ms, oracle_shape(ms), W, H

    return make
