"""The allocation-free training-time-test entry point against the workspace one.

eagle3_ttt_attention_static runs the same kernels as eagle3_ttt_attention with
its scratch in the library's fixed per-device array; on equal inputs the two
outputs must be bit-identical, on two calls in a row (the second smaller, so
the array holds the first call's contents when it starts), on the paths that
use scratch (fp32, bf16 at head size 32) and the fused bf16 path that uses
none; a call that needs more scratch than the array holds is refused before
any launch.
"""
import numpy as np
import pytest
import torch

from speculative_decoding_step_amd import binding as B

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else t.data_ptr()


def _inputs(rng, T, S, Hq, Hkv, hd, tdt):
    def dev(shape):
        return torch.as_tensor(rng.normal(size=shape), dtype=torch.float32).to(tdt).cuda()
    return dev((T, Hq, hd)), dev((Hkv, T, hd)), dev((Hkv, T, hd)), dev((S, Hkv, T, hd)), dev((S, Hkv, T, hd))


@pytest.mark.parametrize("dtype,cases", [
    ("f32", [(300, 3, 4, 2, 64), (100, 2, 4, 2, 64)]),
    ("bf16", [(520, 4, 8, 2, 32), (77, 0, 8, 2, 32)]),
    ("bf16", [(600, 7, 8, 2, 128), (129, 3, 8, 2, 128)]),
])
def test_static_scratch_matches_workspace_call(dtype, cases):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dt = B.BF16 if dtype == "bf16" else B.F32
    stream = torch.cuda.current_stream().cuda_stream
    for i, (T, S, Hq, Hkv, hd) in enumerate(cases):
        print(f"\n[no-alloc ttt {dtype} call {i}: T{T} S{S} Hq{Hq} Hkv{Hkv} hd{hd}]", flush=True)
        rng = np.random.default_rng(1000 * i + T)
        q, k0, v0, ks, vs = _inputs(rng, T, S, Hq, Hkv, hd, tdt)
        ref = torch.full((T, Hq, hd), float("nan"), dtype=tdt, device="cuda")
        out = torch.full((T, Hq, hd), float("nan"), dtype=tdt, device="cuda")
        wsb = B.eagle3_ttt_workspace_bytes(T, Hq, hd)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        ksp, vsp = (_p(ks), _p(vs)) if S else (None, None)
        B.eagle3_ttt_attention(dt, T, S, Hq, Hkv, hd, _p(q), _p(k0), _p(v0), ksp, vsp, _p(ref), _p(ws), wsb, stream)
        B.eagle3_ttt_attention_static(dt, T, S, Hq, Hkv, hd, _p(q), _p(k0), _p(v0), ksp, vsp, _p(out), stream)
        torch.cuda.synchronize()
        assert not torch.isnan(ref.float()).any()
        assert torch.equal(out, ref), (dtype, T, S, hd)


def test_static_scratch_refuses_oversized_calls():
    """fp32 at the 8B draft layer's heads needs ~230 MB of scratch: refused with
    EAGLE3_ECAPACITY before anything runs (the output keeps its contents)."""
    T, S, Hq, Hkv, hd = 2048, 2, 32, 8, 96
    assert B.eagle3_ttt_workspace_bytes(T, Hq, hd) > (32 << 20)
    out = torch.full((T, Hq, hd), 7.0, dtype=torch.float32, device="cuda")
    x = torch.zeros(Hkv * T * hd, dtype=torch.float32, device="cuda")
    with pytest.raises(B.Eagle3Error, match="capacity"):
        B.eagle3_ttt_attention_static(B.F32, T, S, Hq, Hkv, hd, _p(out), _p(x), _p(x), _p(x), _p(x), _p(out),
                                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
