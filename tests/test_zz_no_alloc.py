"""GPU: moe_layer_decode_noalloc (the library's fixed scratch as the workspace) against moe_layer_decode.

Two calls in a row on the same GPU, the second with a smaller step, each
compared bit for bit with moe_layer_decode on a caller workspace: the scratch
keeps the first call's contents, so the second call also shows that nothing
left there leaks into a later step.  A step whose workspace exceeds the
scratch is refused with MOE_EUNSUPPORTED and enqueues nothing.
"""
import numpy as np
import pytest

import synth
from tests._parity import routed_experts, to_dev, to_dev_x, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_routed_ffn_amd as m
    return m


def _case(T, bits, x_dtype, E=512, k=10, H=2048, I=512, seed=0):
    return synth.Workload(f"noalloc_T{T}_b{bits}", E=E, k=k, H=H, I=I, T=T, bits=bits, x_dtype=x_dtype, zipf_s=1.1,
                          seed=seed)


def _both(moe, w, x, lg, ex, residual=None):
    import torch
    layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, to_dev(ex))
    xd, ld = to_dev_x(x), to_dev(lg)
    res = xd if residual else None
    a = moe.layer_decode(layer, xd, ld, w.k, residual=res)
    b = moe.layer_decode_noalloc(layer, xd, ld, w.k, residual=res)
    torch.cuda.synchronize()
    return a, b


def _same(a, b, n):
    for u, v in zip((a[0], a[1], a[3], a[4]), (b[0], b[1], b[3], b[4])):
        assert np.array_equal(to_host(u).view(np.uint32), to_host(v).view(np.uint32))
    for f in ("offsets", "sorted_assign", "assign_pos", "active", "n_active"):
        ta, tb = to_host(getattr(a[2], f)), to_host(getattr(b[2], f))
        if f in ("sorted_assign", "assign_pos"):
            ta, tb = ta[:n], tb[:n]
        if f == "active":
            na = int(to_host(a[2].n_active)[0])
            ta, tb = ta[:na], tb[:na]
        assert np.array_equal(ta, tb), f


@pytest.mark.parametrize("first,second", [((12, 2, "bf16"), (3, 2, "bf16")),  # decode layer: 12 then 3 tokens
                                          ((8, 4, "f32"), (1, 4, "f32"))])  # 4-bit, fp32 x: 8 then 1
def test_noalloc_matches_layer_decode_twice(moe, first, second):
    for T, bits, xdt in (first, second):
        w = _case(T, bits, xdt)
        lg = w.logits()
        ex = routed_experts(w, lg)
        a, b = _both(moe, w, w.x(), lg, ex, residual=True)
        _same(a, b, w.T * w.k)


def test_noalloc_general_shape_then_smaller(moe):
    """A shape that takes the four-launch decode step (H, I not multiples of 2048 and 512)."""
    for T in (7, 2):
        w = _case(T, 3, "bf16", E=48, k=6, H=96, I=64, seed=T)
        x, lg, ex = w.x(), w.logits(), w.experts()
        a, b = _both(moe, w, x, lg, ex)
        _same(a, b, w.T * w.k)


def test_noalloc_refuses_steps_beyond_the_scratch(moe):
    import torch
    w = _case(12, 2, "bf16", E=1024, k=16, H=2048, I=8192)
    layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert moe.decode_workspace_bytes(layer, w.T, w.k) > moe.noalloc_max_bytes()
    x = torch.zeros((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((w.T, w.E), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.layer_decode_noalloc(layer, x, lg, w.k)
    assert ei.value.status == 2  # MOE_EUNSUPPORTED
    assert "scratch" in str(ei.value)
