"""The C ABI library loads without a GPU, exports what include/moe.h declares, and
rejects bad arguments on the host before enqueueing anything."""
import ctypes

import pytest

import expert_routed_ffn_amd as m
from expert_routed_ffn_amd import _lib

L = _lib.lib


def test_every_declared_function_is_exported():
    names = m.header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    assert m.abi_version() == 1
    assert L.moe_status_string(0) == b"MOE_OK"
    assert L.moe_status_string(6) == b"MOE_ECAPACITY"


def test_expert_bytes_formula():
    for H, I, b in [(2048, 512, 2), (2048, 512, 3), (2048, 512, 4), (64, 32, 2), (96, 64, 3), (96, 64, 4)]:
        assert m.expert_bytes(H, I, b) % 256 == 0
        assert m.expert_bytes(H, I, b) >= 3 * H * I * (b / 8 + 4 / 32)
    assert m.expert_bytes(2048, 512, 2) == 1179648
    assert m.expert_bytes(2048, 512, 3) == 1572864  # 3 * 2048 * 512 * (3/8 + 1/8)
    assert m.expert_bytes(2048, 512, 5) == 0  # unsupported width
    assert m.expert_bytes(2048, 512, 1) == 0


NULL = None


def _st(v):
    return int(v)


@pytest.mark.parametrize("E,k,expect", [(0, 1, _lib.MOE_EUNSUPPORTED), (1025, 2, _lib.MOE_EUNSUPPORTED),
                                        (8, 0, _lib.MOE_EUNSUPPORTED), (8, 17, _lib.MOE_EUNSUPPORTED),
                                        (4, 5, _lib.MOE_EUNSUPPORTED), (8, 2, _lib.MOE_EINVAL)])
def test_route_topk_argument_checks(E, k, expect):
    # T = 3 with null pointers: either the sizes or the pointers are rejected on the host.
    assert _st(L.moe_route_topk(NULL, 3, E, k, NULL, NULL, NULL)) == expect
    assert b"moe_route_topk" in L.moe_last_error()


def test_route_topk_negative_T():
    assert _st(L.moe_route_topk(NULL, -1, 8, 2, NULL, NULL, NULL)) == _lib.MOE_EINVAL


def test_zero_tokens_is_a_no_op():
    assert _st(L.moe_route_topk(NULL, 0, 8, 2, NULL, NULL, NULL)) == _lib.MOE_OK


def test_dispatch_argument_checks():
    fake = ctypes.c_void_p(0x1000)
    assert _st(L.moe_dispatch(NULL, 3, 2, 8, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL)) == _lib.MOE_EINVAL
    # large n needs a workspace
    need = int(L.moe_dispatch_workspace_bytes(8192, 10, 512))
    assert need > 0
    assert int(L.moe_dispatch_workspace_bytes(3, 10, 512)) == 0
    st = L.moe_dispatch(fake, 8192, 10, 512, fake, fake, fake, fake, fake, fake, need - 1, NULL)
    assert _st(st) == _lib.MOE_EWORKSPACE


def _q(E=8, H=64, I=32, bits=2, base=0x100, stride=None):
    return _lib.QLayer(E, H, I, bits, base, stride if stride is not None else m.expert_bytes(H, I, bits), None)


def test_expert_ffn_argument_checks():
    fake = ctypes.c_void_p(0x1000)

    def call(q, T=2, k=2, x_t=1, y_t=0, path=0, ws_bytes=1 << 20, x=fake):
        return _st(L.moe_expert_ffn_q(ctypes.byref(q), x, x_t, T, k, fake, fake, fake, fake, fake, y_t, path, fake,
                                      ws_bytes, NULL))

    assert call(_q(bits=5)) == _lib.MOE_EUNSUPPORTED
    assert call(_q(bits=1)) == _lib.MOE_EUNSUPPORTED
    assert call(_q(H=48)) == _lib.MOE_EUNSUPPORTED
    assert call(_q(I=16)) == _lib.MOE_EUNSUPPORTED
    assert call(_q(stride=100)) == _lib.MOE_EINVAL
    assert call(_q(base=0x101)) == _lib.MOE_EINVAL
    assert call(_q(), x=ctypes.c_void_p(0x1004)) == _lib.MOE_EINVAL
    assert call(_q(), x_t=7) == _lib.MOE_EINVAL
    assert call(_q(), path=9) == _lib.MOE_EINVAL
    assert call(_q(), ws_bytes=0) == _lib.MOE_EWORKSPACE
    assert call(_q(), T=0) == _lib.MOE_OK


def test_combine_argument_checks():
    fake = ctypes.c_void_p(0x1000)
    assert _st(L.moe_combine(NULL, 0, NULL, 2, 2, 64, NULL, 0, NULL, NULL, NULL)) == _lib.MOE_EINVAL
    assert _st(L.moe_combine(fake, 0, fake, 2, 17, 64, NULL, 0, fake, NULL, NULL)) == _lib.MOE_EUNSUPPORTED
    assert _st(L.moe_combine(fake, 0, fake, 2, 2, 66, NULL, 0, fake, NULL, NULL)) == _lib.MOE_EUNSUPPORTED
    assert _st(L.moe_combine(fake, 5, fake, 2, 2, 64, NULL, 0, fake, NULL, NULL)) == _lib.MOE_EINVAL


def test_layer_decode_argument_checks():
    fake = ctypes.c_void_p(0x1000)
    q = _q()
    def call(T=3, k=2, ws_bytes=1 << 20):
        return _st(L.moe_layer_decode(ctypes.byref(q), fake, fake, 1, T, k, None, 0, fake, fake, fake, fake, fake,
                                      fake, fake, fake, 0, fake, None, ctypes.c_void_p(0x100000), ws_bytes, None))
    assert call(T=13) == _lib.MOE_EUNSUPPORTED
    assert call(k=17) == _lib.MOE_EUNSUPPORTED
    assert call(T=0) == _lib.MOE_OK
    assert call(ws_bytes=0) == _lib.MOE_EWORKSPACE
    assert int(L.moe_layer_decode_workspace_bytes(ctypes.byref(q), 3, 2)) > 0


def test_auto_path_workspace_follows_routed_rows():
    """AUTO sizes its workspace for GEMV up to 128 routed rows (T * k) and for MFMA above."""
    q = _q(E=512, H=2048, I=512)
    ws = lambda T, k, p: int(L.moe_expert_ffn_workspace_bytes(ctypes.byref(q), T, k, p))
    AUTO, GEMV, MFMA = 0, 1, 2
    for T, k in [(1, 10), (12, 10), (16, 8), (13, 10), (16, 10), (32, 8), (8192, 10)]:
        want = GEMV if T * k <= 128 else MFMA
        assert ws(T, k, AUTO) == ws(T, k, want), (T, k)
    assert ws(26, 10, GEMV) != ws(26, 10, MFMA)


def test_router_argument_checks():
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1008)  # 8-byte aligned only
    F32, BF16 = _lib.MOE_F32, _lib.MOE_BF16
    assert _st(L.moe_router_logits(NULL, BF16, NULL, -1, 64, 8, NULL, NULL)) == _lib.MOE_EINVAL
    assert _st(L.moe_router_logits(NULL, 7, NULL, 3, 64, 8, NULL, NULL)) == _lib.MOE_EINVAL
    assert _st(L.moe_router_logits(NULL, BF16, NULL, 3, 64, 0, NULL, NULL)) == _lib.MOE_EUNSUPPORTED
    assert _st(L.moe_router_logits(NULL, BF16, NULL, 3, 64, 1025, NULL, NULL)) == _lib.MOE_EUNSUPPORTED
    assert _st(L.moe_router_logits(NULL, BF16, NULL, 3, 48, 8, NULL, NULL)) == _lib.MOE_EUNSUPPORTED
    assert _st(L.moe_router_logits(NULL, F32, NULL, 3, 32768, 8, NULL, NULL)) == _lib.MOE_EUNSUPPORTED
    assert _st(L.moe_router_logits(NULL, BF16, NULL, 0, 64, 8, NULL, NULL)) == _lib.MOE_OK
    assert _st(L.moe_router_logits(fake, BF16, NULL, 3, 64, 8, fake, NULL)) == _lib.MOE_EINVAL
    assert _st(L.moe_router_logits(odd, BF16, fake, 3, 64, 8, fake, NULL)) == _lib.MOE_EINVAL
    assert b"aligned" in L.moe_last_error()
    # the top-k wrapper checks E and k first, then the projection's arguments
    assert _st(L.moe_router_topk(fake, BF16, fake, 3, 64, 8, 9, fake, fake, fake, NULL)) == _lib.MOE_EUNSUPPORTED
    assert _st(L.moe_router_topk(fake, BF16, fake, 3, 64, 8, 2, fake, NULL, fake, NULL)) == _lib.MOE_EINVAL
    assert _st(L.moe_router_topk(fake, BF16, fake, 3, 48, 8, 2, fake, fake, fake, NULL)) == _lib.MOE_EUNSUPPORTED
    assert _st(L.moe_router_topk(NULL, BF16, NULL, 0, 64, 8, 2, NULL, NULL, NULL, NULL)) == _lib.MOE_OK
