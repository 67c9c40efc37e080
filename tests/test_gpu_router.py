"""GPU parity of the router projection (logits = x . Wr^T) against the oracle.

The oracle sums in fp64.  The GPU adds bf16 products (exact in fp32) or fused
fp32 products in fp32, in whatever order its kernel uses; for any order of H
such additions the error is at most gamma_H * sum_c |x_c w_c| with
gamma_H = H u / (1 - H u), u = 2^-24.  That bound is the tolerance, per logit.
The routing that follows the projection must equal the oracle's routing of
the GPU's own logits bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from tests._parity import to_dev_x, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_routed_ffn_amd as m
    return m


def _values(x):
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if x.dtype == np.uint16 else \
        x.astype(np.float64)


def _bound(x, wr):
    """gamma_H * sum_c |x_c w_c| for every (t, e)."""
    H = x.shape[1]
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    return gamma * (np.abs(_values(x)) @ np.abs(_values(wr)).T)


def _inputs(T, E, H, x_dtype, seed):
    key_x = synth.stream_key(seed, synth.TAG_X, T, H)
    key_w = synth.stream_key(seed, synth.TAG_ROUTER, E, H)
    x = synth.normal_f32(key_x, (T, H)) if x_dtype == "f32" else synth.normal_bf16_bits(key_x, (T, H))
    wr = synth.normal_bf16_bits_scaled(key_w, (E, H), 1.0 / np.sqrt(H))
    return x, wr


def _dev_x(x):
    return to_dev_x(x)


def _dev_w(wr):
    return to_dev_x(wr)


# (T, E, H, x dtype): decode shape (GEMV), tiny fp32, MFMA with ragged T and E
# and an odd K-step count, fp32 over several token tiles with E not a multiple
# of 4, the smallest MFMA case, a single expert
CASES = [(3, 512, 2048, "bf16"), (4, 8, 64, "f32"), (130, 600, 96, "bf16"), (70, 37, 160, "f32"),
         (64, 7, 32, "bf16"), (17, 1, 32, "bf16"), (200, 1024, 256, "bf16"), (16, 100, 16384, "bf16")]


@pytest.mark.parametrize("T,E,H,x_dtype", CASES)
def test_router_logits_within_the_summation_bound(moe, T, E, H, x_dtype):
    x, wr = _inputs(T, E, H, x_dtype, seed=11)
    got = to_host(moe.router_logits(_dev_x(x), _dev_w(wr))).astype(np.float64)
    ref = oracle.router_logits(x, wr)
    assert got.shape == (T, E)
    assert np.all(np.abs(got - ref) <= _bound(x, wr))


def test_router_logits_prefill_chunk_sampled(moe):
    """Full prefill size (T = 8,192, MFMA path): 64 sampled tokens, every expert."""
    w = synth.prefill()
    x, wr = w.x(), w.router()
    got = to_host(moe.router_logits(_dev_x(x), _dev_w(wr))).astype(np.float64)
    rows = np.unique(np.concatenate([np.arange(0, w.T, w.T // 48), [1, 127, 128, w.T - 129, w.T - 2, w.T - 1]]))
    ref = oracle.router_logits(x[rows], wr)
    assert np.all(np.abs(got[rows] - ref) <= _bound(x[rows], wr))
    # unit-variance logits, as the generator intends
    assert 0.8 < got.std() < 1.2


@pytest.mark.parametrize("T,E,H,k,x_dtype", [(3, 512, 2048, 10, "bf16"), (96, 256, 512, 8, "bf16"),
                                             (5, 64, 128, 16, "f32")])
def test_router_topk_routes_its_own_logits(moe, T, E, H, k, x_dtype):
    x, wr = _inputs(T, E, H, x_dtype, seed=5)
    logits, ids, w = moe.router_topk(_dev_x(x), _dev_w(wr), k)
    lg = to_host(logits)
    ref_ids, ref_w = oracle.route(lg, k)
    assert np.array_equal(to_host(ids), ref_ids)
    assert np.abs(to_host(w) - ref_w).max() <= 1e-6
    assert np.all(np.abs(lg.astype(np.float64) - oracle.router_logits(x, wr)) <= _bound(x, wr))


def test_router_logits_repeatable_and_rows_independent(moe):
    x, wr = _inputs(150, 300, 256, "bf16", seed=3)
    a = to_host(moe.router_logits(_dev_x(x), _dev_w(wr)))
    b = to_host(moe.router_logits(_dev_x(x), _dev_w(wr)))
    assert np.array_equal(a, b)
    # the first 64 tokens alone take the same MFMA path: same bits
    c = to_host(moe.router_logits(_dev_x(np.ascontiguousarray(x[:64])), _dev_w(wr)))
    assert np.array_equal(c, a[:64])
