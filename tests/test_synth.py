"""Checks of the seeded input generators (they feed both the oracle and the GPU path)."""
import numpy as np

import synth


def test_streams_are_deterministic_and_independent():
    k1 = synth.stream_key(0, synth.TAG_WEIGHT, 1, 2, 0)
    k2 = synth.stream_key(0, synth.TAG_WEIGHT, 1, 2, 1)
    a = synth.normal(k1, 1000)
    assert np.array_equal(a, synth.normal(k1, 1000))
    assert np.array_equal(a[500:], synth.normal(k1, 500, first=500))  # counter-based: any slice alone
    b = synth.normal(k2, 1000)
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.1


def test_normal_and_uniform_moments():
    key = synth.stream_key(3, synth.TAG_X)
    u = synth.uniform(key, 200000)
    assert u.min() > 0.0 and u.max() < 1.0 and abs(u.mean() - 0.5) < 0.005
    z = synth.normal(key, 200000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01


def test_f16_encoder_rounds_like_numpy():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
                           [0.0, -0.0, 65504.0, 65519.9, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 6.1e-5]])
    with np.errstate(over="ignore"):
        ref = np.array(vals, np.float64).astype(np.float16).view(np.uint16)
    for v, r in zip(vals, ref):
        assert synth.f64_to_f16_bits(v) == int(r), v


def test_bf16_activations_are_rne_of_fp32():
    key = synth.stream_key(0, synth.TAG_X)
    bits = synth.normal_bf16_bits(key, (4, 256))
    f32 = synth.normal_f32(key, (4, 256))
    u = f32.view(np.uint32).astype(np.uint64)
    lo = u & 0xFFFF
    hi = u >> 16
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    ref = (hi + up).astype(np.uint16)
    assert np.array_equal(bits, ref)


def test_zipf_bias_is_a_permuted_log_rank():
    key = synth.stream_key(0, synth.TAG_RANK)
    r = synth.ranks(key, 512)
    assert sorted(r.tolist()) == list(range(1, 513))
    b = synth.zipf_bias(key, 512, 1.1)
    assert np.allclose(b, (-1.1 * np.log(r)).astype(np.float32), rtol=0, atol=0)


def test_layer_generation_matches_single_expert_and_threads():
    a = synth.layer_experts(0, 2, 6, 64, 32, 2, nthreads=1)
    b = synth.layer_experts(0, 2, 6, 64, 32, 2, nthreads=4)
    assert np.array_equal(a, b)
    assert np.array_equal(a[4], synth.expert(0, 2, 4, 64, 32, 2))
    c = synth.layer_experts(0, 2, 6, 64, 32, 2, which=[1, 4])
    assert np.array_equal(c[4], a[4]) and np.array_equal(c[1], a[1]) and not c[0].any()


def test_drift_walk_matches_drifted_bias():
    w = synth.stack125b()
    walk = synth.drift_walk(w, 3, 6, 0.05)
    for s in range(6):
        assert np.array_equal(walk[s], synth.drifted_bias(w, 3, s, 0.05))
    assert not np.array_equal(walk[0], walk[5])


def test_router_weights_are_seeded_bf16_with_unit_logit_variance():
    w = synth.decode_verify()
    a, b = w.router(0), w.router(0)
    assert a.dtype == np.uint16 and a.shape == (w.E, w.H)
    assert np.array_equal(a, b) and not np.array_equal(a, w.router(1))
    vals = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # N(0, 1/H) entries: H * var is 1 within sampling error
    assert abs(vals.var() * w.H - 1.0) < 0.01
