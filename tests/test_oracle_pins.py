"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something it does not compute itself:
library decoders of IEEE formats, hand-derived closed forms, brute force on
tiny inputs, or invariants of the mathematics.  Each is chosen so that a
plausible slip (a dropped term, a wrong sign, a swapped operand, a wrong bit
position) fails at least one of them.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests import _blob

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- number formats ---------------------------------------------------------

def test_f16_decode_matches_numpy_for_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero survives
    assert math.copysign(1.0, oracle.f16(0x8000)) == -1.0


def test_bf16_decode_matches_float32_upper_half_for_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ---- byte accounting -----------------------------------------------------------

def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([c.strip() for c in line.split("|")])
    return rows


def test_byte_accounting_matches_printed_q4_0_density():
    rows = _golden_rows("byte_accounting.txt")
    per_value = [r for r in rows if len(r) == 4 and not r[0].isdigit()]
    blobs = [r for r in rows if len(r) == 4 and r[0].isdigit()]
    for name, header, bits, bpv in per_value:
        assert (int(header) + 32 * int(bits) / 8) / 32 == float(bpv), name
    for H, I, bits, nbytes in blobs:
        H, I, bits, nbytes = int(H), int(I), int(bits), int(nbytes)
        assert oracle.blob_layout(H, I, bits)[6] == nbytes
        assert 3 * H * I * (bits / 8 + 4 / 32) == nbytes


def test_oracle_layout_matches_hand_layout():
    for H, I, bits in [(64, 32, 2), (64, 32, 4), (2048, 512, 2), (96, 64, 2), (32, 32, 4)]:
        assert oracle.blob_layout(H, I, bits) == _blob.layout(H, I, bits)


# ---- dequantization ---------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_every_code_position_decodes_to_its_own_column(bits):
    """A single nonzero code, swept over every column of a row, must decode at that column only."""
    H, I = 64, 32
    qmax = (1 << bits) - 1
    for mat in range(3):
        R, K = (I, H) if mat < 2 else (H, I)
        r = R // 2 + 1
        for c in range(K):
            q = (c % qmax) + 1
            mats = [_blob.constant_matrix(*((I, H) if m < 2 else (H, I)), 0, 1.0, 0.0) for m in range(3)]
            qm = mats[mat][0].copy()
            qm[r, c] = q
            mats[mat] = (qm, mats[mat][1], mats[mat][2])
            blob = _blob.build_blob(H, I, bits, mats)
            W = oracle.dequant(blob, H, I, bits, mat)
            expect = np.zeros((R, K))
            expect[r, c] = q
            assert np.array_equal(W, expect), (mat, c)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_scale_and_min_take_their_roles(bits):
    """W = s*q + m with s in the low half and m in the high half of the s/m word."""
    H, I = 64, 32
    s, m = 0.125, -0.375
    for q in range(1 << bits):
        mats = [_blob.constant_matrix(*((I, H) if k < 2 else (H, I)), q, s, m) for k in range(3)]
        blob = _blob.build_blob(H, I, bits, mats)
        for mat in range(3):
            W = oracle.dequant(blob, H, I, bits, mat)
            assert np.all(W == s * q + m)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_exactly_representable_blocks_round_trip(bits):
    """Blocks whose values are s*q + m with q spanning 0..qmax encode and decode exactly."""
    rng = np.random.default_rng(1)
    qmax = (1 << bits) - 1
    R, K = 8, 128
    s = 2.0 ** rng.integers(-9, -3, size=(R, K // 32))
    m = -(2.0 ** rng.integers(-6, -2, size=(R, K // 32)))
    q = rng.integers(0, qmax + 1, size=(R, K))
    q[:, ::32] = 0
    q[:, 1::32] = qmax
    w = np.repeat(s, 32, axis=1) * q + np.repeat(m, 32, axis=1)
    codes, sm = synth.quantize_matrix(w, bits)
    H, I = K, R  # the matrix is the Wg plane [I x H] of an expert
    off = oracle.blob_layout(H, I, bits)
    blob = np.zeros(off[6], np.uint8)
    cb, sb = codes.astype("<u4").tobytes(), sm.astype("<u4").tobytes()
    blob[off[0]:off[0] + len(cb)] = np.frombuffer(cb, np.uint8)
    blob[off[1]:off[1] + len(sb)] = np.frombuffer(sb, np.uint8)
    W = oracle.dequant(blob, H, I, bits, 0)
    assert np.array_equal(W, w)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_then_decode_error_within_half_step(bits):
    """|w - deq(quant(w))| <= s/2 plus the fp16 rounding of s and m."""
    qmax = (1 << bits) - 1
    H, I = 64, 32
    blob = synth.expert(0, 0, 3, H, I, bits, 0.02)
    for mat in range(3):
        R, K = (I, H) if mat < 2 else (H, I)
        key = synth.stream_key(0, synth.TAG_WEIGHT, 0, 3, mat)
        w = 0.02 * synth.normal(key, R * K).reshape(R, K)
        W = oracle.dequant(blob, H, I, bits, mat)
        blk_min = w.reshape(R, K // 32, 32).min(axis=2)
        blk_max = w.reshape(R, K // 32, 32).max(axis=2)
        step = (blk_max - blk_min) / qmax
        bound = 0.5 * step * (1 + 2.0 ** -8) + 2.0 ** -10 * (np.abs(blk_min) + qmax * step)
        err = np.abs(W - w).reshape(R, K // 32, 32).max(axis=2)
        assert np.all(err <= bound), (mat, float((err / bound).max()))


# ---- routing ------------------------------------------------------------------------

def _brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


def test_route_matches_brute_force_on_random_inputs():
    rng = np.random.default_rng(2)
    for E, k in [(8, 2), (17, 5), (64, 10), (130, 16), (512, 10)]:
        lg = rng.standard_normal((6, E)).astype(np.float32)
        lg[:, ::7] = np.round(lg[:, ::7])  # plant ties
        ids, w = oracle.route(lg, k)
        for t in range(lg.shape[0]):
            assert list(ids[t]) == _brute_topk(lg[t], k)


def test_route_exhaustive_ties():
    """Every logits vector in {-1, 0, 1}^6, every k: ties go to the lower id."""
    rows = np.array(list(itertools.product([-1.0, 0.0, 1.0], repeat=6)), np.float32)
    for k in range(1, 7):
        ids, _ = oracle.route(rows, k)
        for t in range(rows.shape[0]):
            assert list(ids[t]) == _brute_topk(rows[t], k)
            sel = set(ids[t])
            for a in sel:  # defining property: every kept key beats every dropped key
                for b in set(range(6)) - sel:
                    assert (rows[t, a] > rows[t, b]) or (rows[t, a] == rows[t, b] and a < b)


def test_route_signed_zero_is_a_tie():
    lg = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32)
    ids, w = oracle.route(lg, 2)
    assert ids.tolist() == [[0, 1], [0, 1]]
    assert np.all(w == 0.5)


def test_route_closed_form_golden():
    for k, lgs, ids_s, ws in _golden_rows("route_closed_form.txt"):
        k = int(k)
        lg = np.array([[math.log(float(tok[2:])) for tok in lgs.split()]], np.float32)
        ids, w = oracle.route(lg, k)
        assert ids[0].tolist() == [int(v) for v in ids_s.split()]
        exp = [float(Fraction(v)) for v in ws.split()]
        # fp32 logits of ln(n) carry ~6e-8 relative error into the weights
        assert np.allclose(w[0], exp, rtol=0, atol=1e-6)


def test_softmax_weights_invariants():
    rng = np.random.default_rng(3)
    lg = (np.round(rng.standard_normal((20, 64)) * 1024) / 1024).astype(np.float32)
    for k in [1, 2, 5, 10, 16]:
        ids, w = oracle.route(lg, k)
        assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 1e-15 * k)
        assert np.all(np.diff(w, axis=1) <= 0)  # descending logits -> non-increasing weights
        if k == 1:
            assert np.all(w == 1.0)
        ids2, w2 = oracle.route((lg + np.float32(1.0)).astype(np.float32), k)  # exact shift
        assert np.array_equal(ids, ids2) and np.array_equal(w, w2)
    eq = np.zeros((1, 12), np.float32)
    for k in range(1, 13):
        ids, w = oracle.route(eq, k)
        assert ids[0].tolist() == list(range(k))
        assert np.all(w == 1.0 / k)


# ---- dispatch ------------------------------------------------------------------------

def test_dispatch_is_the_stable_sort_by_expert():
    rng = np.random.default_rng(4)
    for T, k, E in [(1, 1, 1), (4, 2, 8), (3, 10, 512), (37, 6, 33), (200, 8, 16)]:
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
        d = oracle.dispatch(ids, E)
        flat = ids.reshape(-1)
        order = sorted(range(flat.size), key=lambda a: (flat[a], a))
        assert d["sorted_assign"].tolist() == order
        counts = np.bincount(flat, minlength=E)
        assert d["offsets"].tolist() == [0] + np.cumsum(counts).tolist()
        assert np.array_equal(d["assign_pos"][d["sorted_assign"]], np.arange(flat.size))
        assert d["active"].tolist() == [e for e in range(E) if counts[e] > 0]


def test_dispatch_rejects_out_of_range_ids():
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[0, 9]], np.int32), 8)


# ---- expert FFN closed forms ---------------------------------------------------------------

def _silu(z):
    return z / (1.0 + math.exp(-z))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_zero_input_gives_exactly_zero(bits):
    blob = synth.expert(0, 0, 1, 64, 32, bits, 0.02)
    h, y = oracle.expert_ffn(blob, 64, 32, bits, np.zeros(64))
    assert np.all(h == 0.0) and np.all(y == 0.0)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_constant_weight_expert_closed_form(bits):
    H, I = 96, 64
    (qg, sg, mg), (qu, su, mu), (qd, sd, md) = (1, 0.0625, -0.03125), (2, 0.03125, 0.015625), (1, 0.015625, -0.0625)
    cg, cu, cd = sg * qg + mg, su * qu + mu, sd * qd + md
    blob = _blob.build_blob(H, I, bits, [_blob.constant_matrix(I, H, qg, sg, mg), _blob.constant_matrix(I, H, qu, su, mu),
                                          _blob.constant_matrix(H, I, qd, sd, md)])
    x = np.random.default_rng(5).standard_normal(H)
    sx = x.sum()
    h, y = oracle.expert_ffn(blob, H, I, bits, x)
    h_ref = _silu(cg * sx) * (cu * sx)
    assert np.allclose(h, h_ref, rtol=1e-13, atol=0)
    assert np.allclose(y, cd * I * h_ref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("bits,with_min", [(2, False), (2, True), (3, False), (3, True), (4, False), (4, True)])
def test_identity_like_expert_closed_form(bits, with_min):
    """Wg, Wu pick one input column per row, Wd one h entry per output:
    y[n] = c * silu(a * x[pg[s[n]]]) * b * x[pu[s[n]]]."""
    H, I = 64, 32
    rng = np.random.default_rng(6)
    pg, pu = rng.permutation(H)[:I], rng.permutation(H)[:I]
    sel = rng.integers(0, I, size=H)
    a, b, c = 0.5, 2.0, -0.25
    blob = _blob.build_blob(H, I, bits, [_blob.one_hot_matrix(pg, H, a, bits, with_min),
                                          _blob.one_hot_matrix(pu, H, b, bits, with_min),
                                          _blob.one_hot_matrix(sel, I, c, bits, with_min)])
    x = rng.standard_normal(H)
    h, y = oracle.expert_ffn(blob, H, I, bits, x)
    h_ref = np.array([_silu(a * x[pg[i]]) * b * x[pu[i]] for i in range(I)])
    y_ref = np.array([c * h_ref[sel[n]] for n in range(H)])
    assert np.allclose(h, h_ref, rtol=1e-14, atol=0)
    assert np.allclose(y, y_ref, rtol=1e-14, atol=0)


# ---- whole layer ---------------------------------------------------------------------------

def _tiny():
    w = synth.tiny()
    return w, w.x(), w.logits(), w.experts()


def test_layer_k1_is_the_top_expert_alone():
    w, x, lg, ex = _tiny()
    r = oracle.layer(x, lg, ex, 1, w.H, w.I, w.bits)
    assert np.all(r["w"] == 1.0)
    for t in range(w.T):
        e = int(np.argmax(lg[t]))
        _, y = oracle.expert_ffn(ex[e], w.H, w.I, w.bits, x[t].astype(np.float64))
        assert np.array_equal(r["out"][t], y)


def test_layer_all_experts_equal_logits_is_the_mean():
    w, x, lg, ex = _tiny()
    eq = np.zeros_like(lg)
    r = oracle.layer(x, eq, ex, w.E, w.H, w.I, w.bits)
    for t in range(w.T):
        ys = np.stack([oracle.expert_ffn(ex[e], w.H, w.I, w.bits, x[t].astype(np.float64))[1] for e in range(w.E)])
        assert np.allclose(r["out"][t], ys.mean(axis=0), rtol=1e-13, atol=1e-15)


def test_layer_rows_are_independent_and_residual_adds():
    w, x, lg, ex = _tiny()
    res = np.random.default_rng(7).standard_normal((w.T, w.H))
    full = oracle.layer(x, lg, ex, w.k, w.H, w.I, w.bits, residual=res)
    for t in range(w.T):
        one = oracle.layer(x[t:t + 1], lg[t:t + 1], ex, w.k, w.H, w.I, w.bits)
        assert np.array_equal(one["ids"][0], full["ids"][t])
        # the oracle adds the residual first, then the k weighted rows
        assert np.allclose(one["out"][0] + res[t], full["out"][t], rtol=0, atol=4e-16 * (1 + np.abs(res[t])))


def test_layer_combine_is_the_weighted_sum_of_expert_rows():
    w, x, lg, ex = _tiny()
    r = oracle.layer(x, lg, ex, w.k, w.H, w.I, w.bits)
    for t in range(w.T):
        acc = np.zeros(w.H)
        for j in range(w.k):
            _, y = oracle.expert_ffn(ex[r["ids"][t, j]], w.H, w.I, w.bits, x[t].astype(np.float64))
            assert np.array_equal(r["y"][t, j], y)
            acc = acc + r["w"][t, j] * y
        assert np.array_equal(acc, r["out"][t])


def test_bf16_input_rows_decode_like_float32():
    w = synth.decode_verify()
    xb = w.x()[:, :64].copy()
    as_f32 = (xb.astype(np.uint32) << 16).view(np.float32)
    ex = synth.layer_experts(0, 0, 4, 64, 32, 2)
    lg = np.zeros((3, 4), np.float32)
    ra = oracle.layer(xb, lg, ex, 2, 64, 32, 2)
    rb = oracle.layer(as_f32, lg, ex, 2, 64, 32, 2)
    assert np.array_equal(ra["out"], rb["out"])


# ---- router projection ------------------------------------------------------

def _bf16_bits(values) -> np.ndarray:
    """Raw bf16 bits of values that bf16 holds exactly (checked)."""
    f = np.asarray(values, np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), f), "value not exact in bf16"
    return bits


def test_router_one_hot_rows_pick_their_column():
    rng = np.random.default_rng(7)
    T, H, E = 5, 96, 12
    cols = rng.permutation(H)[:E]
    wr = np.zeros((E, H), np.float32)
    wr[np.arange(E), cols] = 1.0
    x = rng.standard_normal((T, H)).astype(np.float32)
    got = oracle.router_logits(x, _bf16_bits(wr))
    assert np.array_equal(got, x[:, cols].astype(np.float64))


def test_router_constant_rows_scale_the_row_sum():
    rng = np.random.default_rng(8)
    T, H, E = 4, 64, 6
    c = np.array([0.5, -2.0, 3.0, 0.0, -0.25, 8.0], np.float32)
    wr = np.repeat(c[:, None], H, axis=1)
    x = rng.integers(-8, 9, (T, H)).astype(np.float32)  # small integers: every sum is exact
    got = oracle.router_logits(x, _bf16_bits(wr))
    want = np.outer(x.astype(np.float64).sum(axis=1), c.astype(np.float64))
    assert np.array_equal(got, want)


def test_router_swapping_operands_transposes_the_logits():
    key_a, key_b = synth.stream_key(3, synth.TAG_ROUTER, 1), synth.stream_key(3, synth.TAG_ROUTER, 2)
    a = synth.normal_bf16_bits(key_a, (7, 64))
    b = synth.normal_bf16_bits(key_b, (9, 64))
    ab = oracle.router_logits(a, b)
    ba = oracle.router_logits(b, a)
    assert ab.shape == (7, 9) and np.array_equal(ab, ba.T)


def test_router_is_linear_in_the_weights_and_tokens_are_independent():
    rng = np.random.default_rng(9)
    T, H, E = 6, 32, 5
    w1 = rng.integers(-4, 5, (E, H)).astype(np.float32)
    w2 = rng.integers(-4, 5, (E, H)).astype(np.float32)
    x = rng.integers(-6, 7, (T, H)).astype(np.float32)
    l1 = oracle.router_logits(x, _bf16_bits(w1))
    l2 = oracle.router_logits(x, _bf16_bits(w2))
    l12 = oracle.router_logits(x, _bf16_bits(w1 + w2))
    assert np.array_equal(l1 + l2, l12)
    # a token's logits do not depend on the other tokens
    assert np.array_equal(oracle.router_logits(x[2:3], _bf16_bits(w1)), l1[2:3])


def test_router_bf16_tokens_decode_like_float32():
    key = synth.stream_key(4, synth.TAG_X, 0)
    xb = synth.normal_bf16_bits(key, (3, 64))
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    wr = synth.normal_bf16_bits(synth.stream_key(4, synth.TAG_ROUTER, 0), (10, 64))
    assert np.array_equal(oracle.router_logits(xb, wr), oracle.router_logits(xf, wr))


# ---- the threaded driver --------------------------------------------------------

@pytest.mark.parametrize("nthreads", [2, 3, 8])
def test_threaded_layer_equals_single_thread_bit_for_bit(nthreads):
    # E = 3, k = 2, T = 450: every expert gets more rows than one work item
    # holds (256), so items of one expert are split across threads
    w = synth.Workload("mt", E=3, k=2, H=64, I=32, T=450, bits=3, x_dtype="bf16", zipf_s=0.0, seed=4)
    x, lg, ex = w.x(), w.logits(), w.experts()
    res = np.random.default_rng(1).standard_normal((w.T, w.H))
    one = oracle.layer(x, lg, ex, w.k, w.H, w.I, w.bits, residual=res)
    assert np.bincount(one["ids"].reshape(-1), minlength=w.E).min() > 256
    many = oracle.layer(x, lg, ex, w.k, w.H, w.I, w.bits, residual=res, nthreads=nthreads)
    for key in ("ids", "w", "y", "out"):
        assert np.array_equal(one[key], many[key]), key
    no_y = oracle.layer(x, lg, ex, w.k, w.H, w.I, w.bits, residual=res, nthreads=nthreads, want_y=False)
    assert np.array_equal(one["out"], no_y["out"])
