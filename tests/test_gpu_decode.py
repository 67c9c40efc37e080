"""GPU parity of the decode / verify path against the CPU oracle.

Routing and dispatch must be bit-exact; expert outputs and layer outputs must
be within DECODE_TOL in the per-row metric max|d| / max|ref| (fp32 path).
"""
import numpy as np
import pytest

import oracle
import synth
from tests._parity import routed_experts, row_rel_err, to_dev, to_dev_x, to_host

pytestmark = pytest.mark.gpu

DECODE_TOL = 2e-3   # layer-output tolerance for the fp32 GEMV path
W_TOL = 1e-6        # fp32 softmax weights vs fp64


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_routed_ffn_amd as m
    return m


def _route_case(kind, T, E, k, seed=0):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":
        return np.round(rng.standard_normal((T, E)) * 2).astype(np.float32) / 2
    if kind == "zeros":
        lg = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0], np.float32), size=(T, E))
        return lg.astype(np.float32)
    if kind == "equal":
        return np.zeros((T, E), np.float32)
    raise ValueError(kind)


ROUTE_CASES = [("normal", 4, 8, 2), ("normal", 3, 512, 10), ("ties", 64, 512, 10), ("zeros", 33, 100, 16),
               ("equal", 5, 1024, 16), ("normal", 7, 1000, 16), ("normal", 9, 64, 1), ("ties", 17, 65, 7),
               ("normal", 1, 1, 1), ("ties", 300, 37, 5)]


@pytest.mark.parametrize("kind,T,E,k", ROUTE_CASES)
def test_route_topk_bit_exact(moe, kind, T, E, k):
    lg = _route_case(kind, T, E, k)
    ids, w = moe.route_topk(to_dev(lg), k)
    ref_ids, ref_w = oracle.route(lg, k)
    assert np.array_equal(to_host(ids), ref_ids)
    assert np.abs(to_host(w) - ref_w).max() <= W_TOL


def test_route_topk_prefill_logits(moe):
    w = synth.prefill()
    lg = w.logits()
    ids, wt = moe.route_topk(to_dev(lg), w.k)
    ref_ids, ref_w = oracle.route(lg, w.k)
    assert np.array_equal(to_host(ids), ref_ids)
    assert np.abs(to_host(wt) - ref_w).max() <= W_TOL


def _check_dispatch(moe, ids_np, E):
    import torch
    d = moe.dispatch(to_dev(ids_np), E)
    torch.cuda.synchronize()
    n = ids_np.size
    ref = oracle.dispatch(np.clip(ids_np, 0, E - 1), E) if ids_np.size else None
    valid = (ids_np >= 0) & (ids_np < E)
    if valid.all():
        assert np.array_equal(to_host(d.offsets), ref["offsets"])
        assert np.array_equal(to_host(d.sorted_assign)[:n], ref["sorted_assign"])
        assert np.array_equal(to_host(d.assign_pos)[:n], ref["assign_pos"])
        na = int(to_host(d.n_active)[0])
        assert na == ref["n_active"]
        assert np.array_equal(to_host(d.active)[:na], ref["active"])
    return d


@pytest.mark.parametrize("T,k,E", [(3, 10, 512), (4, 2, 8), (1, 1, 1), (409, 10, 512), (410, 10, 512),
                                   (512, 8, 256), (8192, 10, 512), (1000, 16, 1024), (2048, 2, 3)])
def test_dispatch_bit_exact(moe, T, k, E):
    rng = np.random.default_rng(T * 131 + k)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    ids = rng.choice(E, size=(T, k), p=p / p.sum()).astype(np.int32)
    _check_dispatch(moe, ids, E)


def test_dispatch_from_routed_prefill(moe):
    w = synth.prefill(0.21)
    ids, _ = oracle.route(w.logits(), w.k)
    _check_dispatch(moe, ids, w.E)


@pytest.mark.parametrize("T,k", [(3, 10), (600, 10)])
def test_dispatch_drops_out_of_range_ids(moe, T, k):
    E = 64
    rng = np.random.default_rng(5)
    ids = rng.integers(-3, E + 3, size=(T, k)).astype(np.int32)
    d = moe.dispatch(to_dev(ids), E)
    flat = ids.reshape(-1)
    ok = (flat >= 0) & (flat < E)
    keep = np.nonzero(ok)[0]
    order = keep[np.argsort(flat[keep], kind="stable")]
    n_ok = int(ok.sum())
    assert int(to_host(d.offsets)[E]) == n_ok
    assert np.array_equal(to_host(d.sorted_assign)[:n_ok], order)
    ap = to_host(d.assign_pos)[:flat.size]
    assert np.all(ap[~ok] == -1)
    assert np.array_equal(ap[order], np.arange(n_ok))


def _run_layer(moe, w: synth.Workload, x, lg, ex, path="gemv", y_dtype=None, residual=None):
    import torch
    base = to_dev(ex)
    layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, base)
    ids, wt, d, y, out = moe.layer_forward(layer, to_dev_x(x), to_dev(lg), w.k, residual=residual,
                                           path=path, y_dtype=y_dtype or torch.float32)
    torch.cuda.synchronize()
    return {"ids": to_host(ids), "w": to_host(wt), "y": to_host(y), "out": to_host(out), "d": d}


def _check_layer(moe, w, x, lg, ex, tol, path="gemv"):
    got = _run_layer(moe, w, x, lg, ex, path)
    ref = oracle.layer(x, lg, ex, w.k, w.H, w.I, w.bits)
    assert np.array_equal(got["ids"], ref["ids"])
    assert np.abs(got["w"] - ref["w"]).max() <= W_TOL
    ey = row_rel_err(got["y"], ref["y"])
    eo = row_rel_err(got["out"], ref["out"])
    print(f"{w.name}: y err {ey:.3e}, out err {eo:.3e}")
    assert ey <= tol and eo <= tol
    return got, ref


def test_layer_tiny(moe):
    w = synth.tiny()
    _check_layer(moe, w, w.x(), w.logits(), w.experts(), DECODE_TOL)


def test_layer_decode_verify(moe):
    w = synth.decode_verify()
    lg = w.logits()
    _check_layer(moe, w, w.x(), lg, routed_experts(w, lg), DECODE_TOL)


@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_layer_decode_sweep_4bit(moe, T):
    w = synth.decode_sweep(T)
    for layer in (0, 1):
        lg = w.logits(layer)
        _check_layer(moe, w, w.x(layer), lg, routed_experts(w, lg, layer), DECODE_TOL)


def _custom(E, k, H, I, T, bits, x_dtype="bf16", zipf=0.0, seed=3):
    return synth.Workload(f"custom_E{E}_k{k}_H{H}_I{I}_T{T}_b{bits}", E=E, k=k, H=H, I=I, T=T, bits=bits,
                          x_dtype=x_dtype, zipf_s=zipf, seed=seed)


@pytest.mark.parametrize("E,k,H,I,T,bits,x_dtype", [
    (16, 4, 96, 64, 3, 2, "bf16"),      # 3 chunks per row: one lane per row
    (8, 2, 4096, 1024, 2, 2, "bf16"),   # two chunks per lane
    (8, 2, 4096, 1024, 2, 4, "f32"),
    (1024, 16, 64, 32, 5, 4, "bf16"),   # largest E and k
    (32, 3, 160, 96, 7, 2, "f32"),      # odd chunk counts, fp32 input
    (4, 1, 128, 64, 1, 4, "bf16"),
    (64, 8, 2048, 512, 3, 3, "bf16"),   # 3-bit codes: wide kernels
    (16, 4, 96, 64, 5, 3, "f32"),       # 3-bit codes: general kernels, fp32 input
    (32, 3, 160, 96, 7, 3, "bf16"),
])
def test_layer_gemv_shapes(moe, E, k, H, I, T, bits, x_dtype):
    w = _custom(E, k, H, I, T, bits, x_dtype)
    _check_layer(moe, w, w.x(), w.logits(), w.experts(), DECODE_TOL)


@pytest.mark.parametrize("T", [5, 8, 13])
def test_layer_gemv_many_rows_per_expert(moe, T):
    """Every token routes to the same experts: rows are processed in several passes."""
    w = _custom(8, 2, 256, 128, T, 2)
    lg = np.tile(np.array([[3.0, 2.0, 0, 0, 0, 0, 0, 0]], np.float32), (T, 1))
    _check_layer(moe, w, w.x(), lg, w.experts(), DECODE_TOL)


def test_combine_residual_and_bf16_out(moe):
    import torch
    rng = np.random.default_rng(9)
    T, k, H = 5, 3, 256
    y = rng.standard_normal((T, k, H)).astype(np.float32)
    wt = rng.random((T, k)).astype(np.float32)
    res = rng.standard_normal((T, H)).astype(np.float32)
    out_b = torch.empty((T, H), dtype=torch.int16, device="cuda")
    out = moe.combine(to_dev(y), to_dev(wt), residual=to_dev(res), out_bf16=out_b)
    ref = oracle.combine(y.astype(np.float64), wt.astype(np.float64), res.astype(np.float64))
    got = to_host(out)
    assert np.abs(got - ref).max() <= 1e-5 * (1 + np.abs(ref).max())
    gb = to_host(out_b).view(np.uint16)
    # bf16 round-to-nearest-even of the fp32 result
    u = got.view(np.uint32).astype(np.uint64)
    up = ((u & 0xFFFF) > 0x8000) | (((u & 0xFFFF) == 0x8000) & (((u >> 16) & 1) == 1))
    assert np.array_equal(gb, ((u >> 16) + up).astype(np.uint16))
    # bf16 residual and bf16 y
    res_b = torch.from_numpy(res).cuda().to(torch.bfloat16)
    y_b = torch.from_numpy(y).cuda().to(torch.bfloat16)
    out2 = moe.combine(y_b, to_dev(wt), residual=res_b)
    ref2 = oracle.combine(to_host(y_b).astype(np.float64), wt.astype(np.float64), to_host(res_b).astype(np.float64))
    assert np.abs(to_host(out2) - ref2).max() <= 1e-5 * (1 + np.abs(ref2).max())


def test_layer_is_deterministic_and_rows_independent(moe):
    w = synth.decode_verify()
    lg = w.logits()
    ex = routed_experts(w, lg)
    x = w.x()
    a = _run_layer(moe, w, x, lg, ex)
    b = _run_layer(moe, w, x, lg, ex)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["y"], b["y"])
    for t in range(w.T):
        one = _run_layer(moe, synth.Workload("one", w.E, w.k, w.H, w.I, 1, w.bits, w.x_dtype), x[t:t + 1],
                         lg[t:t + 1], ex)
        assert np.array_equal(one["out"][0], a["out"][t])


def test_not_resident_expert_gives_nan_rows(moe):
    import torch
    w = _custom(8, 2, 64, 32, 2, 2)
    lg = np.array([[5.0, 4.0, 0, 0, 0, 0, 0, 0], [0, 0, 5.0, 4.0, 0, 0, 0, 0]], np.float32)
    ex = w.experts()
    base = to_dev(ex)
    smap = torch.tensor([0, 1, -1, 3, 4, 5, 6, 7], dtype=torch.int32, device="cuda")
    layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, base, slot_map=smap)
    ids, wt, d, y, out = moe.layer_forward(layer, to_dev_x(w.x()), to_dev(lg), w.k)
    yy = to_host(y)
    assert np.all(np.isnan(yy[1, 0])) and np.all(np.isfinite(yy[0])) and np.all(np.isfinite(yy[1, 1]))


# ---- fused decode step: moe_layer_decode --------------------------------------------

def _four_calls_and_fused(moe, w, x, lg, ex, residual=None, y_dtype=None, out_bf16=False):
    import torch
    y_dtype = y_dtype or torch.float32
    base = to_dev(ex)
    layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, base)
    xd, ld = to_dev_x(x), to_dev(lg)
    res = None if residual is None else residual
    ob4 = torch.zeros((w.T, w.H), dtype=torch.int16, device="cuda") if out_bf16 else None
    obf = torch.zeros((w.T, w.H), dtype=torch.int16, device="cuda") if out_bf16 else None
    a = moe.layer_forward(layer, xd, ld, w.k, residual=res, path="gemv", y_dtype=y_dtype, out_bf16=ob4)
    b = moe.layer_decode(layer, xd, ld, w.k, residual=res, y_dtype=y_dtype, out_bf16=obf)
    torch.cuda.synchronize()
    return a, b, ob4, obf


def _assert_bit_identical(a, b, n):
    ids_a, w_a, d_a, y_a, o_a = a
    ids_b, w_b, d_b, y_b, o_b = b
    assert np.array_equal(to_host(ids_a), to_host(ids_b))
    assert np.array_equal(to_host(w_a).view(np.uint32), to_host(w_b).view(np.uint32))
    for f in ("offsets", "sorted_assign", "assign_pos", "active", "n_active"):
        ta, tb = to_host(getattr(d_a, f)), to_host(getattr(d_b, f))
        if f in ("sorted_assign", "assign_pos"):
            ta, tb = ta[:n], tb[:n]
        if f == "active":
            na = int(to_host(d_a.n_active)[0])
            ta, tb = ta[:na], tb[:na]
        assert np.array_equal(ta, tb), f
    ya, yb = to_host(y_a), to_host(y_b)
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32))
    assert np.array_equal(to_host(o_a).view(np.uint32), to_host(o_b).view(np.uint32))


@pytest.mark.parametrize("case", ["tiny", "decode_verify", "verify4", "verify5", "verify6", "sweep1", "sweep2", "sweep4",
                                  "sweep8"])
def test_layer_decode_bit_identical_to_four_calls(moe, case):
    if case == "tiny":
        w = synth.tiny()
        lg = w.logits()
        ex = w.experts()
    elif case.startswith("verify"):  # 2-bit, bf16 x, four or six tokens: the four-rows-per-wave routed kernel
        w = synth.Workload(f"verify_T{case[6:]}", E=512, k=10, H=2048, I=512, T=int(case[6:]), bits=2,
                           x_dtype="bf16", zipf_s=1.1)
        lg = w.logits()
        ex = routed_experts(w, lg)
    else:
        w = synth.decode_verify() if case == "decode_verify" else synth.decode_sweep(int(case[5:]))
        lg = w.logits()
        ex = routed_experts(w, lg)
    x = w.x()
    a, b, _, _ = _four_calls_and_fused(moe, w, x, lg, ex)
    _assert_bit_identical(a, b, w.T * w.k)
    ref = oracle.layer(x, lg, ex, w.k, w.H, w.I, w.bits)
    assert row_rel_err(to_host(b[4]), ref["out"]) <= DECODE_TOL


@pytest.mark.parametrize("r_dtype,y_bf16", [("f32", False), ("bf16", True)])
def test_layer_decode_residual_bf16_outputs(moe, r_dtype, y_bf16):
    import torch
    w = synth.decode_verify()
    lg = w.logits()
    ex = routed_experts(w, lg)
    x = w.x()
    xr = to_dev_x(x)
    res = xr if r_dtype == "bf16" else xr.float()
    a, b, ob4, obf = _four_calls_and_fused(moe, w, x, lg, ex, residual=res,
                                           y_dtype=torch.bfloat16 if y_bf16 else torch.float32, out_bf16=True)
    _assert_bit_identical(a, b, w.T * w.k)
    assert np.array_equal(to_host(ob4), to_host(obf))


@pytest.mark.parametrize("E,k,H,I,T,bits,x_dtype", [
    (16, 4, 96, 64, 3, 2, "bf16"),
    (8, 2, 4096, 1024, 2, 4, "f32"),
    (1024, 16, 64, 32, 5, 4, "bf16"),
    (32, 3, 160, 96, 7, 2, "f32"),
    (8, 2, 256, 128, 12, 2, "bf16"),
    (512, 10, 2048, 512, 3, 3, "bf16"),  # 3-bit codes through the routed gate/up launch
    (48, 6, 96, 64, 4, 3, "f32"),
])
def test_layer_decode_shapes(moe, E, k, H, I, T, bits, x_dtype):
    w = _custom(E, k, H, I, T, bits, x_dtype)
    x, lg, ex = w.x(), w.logits(), w.experts()
    a, b, _, _ = _four_calls_and_fused(moe, w, x, lg, ex)
    _assert_bit_identical(a, b, w.T * w.k)
    ref = oracle.layer(x, lg, ex, w.k, w.H, w.I, w.bits)
    assert row_rel_err(to_host(b[4]), ref["out"]) <= DECODE_TOL


@pytest.mark.parametrize("E,k,T,x_dtype", [
    (1024, 16, 12, "bf16"),  # T*k = 192 routed rows, the most one step takes; 16 logits per lane
    (600, 16, 12, "f32"),    # E not a multiple of 64
    (8, 2, 3, "bf16"),       # fewer experts than lanes
    (512, 10, 1, "bf16"),
])
def test_layer_decode_routing_in_gateup_limits(moe, E, k, T, x_dtype):
    """Wide shapes route inside every gate/up workgroup: the limits of that path."""
    w = _custom(E, k, 2048, 512, T, 2, x_dtype, zipf=1.1)
    x, lg = w.x(), w.logits()
    ex = routed_experts(w, lg)
    a, b, _, _ = _four_calls_and_fused(moe, w, x, lg, ex)
    _assert_bit_identical(a, b, w.T * w.k)
    ref = oracle.layer(x, lg, ex, w.k, w.H, w.I, w.bits)
    assert np.array_equal(to_host(b[0]), ref["ids"])
    assert row_rel_err(to_host(b[4]), ref["out"]) <= DECODE_TOL


def test_layer_decode_all_rows_on_two_experts(moe):
    """Every token routes to the same two experts: 12 rows per expert, several passes."""
    w = _custom(8, 2, 256, 128, 12, 2)
    lg = np.tile(np.array([[3.0, 2.0, 0, 0, 0, 0, 0, 0]], np.float32), (w.T, 1))
    x, ex = w.x(), w.experts()
    a, b, _, _ = _four_calls_and_fused(moe, w, x, lg, ex)
    _assert_bit_identical(a, b, w.T * w.k)


def test_layer_decode_repeated_calls_reuse_workspace(moe):
    """Counters are cleared by every call: three calls in a row on one workspace agree."""
    import torch
    w = synth.decode_verify()
    lg = w.logits()
    ex = routed_experts(w, lg)
    layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, to_dev(ex))
    xd, ld = to_dev_x(w.x()), to_dev(lg)
    bufs = {"dws": torch.zeros(moe.decode_workspace_bytes(layer, w.T, w.k), dtype=torch.uint8, device="cuda")}
    outs = []
    for _ in range(3):
        outs.append(to_host(moe.layer_decode(layer, xd, ld, w.k, bufs=bufs)[4]).copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
