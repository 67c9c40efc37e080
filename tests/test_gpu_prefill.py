"""GPU parity of the prefill path (grouped GEMM on half-precision MFMA) against the CPU oracle.

The MFMA path rounds decoded weights, x and h to fp16, so outputs are compared
with PREFILL_TOL in the per-row metric max|d| / max|ref|.  At the 8,192-token
size the oracle (on all host threads) checks every row of the 2-bit chunk on
both routings, and for 3- and 4-bit codes one row in every (expert, M-tile)
plus all rows against the GEMV path; smaller cases with ragged tiles are
compared in full.
"""
import numpy as np
import pytest

import oracle
import synth
from tests._parity import row_rel_err, to_dev, to_dev_x, to_host

pytestmark = pytest.mark.gpu

PREFILL_TOL = 5e-3


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_routed_ffn_amd as m
    return m


def _run(moe, w, x, lg, ex, path="mfma", y_dtype=None):
    import torch
    layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, to_dev(ex))
    ids, wt, d, y, out = moe.layer_forward(layer, to_dev_x(x), to_dev(lg), w.k, path=path,
                                           y_dtype=y_dtype or torch.float32)
    torch.cuda.synchronize()
    return ids, wt, d, y, out


_EXPERTS = {}


def _experts(bits):
    """All 512 experts of the prefill layer at `bits` (generated once per module)."""
    if bits not in _EXPERTS:
        _EXPERTS[bits] = synth.prefill(1.0, bits).experts(nthreads=synth.default_threads())
    return _EXPERTS[bits]


def _check_routing(moe, w, lg, ids, d):
    ids_h = to_host(ids)
    ref_ids, _ = oracle.route(lg, w.k)
    assert np.array_equal(ids_h, ref_ids)
    ref_d = oracle.dispatch(ref_ids, w.E)
    assert np.array_equal(to_host(d.offsets), ref_d["offsets"])
    assert np.array_equal(to_host(d.sorted_assign)[:w.T * w.k], ref_d["sorted_assign"])
    counts = np.bincount(ids_h.reshape(-1), minlength=w.E)
    print(f"{w.name}: experts hit {int((counts > 0).sum())}, max rows {counts.max()}, min nonzero "
          f"{counts[counts > 0].min()}")
    return ref_d


@pytest.mark.parametrize("bias_scale,y_bf16", [(1.0, True), (0.21, False)])
def test_prefill_8192_all_rows(moe, bias_scale, y_bf16):
    """The 8,192-token chunk in the benchmark's launch configuration (four calls, MFMA path): every one of the
    8,192 output rows and 81,920 expert rows against the oracle, run on all host threads."""
    import torch
    w = synth.prefill(bias_scale)
    ex = _experts(2)
    x, lg = w.x(), w.logits()
    ids, wt, d, y, out = _run(moe, w, x, lg, ex, y_dtype=torch.bfloat16 if y_bf16 else torch.float32)
    _check_routing(moe, w, lg, ids, d)
    out_h = to_host(out)
    y_h = to_host(y)
    del y
    ref = oracle.layer(x, lg, ex, w.k, w.H, w.I, w.bits, nthreads=oracle.default_threads())
    eo = row_rel_err(out_h, ref["out"])
    ey = row_rel_err(y_h, ref["y"])
    print(f"{w.name}: all {w.T} rows: out err {eo:.3e}; all {w.T * w.k} expert rows: y err {ey:.3e}")
    # the layer output carries the path's tolerance; bf16 y rows carry one more
    # round-to-nearest (at most 2^-9 of the row's largest value)
    assert eo <= PREFILL_TOL
    assert ey <= PREFILL_TOL + (2.0 ** -9 if y_bf16 else 0.0)


def _tile_rows(ref_d, k, bm=128, seed=0):
    """Tokens such that every (expert, M-tile of bm sorted rows) holds at least one of their assignments.
    Both GEMMs run on the same M-tiles.  Returns (tokens, number of tiles)."""
    rng = np.random.default_rng(seed)
    off, sa = ref_d["offsets"], ref_d["sorted_assign"]
    toks, tiles = set(), 0
    for e in range(len(off) - 1):
        for p0 in range(int(off[e]), int(off[e + 1]), bm):
            p1 = min(p0 + bm, int(off[e + 1]))
            toks.add(int(sa[int(rng.integers(p0, p1))]) // k)
            tiles += 1
    return np.array(sorted(toks)), tiles


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("bias_scale", [1.0, 0.21])
def test_prefill_8192_low_bit_every_tile(moe, bits, bias_scale):
    """3- and 4-bit chunks: one checked row in every (expert, M-tile) against the oracle, and all 8,192 rows
    against the GEMV path (fp32 throughout, oracle-checked at 2e-3) on the same inputs."""
    w = synth.prefill(bias_scale, bits)
    ex = _experts(bits)
    x, lg = w.x(), w.logits()
    ids, wt, d, y, out = _run(moe, w, x, lg, ex)
    ref_d = _check_routing(moe, w, lg, ids, d)
    out_h = to_host(out)
    y_h = to_host(y)
    del y, out
    toks, tiles = _tile_rows(ref_d, w.k)
    ref = oracle.layer(x[toks], lg[toks], ex, w.k, w.H, w.I, w.bits, nthreads=oracle.default_threads())
    eo = row_rel_err(out_h[toks], ref["out"])
    ey = row_rel_err(y_h[toks], ref["y"])
    del y_h
    g = _run(moe, w, x, lg, ex, path="gemv")
    eg = row_rel_err(out_h, to_host(g[4]))
    print(f"{w.name}: {tiles} M-tiles covered by {len(toks)} checked tokens: out err {eo:.3e}, y err {ey:.3e}; "
          f"all {w.T} rows against the GEMV path: {eg:.3e}")
    assert eo <= PREFILL_TOL and ey <= PREFILL_TOL and eg <= PREFILL_TOL


def _custom(E, k, H, I, T, bits, x_dtype="bf16", zipf=0.0, seed=5):
    return synth.Workload(f"mfma_E{E}_k{k}_H{H}_I{I}_T{T}_b{bits}", E=E, k=k, H=H, I=I, T=T, bits=bits,
                          x_dtype=x_dtype, zipf_s=zipf, seed=seed)


@pytest.mark.parametrize("E,k,H,I,T,bits,x_dtype,zipf", [
    (8, 2, 64, 32, 4, 2, "f32", 0.0),       # one tile, mostly padding
    (8, 2, 256, 128, 300, 2, "bf16", 0.5),  # several M-tiles per expert, ragged tails
    (16, 4, 256, 96, 257, 4, "bf16", 1.0),  # I not a multiple of 64: partial N-tiles
    (32, 8, 160, 64, 200, 2, "f32", 1.2),   # K = 160: five K-steps, fp32 input
    (4, 1, 128, 64, 129, 4, "f32", 0.0),    # k = 1, one row past a tile
    (16, 4, 256, 128, 300, 3, "bf16", 0.5), # 3-bit codes (the per-K-step loop)
    (8, 2, 160, 96, 130, 3, "f32", 1.0),    # 3-bit, K = 160 and 96
])
def test_mfma_small_cases_full(moe, E, k, H, I, T, bits, x_dtype, zipf):
    w = _custom(E, k, H, I, T, bits, x_dtype, zipf)
    x, lg, ex = w.x(), w.logits(), w.experts()
    ids, wt, d, y, out = _run(moe, w, x, lg, ex)
    ref = oracle.layer(x, lg, ex, w.k, w.H, w.I, w.bits)
    assert np.array_equal(to_host(ids), ref["ids"])
    ey, eo = row_rel_err(to_host(y), ref["y"]), row_rel_err(to_host(out), ref["out"])
    print(f"{w.name}: y err {ey:.3e}, out err {eo:.3e}")
    assert ey <= PREFILL_TOL and eo <= PREFILL_TOL


@pytest.mark.parametrize("bits", [2, 3])
def test_mfma_through_slot_map(moe, bits):
    """The MFMA path with the experts placed in a slot pool by a map (the M-tile
    list resolves each expert's slot): experts in permuted slots give the same
    bits as the plain layout, and an expert marked not resident gives NaN y rows
    for its assignments and leaves every other row unchanged."""
    import torch
    w = _custom(8, 2, 256, 128, 300, bits, "bf16", 0.5)
    x, lg, ex = w.x(), w.logits(), w.experts()
    ref = _run(moe, w, x, lg, ex)
    ids_ref, y_ref = ref[0], to_host(ref[3])
    hit = np.unique(to_host(ids_ref))
    gone = int(hit[len(hit) // 2])  # a routed expert that is then taken out
    eb = w.expert_bytes
    pool = np.zeros((w.E + 1) * eb, np.uint8)  # slot 0 stays unused
    smap = np.empty(w.E, np.int32)
    for e in range(w.E):
        slot = w.E - e  # reversed placement
        smap[e] = slot
        pool[slot * eb:(slot + 1) * eb] = ex.reshape(w.E, eb)[e]
    for case in ("all", "gone"):
        m = smap.copy()
        if case == "gone":
            m[gone] = -1
        layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, to_dev(pool), slot_map=torch.from_numpy(m).cuda())
        ids, wt, d, y, out = moe.layer_forward(layer, to_dev_x(x), to_dev(lg), w.k, path="mfma")
        torch.cuda.synchronize()
        yy = to_host(y)
        assert np.array_equal(to_host(ids), to_host(ids_ref))
        sel = to_host(ids) == gone  # [T, k] assignments to the expert taken out
        if case == "all":
            assert np.array_equal(yy, y_ref)
        else:
            assert sel.any() and np.all(np.isnan(yy[sel]))
            assert np.array_equal(yy[~sel], y_ref[~sel])
        print(f"{w.name} {case}: {int(sel.sum())} assignments to expert {gone}")


def test_decode_and_prefill_paths_agree(moe):
    w = synth.decode_verify()
    lg = w.logits()
    ids, _ = oracle.route(lg, w.k)
    ex = w.experts(which=np.unique(ids))
    x = w.x()
    a = _run(moe, w, x, lg, ex, path="gemv")
    b = _run(moe, w, x, lg, ex, path="mfma")
    ya, yb = to_host(a[3]), to_host(b[3])
    assert row_rel_err(yb, ya) <= PREFILL_TOL


def test_mfma_is_deterministic(moe):
    w = _custom(8, 2, 256, 128, 300, 2, "bf16", 0.5)
    x, lg, ex = w.x(), w.logits(), w.experts()
    a = _run(moe, w, x, lg, ex)
    b = _run(moe, w, x, lg, ex)
    assert np.array_equal(to_host(a[3]), to_host(b[3])) and np.array_equal(to_host(a[4]), to_host(b[4]))


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16)).astype(np.uint16)


def _clip_count(ws) -> int:
    return int(ws[:4].cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("sign", [1, -1])
def test_mfma_rows_far_outside_fp16_range(moe, sign):
    """Token rows scaled by 10^(sign * (t mod 7)): magnitudes up to 1e6 (h up to about 1e11) or down to 1e-6.
    The per-row power-of-two scaling keeps every row within the path's tolerance, with nothing saturated."""
    import torch
    w = _custom(16, 4, 256, 128, 200, 2, "bf16", 0.5, seed=8)
    xb = w.x()
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    scale = (10.0 ** (sign * (np.arange(w.T) % 7))).astype(np.float32)[:, None]
    x = _bf16_bits(xf * scale)
    lg, ex = w.logits(), w.experts()
    layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, to_dev(ex))
    ws = torch.zeros(layer.workspace_bytes(w.T, w.k, "mfma"), dtype=torch.uint8, device="cuda")
    ids, wt, d, y, out = moe.layer_forward(layer, to_dev_x(x), to_dev(lg), w.k, path="mfma", bufs={"ws": ws})
    torch.cuda.synchronize()
    ref = oracle.layer(x, lg, ex, w.k, w.H, w.I, w.bits)
    assert np.array_equal(to_host(ids), ref["ids"])
    ey, eo = row_rel_err(to_host(y), ref["y"]), row_rel_err(to_host(out), ref["out"])
    print(f"rows scaled up to 1e{6 * sign}: largest |out| {np.abs(ref['out']).max():.3e}, y err {ey:.3e}, "
          f"out err {eo:.3e}, saturated {_clip_count(ws)}")
    assert ey <= PREFILL_TOL and eo <= PREFILL_TOL
    assert _clip_count(ws) == 0


def test_mfma_saturation_is_counted(moe):
    """Weights with rows of L1 norm near 1e5 push h beyond the fp16 range even after the row scaling: the values
    saturate and the first word of the workspace counts them (it is cleared by every call)."""
    import torch
    from tests import _blob
    E, k, H, I, T, bits = 2, 1, 64, 32, 160, 2
    big = _blob.build_blob(H, I, bits, [_blob.constant_matrix(I, H, 3, 512.0, 0.0),
                                        _blob.constant_matrix(I, H, 3, 512.0, 0.0),
                                        _blob.constant_matrix(H, I, 1, 1.0, 0.0)])
    small = _blob.build_blob(H, I, bits, [_blob.constant_matrix(I, H, 1, 2.0 ** -10, 0.0),
                                          _blob.constant_matrix(I, H, 1, 2.0 ** -10, 0.0),
                                          _blob.constant_matrix(H, I, 1, 1.0, 0.0)])
    ex = np.stack([big, small])
    x = np.abs(np.random.default_rng(3).standard_normal((T, H))).astype(np.float32) + 0.5
    x_d = torch.from_numpy(x).cuda()
    ws = torch.zeros(moe.ExpertLayer(E, H, I, bits, to_dev(ex)).workspace_bytes(T, k, "mfma"), dtype=torch.uint8,
                     device="cuda")
    layer = moe.ExpertLayer(E, H, I, bits, to_dev(ex))
    to_big = np.tile(np.array([[1.0, 0.0]], np.float32), (T, 1))
    moe.layer_forward(layer, x_d, to_dev(to_big), k, path="mfma", bufs={"ws": ws})
    torch.cuda.synchronize()
    assert _clip_count(ws) == T * I  # g' = u' = 1536 * sum(x') > 2^8, so every h' = g' u' > 65504
    to_small = np.tile(np.array([[0.0, 1.0]], np.float32), (T, 1))
    ids, wt, d, y, out = moe.layer_forward(layer, x_d, to_dev(to_small), k, path="mfma", bufs={"ws": ws})
    torch.cuda.synchronize()
    assert _clip_count(ws) == 0
    ref = oracle.layer(x, to_small, ex, k, H, I, bits)
    assert row_rel_err(to_host(out), ref["out"]) <= PREFILL_TOL
