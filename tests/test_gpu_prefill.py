"""GPU parity of the prefill path (grouped GEMM on half-precision MFMA) against the CPU oracle.

The MFMA path rounds decoded weights, x and h to fp16, so outputs are compared
with PREFILL_TOL in the per-row metric max|d| / max|ref|.  At the 8,192-token
size the oracle computes a seeded sample of token rows one by one (rows are
independent); smaller cases with ragged tiles are compared in full.
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


@pytest.fixture(scope="module")
def prefill_experts():
    return synth.prefill().experts(nthreads=synth.default_threads())


@pytest.mark.parametrize("bias_scale,y_bf16", [(1.0, True), (0.21, False)])
def test_prefill_8192_sampled_rows(moe, prefill_experts, bias_scale, y_bf16):
    import torch
    w = synth.prefill(bias_scale)
    x, lg = w.x(), w.logits()
    ids, wt, d, y, out = _run(moe, w, x, lg, prefill_experts, y_dtype=torch.bfloat16 if y_bf16 else torch.float32)
    ids_h = to_host(ids)
    ref_ids, _ = oracle.route(lg, w.k)
    assert np.array_equal(ids_h, ref_ids)
    counts = np.bincount(ids_h.reshape(-1), minlength=w.E)
    print(f"{w.name}: experts hit {int((counts > 0).sum())}, max rows {counts.max()}, min nonzero "
          f"{counts[counts > 0].min()}")
    out_h = to_host(out)
    assert np.all(np.isfinite(out_h))
    rng = np.random.default_rng(11)
    sample = np.sort(rng.choice(w.T, size=40, replace=False))
    # include rows of the most and least loaded experts
    hot = int(np.argmax(counts))
    sample = np.unique(np.concatenate([sample, np.nonzero((ids_h == hot).any(axis=1))[0][:4],
                                       np.nonzero((ids_h == np.argmin(np.where(counts > 0, counts, 1 << 30))).any(axis=1))[0][:2]]))
    ref = oracle.layer(x[sample], lg[sample], prefill_experts, w.k, w.H, w.I, w.bits)
    y_h = to_host(y)
    ey = row_rel_err(y_h[sample], ref["y"])
    eo = row_rel_err(out_h[sample], ref["out"])
    print(f"{w.name}: sampled {len(sample)} rows, y err {ey:.3e}, out err {eo:.3e}")
    # the layer output carries the path's tolerance; bf16 y rows carry one more
    # round-to-nearest (at most 2^-9 of the row's largest value)
    assert eo <= PREFILL_TOL
    assert ey <= PREFILL_TOL + (2.0 ** -9 if y_bf16 else 0.0)


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
