"""GPU parity in the band between decode and prefill (verify steps of several requests with drafts).

At the decode layer's real shape (512 experts, top-10, hidden 2048,
intermediate 512, 2-bit, Zipf(1.1) routing) the layer runs through
MOE_PATH_AUTO at T from 12 to 512.  AUTO must pick the GEMV path up to 128
routed rows and the MFMA path above (bit-identical to the path named
explicitly), the routing must be bit-exact, and every output row must be
within the chosen path's tolerance of the oracle (on all host threads).
"""
import numpy as np
import pytest

import oracle
import synth
from tests._parity import row_rel_err, to_dev, to_dev_x, to_host

pytestmark = pytest.mark.gpu

DECODE_TOL = 2e-3   # fp32 GEMV path
PREFILL_TOL = 5e-3  # fp16 MFMA path
AUTO_GEMV_MAX_ROWS = 128


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_routed_ffn_amd as m
    return m


@pytest.fixture(scope="module")
def experts():
    return synth.decode_verify().experts(nthreads=synth.default_threads())


def _run(moe, w, x, lg, layer, path):
    import torch
    ids, wt, d, y, out = moe.layer_forward(layer, to_dev_x(x), to_dev(lg), w.k, path=path)
    torch.cuda.synchronize()
    return to_host(ids), to_host(y), to_host(out)


@pytest.mark.parametrize("T", [12, 13, 16, 64, 256, 512])
def test_auto_path_real_shape(moe, experts, T):
    w = synth.Workload(f"verify_band_T{T}", E=512, k=10, H=2048, I=512, T=T, bits=2, x_dtype="bf16", zipf_s=1.1)
    x, lg = w.x(), w.logits()
    layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, to_dev(experts))
    ids, y, out = _run(moe, w, x, lg, layer, "auto")
    chosen = "gemv" if T * w.k <= AUTO_GEMV_MAX_ROWS else "mfma"
    ids_e, y_e, out_e = _run(moe, w, x, lg, layer, chosen)
    assert np.array_equal(ids, ids_e)
    assert np.array_equal(y.view(np.uint32), y_e.view(np.uint32))
    assert np.array_equal(out.view(np.uint32), out_e.view(np.uint32))
    ref = oracle.layer(x, lg, experts, w.k, w.H, w.I, w.bits, nthreads=oracle.default_threads())
    assert np.array_equal(ids, ref["ids"])
    ey, eo = row_rel_err(y, ref["y"]), row_rel_err(out, ref["out"])
    tol = DECODE_TOL if chosen == "gemv" else PREFILL_TOL
    print(f"T={T}: AUTO took the {chosen} path; all {T} rows: y err {ey:.3e}, out err {eo:.3e} (bar {tol:g})")
    assert ey <= tol and eo <= tol
