"""Helpers shared by the GPU parity tests: host<->device marshalling and the error metric."""
import numpy as np

import oracle
import synth


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Max over rows of max|got - ref| / max|ref| along the last axis.
    An all-zero reference row must be matched by an all-zero row."""
    got = np.asarray(got, np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    assert np.all(np.isfinite(got)), "non-finite output"
    num = np.abs(got - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    zero = den == 0
    assert np.all(num[zero] == 0), "nonzero output where the oracle row is zero"
    if (~zero).sum() == 0:
        return 0.0
    return float((num[~zero] / den[~zero]).max())


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_dev_x(x: np.ndarray):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def routed_experts(w: synth.Workload, logits: np.ndarray, layer: int = 0) -> np.ndarray:
    """Experts array [E, eb] with only the experts the oracle routes to filled in."""
    ids, _ = oracle.route(logits, w.k)
    return w.experts(layer, which=np.unique(ids))
