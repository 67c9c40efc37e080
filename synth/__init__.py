"""Seeded synthetic inputs for the routed MoE FFN layer.

A thin ctypes wrapper over ``synth.c`` (compiled to ``libsynth.so`` beside it).
It produces input bytes only: router logits, activations and encoded expert
weights.  Nothing in here decodes weights or computes any part of the layer;
the CPU oracle and the GPU library both consume what it writes.

Stream keys are named by (seed, tag, a, b, c) so any single tensor, e.g. one
expert of one layer, can be regenerated on its own.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

TAG_LOGITS, TAG_X, TAG_WEIGHT, TAG_RANK, TAG_DRIFT, TAG_ROUTER = 1, 2, 3, 4, 5, 6


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-Wall", _SRC, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, dbl, flt, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                       ctypes.c_float, ctypes.c_void_p)
        L.synth_stream_key.restype = u64
        L.synth_stream_key.argtypes = [u64, u64, u64, u64, u64]
        L.synth_u64.argtypes = [u64, u64, i64, vp]
        L.synth_uniform.argtypes = [u64, u64, i64, vp]
        L.synth_normal.argtypes = [u64, u64, i64, vp]
        L.synth_f64_to_f16.restype = ctypes.c_uint16
        L.synth_f64_to_f16.argtypes = [dbl]
        L.synth_normal_f32.argtypes = [u64, i64, flt, vp]
        L.synth_normal_bf16.argtypes = [u64, i64, vp]
        L.synth_normal_bf16_scaled.argtypes = [u64, i64, dbl, vp]
        L.synth_ranks.argtypes = [u64, i32, vp]
        L.synth_zipf_bias.argtypes = [u64, i32, dbl, vp]
        L.synth_logits.argtypes = [u64, i32, i32, vp, vp]
        L.synth_blob_layout.argtypes = [i32, i32, i32, vp]
        L.synth_quantize_matrix.argtypes = [vp, i32, i32, i32, vp, vp]
        L.synth_expert.argtypes = [u64, i32, i32, i32, i32, i32, dbl, vp]
        L.synth_layer.restype = i32
        L.synth_layer.argtypes = [u64, i32, i32, i32, i32, i32, dbl, vp, i64, vp, i32, i32]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def stream_key(seed: int, tag: int, a: int = 0, b: int = 0, c: int = 0) -> int:
    return int(lib().synth_stream_key(seed, tag, a, b, c))


def u64(key: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, np.uint64)
    lib().synth_u64(key, first, n, _p(out))
    return out


def uniform(key: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_uniform(key, first, n, _p(out))
    return out


def normal(key: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_normal(key, first, n, _p(out))
    return out


def f64_to_f16_bits(x: float) -> int:
    return int(lib().synth_f64_to_f16(float(x)))


def normal_f32(key: int, shape, scale: float = 1.0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    lib().synth_normal_f32(key, out.size, scale, _p(out))
    return out


def normal_bf16_bits(key: int, shape) -> np.ndarray:
    """bf16 (round-to-nearest-even of fp32 N(0,1)) as raw uint16 bits."""
    out = np.empty(shape, np.uint16)
    lib().synth_normal_bf16(key, out.size, _p(out))
    return out


def normal_bf16_bits_scaled(key: int, shape, scale: float) -> np.ndarray:
    """bf16 (round-to-nearest-even of fp32 scale * N(0,1)) as raw uint16 bits."""
    out = np.empty(shape, np.uint16)
    lib().synth_normal_bf16_scaled(key, out.size, float(scale), _p(out))
    return out


def ranks(key: int, E: int) -> np.ndarray:
    out = np.empty(E, np.int32)
    lib().synth_ranks(key, E, _p(out))
    return out


def zipf_bias(key: int, E: int, s: float) -> np.ndarray:
    out = np.empty(E, np.float32)
    lib().synth_zipf_bias(key, E, s, _p(out))
    return out


def logits(key: int, T: int, E: int, bias: np.ndarray | None = None) -> np.ndarray:
    out = np.empty((T, E), np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    lib().synth_logits(key, T, E, None if b is None else _p(b), _p(out))
    return out


def blob_layout(H: int, I: int, bits: int) -> list[int]:
    off = np.empty(7, np.int64)
    lib().synth_blob_layout(H, I, bits, _p(off))
    return [int(v) for v in off]


def expert_bytes(H: int, I: int, bits: int) -> int:
    return blob_layout(H, I, bits)[6]


def quantize_matrix(w: np.ndarray, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Encode a float64 [R, K] matrix: (codes uint32 [R, K*bits/32], sm uint32 [R, K/32])."""
    w = np.ascontiguousarray(w, np.float64)
    R, K = w.shape
    codes = np.zeros((R, K * bits // 32), np.uint32)
    sm = np.zeros((R, K // 32), np.uint32)
    lib().synth_quantize_matrix(_p(w), R, K, bits, _p(codes), _p(sm))
    return codes, sm


def expert(seed: int, layer: int, e: int, H: int, I: int, bits: int, std: float = 0.02) -> np.ndarray:
    out = np.empty(expert_bytes(H, I, bits), np.uint8)
    lib().synth_expert(seed, layer, e, H, I, bits, std, _p(out))
    return out


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def layer_experts(seed: int, layer: int, E: int, H: int, I: int, bits: int, std: float = 0.02,
                  which=None, nthreads: int | None = None, out: np.ndarray | None = None) -> np.ndarray:
    """All experts of one layer as uint8 [E, expert_bytes]; with ``which`` only those rows are written."""
    eb = expert_bytes(H, I, bits)
    if out is None:
        out = np.zeros((E, eb), np.uint8)
    assert out.shape == (E, eb) and out.dtype == np.uint8 and out.flags.c_contiguous
    w = None
    if which is not None:
        w = np.ascontiguousarray(np.asarray(which, np.int32))
    rc = lib().synth_layer(seed, layer, E, H, I, bits, std, _p(out), eb, None if w is None else _p(w),
                           0 if w is None else int(w.size), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("synth_layer failed")
    return out


# ---------------------------------------------------------------------------
# Workload recipes
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    E: int
    k: int
    H: int
    I: int
    T: int
    bits: int
    x_dtype: str            # "f32" or "bf16"
    zipf_s: float = 0.0     # popularity bias strength (0: none)
    seed: int = 0
    std: float = 0.02
    layers: int = 1
    extra: dict = field(default_factory=dict)

    def bias(self, layer: int = 0) -> np.ndarray | None:
        if self.zipf_s == 0.0:
            return None
        return zipf_bias(stream_key(self.seed, TAG_RANK, layer), self.E, self.zipf_s)

    def logits(self, layer: int = 0, step: int = 0) -> np.ndarray:
        return logits(stream_key(self.seed, TAG_LOGITS, layer, step), self.T, self.E, self.bias(layer))

    def x(self, layer: int = 0, step: int = 0) -> np.ndarray:
        """Activations [T, H]: float32 values, or raw bf16 bits as uint16."""
        key = stream_key(self.seed, TAG_X, layer, step)
        if self.x_dtype == "f32":
            return normal_f32(key, (self.T, self.H))
        return normal_bf16_bits(key, (self.T, self.H))

    def router(self, layer: int = 0) -> np.ndarray:
        """Router weights [E, H] as raw bf16 bits: N(0, 1/H) entries, so that with
        N(0,1) activations every logit has unit variance."""
        return normal_bf16_bits_scaled(stream_key(self.seed, TAG_ROUTER, layer), (self.E, self.H),
                                       1.0 / np.sqrt(self.H))

    def experts(self, layer: int = 0, which=None, nthreads=None) -> np.ndarray:
        return layer_experts(self.seed, layer, self.E, self.H, self.I, self.bits, self.std, which, nthreads)

    @property
    def expert_bytes(self) -> int:
        return expert_bytes(self.H, self.I, self.bits)


def tiny() -> Workload:
    """8 experts, top-2, hidden 64, intermediate 32, 4 tokens, fp32 activations, 2-bit."""
    return Workload("tiny", E=8, k=2, H=64, I=32, T=4, bits=2, x_dtype="f32")


def decode_verify(bits: int = 2) -> Workload:
    """512 experts, top-10, hidden 2048, intermediate 512, T=3 (1 token + 2 drafts), 2-bit (or `bits`), Zipf(1.1)."""
    return Workload("decode_verify" if bits == 2 else f"decode_verify_b{bits}", E=512, k=10, H=2048, I=512, T=3,
                    bits=bits, x_dtype="bf16", zipf_s=1.1)


def decode_sweep(T: int) -> Workload:
    """256 experts, top-8, hidden 2048, intermediate 512, 40 layers, 4-bit, Zipf(1.0)."""
    return Workload(f"decode_sweep_T{T}", E=256, k=8, H=2048, I=512, T=T, bits=4, x_dtype="bf16", zipf_s=1.0,
                    layers=40)


def stack125b() -> Workload:
    """48 layers x 512 experts, top-10, T=3 per step, 2-bit, Zipf(1.2) with per-step drift."""
    return Workload("stack125b", E=512, k=10, H=2048, I=512, T=3, bits=2, x_dtype="bf16", zipf_s=1.2, layers=48,
                    extra={"steps": 256, "drift_sigma": 0.05, "slots": 4096})


def prefill(bias_scale: float = 1.0, bits: int = 2) -> Workload:
    """8,192 tokens, 512 experts, top-10, hidden 2048, intermediate 512, 2-bit (or `bits`), Zipf(1.1 * bias_scale)."""
    name = "prefill" if bias_scale == 1.0 else f"prefill_l{bias_scale:g}"
    return Workload(name if bits == 2 else f"{name}_b{bits}", E=512, k=10, H=2048, I=512, T=8192, bits=bits,
                    x_dtype="bf16", zipf_s=1.1 * bias_scale)


def drifted_bias(w: Workload, layer: int, step: int, sigma: float) -> np.ndarray:
    """Zipf bias of ``layer`` after ``step`` Gaussian random-walk steps of size ``sigma`` (fp32 adds)."""
    b = w.bias(layer).astype(np.float32)
    for s in range(step):
        b = (b + normal_f32(stream_key(w.seed, TAG_DRIFT, layer, s), (w.E,), sigma)).astype(np.float32)
    return b


def drift_walk(w: Workload, layer: int, steps: int, sigma: float) -> np.ndarray:
    """Biases of ``layer`` at steps 0 .. steps-1 as float32 [steps, E]; row s equals drifted_bias(w, layer, s, sigma)."""
    out = np.empty((steps, w.E), np.float32)
    b = w.bias(layer).astype(np.float32)
    for s in range(steps):
        out[s] = b
        b = (b + normal_f32(stream_key(w.seed, TAG_DRIFT, layer, s), (w.E,), sigma)).astype(np.float32)
    return out
