#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN layer on one MI355X.

Workload (decode / speculative verify): 512 experts, top-10, hidden 2048,
expert intermediate 512, SwiGLU, T = 3 tokens per step (one token plus two
drafts), 2-bit block-32 weights with fp16 scale and min drawn from N(0, 0.02),
bf16 activations N(0, 1), fp32 router logits N(0, 1) plus a Zipf(1.1)
popularity bias.  All inputs are seeded synthetic data (no trained weights).

A step is one pass of the whole layer: route + dispatch + expert FFN +
combine, issued as moe_layer_decode (three launches: routing and dispatch in one
workgroup, the gate/up GEMV, the down GEMV with the combine folded in); the
same step as four separate calls is timed beside it.  Step i uses layer copy i mod --copies (independent allocations of
the same layer, 48 by default, about 1 GB of touched weights per cycle) so
that the 256 MB on-package cache cannot serve one step from the previous one;
this is the 48-layer stack of the 125B-shaped model with identical weights.
The K timed steps are captured once in a HIP graph and replayed.

The JSON line also carries:
  roofline      the dominant kernel (the gate/up dequant-GEMV): algorithmic
                bytes per launch / its mean duration, timed with HIP events attached
                to that kernel's own launch (moe_profile_next_launch);
  cpu_baseline  the CPU oracle (scalar C, fp64, one thread) on a bounded
                sample of the same layer steps;
  prefill       the 8,192-token prompt-chunk layer on the MFMA path (tokens/s,
                and the gate/up GEMM against the 2.5 PFLOP/s dense half-precision
                MFMA peak); --no-prefill skips it.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "MoE-layer tokens/s (decode T=1–3, prefill 8192) + % of HBM / MFMA roofline"


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


class KernelTimer:
    """Pairs of HIP events attached to individual kernel launches."""

    def __init__(self, n: int):
        self.hip = _hip()
        self.ev = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0 and self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.ev.append((a, b))

    def arm(self, i: int, kernel: str):
        from expert_routed_ffn_amd import profile_next_launch
        profile_next_launch(kernel, self.ev[i][0], self.ev[i][1])

    def times_ms(self) -> list[float]:
        out = []
        for a, b in self.ev:
            assert self.hip.hipEventSynchronize(b) == 0
            ms = ctypes.c_float()
            assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
            out.append(ms.value)
        return out

    def close(self):
        for a, b in self.ev:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)


def decode_bench(args, torch, moe, synth, oracle):
    import numpy as np

    w = synth.decode_verify()
    dev = torch.device("cuda:0")
    eb = w.expert_bytes
    t0 = time.time()
    ex = w.experts(nthreads=synth.default_threads())
    x_np, lg_np = w.x(), w.logits()
    gen_s = time.time() - t0

    NL = args.copies
    layer_bytes = w.E * eb
    big = torch.empty(NL * layer_bytes, dtype=torch.uint8, device=dev)
    big[:layer_bytes].copy_(torch.from_numpy(ex.reshape(-1)))
    for c in range(1, NL):
        big[c * layer_bytes:(c + 1) * layer_bytes].copy_(big[:layer_bytes])
    layers = [moe.ExpertLayer(w.E, w.H, w.I, w.bits, big, eb, base_offset=c * layer_bytes) for c in range(NL)]

    x = torch.from_numpy(x_np.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    lg = torch.from_numpy(lg_np).to(dev)
    T, k = w.T, w.k
    bufs = {
        "ids": torch.empty((T, k), dtype=torch.int32, device=dev),
        "w": torch.empty((T, k), dtype=torch.float32, device=dev),
        "dispatch": moe.Dispatch(T, k, w.E, dev),
        "y": torch.empty((T, k, w.H), dtype=torch.float32, device=dev),
        "ws": torch.empty(layers[0].workspace_bytes(T, k, "gemv"), dtype=torch.uint8, device=dev),
        "out": torch.empty((T, w.H), dtype=torch.float32, device=dev),
    }

    bufs["dws"] = torch.empty(moe.decode_workspace_bytes(layers[0], T, k), dtype=torch.uint8, device=dev)

    def step(i, stream=None):
        moe.layer_decode(layers[i % NL], x, lg, k, bufs=bufs, stream=stream)

    def step4(i, stream=None):
        moe.layer_forward(layers[i % NL], x, lg, k, bufs=bufs, path="gemv", stream=stream)

    # correctness guard on the benchmarked buffers: copy NL-1 against the oracle
    step(NL - 1)
    torch.cuda.synchronize()
    ref = oracle.layer(x_np, lg_np, ex, k, w.H, w.I, w.bits, want_y=False)
    got = bufs["out"].cpu().numpy().astype(np.float64)
    err = float((np.abs(got - ref["out"]).max(axis=1) / np.abs(ref["out"]).max(axis=1)).max())
    if not np.array_equal(bufs["ids"].cpu().numpy(), ref["ids"]) or err > 2e-3:
        raise SystemExit(f"bench: layer output does not match the oracle (row error {err:.3e})")
    U = int(bufs["dispatch"].n_active.item())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # capture the K timed steps in one graph
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        for i in range(args.steps):
            step(i)
    g.replay()  # one untimed replay (graph upload)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    got2 = bufs["out"].cpu().numpy().astype(np.float64)
    if not np.array_equal(got, got2):
        raise SystemExit("bench: graph replay output differs from the eager step")

    # the same step as four separate calls, for comparison
    k4 = max(NL, args.steps // 4)
    g4 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g4, stream=cap):
        for i in range(k4):
            step4(i)
    g4.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g4.replay()
    torch.cuda.synchronize()
    four_call_us = (time.perf_counter() - t0) / k4 * 1e6
    if not np.array_equal(got, bufs["out"].cpu().numpy().astype(np.float64)):
        raise SystemExit("bench: the four-call step differs from the fused step")

    # dominant kernel: the gate/up GEMV (two thirds of the bytes); the down
    # kernel (with the folded combine) is timed on alternate steps
    nprof = 2 * max(NL, 96)
    timer = KernelTimer(nprof)
    for i in range(nprof):
        timer.arm(i, "gemv_gateup" if i % 2 == 0 else "gemv_down")
        step(i // 2)
    torch.cuda.synchronize()
    kt = timer.times_ms()
    timer.close()
    # the first cycle of copies pays first-touch costs; use the rest
    gu = kt[0::2][NL:] if len(kt) // 2 > NL else kt[0::2]
    dn = kt[1::2][NL:] if len(kt) // 2 > NL else kt[1::2]
    gu_ms = sum(gu) / len(gu)
    dn_ms = sum(dn) / len(dn)
    gu_plane = w.I * w.H * w.bits // 8 + w.I * (w.H // 32) * 4  # one [I x H] matrix: codes + scale/min
    gu_bytes = U * 2 * gu_plane + T * w.H * 2 + T * k * w.I * 4  # Wg, Wu of the unique experts; x; h written
    dn_bytes = U * (eb - 2 * gu_plane) + T * k * w.I * 4 + T * k * w.H * 4 + T * w.H * 4  # Wd; h; y; out

    res = {
        "value": T * args.steps / elapsed,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "U": U,
        "err": err,
        "gen_s": gen_s,
        "roofline": {
            "bound": "hbm",
            "achieved": gu_bytes / (gu_ms * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gu_bytes / (gu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": None,
            "kernel": "ffn_gateup_kernel (expert gate/up dequant-GEMV + SwiGLU)",
            "bytes_per_launch": gu_bytes,
            "mean_us": gu_ms * 1e3,
            "launches": len(gu),
            "down_kernel_mean_us": dn_ms * 1e3,
            "down_kernel_gbs": dn_bytes / (dn_ms * 1e-3) / 1e9,
        },
        "layer_hbm_frac": (U * eb + T * w.H * 2 + T * w.E * 4 + T * w.H * 4) / (elapsed / args.steps) / 1e9
        / HBM_PEAK_GBS,
        "four_call_us_per_step": four_call_us,
    }
    return res, (x_np, lg_np, ex, w)


def prefill_bench(args, torch, moe, synth, oracle):
    """8,192-token prompt chunk through one layer (MFMA path)."""
    import numpy as np

    w = synth.prefill(args.prefill_bias)
    dev = torch.device("cuda:0")
    ex = w.experts(nthreads=synth.default_threads())
    x_np, lg_np = w.x(), w.logits()
    base = torch.from_numpy(ex.reshape(-1)).to(dev)
    layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, base)
    x = torch.from_numpy(x_np.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    lg = torch.from_numpy(lg_np).to(dev)
    T, k = w.T, w.k
    bufs = {
        "ids": torch.empty((T, k), dtype=torch.int32, device=dev),
        "w": torch.empty((T, k), dtype=torch.float32, device=dev),
        "dispatch": moe.Dispatch(T, k, w.E, dev),
        "y": torch.empty((T, k, w.H), dtype=torch.bfloat16, device=dev),
        "ws": torch.empty(layer.workspace_bytes(T, k, "mfma"), dtype=torch.uint8, device=dev),
        "out": torch.empty((T, w.H), dtype=torch.float32, device=dev),
    }

    def step():
        moe.layer_forward(layer, x, lg, k, bufs=bufs, path="mfma", y_dtype=torch.bfloat16)

    step()
    torch.cuda.synchronize()
    sample = np.array([0, 1, T // 2, T - 1])
    ref = oracle.layer(x_np[sample], lg_np[sample], ex, k, w.H, w.I, w.bits, want_y=False)
    got = bufs["out"].cpu().numpy()[sample].astype(np.float64)
    err = float((np.abs(got - ref["out"]).max(axis=1) / np.abs(ref["out"]).max(axis=1)).max())
    if err > 5e-3:
        raise SystemExit(f"bench: prefill output does not match the oracle (row error {err:.3e})")
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.prefill_steps):
        step()
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / args.prefill_steps

    n = T * k
    timer = KernelTimer(2 * args.prefill_steps)
    for i in range(args.prefill_steps):
        timer.arm(2 * i, "mfma_gateup")
        moe.expert_ffn_q(layer, x, k, bufs["dispatch"], bufs["y"], path="mfma", ws=bufs["ws"])
        timer.arm(2 * i + 1, "mfma_down")
        moe.expert_ffn_q(layer, x, k, bufs["dispatch"], bufs["y"], path="mfma", ws=bufs["ws"])
    torch.cuda.synchronize()
    kt = timer.times_ms()
    timer.close()
    gu_ms = sum(kt[0::2]) / len(kt[0::2])
    dn_ms = sum(kt[1::2]) / len(kt[1::2])
    gu_flops = 2.0 * n * w.H * 2 * w.I
    dn_flops = 2.0 * n * w.I * w.H
    counts = np.bincount(bufs["ids"].cpu().numpy().reshape(-1), minlength=w.E)
    return {
        "workload": f"prefill chunk: T=8192, 512 experts, top-10, hidden 2048, intermediate 512, 2-bit, "
                    f"Zipf({1.1 * args.prefill_bias:g}) router bias",
        "value": T / el,
        "unit": "tokens/s",
        "ms_per_step": el * 1e3,
        "layer_tflops": (gu_flops + dn_flops) / el / 1e12,
        "experts_hit": int((counts > 0).sum()),
        "max_rows_per_expert": int(counts.max()),
        "sample_row_err": err,
        "roofline": {
            "bound": "mfma",
            "achieved": gu_flops / (gu_ms * 1e-3) / 1e12,
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": gu_flops / (gu_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "traffic": None,
            "kernel": "mfma_ffn_kernel gate/up (fp16 MFMA, weights decoded in LDS)",
            "flops_per_launch": gu_flops,
            "mean_us": gu_ms * 1e3,
            "down_mean_us": dn_ms * 1e3,
            "down_tflops": dn_flops / (dn_ms * 1e-3) / 1e12,
        },
    }


def cpu_baseline(args, oracle, data):
    x_np, lg_np, ex, w = data
    n = args.cpu_steps
    t0 = time.perf_counter()
    for _ in range(n):
        oracle.layer(x_np, lg_np, ex, w.k, w.H, w.I, w.bits, want_y=False)
    dt = time.perf_counter() - t0
    return {"value": w.T * n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} layer steps of the same workload (T={w.T}), scalar C fp64 oracle on one thread, "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=960)
    ap.add_argument("--warmup", type=int, default=96)
    ap.add_argument("--copies", type=int, default=48)
    ap.add_argument("--cpu-steps", type=int, default=12)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--prefill-bias", type=float, default=1.0, help="scale of the Zipf(1.1) router bias")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import __graft_entry__
    __graft_entry__._ensure_built()
    import torch

    import oracle
    import synth
    import expert_routed_ffn_amd as moe

    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(1)

    res, data = decode_bench(args, torch, moe, synth, oracle)
    pre = None if args.no_prefill else prefill_bench(args, torch, moe, synth, oracle)
    cpu = None if args.no_cpu else cpu_baseline(args, oracle, data)
    out = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode/verify layer: 512 experts, top-10, hidden 2048, intermediate 512, SwiGLU, T=3, "
                        "2-bit block-32 weights (fp16 scale/min), bf16 activations, Zipf(1.1) router bias",
            "E": 512, "k": 10, "H": 2048, "I": 512, "T": 3, "bits": 2,
            "layer_copies": args.copies, "hip_graph": True, "unique_experts_per_step": res["U"],
            "layer_hbm_frac": res["layer_hbm_frac"], "entry": "moe_layer_decode",
            "four_call_us_per_step": res["four_call_us_per_step"],
        },
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "prefill": pre,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
