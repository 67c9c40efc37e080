#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN layer on one MI355X.

Workload (decode / speculative verify): 512 experts, top-10, hidden 2048,
expert intermediate 512, SwiGLU, T = 3 tokens per step (one token plus two
drafts), 2-bit block-32 weights with fp16 scale and min drawn from N(0, 0.02),
bf16 activations N(0, 1), fp32 router logits N(0, 1) plus a Zipf(1.1)
popularity bias.  All inputs are seeded synthetic data (no trained weights).

A step is one pass of the whole layer: route + dispatch + expert FFN +
combine, issued as moe_layer_decode (two launches: the gate/up GEMV, whose
workgroups route the tokens themselves, then the down GEMV with the combine
folded in); the same step as four separate calls is timed beside it.  Step i
uses layer copy i mod --copies (independent allocations of
the same layer, 48 by default, about 1 GB of touched weights per cycle) so
that the 256 MB on-package cache cannot serve one step from the previous one;
this is the 48-layer stack of the 125B-shaped model with identical weights.
The K timed steps are captured once in a HIP graph and replayed.

The JSON line also carries:
  roofline      the dominant kernel (routing + gate/up dequant-GEMV): algorithmic
                bytes per launch / its mean duration, timed with HIP events attached
                to that kernel's own launch (moe_profile_next_launch);
  cpu_baseline  the CPU oracle (scalar C, fp64, one thread) on a bounded
                sample of the same layer steps;
  prefill       the 8,192-token prompt-chunk layer on the MFMA path (tokens/s,
                and the gate/up GEMM against the 2.5 PFLOP/s dense half-precision
                MFMA peak); --no-prefill skips it.

--workload stack125b runs decode steps through a 48-layer x 512-expert stack
(fully resident, then through a 4,096-slot resident-expert table with misses
copied from page-locked host memory); --workload sweep runs the 40-layer
4-bit stack at T = 1, 2, 4, 8.  Each prints its own JSON line.
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
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 (and bf16) MFMA, MI355X
ROUNDS = 3  # timed rounds per measurement; the value is their median

# Memory traffic per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch, two runs), scaled
# by what the same counters read for a plain 256 MiB device-to-device copy in the same runs (FETCH_SIZE reads
# 131,093.4 KiB for it: x1.99970; WRITE_SIZE reads 262,144 KiB: x1.0).  Each entry is valid only for the kernel
# sources it was measured on (first 16 hex digits of their SHA-256); after a change the traffic is reported null.
FETCH_SCALE = 262144.0 / 131093.4
WRITE_SCALE = 1.0
TRAFFIC = {
    "gemv_gateup": {"sources": ["ffn_gemv.hip", "route_dispatch_dev.hpp", "slot_dev.hpp"],
                    "sha": "f9f3b89b37ce3455", "fetch_kib": 7632.875, "write_kib": 62.9375},
    "mfma_gateup": {"sources": ["ffn_mfma.hip"], "sha": "331d90259eb66f12", "fetch_kib": 292906.25,
                    "write_kib": 81920.625},
    # the same kernel on the chunk whose router bias is scaled by 0.21 (every expert hit)
    "mfma_gateup_flat": {"sources": ["ffn_mfma.hip"], "sha": "331d90259eb66f12", "fetch_kib": 520170.75,
                         "write_kib": 81927.15625},
}


def _sources_sha(names) -> str:
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "expert_routed_ffn_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the counter runs, or None if its sources have changed since."""
    t = TRAFFIC.get(kernel)
    if t is None or _sources_sha(t["sources"]) != t["sha"]:
        return None
    return (t["fetch_kib"] * FETCH_SCALE + t["write_kib"] * WRITE_SCALE) * 1024.0


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


def decode_bench(args, torch, moe, synth, oracle, bits: int = 2):
    import numpy as np

    w = synth.decode_verify(bits)
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

    bufs["dws"] = torch.zeros(moe.decode_workspace_bytes(layers[0], T, k), dtype=torch.uint8, device=dev)

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
    rounds = []
    for _ in range(ROUNDS):
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        rounds.append(time.perf_counter() - t0)
    elapsed = sorted(rounds)[len(rounds) // 2]
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

    # dominant kernel: the routed gate/up GEMV (routing + two thirds of the bytes); the down kernel (with the
    # combine folded in) is timed on alternate steps; the first cycle of copies pays first-touch costs
    nprof = 2 * max(NL, 96)
    timer = KernelTimer(nprof)
    for i in range(nprof):
        timer.arm(i, "gemv_gateup" if i % 2 == 0 else "gemv_down")
        step(i // 2)
    torch.cuda.synchronize()
    kt = timer.times_ms()
    timer.close()
    gu = kt[0::2][NL:] if len(kt) // 2 > NL else kt[0::2]
    dn = kt[1::2][NL:] if len(kt) // 2 > NL else kt[1::2]
    gu_ms = sum(gu) / len(gu)
    dn_ms = sum(dn) / len(dn)
    gu_plane = w.I * w.H * w.bits // 8 + w.I * (w.H // 32) * 4  # one [I x H] matrix: codes + scale/min
    # Wg, Wu of the unique experts; logits (routed inside the same launch); x; h written
    gu_bytes = U * 2 * gu_plane + T * w.E * 4 + T * w.H * 2 + T * k * w.I * 4
    dn_bytes = U * (eb - 2 * gu_plane) + T * k * w.I * 4 + T * k * w.H * 4 + T * w.H * 4  # Wd; h; y; out

    res = {
        "value": T * args.steps / elapsed,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "rounds_us_per_step": {"median": elapsed * 1e6 / args.steps, "min": min(rounds) * 1e6 / args.steps,
                               "max": max(rounds) * 1e6 / args.steps, "n": len(rounds)},
        "U": U,
        "err": err,
        "gen_s": gen_s,
        "roofline": {
            "bound": "hbm",
            "achieved": gu_bytes / (gu_ms * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gu_bytes / (gu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": measured_traffic("gemv_gateup") if bits == 2 else None,
            "kernel": "ffn_route_gateup_kernel (routing + expert gate/up dequant-GEMV + SwiGLU)",
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


def prefill_bench(args, torch, moe, synth, oracle, bits: int = 2, bias: float | None = None):
    """8,192-token prompt chunk through one layer (MFMA path)."""
    import numpy as np

    bias = args.prefill_bias if bias is None else bias
    w = synth.prefill(bias, bits)
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
    eager = (time.perf_counter() - t0) / args.prefill_steps
    eager_out = bufs["out"].clone()

    # the same steps captured in one graph, as a serving loop replays a chunk's launches: no host gaps between
    # the nine kernels of a step; two replays, each checked against the eager result
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        for _ in range(args.prefill_steps):
            step()
    g.replay()  # untimed (graph upload)
    torch.cuda.synchronize()
    if not torch.equal(bufs["out"], eager_out):
        raise SystemExit("bench: prefill graph replay differs from the eager step")
    rounds = []
    for _ in range(ROUNDS):
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        rounds.append((time.perf_counter() - t0) / args.prefill_steps)
        if not torch.equal(bufs["out"], eager_out):
            raise SystemExit("bench: prefill graph replay differs from the eager step")
    el = sorted(rounds)[len(rounds) // 2]
    del g

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
        "workload": f"prefill chunk: T=8192, 512 experts, top-10, hidden 2048, intermediate 512, {bits}-bit, "
                    f"Zipf({1.1 * bias:g}) router bias",
        "value": T / el,
        "unit": "tokens/s",
        "dtype": "f16 MFMA (weights, x, h), f32 accumulation; bf16 y",
        "ms_per_step": el * 1e3,
        "rounds_ms_per_step": {"median": el * 1e3, "min": min(rounds) * 1e3, "max": max(rounds) * 1e3,
                               "n": len(rounds)},
        "hip_graph": True,
        "eager_ms_per_step": eager * 1e3,
        "layer_tflops": (gu_flops + dn_flops) / el / 1e12,
        "experts_hit": int((counts > 0).sum()),
        "max_rows_per_expert": int(counts.max()),
        "min_rows_per_hit_expert": int(counts[counts > 0].min()),
        "sample_row_err": err,
        "_data": (x_np, lg_np, ex, w),
        "roofline": {
            "bound": "mfma",
            "achieved": gu_flops / (gu_ms * 1e-3) / 1e12,
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": gu_flops / (gu_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "traffic": (measured_traffic("mfma_gateup") if bias == 1.0 else
                        measured_traffic("mfma_gateup_flat") if abs(bias - 0.21) < 1e-9 else None) if bits == 2 else None,
            "kernel": "mfma_rb_kernel gate/up (fp16 32x32x16 MFMA, weights decoded into registers)",
            "flops_per_launch": gu_flops,
            "mean_us": gu_ms * 1e3,
            "down_mean_us": dn_ms * 1e3,
            "down_tflops": dn_flops / (dn_ms * 1e-3) / 1e12,
        },
    }


def router_bench(args, torch, moe, synth, oracle):
    """Router projection: decode step (T=3, GEMV) over rotated weight copies, and a prefill chunk
    (T=8192, MFMA)."""
    import numpy as np

    dev = torch.device("cuda:0")
    wd, wp = synth.decode_verify(), synth.prefill(args.prefill_bias)
    E, H = wd.E, wd.H
    copies = 160  # 160 x 2 MB: more than the last-level cache, so each launch streams from HBM
    wr_np = wd.router()
    wr = torch.from_numpy(wr_np.view(np.int16)).view(torch.bfloat16).to(dev)
    wrs = wr.unsqueeze(0).repeat(copies, 1, 1).contiguous()
    res = {}
    for name, w, n in (("decode", wd, 4 * copies), ("prefill", wp, 20)):
        x_np = w.x()
        x = torch.from_numpy(x_np.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        logits = torch.empty((w.T, E), dtype=torch.float32, device=dev)
        moe.router_logits(x, wrs[0], logits)
        torch.cuda.synchronize()
        rows = np.array([0, w.T - 1])
        ref = oracle.router_logits(x_np[rows], wr_np)
        err = float(np.abs(logits.cpu().numpy()[rows].astype(np.float64) - ref).max())
        if err > 1e-3:
            raise SystemExit(f"bench: router logits do not match the oracle ({err:.3e})")
        for i in range(copies):
            moe.router_logits(x, wrs[i % copies], logits)
        timer = KernelTimer(n)
        for i in range(n):
            timer.arm(i, "router")
            moe.router_logits(x, wrs[i % copies], logits)
        torch.cuda.synchronize()
        ms = timer.times_ms()
        timer.close()
        us = 1e3 * sum(ms) / len(ms)
        nbytes = E * H * 2 + w.T * H * 2 + w.T * E * 4
        flops = 2.0 * w.T * E * H
        res[name] = {"T": w.T, "mean_us": us, "gbs": nbytes / (us * 1e-6) / 1e9, "tflops": flops / (us * 1e-6) / 1e12,
                     "kernel": "router_gemv_kernel" if w.T < 64 else "router_mfma_kernel"}
    res["decode"]["hbm_frac"] = res["decode"]["gbs"] / HBM_PEAK_GBS
    res["prefill"]["mfma_frac"] = res["prefill"]["tflops"] / MFMA_F16_PEAK_TFLOPS
    res["workload"] = "router projection, E=512, H=2048, bf16 weights and activations, fp32 logits"
    return res


def bits3_bench(args, torch, moe, synth, oracle):
    """The decode/verify layer and the prefill chunk with 3-bit weights (same routing and shapes)."""
    res, _ = decode_bench(args, torch, moe, synth, oracle, 3)
    pre = None if args.no_prefill else prefill_bench(args, torch, moe, synth, oracle, 3)
    if pre is not None:
        pre.pop("_data")
    return {"metric": "MoE-layer tokens/s, 3-bit weights", "unit": "tokens/s",
            "decode": {"workload": "decode/verify layer, T=3, 512 experts, top-10, 2048 x 512, 3-bit",
                       "value": res["value"], "ms_per_step": res["ms_per_step"], "unique_experts_per_step": res["U"],
                       "layer_hbm_frac": res["layer_hbm_frac"], "roofline": res["roofline"]},
            "prefill": pre}


def prefill4_bench(args, torch, moe, synth, oracle):
    """The prefill chunk with 4-bit weights (same routing and shapes)."""
    pre = prefill_bench(args, torch, moe, synth, oracle, 4)
    pre.pop("_data")
    return {"metric": "MoE-layer prefill tokens/s, 4-bit weights", **pre}


# ---- stacks of layers (decode steps through many layers) ------------------------------------

def _placed_stack(torch, synth, w, dev, nthreads):
    """Device-resident [L, E, expert_bytes] stack: a pool of E generated expert blobs (layer 0's), and
    every (layer, expert) at its own address holding pool[perm_l(e)] for a fixed per-layer permutation."""
    import numpy as np
    pool = w.experts(0, nthreads=nthreads)
    pool_d = torch.from_numpy(pool).to(dev)
    rng = np.random.Generator(np.random.PCG64(w.seed + 0x5EED))
    perms = [np.arange(w.E)] + [rng.permutation(w.E) for _ in range(w.layers - 1)]
    big = torch.empty((w.layers, w.E, w.expert_bytes), dtype=torch.uint8, device=dev)
    for l in range(w.layers):
        torch.index_select(pool_d, 0, torch.from_numpy(perms[l]).to(dev), out=big[l])
    del pool_d
    return big, pool, perms


def _stack_inputs(torch, synth, w, steps, sigma, dev):
    """x [steps, L, T, H] bf16 (a seeded input for every step and layer: chaining the layers through the residual
    makes these synthetic activations grow without bound) and logits [steps, L, T, E] fp32 on the device, plus the
    per-(step, layer) count of unique routed experts (numpy top-k on the same logits; ties are immaterial here)."""
    import numpy as np
    xs = np.stack([np.stack([w.x(l, s) for l in range(w.layers)]) for s in range(steps)])
    lg = np.empty((steps, w.layers, w.T, w.E), np.float32)
    for l in range(w.layers):
        walk = synth.drift_walk(w, l, steps, sigma) if sigma > 0 else np.repeat(w.bias(l)[None], steps, 0)
        for s in range(steps):
            lg[s, l] = synth.logits(synth.stream_key(w.seed, synth.TAG_LOGITS, l, s), w.T, w.E, walk[s])
    top = np.argpartition(-lg, w.k - 1, axis=-1)[..., :w.k]
    U = np.array([[len(np.unique(top[s, l])) for l in range(w.layers)] for s in range(steps)])
    x_d = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(dev)
    return x_d, torch.from_numpy(lg).to(dev), U, xs, lg


def _check_layers(w):
    return sorted({0, w.layers // 2, w.layers - 1})


def _resident_stack_run(torch, moe, w, big, x_d, lg_d, steps, chunk):
    """Every step through all layers with moe_layer_decode (residual = the layer input, bf16 output of every
    (step, layer) kept); graphs of `chunk` steps.  Returns (seconds per step, bf16 outputs [steps, L, T, H],
    fp32 outputs of step 0 at the check layers)."""
    dev = big.device
    L, E, T, k, H = w.layers, w.E, w.T, w.k, w.H
    eb = w.expert_bytes
    layers = [moe.ExpertLayer(E, H, w.I, w.bits, big, eb, base_offset=l * E * eb) for l in range(L)]
    bufs = {
        "ids": torch.empty((T, k), dtype=torch.int32, device=dev),
        "w": torch.empty((T, k), dtype=torch.float32, device=dev),
        "dispatch": moe.Dispatch(T, k, E, dev),
        "y": torch.empty((T, k, H), dtype=torch.float32, device=dev),
        "out": torch.empty((T, H), dtype=torch.float32, device=dev),
        "dws": torch.zeros(moe.decode_workspace_bytes(layers[0], T, k), dtype=torch.uint8, device=dev),
    }
    rec = torch.empty((steps, L, T, H), dtype=torch.bfloat16, device=dev)
    out0 = {l: torch.empty((T, H), dtype=torch.float32, device=dev) for l in _check_layers(w)}

    def run(s, keep=None):
        for l in range(L):
            moe.layer_decode(layers[l], x_d[s, l], lg_d[s, l], k, residual=x_d[s, l], out_bf16=rec[s, l], bufs=bufs)
            if keep is not None and l in keep:
                keep[l].copy_(bufs["out"])

    check_steps = sorted({0, 1, steps - 1})
    for s in check_steps:
        run(s, out0 if s == 0 else None)
    torch.cuda.synchronize()
    eager = {s: rec[s].clone() for s in check_steps}
    cap = torch.cuda.Stream()
    graphs = []
    for c0 in range(0, steps, chunk):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for s in range(c0, min(steps, c0 + chunk)):
                run(s)
        graphs.append(g)
    graphs[0].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    for s, f in eager.items():
        if not torch.equal(rec[s].view(torch.int16), f.view(torch.int16)):
            raise SystemExit(f"bench: graph replay of stack step {s} differs from the eager step")
    return sec, rec, out0


def _check_against_oracle(oracle, w, pool, perms, xs, lg, out0, tol=2e-3):
    """Step 0 at the check layers: fp32 layer outputs against the oracle on the same bytes."""
    import numpy as np
    worst = 0.0
    for l, o in out0.items():
        ex = pool[perms[l]]
        res = (xs[0, l].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ref = oracle.layer(xs[0, l], lg[0, l], ex, w.k, w.H, w.I, w.bits, residual=res, want_y=False)
        got = o.cpu().numpy().astype(np.float64)
        err = float((np.abs(got - ref["out"]).max(axis=1) / np.abs(ref["out"] - res).max(axis=1)).max())
        if err > tol:
            raise SystemExit(f"bench: stack layer {l} does not match the oracle (row error {err:.3e})")
        worst = max(worst, err)
    return worst


def stack125b_bench(args, torch, moe, synth, oracle):
    """48 layers x 512 experts, T=3, Zipf(1.2) routing with per-step drift: fully resident, then through a
    4,096-slot resident-expert table with misses copied from page-locked host memory."""
    import numpy as np
    w = synth.stack125b()
    steps = args.stack_steps or w.extra["steps"]
    sigma, n_slots = w.extra["drift_sigma"], w.extra["slots"]
    dev = torch.device("cuda:0")
    L, E, T, k, H, eb = w.layers, w.E, w.T, w.k, w.H, w.expert_bytes
    t0 = time.time()
    big, pool, perms = _placed_stack(torch, synth, w, dev, synth.default_threads())
    x_d, lg_d, U, xs, lg = _stack_inputs(torch, synth, w, steps, sigma, dev)
    print(f"[stack125b] inputs ready in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    sec, rec, out0 = _resident_stack_run(torch, moe, w, big, x_d, lg_d, steps, args.stack_chunk)
    err = _check_against_oracle(oracle, w, pool, perms, xs, lg, out0)
    ref_rec = rec.view(torch.int16).cpu()
    del rec
    algo = float(U.mean()) * L * eb
    resident = {"us_per_step": sec * 1e6, "stack_tokens_per_s": T / sec, "layer_tokens_per_s": T * L / sec,
                "algorithmic_GBs": algo / sec / 1e9, "hbm_frac": algo / sec / 1e9 / HBM_PEAK_GBS,
                "mean_unique_experts_per_layer": float(U.mean()), "checked_layers_row_err": err}
    print(f"[stack125b] resident: {sec * 1e6:.1f} us/step", file=sys.stderr, flush=True)

    # slot-table mode: page-locked host master copy, 4,096 device slots
    host = torch.empty((L, E, eb), dtype=torch.uint8, pin_memory=True)
    host.copy_(big)
    del big
    torch.cuda.empty_cache()
    probe = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    hsrc = host.view(-1)[: 1 << 30]
    probe.copy_(hsrc, non_blocking=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(3):
        probe.copy_(hsrc, non_blocking=True)
    torch.cuda.synchronize()
    h2d_gbs = 3 * (1 << 30) / (time.perf_counter() - t1) / 1e9
    del probe
    slots = torch.empty((n_slots, eb), dtype=torch.uint8, device=dev)
    smap = torch.empty(L * E, dtype=torch.int32, device=dev)
    table = moe.SlotTable(L, E, n_slots, eb, host, slots, smap)
    b0 = np.stack([w.bias(l) for l in range(L)]).reshape(-1)
    hot = np.lexsort((np.arange(L * E), -b0))[:n_slots]  # hottest by step-0 bias, ties to the lower (layer, expert)
    table.preload([(int(i) // E, int(i) % E) for i in hot])
    torch.cuda.synchronize()
    base = table.stats()
    views = [table.layer(l, H, w.I, w.bits) for l in range(L)]
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wt = torch.empty((T, k), dtype=torch.float32, device=dev)
    d = moe.Dispatch(T, k, E, dev)
    y = torch.empty((T, k, H), dtype=torch.float32, device=dev)
    ws = torch.empty(views[0].workspace_bytes(T, k, "gemv"), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    rec = torch.empty((steps, L, T, H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(steps):
        for l in range(L):
            moe.route_topk(lg_d[s, l], k, ids=ids, w=wt)
            moe.dispatch(ids, E, out=d)
            table.resolve(l, d)
            moe.expert_ffn_q(views[l], x_d[s, l], k, d, y=y, path="gemv", ws=ws)
            moe.combine(y, wt, residual=x_d[s, l], out=out, out_bf16=rec[s, l])
    torch.cuda.synchronize()
    sec_s = (time.perf_counter() - t1) / steps
    st = table.stats()
    table.close()
    got = rec.view(torch.int16).cpu()
    if not torch.equal(got, ref_rec):
        bad = [s for s in range(steps) if not torch.equal(got[s], ref_rec[s])]
        raise SystemExit(f"bench: the slot-table stack differs from the resident stack at {len(bad)} of {steps} "
                         f"steps (first {bad[:5]}); stats {st}")
    hits, misses = st["hits"] - base["hits"], st["misses"] - base["misses"]
    h2d = st["bytes_h2d"] - base["bytes_h2d"]
    slot = {"us_per_step": sec_s * 1e6, "stack_tokens_per_s": T / sec_s, "hit_rate": hits / max(1, hits + misses),
            "misses_per_step": misses / steps, "h2d_MB_per_step": h2d / steps / 1e6,
            "h2d_link_GBs_measured": h2d_gbs,
            "h2d_time_share": (h2d / steps / (h2d_gbs * 1e9)) / sec_s,
            "bit_identical_to_resident": True,
            "note": "eager: the host waits for each layer's routing before resolving it"}
    print(f"[stack125b] slots, host policy: {sec_s * 1e6:.1f} us/step", file=sys.stderr, flush=True)

    # the same table with its policy on the GPU (moe_slot_table_resolve_device): no host round trip, so the
    # steps are captured in graphs like the resident run; every graph is replayed once (the policy state moves on)
    table = moe.SlotTable(L, E, n_slots, eb, host, slots, smap)
    table.preload([(int(i) // E, int(i) % E) for i in hot])
    table.enable_device()
    views = [table.layer(l, H, w.I, w.bits) for l in range(L)]
    dbufs = {"ids": ids, "w": wt, "dispatch": d, "y": y, "out": out,
             "dws": torch.zeros(moe.decode_workspace_bytes(views[0], T, k), dtype=torch.uint8, device=dev)}

    def dstep(s):  # moe_layer_decode_slots: routing, resolve and miss staging inside gate/up, then down
        for l in range(L):
            moe.layer_decode_slots(table, l, views[l], x_d[s, l], lg_d[s, l], k, residual=x_d[s, l],
                                   out_bf16=rec[s, l], bufs=dbufs)

    rec.zero_()
    cap = torch.cuda.Stream()
    graphs = []
    for c0 in range(0, steps, args.stack_chunk):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for s in range(c0, min(steps, c0 + args.stack_chunk)):
                dstep(s)
        graphs.append(g)
    torch.cuda.synchronize()
    base = table.stats()
    t1 = time.perf_counter()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    sec_d = (time.perf_counter() - t1) / steps
    st = table.stats()
    table.close()
    got = rec.view(torch.int16).cpu()
    if not torch.equal(got, ref_rec):
        bad = [s for s in range(steps) if not torch.equal(got[s], ref_rec[s])]
        raise SystemExit(f"bench: the device-policy slot stack differs from the resident stack at {len(bad)} of "
                         f"{steps} steps (first {bad[:5]}); stats {st}")
    hits, misses = st["hits"] - base["hits"], st["misses"] - base["misses"]
    h2d = st["bytes_h2d"] - base["bytes_h2d"]
    slot_dev = {"us_per_step": sec_d * 1e6, "stack_tokens_per_s": T / sec_d,
                "hit_rate": hits / max(1, hits + misses), "misses_per_step": misses / steps,
                "h2d_MB_per_step": h2d / steps / 1e6, "h2d_GBs_effective_share": h2d / steps / sec_d / 1e9,
                "bit_identical_to_resident": True,
                "note": "moe_layer_decode_slots, two launches per layer: in the gate/up launch one workgroup "
                        "routes, resolves and publishes the outcome; resident experts' rows start at once, missed "
                        "experts' rows wait for it, then read the page-locked master copy (device mapping) and "
                        "write their new slot as they go, while copy workgroups move the rest of each missed blob; "
                        "the down launch writes the table's map and counters; steps captured in graphs"}
    print(f"[stack125b] slots, device policy: {sec_d * 1e6:.1f} us/step", file=sys.stderr, flush=True)
    return {
        "metric": "MoE stack tokens/s (125B-shaped stack, decode T=3)",
        "workload": f"48 layers x 512 experts, top-10, hidden 2048, intermediate 512, T=3, 2-bit, Zipf(1.2) routing "
                    f"with per-step drift 0.05, {steps} steps; {n_slots}-slot table for the slot mode",
        "unit": "tokens/s", "steps": steps, "resident": resident, "slots": slot, "slots_device": slot_dev,
        "data": "synthetic; a pool of 512 generated experts placed at every (layer, expert) address under "
                "per-layer permutations",
    }


def sweep_bench(args, torch, moe, synth, oracle):
    """40 layers x 256 experts, 4-bit, T in {1, 2, 4, 8}: decode steps through the stack."""
    import numpy as np
    dev = torch.device("cuda:0")
    w1 = synth.decode_sweep(1)
    steps = args.stack_steps or 64
    big, pool, perms = _placed_stack(torch, synth, w1, dev, synth.default_threads())
    rows = []
    for T in (1, 2, 4, 8):
        w = synth.decode_sweep(T)
        x_d, lg_d, U, xs, lg = _stack_inputs(torch, synth, w, steps, 0.0, dev)
        sec, rec, out0 = _resident_stack_run(torch, moe, w, big, x_d, lg_d, steps, args.stack_chunk)
        err = _check_against_oracle(oracle, w, pool, perms, xs, lg, out0)
        del rec
        algo = float(U.mean()) * w.layers * w.expert_bytes
        rows.append({"T": T, "us_per_step": sec * 1e6, "stack_tokens_per_s": T / sec,
                     "algorithmic_GBs": algo / sec / 1e9, "hbm_frac": algo / sec / 1e9 / HBM_PEAK_GBS,
                     "mean_unique_experts_per_layer": float(U.mean()), "checked_layers_row_err": err})
        print(f"[sweep] T={T}: {sec * 1e6:.1f} us/step", file=sys.stderr, flush=True)
    return {
        "metric": "MoE stack tokens/s (40-layer 4-bit decode sweep)",
        "workload": f"40 layers x 256 experts, top-8, hidden 2048, intermediate 512, 4-bit, Zipf(1.0), {steps} steps",
        "unit": "tokens/s", "steps": steps, "per_T": rows,
        "data": "synthetic; a pool of 256 generated experts placed at every (layer, expert) address under "
                "per-layer permutations",
    }


def crossover_bench(args, torch, moe, synth, oracle):
    """Layer step time against T on the decode layer shape: the GEMV and MFMA expert-FFN paths (four calls each)
    and moe_layer_decode (T <= 12).  Sets where MOE_PATH_AUTO switches from GEMV to MFMA."""
    import numpy as np
    dev = torch.device("cuda:0")
    w0 = synth.decode_verify()
    ex = w0.experts(nthreads=synth.default_threads())
    eb, E, k, nc = w0.expert_bytes, w0.E, w0.k, 16
    lb = E * eb
    big = torch.empty(nc * lb, dtype=torch.uint8, device=dev)
    big[:lb].copy_(torch.from_numpy(ex.reshape(-1)))
    for c in range(1, nc):
        big[c * lb:(c + 1) * lb].copy_(big[:lb])
    layers = [moe.ExpertLayer(E, w0.H, w0.I, w0.bits, big[c * lb:(c + 1) * lb]) for c in range(nc)]
    rows = []
    for T in (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128, 256, 512):
        w = synth.Workload(f"crossover_T{T}", E=E, k=k, H=w0.H, I=w0.I, T=T, bits=w0.bits, x_dtype="bf16",
                           zipf_s=1.1)
        x = torch.from_numpy(w.x().view(np.int16).copy()).view(torch.bfloat16).to(dev)
        lg = torch.from_numpy(w.logits()).to(dev)
        row = {"T": T}
        for mode in ("gemv", "mfma", "decode"):
            if mode == "decode" and T > 12:
                continue
            bufs = {}
            if mode == "decode":
                bufs["dws"] = torch.zeros(moe.decode_workspace_bytes(layers[0], T, k), dtype=torch.uint8,
                                          device=dev)

                def step(i):
                    moe.layer_decode(layers[i % nc], x, lg, k, bufs=bufs)
            else:
                ids, wt, d, y, out = moe.layer_forward(layers[0], x, lg, k, path=mode)
                bufs.update(ids=ids, w=wt, dispatch=d, y=y, out=out,
                            ws=torch.empty(max(1, layers[0].workspace_bytes(T, k, mode)), dtype=torch.uint8,
                                           device=dev))

                def step(i, mode=mode):
                    moe.layer_forward(layers[i % nc], x, lg, k, path=mode, bufs=bufs)
            for i in range(2 * nc):
                step(i)
            torch.cuda.synchronize()
            n = 64 if T <= 64 else 16
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                for i in range(n):
                    step(i)
            g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            row[f"{mode}_us"] = (time.perf_counter() - t0) / n * 1e6
            del g
        rows.append(row)
        print(f"[crossover] {row}", file=sys.stderr, flush=True)
    return {
        "metric": "MoE layer step time against T (decode layer shape)",
        "workload": "512 experts, top-10, hidden 2048, intermediate 512, 2-bit, Zipf(1.1), bf16 x; 16 rotated "
                    "layer copies, graph-replayed steps",
        "unit": "us per layer step", "per_T": rows,
        "first_T_mfma_faster": next((r["T"] for r in rows if r["mfma_us"] < r["gemv_us"]), None),
        "data": "synthetic",
    }


def _cpu_info() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(args, oracle, data, pre_data=None):
    """The oracle (scalar C, fp64) on the host cores: the decode layer on one thread and on all threads, and the
    prefill chunk on all threads (in full) with a one-thread figure built from measured per-expert and per-row
    costs.  Each timing is the median of ROUNDS rounds."""
    import numpy as np
    x_np, lg_np, ex, w = data
    nt = oracle.default_threads()

    def timed(fn, rounds=ROUNDS):
        ts = []
        for _ in range(rounds):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[len(ts) // 2], min(ts), max(ts)

    n1, nm = max(1, args.cpu_steps // 4), args.cpu_steps
    med1, lo1, hi1 = timed(lambda: [oracle.layer(x_np, lg_np, ex, w.k, w.H, w.I, w.bits, want_y=False)
                                    for _ in range(n1)])
    medm, lom, him = timed(lambda: [oracle.layer(x_np, lg_np, ex, w.k, w.H, w.I, w.bits, want_y=False, nthreads=nt)
                                    for _ in range(nm)])
    out = {"value": w.T * nm / medm, "unit": "tokens/s", "cores": nt, "kind": "oracle",
           "sample": f"decode/verify layer (T={w.T}), {nm} layer steps per round on {nt} threads "
                     f"(oracle_layer_mt), median of {ROUNDS} rounds ({medm:.2f} s; min {lom:.2f}, max {him:.2f})",
           "single_thread": {"value": w.T * n1 / med1, "unit": "tokens/s", "cores": 1,
                             "sample": f"{n1} layer steps per round, median of {ROUNDS} rounds ({med1:.2f} s; "
                                       f"min {lo1:.2f}, max {hi1:.2f})"},
           **_cpu_info()}
    if pre_data is not None:
        px, plg, pex, pw = pre_data
        medp, lop, hip = timed(lambda: oracle.layer(px, plg, pex, pw.k, pw.H, pw.I, pw.bits, want_y=False,
                                                    nthreads=nt), rounds=1)
        # one thread: the oracle decodes each routed expert once and runs every routed row through the decoded
        # matrices; time both pieces on this host and scale them to the chunk's counts
        ids, _ = oracle.route(plg, pw.k)
        hit = np.unique(ids)
        t0 = time.perf_counter()
        mats = [oracle.dequant(pex[hit[0]], pw.H, pw.I, pw.bits, m) for m in range(3)]
        t_dec = time.perf_counter() - t0
        xr = (px[:64].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        t0 = time.perf_counter()
        for r in range(64):
            oracle.ffn_decoded(*mats, xr[r])
        t_row = (time.perf_counter() - t0) / 64
        est = len(hit) * t_dec + ids.size * t_row
        out["prefill"] = {
            "value": pw.T / medp, "unit": "tokens/s", "cores": nt, "kind": "oracle",
            "sample": f"the whole 8,192-token chunk (Zipf({1.1 * args.prefill_bias:g}), {len(hit)} experts hit) on "
                      f"{nt} threads, one round: {medp:.1f} s",
            "single_thread_estimate": {
                "value": pw.T / est, "unit": "tokens/s", "cores": 1,
                "sample": f"extrapolated: {len(hit)} expert decodes x {t_dec * 1e3:.1f} ms (one measured) + "
                          f"{ids.size} routed rows x {t_row * 1e3:.2f} ms (64 rows measured) = {est:.0f} s"}}
    return out


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
    ap.add_argument("--workload", choices=["layer", "stack125b", "sweep", "crossover", "prefill4", "bits3"],
                    default="layer",
                    help="layer: the decode/verify layer (+ prefill), the default; stack125b / sweep: decode "
                         "steps through a 48- or 40-layer stack; crossover: layer step time against T for the "
                         "GEMV and MFMA paths; prefill4: the prefill chunk with 4-bit weights; bits3: decode layer "
                         "and prefill chunk with 3-bit weights; all but layer print "
                         "their own JSON line")
    ap.add_argument("--stack-steps", type=int, default=0, help="steps of a stack run (default 256 / 64)")
    ap.add_argument("--stack-chunk", type=int, default=16, help="steps per captured graph in stack runs")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device once (a reference for memory-traffic counters)")
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

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.workload != "layer":
        fn = {"stack125b": stack125b_bench, "sweep": sweep_bench, "crossover": crossover_bench,
              "prefill4": prefill4_bench, "bits3": bits3_bench}[args.workload]
        print(json.dumps({**fn(args, torch, moe, synth, oracle), "n_gpus": 1}), flush=True)
        return

    res, data = decode_bench(args, torch, moe, synth, oracle)
    pre = flat = pre_data = None
    if not args.no_prefill:
        pre = prefill_bench(args, torch, moe, synth, oracle)
        pre_data = pre.pop("_data")
        flat = prefill_bench(args, torch, moe, synth, oracle, bias=0.21)
        flat.pop("_data")
        flat["note"] = ("the Zipf bias scaled by 0.21: every expert is hit and the per-expert row counts span "
                        f"{flat['min_rows_per_hit_expert']} to {flat['max_rows_per_expert']}")
        torch.cuda.empty_cache()
    rtr = None if args.no_prefill else router_bench(args, torch, moe, synth, oracle)
    cpu = None if args.no_cpu else cpu_baseline(args, oracle, data, pre_data)
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
        "rounds_us_per_step": res["rounds_us_per_step"],
        "cpu_baseline": cpu,
        "prefill": pre,
        "prefill_flat": flat,
        "router": rtr,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
