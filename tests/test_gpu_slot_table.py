"""GPU: the resident-expert slot table changes placement only, never results.

A small chained stack (layers feed each other through combine's residual and
bf16 output) runs once with every expert resident in device memory and once
through a slot table holding only part of them, misses copied from
page-locked host memory; every layer's outputs must be bit-identical.  Every
layer output of the slot-table runs is also checked against the oracle on the
same input bytes (each layer's bf16 input, its logits and its master blobs).
"""
import numpy as np
import pytest

import oracle
import synth
from tests._parity import row_rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_routed_ffn_amd as m
    return m


def _stack(L=4, E=64, H=256, I=128, bits=2, T=3, k=6):
    return synth.Workload("small_stack", E=E, k=k, H=H, I=I, T=T, bits=bits, x_dtype="bf16", zipf_s=1.2, layers=L)


def _host_master(w, torch):
    eb = w.expert_bytes
    host = torch.empty(w.layers * w.E * eb, dtype=torch.uint8, pin_memory=True)
    hv = host.numpy().reshape(w.layers, w.E, eb)
    for l in range(w.layers):
        synth.layer_experts(w.seed, l, w.E, w.H, w.I, w.bits, out=hv[l])
    return host


DECODE_TOL = 2e-3


def _bf16_to_f64(bits_u16):
    return (np.asarray(bits_u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _check_against_oracle(w, host, cases):
    """cases: (layer, x as raw bf16 bits or fp32 values, logits, layer output with x as residual).
    The oracle runs each layer on the same bytes; the per-row error of out - x is held to DECODE_TOL."""
    ex_all = host.numpy().reshape(w.layers, w.E, w.expert_bytes)
    worst = 0.0
    for l, x_np, lg_np, out in cases:
        res = _bf16_to_f64(x_np) if x_np.dtype == np.uint16 else x_np.astype(np.float64)
        ref = oracle.layer(x_np, lg_np, ex_all[l], w.k, w.H, w.I, w.bits, residual=res, want_y=False,
                           nthreads=oracle.default_threads())
        worst = max(worst, row_rel_err(out - res, ref["out"] - res))
    print(f"{len(cases)} layer steps against the oracle: max row error {worst:.3e}")
    assert worst <= DECODE_TOL


def _run(moe, torch, w, layer_of, steps, resolve=None, record=None):
    """Run `steps` decode steps through the stack; returns every layer's (y, out) per step.
    With `record` (a list), appends (layer, x bits, logits, out) of every layer step."""
    dev = torch.device("cuda")
    outs = []
    for s in range(steps):
        x = torch.from_numpy(w.x(0, s).view(np.int16).copy()).view(torch.bfloat16).to(dev)
        for l in range(w.layers):
            lg_np = synth.logits(synth.stream_key(w.seed, synth.TAG_LOGITS, l, s), w.T, w.E,
                                 synth.drifted_bias(w, l, s, 0.05))
            lg = torch.from_numpy(lg_np).to(dev)
            ids, wt = moe.route_topk(lg, w.k)
            d = moe.dispatch(ids, w.E)
            if resolve is not None:
                resolve(l, d)
            y = moe.expert_ffn_q(layer_of(l), x, w.k, d, path="gemv")
            nxt = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
            out = moe.combine(y, wt, residual=x, out_bf16=nxt.view(torch.int16))
            torch.cuda.synchronize()
            outs.append((to_host(y).copy(), to_host(out).copy()))
            if record is not None:
                record.append((l, x.view(torch.int16).cpu().numpy().view(np.uint16).copy(), lg_np, outs[-1][1]))
            x = nxt
    return outs


@pytest.mark.parametrize("n_slots", [64, 24])
def test_slot_table_matches_resident_bit_for_bit(moe, n_slots):
    import torch
    w = _stack()
    eb = w.expert_bytes
    host = _host_master(w, torch)
    dev_all = host.to("cuda")
    resident = [moe.ExpertLayer(w.E, w.H, w.I, w.bits, dev_all, eb, base_offset=l * w.E * eb) for l in range(w.layers)]
    ref = _run(moe, torch, w, lambda l: resident[l], steps=4)

    slots = torch.empty(n_slots * eb, dtype=torch.uint8, device="cuda")
    smap = torch.empty(w.layers * w.E, dtype=torch.int32, device="cuda")
    table = moe.SlotTable(w.layers, w.E, n_slots, eb, host, slots, smap)
    # warm start: the most popular experts of each layer by the step-0 bias
    pairs = []
    for l in range(w.layers):
        order = np.argsort(-w.bias(l), kind="stable")[: n_slots // (2 * w.layers)]
        pairs += [(l, int(e)) for e in order]
    table.preload(pairs)
    rec = []
    got = _run(moe, torch, w, lambda l: table.layer(l, w.H, w.I, w.bits), steps=4,
               resolve=lambda l, d: table.resolve(l, d), record=rec)
    st = table.stats()
    table.close()
    assert st["misses"] > 0 and st["resolves"] == 4 * w.layers
    if n_slots < 64:
        assert st["evictions"] > 0
    for (ya, oa), (yb, ob) in zip(ref, got):
        assert np.array_equal(ya, yb) and np.array_equal(oa, ob)
    _check_against_oracle(w, host, rec)


def test_slot_table_rejects_pageable_host_memory(moe):
    import torch
    w = _stack(L=1, E=8, H=64, I=32)
    eb = w.expert_bytes
    host = torch.empty(w.E * eb, dtype=torch.uint8)  # pageable
    slots = torch.empty(4 * eb, dtype=torch.uint8, device="cuda")
    smap = torch.empty(w.E, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.SlotTable(1, w.E, 4, eb, host, slots, smap)
    assert ei.value.status == 5  # MOE_ENOTPINNED


def test_slot_table_capacity_error(moe):
    import torch
    w = _stack(L=1, E=16, H=64, I=32, T=3, k=4)
    eb = w.expert_bytes
    host = _host_master(w, torch)
    slots = torch.empty(2 * eb, dtype=torch.uint8, device="cuda")
    smap = torch.empty(w.E, dtype=torch.int32, device="cuda")
    table = moe.SlotTable(1, w.E, 2, eb, host, slots, smap)
    ids = torch.tensor([[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11]], dtype=torch.int32, device="cuda")
    d = moe.dispatch(ids, w.E)
    with pytest.raises(moe.MoeError) as ei:
        table.resolve(0, d)
    assert ei.value.status == 6  # MOE_ECAPACITY
    table.close()


# ---- device mode: the policy on the GPU ------------------------------------------------

def _warm_pairs(w, n_slots):
    pairs = []
    for l in range(w.layers):
        order = np.argsort(-w.bias(l), kind="stable")[: n_slots // (2 * w.layers)]
        pairs += [(l, int(e)) for e in order]
    return pairs


@pytest.mark.parametrize("n_slots", [64, 24])
def test_slot_table_device_mode_matches_resident_bit_for_bit(moe, n_slots):
    import torch
    w = _stack()
    eb = w.expert_bytes
    host = _host_master(w, torch)
    dev_all = host.to("cuda")
    resident = [moe.ExpertLayer(w.E, w.H, w.I, w.bits, dev_all, eb, base_offset=l * w.E * eb) for l in range(w.layers)]
    ref = _run(moe, torch, w, lambda l: resident[l], steps=4)
    slots = torch.empty(n_slots * eb, dtype=torch.uint8, device="cuda")
    smap = torch.empty(w.layers * w.E, dtype=torch.int32, device="cuda")
    table = moe.SlotTable(w.layers, w.E, n_slots, eb, host, slots, smap)
    table.preload(_warm_pairs(w, n_slots))
    table.enable_device()
    rec = []
    got = _run(moe, torch, w, lambda l: table.layer(l, w.H, w.I, w.bits), steps=4,
               resolve=lambda l, d: table.resolve_device(l, d), record=rec)
    st = table.stats()
    table.close()
    assert st["misses"] > 0 and st["resolves"] == 4 * w.layers
    if n_slots < 64:
        assert st["evictions"] > 0
    for (ya, oa), (yb, ob) in zip(ref, got):
        assert np.array_equal(ya, yb) and np.array_equal(oa, ob)
    _check_against_oracle(w, host, rec)


def test_slot_table_device_policy_equals_host_policy(moe):
    """Random active sets through the device table and a host-only table: same map and counters after every
    resolve, and every occupied slot holds its blob."""
    import torch
    w = _stack(L=3, E=40, H=64, I=32)
    eb, n_slots = w.expert_bytes, 20
    host = _host_master(w, torch)
    slots = torch.zeros(n_slots * eb, dtype=torch.uint8, device="cuda")
    smap = torch.empty(w.layers * w.E, dtype=torch.int32, device="cuda")
    table = moe.SlotTable(w.layers, w.E, n_slots, eb, host, slots, smap)
    ref = moe.HostSlotTable(w.layers, w.E, n_slots)
    pairs = [(0, 3), (1, 7), (2, 1), (0, 5)]
    table.preload(pairs)
    ref.preload(pairs)
    table.enable_device()
    rng = np.random.default_rng(11)
    d = moe.Dispatch(1, n_slots, w.E, "cuda")
    for it in range(60):
        layer = int(rng.integers(0, w.layers))
        n = int(rng.integers(0, n_slots + 1))
        act = np.sort(rng.choice(w.E, size=n, replace=False)).astype(np.int32)
        d.active[:n] = torch.from_numpy(act).cuda()
        d.n_active.fill_(n)
        table.resolve_device(layer, d, max_active=n_slots)
        ref.resolve(layer, act)
        torch.cuda.synchronize()
        assert np.array_equal(table.map_host(), ref.map_host()), it
        a, b = table.stats(), ref.stats()
        assert a["bytes_h2d"] == b["bytes_h2d"] // 256 * eb  # the host-only table counts 256 bytes a copy
        a.pop("bytes_h2d"), b.pop("bytes_h2d")
        assert a == b, it
    m = table.map_host()
    blobs = host.numpy().reshape(w.layers * w.E, eb)
    sl = slots.cpu().numpy().reshape(n_slots, eb)
    for idx in np.nonzero(m >= 0)[0]:
        assert np.array_equal(sl[m[idx]], blobs[idx]), idx
    table.close()
    ref.close()


def test_slot_table_device_mode_errors(moe):
    import torch
    w = _stack(L=1, E=16, H=64, I=32, T=3, k=4)
    eb = w.expert_bytes
    host = _host_master(w, torch)
    slots = torch.empty(4 * eb, dtype=torch.uint8, device="cuda")
    smap = torch.empty(w.E, dtype=torch.int32, device="cuda")
    table = moe.SlotTable(1, w.E, 4, eb, host, slots, smap)
    ids = torch.tensor([[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11]], dtype=torch.int32, device="cuda")
    d = moe.dispatch(ids, w.E)
    with pytest.raises(moe.MoeError) as ei:
        table.resolve_device(0, d)  # not in device mode yet
    assert ei.value.status == 1  # MOE_EINVAL
    table.enable_device()
    with pytest.raises(moe.MoeError) as ei:
        table.resolve_device(0, d, max_active=12)
    assert ei.value.status == 6  # MOE_ECAPACITY
    with pytest.raises(moe.MoeError) as ei:
        table.resolve(0, d)
    assert ei.value.status == 1
    table.close()


@pytest.mark.parametrize("bits,T,n_slots,xf32", [(2, 3, 64, False), (2, 3, 30, False), (3, 5, 64, False),
                                                  (4, 12, 64, False), (2, 7, 64, True)])
def test_layer_decode_slots_matches_resident_layer_decode(moe, bits, T, n_slots, xf32):
    """moe_layer_decode_slots (router + resolve in one workgroup, then the gate/up launch that also stages the
    misses, then down) against moe_layer_decode on resident weights, and the table's counters against the
    stand-alone device resolve on the same steps.  T above 3 takes several gate/up passes per item, of which
    only the first fills the slot."""
    import torch
    w = _stack(H=2048, I=512, E=64, k=10, bits=bits, T=T)  # wide shape: the combine is folded into the down kernel
    eb = w.expert_bytes
    host = _host_master(w, torch)
    dev_all = host.to("cuda")
    resident = [moe.ExpertLayer(w.E, w.H, w.I, w.bits, dev_all, eb, base_offset=l * w.E * eb) for l in range(w.layers)]
    tables = []
    for _ in range(2):
        slots = torch.empty(n_slots * eb, dtype=torch.uint8, device="cuda")
        smap = torch.empty(w.layers * w.E, dtype=torch.int32, device="cuda")
        t = moe.SlotTable(w.layers, w.E, n_slots, eb, host, slots, smap)
        t.preload(_warm_pairs(w, n_slots))
        t.enable_device()
        tables.append(t)
    fused, split = tables
    rec = []
    for s in range(3):
        x = torch.from_numpy(w.x(0, s).view(np.int16).copy()).view(torch.bfloat16).cuda()
        for l in range(w.layers):
            if xf32:
                x = x.float()
            lg = torch.from_numpy(synth.logits(synth.stream_key(w.seed, synth.TAG_LOGITS, l, s), w.T, w.E,
                                               synth.drifted_bias(w, l, s, 0.05))).cuda()
            a = moe.layer_decode(resident[l], x, lg, w.k, residual=x)
            b = moe.layer_decode_slots(fused, l, fused.layer(l, w.H, w.I, w.bits), x, lg, w.k, residual=x)
            d = moe.dispatch(a[0], w.E)
            split.resolve_device(l, d)
            torch.cuda.synchronize()
            for u, v in zip((a[0], a[1], a[3], a[4]), (b[0], b[1], b[3], b[4])):
                assert np.array_equal(to_host(u).view(np.uint32), to_host(v).view(np.uint32)), (s, l)
            x_np = x.cpu().numpy() if xf32 else x.view(torch.int16).cpu().numpy().view(np.uint16)
            rec.append((l, x_np.copy(), to_host(lg).copy(), to_host(b[4]).copy()))
            x = a[4].to(torch.bfloat16)
    assert fused.stats() == split.stats()
    assert np.array_equal(fused.map_host(), split.map_host())
    assert fused.stats()["misses"] > 0
    # every filled slot holds its expert's master blob: the gate and up planes
    # written by the gate/up items that read the master copy, the rest by the
    # copy workgroups of the same launch
    smap = fused.map_host().reshape(-1)
    slots_h = fused.slots.cpu().numpy()
    host_h = host.numpy()
    filled = np.flatnonzero(smap >= 0)
    assert len(filled) == n_slots
    for g in filled:
        sl = int(smap[g])
        assert np.array_equal(slots_h[sl * eb:(sl + 1) * eb], host_h[g * eb:(g + 1) * eb]), (g, sl)
    for t in tables:
        t.close()
    _check_against_oracle(w, host, rec)


def test_layer_decode_slots_table_above_register_stamps(moe):
    """A table of 4,160 slots, more than the in-launch resolve holds in registers (256 threads x 16 stamps),
    so its victim search reads the stamps from memory.  Preload fills every slot, the experts of the two
    computed layers first (oldest, the most popular among them), so misses evict, and the most popular
    experts are the oldest: a hit among them must not be taken as a victim in the same resolve.  Outputs
    bit-identical to resident weights, map and counters equal to those of the stand-alone device resolve,
    filled slots of the computed layers hold their blobs, and the oracle agrees."""
    import torch
    L, E, n_slots, run = 33, 128, 4160, 2
    assert n_slots > 256 * 16 and n_slots <= L * E
    w = synth.Workload("large_table", E=E, k=10, H=2048, I=512, T=3, bits=2, x_dtype="bf16", zipf_s=1.2, layers=L)
    eb = w.expert_bytes
    host = torch.empty(L * E * eb, dtype=torch.uint8, pin_memory=True)
    hv = host.numpy().reshape(L, E, eb)
    for l in range(run):
        synth.layer_experts(w.seed, l, E, w.H, w.I, w.bits, out=hv[l])
    hv[run:] = 0  # layers never computed: their blobs are only placed and copied
    dev_run = host[: run * E * eb].to("cuda")
    resident = [moe.ExpertLayer(E, w.H, w.I, w.bits, dev_run, eb, base_offset=l * E * eb) for l in range(run)]
    pairs = []
    for l in range(run):  # by popularity, ranks 8..39 left out so that they miss
        order = np.argsort(-w.bias(l), kind="stable")
        pairs += [(l, int(e)) for e in np.concatenate([order[:8], order[40:]])]
    pairs += [(l, e) for l in range(run, L) for e in range(E)]
    assert len(pairs) == n_slots
    tables = []
    for _ in range(2):
        slots = torch.empty(n_slots * eb, dtype=torch.uint8, device="cuda")
        smap = torch.empty(L * E, dtype=torch.int32, device="cuda")
        t = moe.SlotTable(L, E, n_slots, eb, host, slots, smap)
        t.preload(pairs)
        t.enable_device()
        tables.append(t)
    fused, split = tables
    rec = []
    for s in range(3):
        x = torch.from_numpy(w.x(0, s).view(np.int16).copy()).view(torch.bfloat16).cuda()
        for l in range(run):
            lg = torch.from_numpy(synth.logits(synth.stream_key(w.seed, synth.TAG_LOGITS, l, s), w.T, E,
                                               synth.drifted_bias(w, l, s, 0.05))).cuda()
            a = moe.layer_decode(resident[l], x, lg, w.k, residual=x)
            b = moe.layer_decode_slots(fused, l, fused.layer(l, w.H, w.I, w.bits), x, lg, w.k, residual=x)
            split.resolve_device(l, moe.dispatch(a[0], E))
            torch.cuda.synchronize()
            for u, v in zip((a[0], a[1], a[3], a[4]), (b[0], b[1], b[3], b[4])):
                assert np.array_equal(to_host(u).view(np.uint32), to_host(v).view(np.uint32)), (s, l)
            rec.append((l, x.view(torch.int16).cpu().numpy().view(np.uint16).copy(), to_host(lg).copy(),
                        to_host(b[4]).copy()))
            x = a[4].to(torch.bfloat16)
    st = fused.stats()
    assert st == split.stats()
    assert np.array_equal(fused.map_host(), split.map_host())
    assert st["misses"] > 0 and st["evictions"] > 0, st
    smap = fused.map_host().reshape(-1)
    filled = np.flatnonzero(smap[: run * E] >= 0)
    got = fused.slots.view(n_slots, eb)[torch.from_numpy(smap[filled].astype(np.int64)).cuda()].cpu().numpy()
    assert np.array_equal(got, host.numpy().reshape(L * E, eb)[filled])
    assert (smap >= 0).sum() == n_slots
    for t in tables:
        t.close()
    _check_against_oracle(w, host, rec)
