"""GPU: layer steps captured in a HIP graph and replayed give the eager results bit for bit.

The decode step, the prefill (MFMA) step and the slot-table step with its
misses staged inside the gate/up launch are each captured once and replayed
three times.  Before every replay the outputs are overwritten by eager work
and the host synchronises; after it, every output is compared bit for bit
with the eager run (the library records no memset nodes, whose replays are
the known hazard).
"""
import pytest

import synth
from tests._parity import routed_experts, to_dev, to_dev_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_routed_ffn_amd as m
    return m


def _bits(t):
    import torch
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _replay_and_check(torch, g, outs):
    """outs: (tensor, eager copy) pairs; three replays, each after the tensors are overwritten."""
    for r in range(3):
        for t, _ in outs:
            _bits(t).fill_(-1)  # eager work between replays: a fill kernel, then a sync
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, ref) in enumerate(outs):
            assert torch.equal(_bits(t), _bits(ref)), (r, i)


def _capture(torch, step):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        step()
    torch.cuda.synchronize()
    return g


def test_layer_decode_graph_replays(moe):
    import torch
    w = synth.decode_verify()
    lg = w.logits()
    layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, to_dev(routed_experts(w, lg)))
    x, lgd = to_dev_x(w.x()), to_dev(lg)
    T, k = w.T, w.k
    bufs = {"ids": torch.empty((T, k), dtype=torch.int32, device="cuda"),
            "w": torch.empty((T, k), dtype=torch.float32, device="cuda"),
            "dispatch": moe.Dispatch(T, k, w.E, torch.device("cuda")),
            "y": torch.empty((T, k, w.H), dtype=torch.float32, device="cuda"),
            "out": torch.empty((T, w.H), dtype=torch.float32, device="cuda"),
            "dws": torch.zeros(moe.decode_workspace_bytes(layer, T, k), dtype=torch.uint8, device="cuda")}

    def step():
        moe.layer_decode(layer, x, lgd, k, residual=x, bufs=bufs)

    step()
    torch.cuda.synchronize()
    names = ("ids", "w", "y", "out")
    outs = [(bufs[n], bufs[n].clone()) for n in names]
    _replay_and_check(torch, _capture(torch, step), outs)


def test_prefill_graph_replays(moe):
    import torch
    w = synth.Workload("graph_prefill", E=16, k=4, H=256, I=128, T=300, bits=2, x_dtype="bf16", zipf_s=0.8)
    lg = w.logits()
    layer = moe.ExpertLayer(w.E, w.H, w.I, w.bits, to_dev(w.experts()))
    x, lgd = to_dev_x(w.x()), to_dev(lg)
    T, k = w.T, w.k
    bufs = {"ids": torch.empty((T, k), dtype=torch.int32, device="cuda"),
            "w": torch.empty((T, k), dtype=torch.float32, device="cuda"),
            "dispatch": moe.Dispatch(T, k, w.E, torch.device("cuda")),
            "y": torch.empty((T, k, w.H), dtype=torch.bfloat16, device="cuda"),
            "ws": torch.empty(layer.workspace_bytes(T, k, "mfma"), dtype=torch.uint8, device="cuda"),
            "out": torch.empty((T, w.H), dtype=torch.float32, device="cuda")}

    def step():
        moe.layer_forward(layer, x, lgd, k, bufs=bufs, path="mfma", y_dtype=torch.bfloat16)

    step()
    torch.cuda.synchronize()
    outs = [(bufs[n], bufs[n].clone()) for n in ("ids", "w", "y", "out")]
    _replay_and_check(torch, _capture(torch, step), outs)


def test_layer_decode_slots_graph_replays(moe):
    """Two layers through a slot table too small for both layers' experts, so every replay evicts and stages
    misses again (the policy state moves on between replays); each replay's outputs must equal the resident
    run's."""
    import torch
    w = synth.Workload("graph_slots", E=64, k=10, H=2048, I=512, T=3, bits=2, x_dtype="bf16", zipf_s=0.3, layers=2)
    eb, T, k, dev = w.expert_bytes, w.T, w.k, torch.device("cuda")
    host = torch.empty(w.layers * w.E * eb, dtype=torch.uint8, pin_memory=True)
    hv = host.numpy().reshape(w.layers, w.E, eb)
    for l in range(w.layers):
        synth.layer_experts(w.seed, l, w.E, w.H, w.I, w.bits, out=hv[l])
    dev_all = host.to(dev)
    x = to_dev_x(w.x())
    lgs = [to_dev(w.logits(l)) for l in range(w.layers)]

    def mkbufs(layer):
        return {"ids": torch.empty((T, k), dtype=torch.int32, device=dev),
                "w": torch.empty((T, k), dtype=torch.float32, device=dev),
                "dispatch": moe.Dispatch(T, k, w.E, dev),
                "y": torch.empty((T, k, w.H), dtype=torch.float32, device=dev),
                "out": torch.empty((T, w.H), dtype=torch.float32, device=dev),
                "dws": torch.zeros(moe.decode_workspace_bytes(layer, T, k), dtype=torch.uint8, device=dev)}

    refs = []
    for l in range(w.layers):
        res = moe.ExpertLayer(w.E, w.H, w.I, w.bits, dev_all, eb, base_offset=l * w.E * eb)
        b = mkbufs(res)
        moe.layer_decode(res, x, lgs[l], k, residual=x, bufs=b)
        torch.cuda.synchronize()
        refs.append({n: b[n].clone() for n in ("ids", "w", "y", "out")})

    n_slots = 32  # at least T*k = 30 (the most one layer can route), fewer than the two layers need together
    slots = torch.empty(n_slots * eb, dtype=torch.uint8, device=dev)
    smap = torch.empty(w.layers * w.E, dtype=torch.int32, device=dev)
    table = moe.SlotTable(w.layers, w.E, n_slots, eb, host, slots, smap)
    table.enable_device()
    views = [table.layer(l, w.H, w.I, w.bits) for l in range(w.layers)]
    bufs = [mkbufs(views[l]) for l in range(w.layers)]

    def step():
        for l in range(w.layers):
            moe.layer_decode_slots(table, l, views[l], x, lgs[l], k, residual=x, bufs=bufs[l])

    step()
    torch.cuda.synchronize()
    for l in range(w.layers):
        for n in ("ids", "w", "y", "out"):
            assert torch.equal(_bits(bufs[l][n]), _bits(refs[l][n])), (l, n)
    before = table.stats()["misses"]
    g = _capture(torch, step)
    outs = [(bufs[l][n], refs[l][n]) for l in range(w.layers) for n in ("ids", "w", "y", "out")]
    _replay_and_check(torch, g, outs)
    assert table.stats()["misses"] > before + 3  # every replay staged misses again
    table.close()
