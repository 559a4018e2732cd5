"""The C ABI under HIP graph capture: a per-layer loop of compress and decode calls (one
call per layer's K and V, the serving pattern) is captured once on a side stream and
replayed on successive steps. Every replay must reproduce an eager run bit for bit.
Between replays the test does eager work of its own and synchronises, so a graph that
only works when replayed back to back would fail."""
from __future__ import annotations

import pytest
import torch

import gen
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cf():
    from activation_residual_compression_cf_amd import cf as _cf

    return _cf


@pytest.mark.parametrize("bits", [1, 2])
def test_per_layer_loop_graph_matches_eager(cf, bits):
    dev = cf.require_device()
    wl = gen.Workload("graph", 256, 3072, 6, 5, "bf16", True)  # 3 layers x (K, V)
    tr = gen.Trajectory(wl, 11)
    A = [to_dev(tr.next(), dev) for _ in range(wl.steps)]
    say(f"graph capture of the per-layer loop, bits={bits}")
    eager_tx = cf.Slab(wl.slots, wl.numel, bits, dev)
    eager_rx = cf.Slab(wl.slots, wl.numel, bits, dev, receiver=True)
    graph_tx = cf.Slab(wl.slots, wl.numel, bits, dev)
    graph_rx = cf.Slab(wl.slots, wl.numel, bits, dev, receiver=True)
    for s in (eager_tx, eager_rx, graph_tx, graph_rx):
        s.init(A[0], per_call=2)
    static_a = torch.empty_like(A[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        graph_tx.compress(static_a, per_call=2)
        graph_rx.decompress(graph_tx.codes, graph_tx.scales, per_call=2)
    torch.cuda.synchronize()
    for t in range(1, wl.steps):
        static_a.copy_(A[t])
        g.replay()
        eager_tx.compress(A[t], per_call=2)
        eager_rx.decompress(eager_tx.codes, eager_tx.scales, per_call=2)
        junk = (A[t].float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for x, y in ((graph_tx.ahat, eager_tx.ahat), (graph_tx.err, eager_tx.err),
                     (graph_tx.codes, eager_tx.codes), (graph_tx.scales, eager_tx.scales),
                     (graph_rx.ahat, eager_rx.ahat)):
            assert torch.equal(x, y), f"replay {t} differs from the eager run"
        assert torch.equal(graph_rx.ahat, graph_tx.ahat)


def test_topk_graph_matches_eager(cf):
    dev = cf.require_device()
    wl = gen.Workload("graphk", 256, 3072, 4, 4, "bf16", True)
    tr = gen.Trajectory(wl, 12)
    A = [to_dev(tr.next().reshape(-1), dev) for _ in range(wl.steps)]
    say("graph capture of top-k compress + decode")
    n, k = A[0].numel(), 12
    st = {}
    for name in ("eager", "graph"):
        ah = torch.empty(n, dtype=torch.float32, device=dev)
        er = torch.empty_like(ah)
        rx = torch.empty_like(ah)
        cf.init_state(A[0], ah, er)
        cf.init_state(A[0], rx)
        idx = torch.empty(n // 128 * k, dtype=torch.uint8, device=dev)
        vals = torch.empty(n // 128 * k, dtype=torch.int16, device=dev)
        st[name] = (ah, er, rx, idx, vals)
    static_a = torch.empty_like(A[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    ah, er, rx, idx, vals = st["graph"]
    with torch.cuda.graph(g, stream=side):
        cf.topk_compress(k, static_a, ah, er, idx, vals)
        cf.topk_decompress(k, idx, vals, rx)
    torch.cuda.synchronize()
    for t in range(1, wl.steps):
        static_a.copy_(A[t])
        g.replay()
        e = st["eager"]
        cf.topk_compress(k, A[t], e[0], e[1], e[3], e[4])
        cf.topk_decompress(k, e[3], e[4], e[2])
        torch.cuda.synchronize()
        for x, y in zip(st["graph"], st["eager"]):
            assert torch.equal(x, y), f"replay {t} differs from the eager run"


def test_lowrank_split_call_graph_matches_eager(cf):
    """A low-rank call large enough to run as two halves on two streams, captured into a
    graph (the library's side stream joins the capture through its events) and replayed
    on successive steps: every replay equals an eager run bit for bit."""
    import numpy as np

    dev = cf.require_device()
    B, m, n, k = 8, 1024, 3072, 32  # 25M elements: two halves of 4 tensors
    wl = gen.Workload("graphlr", m, n, B, 4, "bf16", True)
    tr = gen.Trajectory(wl, 13)
    A = [to_dev(tr.next(), dev).view(B, m, n) for _ in range(wl.steps)]
    q0 = torch.from_numpy(np.stack([gen.start_basis(13, s, n, k) for s in range(B)])).to(dev)
    say("graph capture of a two-stream low-rank call")
    st = {}
    for name in ("eager", "graph", "first"):
        ah = torch.empty((B, m, n), dtype=torch.float32, device=dev)
        er = torch.empty_like(ah)
        cf.init_state(A[0], ah, er)
        ws = torch.empty(cf.lowrank_workspace_bytes(m, n, k, B), dtype=torch.uint8, device=dev)
        st[name] = (ah, er, q0.clone(), cf.lowrank_payload(B, m, n, k, 4, dev), ws)
    # one eager call on this thread before the capture: the side stream and events of
    # the split are made then, not during the capture
    f = st.pop("first")
    cf.lowrank_compress(A[1], f[0], f[1], f[2], k, 2, 4, f[3], f[4])
    torch.cuda.synchronize()
    del f
    static_a = torch.empty_like(A[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    ah, er, q, pay, ws = st["graph"]
    with torch.cuda.graph(g, stream=side):
        cf.lowrank_compress(static_a, ah, er, q, k, 2, 4, pay, ws)
    torch.cuda.synchronize()
    for t in range(1, wl.steps):
        static_a.copy_(A[t])
        g.replay()
        e = st["eager"]
        cf.lowrank_compress(A[t], e[0], e[1], e[2], k, 2, 4, e[3], e[4])
        junk = (A[t].float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        gx, ex = st["graph"], st["eager"]
        for x, y in zip((gx[0], gx[1], gx[2], *gx[3]), (ex[0], ex[1], ex[2], *ex[3])):
            assert torch.equal(x, y), f"replay {t} differs from the eager run"


def test_two_stream_per_layer_graph_matches_eager(cf):
    """The per-layer calls alternating over two streams, forked from and joined to the
    capture stream, captured as a graph with two parallel branches: every replay equals
    the eager one-stream run bit for bit."""
    dev = cf.require_device()
    wl = gen.Workload("graph2", 256, 3072, 6, 5, "bf16", True)
    tr = gen.Trajectory(wl, 13)
    A = [to_dev(tr.next(), dev) for _ in range(wl.steps)]
    say("graph capture of the per-layer loop over two streams, 1-bit")
    eager = cf.Slab(wl.slots, wl.numel, 1, dev)
    graph = cf.Slab(wl.slots, wl.numel, 1, dev)
    for s in (eager, graph):
        s.init(A[0], per_call=2)
    static_a = torch.empty_like(A[0])
    side = torch.cuda.Stream()
    pair = [torch.cuda.Stream(), torch.cuda.Stream()]
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        cur = torch.cuda.current_stream()
        for x in pair:
            x.wait_stream(cur)
        graph.compress(static_a, per_call=2, streams=pair)
        for x in pair:
            cur.wait_stream(x)
    torch.cuda.synchronize()
    for t in range(1, wl.steps):
        static_a.copy_(A[t])
        g.replay()
        eager.compress(A[t], per_call=2)
        junk = (A[t].float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for x, y in ((graph.ahat, eager.ahat), (graph.err, eager.err), (graph.codes, eager.codes),
                     (graph.scales, eager.scales)):
            assert torch.equal(x, y), f"replay {t} differs from the eager run"
