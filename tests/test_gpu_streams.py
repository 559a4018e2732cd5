"""Calls on different streams with disjoint buffers may run concurrently (C ABI
convention): the same work issued on two streams, interleaved call by call, gives
bit-identical results to running it on one stream."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gen
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cf():
    from activation_residual_compression_cf_amd import cf as _cf

    return _cf


def _state(cf, dev, A0, n):
    ah = torch.empty(n, dtype=torch.float32, device=dev)
    er = torch.empty_like(ah)
    cf.init_state(A0, ah, er)
    return ah, er


def test_two_streams_match_one_stream(cf):
    dev = cf.require_device()
    wl = gen.Workload("streams", 512, 3072, 4, 4, "bf16", True)
    tr = gen.Trajectory(wl, 21)
    A = [to_dev(tr.next(), dev) for _ in range(wl.steps)]
    n = A[0].numel()
    say("two streams vs one stream: 1-bit, 2-bit, top-k and low rank interleaved")
    q0 = torch.from_numpy(np.stack([gen.start_basis(21, s, 3072, 8) for s in range(4)])).to(dev)
    results = []
    for streams in (1, 2):
        ss = [torch.cuda.Stream() for _ in range(streams)]
        for s in ss:
            s.wait_stream(torch.cuda.current_stream())
        pick = lambda i: ss[i % streams]
        s1, s2, sk, sl = (_state(cf, dev, A[0].reshape(-1), n) for _ in range(4))
        ql = q0.clone()
        ws = torch.empty(cf.lowrank_workspace_bytes(512, 3072, 8, 4), dtype=torch.uint8, device=dev)
        c1 = torch.empty(n // 8, dtype=torch.uint8, device=dev)
        sc1 = torch.empty(n // 128, dtype=torch.float32, device=dev)
        c2 = torch.empty(n // 4, dtype=torch.uint8, device=dev)
        sc2 = torch.empty(n // 128, dtype=torch.float32, device=dev)
        ik = torch.empty(n // 128 * 12, dtype=torch.uint8, device=dev)
        vk = torch.empty(n // 128 * 12, dtype=torch.int16, device=dev)
        # every buffer is allocated up front: nothing a side stream writes is freed and
        # handed out again by the caching allocator while that stream may still use it
        pay = cf.lowrank_payload(4, 512, 3072, 8, 4, dev)
        for t in range(1, wl.steps):
            a = A[t].reshape(-1)
            cf.compress(1, a, s1[0], s1[1], c1, sc1, stream=pick(0))
            cf.compress(2, a, s2[0], s2[1], c2, sc2, stream=pick(1))
            cf.topk_compress(12, a, sk[0], sk[1], ik, vk, stream=pick(2))
            cf.lowrank_compress(A[t], sl[0].view(4, 512, 3072), sl[1].view(4, 512, 3072), ql, 8, 2, 4,
                                payload=pay, workspace=ws, stream=pick(3))
        torch.cuda.synchronize()
        results.append([x.clone() for x in (*s1, c1, sc1, *s2, c2, sc2, *sk, ik, vk, *sl, ql, *pay)])
    for x, y in zip(*results):
        assert torch.equal(x, y)


def test_side_stream_call_with_its_own_workspace(cf):
    """The binding allocates the low-rank workspace (and payload) itself, launches on a
    side stream and frees the workspace when the call returns.  Memory the current stream
    allocates and fills straight after the call must not be that workspace while the side
    stream still uses it: the results equal those of the same call with a workspace
    allocated up front."""
    dev = cf.require_device()
    B, m, n, k = 8, 1024, 3072, 32
    wl = gen.Workload("ws", m, n, B, 2, "bf16", True)
    tr = gen.Trajectory(wl, 3)
    A0, A1 = (to_dev(tr.next(), dev).view(B, m, n) for _ in range(2))
    q0 = torch.from_numpy(np.stack([gen.start_basis(3, s, n, k) for s in range(B)])).to(dev)
    need = cf.lowrank_workspace_bytes(m, n, k, B)
    say("low rank on a side stream with the binding's own workspace")
    outs = []
    for own in (False, True):
        ah = torch.empty((B, m, n), dtype=torch.float32, device=dev)
        er = torch.empty_like(ah)
        cf.init_state(A0, ah, er)
        q = q0.clone()
        torch.cuda.synchronize()
        if not own:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            pay = cf.lowrank_compress(A1, ah, er, q, k, 2, 4, workspace=ws)
            torch.cuda.synchronize()
        else:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            pay = cf.lowrank_compress(A1, ah, er, q, k, 2, 4, stream=side)
            junk = [torch.empty(need, dtype=torch.uint8, device=dev) for _ in range(2)]
            for j in junk:
                j.fill_(0xFF)  # NaN patterns wherever the workspace was reused too early
            torch.cuda.synchronize()
            del junk
        outs.append([ah.clone(), er.clone(), q.clone(), *[p.clone() for p in pay]])
    for x, y in zip(*outs):
        assert torch.equal(x, y)


def test_slab_calls_over_two_streams_match_one_stream(cf):
    """The per-layer pattern with its calls alternating over two streams (Slab.compress
    with `streams`): every tensor's Ahat, e, codes and scales equal those of the same
    calls on one stream, over several steps."""
    dev = cf.require_device()
    wl = gen.Workload("slab_streams", 256, 3072, 6, 4, "bf16", True)
    tr = gen.Trajectory(wl, 23)
    A = [to_dev(tr.next(), dev) for _ in range(wl.steps)]
    n = wl.m * wl.n
    say("Slab.compress, 6 tensors in calls of 2, one stream vs two alternating streams")
    out = []
    for two in (False, True):
        slab = cf.Slab(wl.slots, n, 1, dev)
        slab.init(A[0].reshape(-1), 2)
        pair = [torch.cuda.Stream(), torch.cuda.Stream()] if two else None
        for t in range(1, wl.steps):
            cur = torch.cuda.current_stream()
            if pair:
                for x in pair:
                    x.wait_stream(cur)
            slab.compress(A[t].reshape(-1), 2, streams=pair)
            if pair:
                for x in pair:
                    cur.wait_stream(x)
        torch.cuda.synchronize()
        out.append([x.cpu() for x in (slab.ahat, slab.err, slab.codes, slab.scales)])
    for x, y in zip(*out):
        assert torch.equal(x, y)
