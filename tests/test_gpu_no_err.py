"""Senders without the error buffer (err = NULL): the error feedback lives in ahat, so
every other output must be bit-identical to the same step with err given."""
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


@pytest.mark.parametrize("bits", [1, 2])
@pytest.mark.parametrize("slots", [2, 48])  # 49,152 groups (small-call shape) and 1.18 M (large)
def test_quantizer_without_err(cf, bits, slots):
    dev = cf.require_device()
    wl = gen.Workload("noerr", 1024, 3072, slots, 3, "bf16", True)
    tr = gen.Trajectory(wl, 31)
    A = [to_dev(tr.next().reshape(-1), dev) for _ in range(3)]
    say(f"quantizer without err, bits={bits}, slots={slots}")
    n = A[0].numel()
    s1, s2 = cf.SenderState.create(n, dev), cf.SenderState.create(n, dev)
    cf.init_state(A[0], s1.ahat, s1.err)
    cf.init_state(A[0], s2.ahat)
    for t in (1, 2):
        c1, k1 = cf.compress(bits, A[t], s1.ahat, s1.err)
        c2, k2 = cf.compress(bits, A[t], s2.ahat, None)
        torch.cuda.synchronize()
        assert torch.equal(c1, c2) and torch.equal(k1, k2) and torch.equal(s1.ahat, s2.ahat)


@pytest.mark.parametrize("offset", [0, 1])  # staged payload, and the direct-store path
def test_topk_without_err(cf, offset):
    dev = cf.require_device()
    wl = gen.Workload("noerrk", 1024, 3072, 4, 3, "bf16", True)
    tr = gen.Trajectory(wl, 32)
    A = [to_dev(tr.next().reshape(-1), dev) for _ in range(3)]
    n, k = A[0].numel(), 12
    say(f"top-k without err, payload offset {offset}")
    outs = []
    for with_err in (True, False):
        ah = torch.empty(n, dtype=torch.float32, device=dev)
        er = torch.empty_like(ah) if with_err else None
        cf.init_state(A[0], ah, er)
        ib = torch.zeros(n // 128 * k + 8, dtype=torch.uint8, device=dev)
        vb = torch.zeros(n // 128 * k + 8, dtype=torch.int16, device=dev)
        idx, vals = ib[offset:offset + n // 128 * k], vb[offset:offset + n // 128 * k]
        for t in (1, 2):
            cf.topk_compress(k, A[t], ah, er, idx, vals)
        torch.cuda.synchronize()
        outs.append((ah, ib, vb))
    for x, y in zip(*outs):
        assert torch.equal(x, y)


@pytest.mark.parametrize("rank,iters,fb", [(32, 2, 4), (8, 2, 16), (8, 2, 4)])
def test_lowrank_without_err(cf, rank, iters, fb):
    dev = cf.require_device()
    wl = gen.Workload("noerrl", 512, 3072, 3, 3, "bf16", True)
    tr = gen.Trajectory(wl, 33)
    A = [to_dev(tr.next(), dev) for _ in range(3)]
    say(f"low rank without err, r{rank} q{iters} fb{fb}")
    q0 = torch.from_numpy(np.stack([gen.start_basis(33, s, 3072, rank) for s in range(3)])).to(dev)
    outs = []
    for with_err in (True, False):
        ah = torch.empty((3, 512, 3072), dtype=torch.float32, device=dev)
        er = torch.empty_like(ah) if with_err else None
        cf.init_state(A[0], ah, er)
        q = q0.clone()
        for t in (1, 2):
            pay = cf.lowrank_compress(A[t], ah, er, q, rank, iters, fb)
        torch.cuda.synchronize()
        outs.append((ah, q, *[x for x in pay if x is not None]))
    for x, y in zip(*outs):
        assert torch.equal(x, y)
