"""cf_lowrank_compress_noalloc, the entry point that allocates nothing (it uses the
library's fixed device scratch instead of a caller workspace), against
cf_lowrank_compress with a workspace, through the C ABI: the same kernels on the same
inputs, so every output must agree bit for bit.  Two calls in a row, the second smaller
and of another shape, so the second runs on what the first left in the scratch; then a
call too large for the scratch, which must fail with CF_E_SCRATCH and write nothing."""
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


def _case(cf, dev, batch, m, n, rank, seed):
    wl = gen.Workload("noalloc", m, n, batch, 2, "bf16", True)
    tr = gen.Trajectory(wl, seed)
    A0, A1 = (to_dev(tr.next(), dev).view(batch, m, n) for _ in range(2))
    q0 = torch.from_numpy(np.stack([gen.start_basis(seed, s, n, rank) for s in range(batch)])).to(dev)
    return A0, A1, q0


def _run(cf, dev, A0, A1, q0, rank, iters, fb, noalloc):
    batch, m, n = A1.shape
    ah = torch.empty((batch, m, n), dtype=torch.float32, device=dev)
    er = torch.empty_like(ah)
    cf.init_state(A0, ah, er)
    q = q0.clone()
    pay = cf.lowrank_payload(batch, m, n, rank, fb, dev)
    if noalloc:
        cf.lowrank_compress_noalloc(A1, ah, er, q, rank, iters, fb, pay)
    else:
        ws = torch.empty(cf.lowrank_workspace_bytes(m, n, rank, batch), dtype=torch.uint8, device=dev)
        cf.lowrank_compress(A1, ah, er, q, rank, iters, fb, pay, ws)
    torch.cuda.synchronize()
    return [ah, er, q, *[p for p in pay if p is not None]]


def test_noalloc_matches_workspace_call(cf):
    dev = cf.require_device()
    # first call: four FLUX-shard tensors at rank 32 (53 MiB of the 64 MiB scratch);
    # second: a smaller call of another shape, rank and factor width
    for batch, m, n, rank, iters, fb, seed in ((4, 1024, 3072, 32, 2, 4, 11), (2, 256, 768, 8, 3, 16, 12)):
        need = cf.lowrank_workspace_bytes(m, n, rank, batch)
        assert need <= cf.NOALLOC_SCRATCH_BYTES
        say(f"noalloc low rank: batch={batch} {m}x{n} rank={rank} iters={iters} fb={fb} ({need} B of scratch)")
        A0, A1, q0 = _case(cf, dev, batch, m, n, rank, seed)
        want = _run(cf, dev, A0, A1, q0, rank, iters, fb, noalloc=False)
        got = _run(cf, dev, A0, A1, q0, rank, iters, fb, noalloc=True)
        for i, (x, y) in enumerate(zip(got, want)):
            assert torch.equal(x, y), f"output {i} differs"


def test_noalloc_rejects_a_call_beyond_its_scratch(cf):
    dev = cf.require_device()
    batch, m, n, rank = 5, 1024, 3072, 32
    assert cf.lowrank_workspace_bytes(m, n, rank, batch) > cf.NOALLOC_SCRATCH_BYTES
    say("noalloc low rank: a call beyond the fixed scratch")
    A0, A1, q0 = _case(cf, dev, batch, m, n, rank, 13)
    ah = torch.empty((batch, m, n), dtype=torch.float32, device=dev)
    er = torch.empty_like(ah)
    cf.init_state(A0, ah, er)
    q = q0.clone()
    pay = cf.lowrank_payload(batch, m, n, rank, 4, dev)
    for p in pay:
        p.fill_(0x5A if p.dtype == torch.uint8 else 3.0)
    snap = [x.clone() for x in (ah, er, q, *pay)]
    with pytest.raises(cf.CFError) as ei:
        cf.lowrank_compress_noalloc(A1, ah, er, q, rank, 2, 4, pay)
    assert ei.value.status == -9
    torch.cuda.synchronize()
    for x, y in zip((ah, er, q, *pay), snap):
        assert torch.equal(x, y)
