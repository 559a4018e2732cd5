"""GPU parity of the 1/2-bit path (cf_init_state, cf_compress, cf_decompress) against
the CPU oracle, through the C ABI.

The bar is bit-exact: the oracle and the kernels take every decision in fp32 with
the same operation order (no FMA contraction on either side), so codes, scales, the
reconstruction and the error buffer must match bit for bit - stricter than the
tolerance the method needs (codes exact except within 1 ulp of a boundary; scales,
reconstruction and error within 1e-5 relative).  Trajectories evolve independently on
both sides from the same seeded inputs.  Full-size workloads are checked on sampled
tensors (the oracle computes any tensor on its own) plus properties that hold for
every element (receiver == sender, err == a - ahat).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import host, mismatch, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cf():
    from activation_residual_compression_cf_amd import cf as _cf

    return _cf


@pytest.fixture(scope="module")
def dev(cf):
    return cf.require_device()


@pytest.fixture(scope="module")
def O():
    return oracle.default()


def run_trajectory(cf, dev, O, wl: gen.Workload, bits: int, warmup: int, steps: int,
                   per_call: int, samples, seed: int = 0):
    say(f"trajectory {wl.name} {wl.m}x{wl.n} x{wl.slots} bits={bits} W={warmup} "
        f"steps={steps} per_call={per_call} samples={list(samples)}")
    tr = gen.Trajectory(wl, seed)
    numel = wl.m * wl.n
    tx = cf.Slab(wl.slots, numel, bits, dev)
    rx = cf.Slab(wl.slots, numel, bits, dev, receiver=True)
    ost = {s: (np.empty((wl.m, wl.n), np.float32), np.empty((wl.m, wl.n), np.float32))
           for s in samples}
    for t in range(steps):
        A = tr.next()
        a_d = to_dev(A, dev)
        if t < warmup:
            tx.init(a_d, per_call)
            rx.init(a_d, per_call)
            for s, (ah, er) in ost.items():
                O.init_state(A[s], ah, er)
            continue
        tx.compress(a_d, per_call)
        rx.decompress(tx.codes, tx.scales, per_call)
        torch.cuda.synchronize()
        for s, (ah, er) in ost.items():
            c_o, s_o = O.compress(bits, A[s], ah, er)
            tag = f"step {t} slot {s}"
            assert np.array_equal(host(tx.codes[s]), c_o), f"{tag} codes: {mismatch(host(tx.codes[s]), c_o)}"
            assert np.array_equal(host(tx.scales[s]), s_o), f"{tag} scales: {mismatch(host(tx.scales[s]), s_o)}"
            assert np.array_equal(host(tx.ahat[s]), ah.reshape(-1)), f"{tag} ahat: {mismatch(host(tx.ahat[s]), ah)}"
            assert np.array_equal(host(tx.err[s]), er.reshape(-1)), f"{tag} err: {mismatch(host(tx.err[s]), er)}"
        # every element: the receiver mirrors the sender, and err = a - ahat
        assert torch.equal(rx.ahat, tx.ahat), f"step {t}: receiver differs from sender"
        a32 = a_d.reshape(wl.slots, numel).float()
        assert torch.equal(tx.err, a32 - tx.ahat), f"step {t}: err != a - ahat"
        del a32
    return tx, rx


@pytest.mark.parametrize("bits", [1, 2])
def test_tiny_trajectory(cf, dev, O, bits):
    """256x128 fp32, A_0 ~ N(0,1), drift N(0, 0.05^2), 1 warmup step."""
    run_trajectory(cf, dev, O, gen.WORKLOADS["tiny"], bits, warmup=1, steps=4, per_call=1,
                   samples=[0])


@pytest.mark.parametrize("bits,dtype", [(1, "bf16"), (2, "bf16"), (1, "f32"), (2, "f32")])
def test_several_tiles_ragged_tail(cf, dev, O, bits, dtype):
    """173 groups per tensor (5 full blocks of 32 groups + 13), 3 tensors per call."""
    wl = gen.Workload("ragged", 173, 128, 3, 4, dtype, dtype == "bf16")
    run_trajectory(cf, dev, O, wl, bits, warmup=1, steps=4, per_call=3, samples=[0, 1, 2])


@pytest.mark.parametrize("bits", [1, 2])
@pytest.mark.parametrize("rows", [1567, 44001])
def test_partial_round_of_block_runs(cf, dev, O, bits, rows):
    """Grids that end inside a round of the per-XCD block runs, with a ragged last tile.
    3 tensors of rows x 128 in one call: 1567 rows give 4701 groups, so the sender's
    2351 one-wave blocks fill one round of 2048 and part of the next; 44001 rows give
    132003 groups, enough for the decode's large launch (16501 blocks of 256 threads,
    32 rounds of 512 and a partial one) and 66002 sender blocks (32 rounds of 2048 and
    a partial one)."""
    wl = gen.Workload(f"runs{rows}", rows, 128, 3, 4, "bf16", True)
    run_trajectory(cf, dev, O, wl, bits, warmup=1, steps=4, per_call=3, samples=[0, 1, 2])


@pytest.mark.parametrize("bits", [1, 2])
def test_single_group_special_values(cf, dev, O, bits):
    """One group: zero residual, exact 2-bit ties, signed zeros, subnormals."""
    cases = []
    z = np.zeros(128, np.float32)
    cases.append((z.copy(), z.copy()))                              # zero residual
    r = np.zeros(128, np.float32)
    r[:3] = [3.0, 2.0, -2.0]                                        # |r| == s ties (s = 2)
    r[3:] = 0.5
    cases.append((r, np.zeros(128, np.float32)))
    m = np.full(128, -0.0, np.float32)
    cases.append((m, np.zeros(128, np.float32)))                    # r = -0 everywhere
    sub = (np.arange(128, dtype=np.float32) - 64) * np.float32(1e-40)  # subnormal residuals
    cases.append((sub.astype(np.float32), np.zeros(128, np.float32)))
    rng = np.random.default_rng(9)
    a = rng.standard_normal(128).astype(np.float32)
    cases.append((a, a.copy()))                                     # a == ahat
    for i, (a, ah0) in enumerate(cases):
        say(f"single group case {i} bits={bits}")
        ah_o, er_o = ah0.copy(), np.zeros(128, np.float32)
        c_o, s_o = O.compress(bits, a, ah_o, er_o)
        a_d, ah_d = to_dev(a, dev), to_dev(ah0, dev)
        er_d = torch.full((128,), 7.0, device=dev)
        codes, scales = cf.compress(bits, a_d, ah_d, er_d)
        torch.cuda.synchronize()
        assert np.array_equal(host(codes), c_o), (i, mismatch(host(codes), c_o))
        assert np.array_equal(host(scales), s_o), (i, host(scales), s_o)
        assert np.array_equal(host(ah_d).view(np.uint32), ah_o.view(np.uint32)), i
        assert np.array_equal(host(er_d).view(np.uint32), er_o.view(np.uint32)), i


def test_flux_1bit_full_shape(cf, dev, O):
    """114 x (1024 x 3072) bf16 per step, Compact-1bit, 1 warmup step, one call per
    layer (K and V), as the benchmark's per-layer row times it."""
    run_trajectory(cf, dev, O, gen.WORKLOADS["flux"], 1, warmup=1, steps=3, per_call=2,
                   samples=[0, 1, 57, 113])


def test_flux_1bit_full_shape_one_call(cf, dev, O):
    """The benchmark's headline launch: Compact-1bit, the whole step of 114 tensors as
    one call, 1 warmup step."""
    run_trajectory(cf, dev, O, gen.WORKLOADS["flux"], 1, warmup=1, steps=3, per_call=114,
                   samples=[0, 56, 113])


def test_flux_1bit_whole_trajectory(cf, dev, O):
    """All 28 denoising steps of the FLUX shard (1 warmup, 27 compressed), the headline
    launch, with two sampled tensors replayed on the oracle at every step: bit-exact
    over the whole horizon, where the error feedback has had every step to accumulate."""
    run_trajectory(cf, dev, O, gen.WORKLOADS["flux"], 1, warmup=1, steps=28, per_call=114,
                   samples=[3, 110])


def test_flux_2bit_full_shape_one_call(cf, dev, O):
    """Compact-2bit, 2 warmup steps, the whole step as one slab call."""
    run_trajectory(cf, dev, O, gen.WORKLOADS["flux"], 2, warmup=2, steps=4, per_call=114,
                   samples=[0, 77, 113])


def test_cogvideo_2bit_whole_trajectory(cf, dev, O):
    """All 50 CogVideoX-2b shard steps (2 warmup, 48 compressed) of 60 tensors of
    2925 x 1920, Compact-2bit, the whole step as one call; two sampled tensors replayed
    on the oracle at every step."""
    run_trajectory(cf, dev, O, gen.WORKLOADS["cogvideo"], 2, warmup=2, steps=50, per_call=60,
                   samples=[1, 58])


def test_cogvideo_2bit_full_shape(cf, dev, O):
    """60 x (2925 x 1920) bf16 per step, Compact-2bit, 2 warmup steps."""
    run_trajectory(cf, dev, O, gen.WORKLOADS["cogvideo"], 2, warmup=2, steps=4, per_call=2,
                   samples=[0, 31, 59])


def test_deterministic(cf, dev):
    wl = gen.Workload("det", 512, 3072, 2, 2, "bf16", True)
    tr = gen.Trajectory(wl, 4)
    a0, a1 = to_dev(tr.next(), dev), to_dev(tr.next(), dev)
    outs = []
    for _ in range(2):
        say("determinism run")
        s = cf.Slab(2, wl.numel, 2, dev)
        s.init(a0)
        s.compress(a1)
        torch.cuda.synchronize()
        outs.append([x.clone() for x in (s.ahat, s.err, s.codes, s.scales)])
    for x, y in zip(*outs):
        assert torch.equal(x, y)


@pytest.mark.parametrize("bits", [1, 2])
def test_guard_bytes_untouched(cf, dev, bits):
    """Canary bytes around every output stay intact (ragged size)."""
    n = 128 * 45
    pad = 4096
    rng = np.random.default_rng(10)
    a = to_dev(rng.standard_normal(n).astype(np.float32), dev)

    def guarded(nbytes):
        buf = torch.full((nbytes + 2 * pad,), 0xA5, dtype=torch.uint8, device=dev)
        return buf, buf[pad:pad + nbytes]

    hb, h = guarded(n * 4)
    eb, e = guarded(n * 4)
    cb, c = guarded(n * bits // 8)
    sb, sc = guarded(n // 128 * 4)
    h.view(torch.float32).zero_()
    say(f"guard bytes bits={bits}")
    cf.compress(bits, a, h.view(torch.float32), e.view(torch.float32), c, sc.view(torch.float32))
    cf.decompress(bits, c, sc.view(torch.float32), h.view(torch.float32))
    torch.cuda.synchronize()
    for buf in (hb, eb, cb, sb):
        g = host(buf)
        assert (g[:pad] == 0xA5).all() and (g[-pad:] == 0xA5).all()


def test_failed_call_writes_nothing(cf, dev):
    n = 128 * 8
    a = torch.randn(n, device=dev)
    ah = torch.zeros(n, device=dev)
    er = torch.full((n,), 3.0, device=dev)
    codes = torch.full((n // 8,), 0x5A, dtype=torch.uint8, device=dev)
    sc = torch.full((n // 128,), 2.0, device=dev)
    snap = [x.clone() for x in (ah, er, codes, sc)]
    with pytest.raises(cf.CFError) as ei:
        cf.compress(1, a, ah, ah, codes, sc)  # err aliases ahat
    assert ei.value.status == -5
    with pytest.raises(cf.CFError):
        cf.compress(3, a, ah, er, codes, sc)
    with pytest.raises(cf.CFError):
        cf.compress(1, a[:1000], ah[:1000], er[:1000], codes, sc)  # not a multiple of 128
    with pytest.raises(ValueError):
        cf.compress(2, a, ah, er, codes, sc)  # 2-bit codes need twice the bytes: refused by the binding
    with pytest.raises(ValueError):
        cf.decompress(1, codes[:64], sc, ah)  # codes too short for ahat
    torch.cuda.synchronize()
    for x, y in zip((ah, er, codes, sc), snap):
        assert torch.equal(x, y)


def test_index_beyond_2_31_elements(cf, dev, O):
    """A single call over 2^31 + 2^20 elements (64-bit indexing); sampled groups at the
    start, around 2^31 and at the end are checked against the oracle, and a receiver
    decoding the same payload matches the sender on every element."""
    wl = gen.Workload("big", 1024, 3072, 1, 2, "bf16", True)
    tr = gen.Trajectory(wl, 5)
    t0, t1 = tr.next()[0].reshape(-1), tr.next()[0].reshape(-1)
    numel = (1 << 31) + (1 << 20)
    reps = -(-numel // t0.size)
    a0 = np.tile(t0, reps)[:numel]
    a1 = np.tile(t1, reps)[:numel]
    say(f"index beyond 2^31: numel={numel}")
    a0_d = to_dev(a0, dev)
    ah = torch.empty(numel, dtype=torch.float32, device=dev)
    er = torch.empty(numel, dtype=torch.float32, device=dev)
    cf.init_state(a0_d, ah, er)
    rx = torch.empty(numel, dtype=torch.float32, device=dev)
    cf.init_state(a0_d, rx)
    del a0_d
    a1_d = to_dev(a1, dev)
    codes, scales = cf.compress(1, a1_d, ah, er)
    cf.decompress(1, codes, scales, rx)
    torch.cuda.synchronize()
    assert torch.equal(rx, ah), "receiver != sender beyond 2^31 elements"
    del rx
    ng = numel // 128
    for g0 in (0, (1 << 31) // 128 - 8, ng - 64):
        sl = slice(g0 * 128, (g0 + 64) * 128)
        ah_o = gen.as_f32(a0[sl]).copy()
        er_o = np.zeros_like(ah_o)
        c_o, s_o = O.compress(1, np.ascontiguousarray(a1[sl]), ah_o, er_o)
        assert np.array_equal(host(codes[g0 * 16:(g0 + 64) * 16]), c_o)
        assert np.array_equal(host(scales[g0:g0 + 64]), s_o)
        assert np.array_equal(host(ah[sl]), ah_o)
        assert np.array_equal(host(er[sl]), er_o)
