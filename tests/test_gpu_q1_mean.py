"""GPU parity of the 1-bit group scale: the exact mean of |r| over a group, rounded once
to fp32 (to nearest, ties to even).

The page ("Accelerating Parallel Diffusion Model Serving with Residual Compression",
Approach; Compact-1bit in the measured-effects table) names the scale mean|r| and fixes
no summation order.  The oracle sums exactly; the kernel sums truncated terms in fp64,
which is exact, and falls back to an exact 288-bit sum only when the cut-off bits could
move the rounding.  Both must give the same scale bit for bit.  The groups below drive
the kernel through both paths: sums at rounding ties, ties broken by terms far below
fp64 precision, subnormal means, sums beyond fp32's range, and spans of up to 2^250
inside one group.

The bar the method sets (codes exact except within 1 ulp of a decision boundary;
scales, reconstruction and error within 1e-5 relative) is written out in
``assert_within_bar``; the kernel is expected to meet it with no difference at all.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gen
import oracle
import pins
from gpu_util import host, mismatch, say, to_dev

pytestmark = pytest.mark.gpu

REL = 1e-5  # scales, reconstruction and error: max|diff| / max|oracle| per tensor
CODE_FRAC = 1e-5  # code mismatches allowed, as a share of the elements


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


def golden_groups() -> np.ndarray:
    g = pins.load_golden("q1_exact_mean.txt")
    out = []
    for case in sorted({k.split("_")[0] for k in g}):
        a = np.zeros(128, np.float32)
        r = pins._golden_floats(g[f"{case}_r"])
        a[: r.size] = r
        out.append(a)
    return np.stack(out)


def assert_within_bar(tag, r_orc, c_gpu, c_orc, s_gpu, s_orc, ah_gpu, ah_orc, e_gpu, e_orc):
    """The tolerance the method states, then bit-exactness (what the design gives)."""
    bits_g = np.unpackbits(c_gpu, bitorder="little")
    bits_o = np.unpackbits(c_orc, bitorder="little")
    bad = np.flatnonzero(bits_g != bits_o)
    assert bad.size <= CODE_FRAC * bits_o.size, f"{tag}: {bad.size} code mismatches"
    if bad.size:
        near0 = np.abs(r_orc.reshape(-1)[bad]) <= np.spacing(np.float32(0)) * 2
        assert near0.all(), f"{tag}: codes differ away from a decision boundary"
    for nm, x, y in (("scales", s_gpu, s_orc), ("ahat", ah_gpu, ah_orc), ("err", e_gpu, e_orc)):
        den = float(np.abs(y).max()) or 1.0
        d = float(np.abs(x.astype(np.float64) - y.astype(np.float64)).max()) / den
        assert d <= REL, f"{tag}: {nm} differs by {d:.3g} relative"
    assert np.array_equal(c_gpu, c_orc), f"{tag} codes: {mismatch(c_gpu, c_orc)}"
    assert np.array_equal(s_gpu.view(np.uint32), s_orc.view(np.uint32)), f"{tag} scales: {mismatch(s_gpu, s_orc)}"
    assert np.array_equal(ah_gpu.view(np.uint32), ah_orc.view(np.uint32)), f"{tag} ahat: {mismatch(ah_gpu, ah_orc)}"
    assert np.array_equal(e_gpu.view(np.uint32), e_orc.view(np.uint32)), f"{tag} err: {mismatch(e_gpu, e_orc)}"


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_scale_stress_groups(cf, dev, O, sign):
    """Golden groups and the oracle pins' stress groups, given as a = r with Ahat = 0
    (and negated): scales, codes, reconstruction and error equal the oracle's."""
    r = np.concatenate([golden_groups(), pins._q1_test_groups(np.random.default_rng(21)),
                        pins._q1_test_groups(np.random.default_rng(22))]).astype(np.float32)
    a = (sign * r).reshape(-1).astype(np.float32)
    say(f"1-bit stress groups: {a.size // 128} groups, sign {sign:+.0f}")
    ah_o, er_o = np.zeros_like(a), np.zeros_like(a)
    c_o, s_o = O.compress(1, a, ah_o, er_o)
    a_d = to_dev(a, dev)
    ah_d = torch.zeros_like(a_d)
    er_d = torch.full_like(a_d, 7.0)
    codes, scales = cf.compress(1, a_d, ah_d, er_d)
    torch.cuda.synchronize()
    assert_within_bar("stress", a, host(codes), c_o, host(scales), s_o, host(ah_d), ah_o, host(er_d), er_o)


def tie_groups(G: int, seed: int = 5) -> np.ndarray:
    """G groups whose exact sum lies halfway between two fp32 values (integers near 2^19,
    sum in [2^26, 2^27) adjusted to 4 mod 8, scaled by a power of two), with element 127
    zero; in every other group element 127 is set to a term 2^-60 .. 2^-120 of the
    group's largest, which breaks the tie upwards."""
    rng = np.random.default_rng(seed)
    g = rng.integers(2 ** 18, 2 ** 20, (G, 128)).astype(np.int64)
    g[:, 127] = 0
    g[:, 0] -= g.sum(1) % 8 - 4
    s = g.sum(1)
    assert np.all((s % 8 == 4) & (s >= 2 ** 26) & (s < 2 ** 27))
    x = g.astype(np.float64) * 2.0 ** rng.integers(-10, 40, (G, 1))
    brk = np.arange(G) % 2 == 1
    x[brk, 127] = x[brk].max(1) * 2.0 ** -rng.integers(60, 121, int(brk.sum()))
    return x.astype(np.float32)


def test_scale_ties_every_group(cf, dev, O):
    """Every group's mean sits on a rounding tie, and every other group has the tie
    broken by a term far below fp64 precision of the sum: the unbroken ones go to the
    even value on the kernel's fast path, the broken ones take its exact path, in both
    halves of a wave and in neighbouring waves."""
    x = tie_groups(4096)
    a = x.reshape(-1)
    say(f"1-bit tie groups: {x.shape[0]}")
    ah_o, er_o = np.zeros_like(a), np.zeros_like(a)
    c_o, s_o = O.compress(1, a, ah_o, er_o)
    a_d = to_dev(a, dev)
    ah_d = torch.zeros_like(a_d)
    er_d = torch.zeros_like(a_d)
    codes, scales = cf.compress(1, a_d, ah_d, er_d)
    torch.cuda.synchronize()
    assert_within_bar("ties", a, host(codes), c_o, host(scales), s_o, host(ah_d), ah_o, host(er_d), er_o)


def test_flux_per_step_from_gpu_state(cf, dev, O):
    """The FLUX shard's headline launch (114 tensors in one call), step by step: before
    each step the oracle takes the GPU's own reconstruction of the sampled tensors, then
    both compress the same activation; codes, scales, reconstruction and error meet the
    bar (and agree bit for bit)."""
    wl = gen.WORKLOADS["flux"]
    tr = gen.Trajectory(wl, 0)
    numel = wl.numel
    tx = cf.Slab(wl.slots, numel, 1, dev)
    samples = (0, 31, 77, 113)
    for t in range(6):
        A = tr.next()
        a_d = to_dev(A, dev)
        if t == 0:
            tx.init(a_d, wl.slots)
            continue
        before = {s: host(tx.ahat[s]).copy() for s in samples}
        say(f"flux 1-bit per-step check, step {t}")
        tx.compress(a_d, wl.slots)
        torch.cuda.synchronize()
        for s in samples:
            ah = before[s].reshape(wl.m, wl.n).copy()
            er = np.empty_like(ah)
            r = (gen.as_f32(A[s]).astype(np.float32) - ah).astype(np.float32)
            c_o, s_o = O.compress(1, A[s], ah, er)
            assert_within_bar(f"step {t} slot {s}", r, host(tx.codes[s]), c_o, host(tx.scales[s]), s_o,
                              host(tx.ahat[s]), ah.reshape(-1), host(tx.err[s]), er.reshape(-1))
        del a_d
