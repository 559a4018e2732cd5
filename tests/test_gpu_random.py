"""Randomised bit-exact parity of the 1/2-bit, top-k and ablation paths over wide value
ranges.

Each case draws its size, activation dtype, compressor and data from a seeded
generator: per-group magnitudes spread over 60 decades of the fp32 exponent range
(10^-30 to 10^30), reconstructions that sit close to the activation in some groups and
are unrelated in others, and exact zeros, negative zeros and repeated values sprinkled
in.  Sizes run from one group to a few thousand.  The GPU's codes, scales, index bytes,
values, reconstruction, error and receiver mirror (and, for half the quantizer cases, the
mirror's round-to-nearest-even bf16 copy) must equal the oracle's bit for bit;
the ablation modes (no error feedback against a previous activation, naive quantization
of the activation itself) compare their codes, scales and reconstruction.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import explain_int4_ties, host, mismatch, rel, say, to_dev

pytestmark = pytest.mark.gpu

CASES = 30


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


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even bf16 bits of finite fp32 values (the test's input encoding)."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _widen(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def draw_case(seed: int):
    rng = np.random.default_rng(1000 + seed)
    groups = int(rng.integers(1, 3000))
    n = 128 * groups
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    mag = np.repeat(10.0 ** rng.uniform(-30, 30, size=groups), 128)
    x = rng.standard_normal(n) * mag
    u = rng.random(n)
    x[u < 0.02] = 0.0
    x[(u >= 0.02) & (u < 0.03)] = -0.0
    rep = (u >= 0.03) & (u < 0.06)
    x[rep] = mag[rep]  # ties inside a group
    a32 = x.astype(np.float32)
    a = _bf16_bits(a32) if dtype == "bf16" else a32
    a_f = _widen(a) if dtype == "bf16" else a
    # reconstruction: near the activation in half the groups, unrelated in the others
    near = np.repeat(rng.random(groups) < 0.5, 128)
    other = (rng.standard_normal(n) * np.repeat(10.0 ** rng.uniform(-30, 30, size=groups), 128))
    ahat = np.where(near, a_f * (1 + 1e-3 * rng.standard_normal(n)), other).astype(np.float32)
    kind = ("q1", "q2", "topk", "noef", "naive")[seed % 5]
    k = {2: 1, 7: 128}.get(seed, int(rng.integers(1, 129)))
    prev = a_f * (1 + 1e-2 * rng.standard_normal(n))  # the previous step's activation
    a_prev = _bf16_bits(prev.astype(np.float32)) if dtype == "bf16" else prev.astype(np.float32)
    return n, dtype, a, ahat, kind, k, a_prev


def _same_bits(x: np.ndarray, y: np.ndarray) -> bool:
    return np.array_equal(np.asarray(x).view(np.uint32), np.asarray(y).view(np.uint32))


@pytest.mark.parametrize("seed", range(CASES))
def test_random_case(cf, dev, O, seed):
    n, dtype, a, ahat0, kind, k, a_prev = draw_case(seed)
    say(f"random case {seed}: {kind} n={n} dtype={dtype}" + (f" k={k}" if kind == "topk" else ""))
    if kind in ("noef", "naive"):
        bits = 1 + seed % 2
        ah_o = ahat0.copy()
        a_d, ah_d = to_dev(a, dev), to_dev(ahat0, dev)
        if kind == "noef":
            codes_o, scales_o = O.compress_noef(bits, a, a_prev, ah_o)
            codes, scales = cf.compress_ablation(cf.CF_MODE_NOEF, bits, a_d, ah_d, to_dev(a_prev, dev))
        else:
            ah_o, codes_o, scales_o = O.quantize_naive(bits, a)
            codes, scales = cf.compress_ablation(cf.CF_MODE_NAIVE, bits, a_d, ah_d)
        torch.cuda.synchronize()
        assert np.array_equal(host(codes), codes_o), mismatch(host(codes), codes_o)
        assert _same_bits(host(scales), scales_o), mismatch(host(scales), scales_o)
        assert _same_bits(host(ah_d), ah_o), mismatch(host(ah_d).view(np.uint32), ah_o.view(np.uint32))
        return
    ah_o, er_o, rx_o = ahat0.copy(), np.zeros(n, np.float32), ahat0.copy()
    a_d = to_dev(a, dev)
    ah_d, rx_d = to_dev(ahat0, dev), to_dev(ahat0, dev)
    er_d = torch.full((n,), 7.0, device=dev)
    if kind == "topk":
        idx_o, vals_o = O.topk_compress(k, a, ah_o, er_o)
        O.topk_decompress(k, idx_o, vals_o, rx_o)
        idx, vals = cf.topk_compress(k, a_d, ah_d, er_d)
        cf.topk_decompress(k, idx, vals, rx_d)
        torch.cuda.synchronize()
        assert np.array_equal(host(idx), idx_o), mismatch(host(idx), idx_o)
        assert np.array_equal(host(vals).view(np.uint16), vals_o), mismatch(host(vals).view(np.uint16), vals_o)
    else:
        bits = 1 if kind == "q1" else 2
        codes_o, scales_o = O.compress(bits, a, ah_o, er_o)
        O.decompress(bits, codes_o, scales_o, rx_o)
        codes, scales = cf.compress(bits, a_d, ah_d, er_d)
        # even seeds decode with the bf16 copy of the mirror (cf_decompress_bf16)
        out16 = torch.empty(n, dtype=torch.bfloat16, device=dev) if seed % 2 == 0 else None
        cf.decompress(bits, codes, scales, rx_d, out_bf16=out16)
        torch.cuda.synchronize()
        assert np.array_equal(host(codes), codes_o), mismatch(host(codes), codes_o)
        assert _same_bits(host(scales), scales_o), mismatch(host(scales), scales_o)
        if out16 is not None:
            got16 = host(out16.view(torch.int16)).view(np.uint16)
            assert np.array_equal(got16, _bf16_bits(rx_o)), mismatch(got16, _bf16_bits(rx_o))
    assert _same_bits(host(ah_d), ah_o), mismatch(host(ah_d).view(np.uint32), ah_o.view(np.uint32))
    assert _same_bits(host(er_d), er_o), mismatch(host(er_d).view(np.uint32), er_o.view(np.uint32))
    assert _same_bits(host(rx_d), rx_o), mismatch(host(rx_d).view(np.uint32), rx_o.view(np.uint32))


LOWRANK_CASES = 12


def draw_lowrank_case(seed: int):
    rng = np.random.default_rng(2000 + seed)
    m, n = 16 * int(rng.integers(1, 40)), 16 * int(rng.integers(1, 40))
    fb = (4, 16, 32)[seed % 3]
    rank = int(rng.integers(1, min(m, n, 64) + 1))
    if fb == 4:
        rank = max(2, rank - rank % 2)
    iters = int(rng.integers(1, 7))
    batch = int(rng.integers(1, 4))
    dtype = "bf16" if seed % 2 == 0 else "f32"
    scale = 10.0 ** rng.uniform(-8, 8, size=(batch, 1, 1))
    a32 = (rng.standard_normal((batch, m, n)) * scale).astype(np.float32)
    a = _bf16_bits(a32) if dtype == "bf16" else a32
    a_f = _widen(a) if dtype == "bf16" else a
    ahat = (a_f * (1 + 0.1 * rng.standard_normal((batch, m, n)))).astype(np.float32)
    q = rng.standard_normal((batch, n, rank)).astype(np.float32)
    return m, n, rank, iters, fb, batch, dtype, a, ahat, q


@pytest.mark.parametrize("seed", range(LOWRANK_CASES))
def test_random_lowrank_case(cf, dev, O, seed):
    """Random shapes (multiples of 16 up to 624), ranks, iteration counts, factor widths,
    batches and per-tensor magnitudes (10^-8 to 10^8): the reconstruction update agrees
    with the oracle's to the low-rank tolerance (INT4 codes at rounding ties accepted as in
    the trajectory tests), e == a - Ahat exactly, and the receiver equals the sender bit
    for bit."""
    m, n, rank, iters, fb, batch, dtype, a, ahat0, q0 = draw_lowrank_case(seed)
    say(f"random low-rank case {seed}: {batch} x {m}x{n} rank={rank} iters={iters} fb={fb} dtype={dtype}")
    a_d, ah_d, rx_d = to_dev(a, dev), to_dev(ahat0, dev), to_dev(ahat0, dev)
    er_d = torch.empty_like(ah_d)
    q_d = to_dev(q0, dev)
    payload = cf.lowrank_compress(a_d, ah_d, er_d, q_d, rank, iters, fb)
    cf.lowrank_decompress(fb, payload, rx_d, rank)
    torch.cuda.synchronize()
    assert torch.equal(rx_d, ah_d), "receiver differs from sender"
    assert torch.equal(er_d, a_d.float() - ah_d), "err != a - ahat"
    tol = 2e-4 if fb == 32 else 1e-3
    for s in range(batch):
        ah_o, er_o, q_o = ahat0[s].copy(), np.zeros((m, n), np.float32), q0[s].copy()
        O.lowrank_compress(np.ascontiguousarray(a[s]), ah_o, er_o, q_o, rank, iters, fb)
        r_gpu = host(ah_d[s]).astype(np.float64) - ahat0[s]
        r_orc = ah_o.astype(np.float64) - ahat0[s]
        e = rel(r_gpu, r_orc)
        say(f"  tensor {s}: rel(R_gpu, R_oracle) = {e:.2e}")
        if e > tol and fb == 4:
            u, us, v, vs = (host(x) for x in payload)
            hu, hv = m * rank // 2, n * rank // 2
            gpu_pay = (u[s * hu:(s + 1) * hu], us[s * rank:(s + 1) * rank],
                       v[s * hv:(s + 1) * hv], vs[s * rank:(s + 1) * rank])
            # the same batch from the same state with fp32 factors: the same launches and factors
            f32 = cf.lowrank_compress(a_d, to_dev(ahat0, dev), torch.empty_like(ah_d), to_dev(q0, dev), rank,
                                      iters, 32)
            torch.cuda.synchronize()
            gpu_f32 = (host(f32[0]).reshape(batch, m, rank)[s], host(f32[2]).reshape(batch, n, rank)[s])
            flips, d, e = explain_int4_ties(O, np.ascontiguousarray(a[s]), ahat0[s], q0[s], rank, iters,
                                            gpu_pay, gpu_f32, r_gpu, cold=True)
            say(f"  tensor {s}: {flips} INT4 codes at rounding ties (factors within {d:.2e}); with them rel = {e:.2e}")
        assert e <= tol, f"tensor {s}: reconstruction update differs by {e:.3e}"
