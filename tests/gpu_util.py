"""Helpers shared by the GPU tests: host <-> device copies, labelled progress, relative
error, and the check that explains INT4 code differences by rounding ties."""
from __future__ import annotations

import sys

import numpy as np
import torch


def say(msg: str):
    """Print and flush a line naming the case about to run on the GPU."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dev) -> torch.Tensor:
    """uint16 arrays hold raw bf16 bits and become bfloat16 tensors; float32 stays."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(x).to(dev)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def mismatch(a: np.ndarray, b: np.ndarray) -> str:
    a = np.asarray(a).reshape(-1)
    b = np.asarray(b).reshape(-1)
    bad = np.flatnonzero(a != b)
    if bad.size == 0:
        return "equal"
    i = bad[0]
    return f"{bad.size} of {a.size} differ; first at {i}: {a[i]!r} vs {b[i]!r}"


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# An INT4 code is rint(x / s) in fp32 on both sides, but the fp32 factor x itself is
# determined only to rounding: the GPU forms Y = r Q and Q = r^T P as fp32 dot products of
# n = 3072 and m = 1024 terms (each good to about sqrt(terms) * 2^-24, a few 1e-6 of the
# operands' scale) and orthonormalises in fp64 Cholesky QR, the oracle does everything in
# fp64 with Householder QR; the orthonormalisation passes Y's error on, scaled by Y's
# conditioning.  Where x / s lies within that difference of a half-integer, the two sides
# may round to neighbouring codes, and one flipped code can move the reconstruction by a
# few 1e-3 of its norm (one outer product of a factor column).  Such a flip is accepted
# only where the GPU's fp32 factors (from the same step with fp32 factors: the kernels up
# to the quantizer are the same, and deterministic) agree with the oracle's to FACTOR_TOL
# of their column's largest element, each side's codes are the rounding of its own
# factors, and the two values lie on the two sides of the tie between the two codes.
# Measured on the FLUX trajectory (6 sampled tensors): warm-started steps agree to
# 0.5-2.2e-6; the first step, from a random start basis, to at most 7.5e-5 (rank 32, two
# iterations: the weakest directions of Y are still poorly separated, and the
# orthonormalisation magnifies Y's rounding along them).
FACTOR_TOL = {"warm": 1e-5, "cold": 2e-4}


def int4_codes(O, packed, rows, k):
    return O.int4_dequantize(packed, np.ones(k, np.float32), rows, k).astype(np.int32)


def explain_int4_ties(O, a, ah_before, q_before, rank, iters, gpu_pay, gpu_f32, r_gpu, cold):
    """Where the GPU's INT4 codes differ from the oracle's, explain each difference by the
    two sides' fp32 factors (gpu_f32 = the GPU's P, Q of the same step) lying on the two
    sides of one rounding tie (`cold`: q_before is a start basis, not a previous step's
    factor); the GPU's reconstruction must then equal the oracle's
    reconstruction of the GPU's codes with the oracle's scales.  Returns (number of
    flipped codes, the factors' largest difference relative to their column's largest
    element, that relative error)."""
    m, n = ah_before.shape
    er = np.zeros_like(ah_before)
    P, _, Q, _ = O.lowrank_compress(a, ah_before.copy(), er, q_before.copy(), rank, iters, 32)
    u_o, us_o, v_o, vs_o = O.lowrank_compress(a, ah_before.copy(), er, q_before.copy(), rank, iters, 4)
    u_g, us_g, v_g, vs_g = gpu_pay
    assert rel(us_g, us_o) <= 1e-5 and rel(vs_g, vs_o) <= 1e-5, "INT4 scales differ"
    flips, worst = 0, 0.0
    for X, Xg, so, sg, po, pg, rows in ((P, gpu_f32[0], us_o, us_g, u_o, u_g, m),
                                        (Q, gpu_f32[1], vs_o, vs_g, v_o, v_g, n)):
        X = np.asarray(X, np.float32).reshape(rows, rank)
        Xg = np.asarray(Xg, np.float32).reshape(rows, rank)
        cm = np.abs(X).max(axis=0)
        d = (np.abs(Xg.astype(np.float64) - X) / np.where(cm > 0, cm, 1.0)).max()
        worst = max(worst, float(d))
        tol = FACTOR_TOL["cold" if cold else "warm"]
        assert d <= tol, f"fp32 factors differ by {d:.3g} of their column maximum"
        qg, sq = O.int4_quantize(Xg)
        assert np.array_equal(qg, pg) and np.array_equal(sq, sg), "GPU codes are not its own factors' rounding"
        co, cg = int4_codes(O, po, rows, rank), int4_codes(O, pg, rows, rank)
        diff = co != cg
        if diff.any():
            cols = np.nonzero(diff)[1]
            assert np.all(np.abs(co[diff] - cg[diff]) == 1), "INT4 codes differ by more than one step"
            tie = (co[diff] + cg[diff]) / 2.0
            t_o = (X[diff] / so[cols]).astype(np.float32).astype(np.float64)
            t_g = (Xg[diff] / sg[cols]).astype(np.float32).astype(np.float64)
            assert np.all((t_o - tie) * (t_g - tie) <= 0), "INT4 codes differ away from a tie"
            flips += int(diff.sum())
    r_ties = np.zeros((m, n), np.float32)
    O.lowrank_decompress(4, u_g, us_o, v_g, vs_o, r_ties, rank)
    return flips, worst, rel(r_gpu, r_ties)
