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


# An INT4 code is decided by rint(x / s) in fp32 on both sides, but the fp32 factor x
# itself is only determined to about 1e-6 of its column's largest element (Householder
# QR in fp64 against Cholesky QR with fp32 MFMA products), and so is s = max|x| / 7.
# With |x / s| <= 7 the two sides' x / s then differ by at most about 7 * 1e-6.  Where
# x / s lies that close to a half-integer, both neighbouring codes are valid roundings,
# and one flipped code can move the reconstruction by a few 1e-3 of its norm (one outer
# product of a factor column).
TIE = 1e-5  # |x / s - (j + 1/2)| below which either rounding is accepted


def int4_codes(O, packed, rows, k):
    return O.int4_dequantize(packed, np.ones(k, np.float32), rows, k).astype(np.int32)


def explain_int4_ties(O, a, ah_before, q_before, rank, iters, gpu_pay, r_gpu, tol):
    """Where the GPU's INT4 codes differ from the oracle's, the oracle's own fp32 factor
    must sit at a rounding tie and the codes must be neighbours; the GPU's reconstruction
    must then equal the oracle's reconstruction of those codes with the oracle's scales.
    Returns (number of tie flips, that relative error)."""
    m, n = ah_before.shape
    er = np.zeros_like(ah_before)
    P, _, Q, _ = O.lowrank_compress(a, ah_before.copy(), er, q_before.copy(), rank, iters, 32)
    u_o, us_o, v_o, vs_o = O.lowrank_compress(a, ah_before.copy(), er, q_before.copy(), rank, iters, 4)
    u_g, us_g, v_g, vs_g = gpu_pay
    assert rel(us_g, us_o) <= 1e-5 and rel(vs_g, vs_o) <= 1e-5, "INT4 scales differ"
    flips = 0
    for X, sc, po, pg, rows in ((P, us_o, u_o, u_g, m), (Q, vs_o, v_o, v_g, n)):
        co, cg = int4_codes(O, po, rows, rank), int4_codes(O, pg, rows, rank)
        diff = co != cg
        if diff.any():
            t = (np.asarray(X, np.float32).reshape(rows, rank)[diff] / sc[np.nonzero(diff)[1]]).astype(np.float32)
            assert np.all(np.abs(co[diff] - cg[diff]) == 1), "INT4 codes differ by more than one step"
            assert np.all(np.abs(np.abs(t - np.trunc(t)) - 0.5) <= TIE), "INT4 codes differ away from a tie"
            flips += int(diff.sum())
    r_ties = np.zeros((m, n), np.float32)
    O.lowrank_decompress(4, u_g, us_o, v_g, vs_o, r_ties, rank)
    return flips, rel(r_gpu, r_ties)
