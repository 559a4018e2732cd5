"""CPU oracle for CompactFusion residual compression (TEST INFRASTRUCTURE ONLY).

Thin numpy/ctypes wrapper over ``libcforacle.so`` (built from ``cf_oracle.c`` with
``gcc -O2 -ffp-contract=off``).  Only the test suite, ``__graft_entry__.smoke()`` and
``bench.py``'s CPU-baseline leg may import this package; the GPU library never does,
and the two share no code.

Every function follows "Accelerating Parallel Diffusion Model Serving with Residual
Compression" (CompactFusion summary), section Approach (residual against the previous
reconstruction, sender-side error feedback, low rank with INT4 factors) and its
measured-effects table (1-bit / 2-bit variants, warmup, rank 32, iterations), and the
Limitations list, which names sparsity as the other fast compressor family (read here as
per-group top-k of the residual with the same error feedback); the readings the pages leave open are listed at the top of ``cf_oracle.c``.

Activations are numpy arrays: ``uint16`` holds raw bf16 bits, ``float32`` is fp32.
State arrays (``ahat``, ``err``) are float32 and updated in place.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcforacle.so")
GROUP = 128
BF16, F32 = 0, 1

_SIG = {
    "cfo_init_state": "ipppl",
    "cfo_compress": "iipppppl",
    "cfo_decompress": "ipppl",
    "cfo_compress_explicit_ef": "iippppppl",
    "cfo_compress_noef": "iipppppl",
    "cfo_quantize_naive": "iippppl",
    "cfo_int4_quantize": "plipp",
    "cfo_int4_dequantize": "pplip",
    "cfo_lowrank_compress": "ippplliiippppp",
    "cfo_lowrank_decompress": "ippppplli",
    "cfo_topk_compress": "iipppppl",
    "cfo_topk_decompress": "ipppl",
}
_CT = {"i": ctypes.c_int, "l": ctypes.c_int64, "p": ctypes.c_void_p}


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"activation dtype {a.dtype} (want uint16 bf16 bits or float32)")


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"{what} failed with status {rc}")


def codes_bytes(numel: int, bits: int) -> int:
    return numel * bits // 8


class Oracle:
    """The oracle functions bound to one build of the C library."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        for name, sig in _SIG.items():
            f = getattr(L, name)
            f.argtypes = [_CT[c] for c in sig]
            f.restype = ctypes.c_int
        self.L = L

    def init_state(self, a, ahat, err=None):
        _check(self.L.cfo_init_state(_dtype_code(a), _p(a), _p(ahat), _p(err), a.size),
               "init_state")

    def compress(self, bits, a, ahat, err, codes=None, scales=None):
        """One sender step; returns (codes uint8[numel*bits/8], scales float32[numel/128])."""
        n = a.size
        codes = np.zeros(codes_bytes(n, bits), np.uint8) if codes is None else codes
        scales = np.zeros(n // GROUP, np.float32) if scales is None else scales
        _check(self.L.cfo_compress(bits, _dtype_code(a), _p(a), _p(ahat), _p(err), _p(codes),
                                   _p(scales), n), "compress")
        return codes, scales

    def decompress(self, bits, codes, scales, ahat):
        _check(self.L.cfo_decompress(bits, _p(codes), _p(scales), _p(ahat), ahat.size),
               "decompress")

    def compress_explicit_ef(self, bits, a, a_prev, ahat, err):
        n = a.size
        codes = np.zeros(codes_bytes(n, bits), np.uint8)
        scales = np.zeros(n // GROUP, np.float32)
        _check(self.L.cfo_compress_explicit_ef(bits, _dtype_code(a), _p(a), _p(a_prev), _p(ahat),
                                               _p(err), _p(codes), _p(scales), n), "explicit_ef")
        return codes, scales

    def compress_noef(self, bits, a, a_prev, ahat):
        n = a.size
        codes = np.zeros(codes_bytes(n, bits), np.uint8)
        scales = np.zeros(n // GROUP, np.float32)
        _check(self.L.cfo_compress_noef(bits, _dtype_code(a), _p(a), _p(a_prev), _p(ahat),
                                        _p(codes), _p(scales), n), "noef")
        return codes, scales

    def quantize_naive(self, bits, a):
        n = a.size
        out = np.zeros(n, np.float32)
        codes = np.zeros(codes_bytes(n, bits), np.uint8)
        scales = np.zeros(n // GROUP, np.float32)
        _check(self.L.cfo_quantize_naive(bits, _dtype_code(a), _p(a), _p(out), _p(codes),
                                         _p(scales), n), "naive")
        return out.reshape(a.shape), codes, scales

    def int4_quantize(self, x):
        rows, k = x.shape
        x = np.ascontiguousarray(x, np.float32)
        packed = np.zeros(rows * k // 2, np.uint8)
        scales = np.zeros(k, np.float32)
        _check(self.L.cfo_int4_quantize(_p(x), rows, k, _p(packed), _p(scales)), "int4_quantize")
        return packed, scales

    def int4_dequantize(self, packed, scales, rows, k):
        x = np.zeros((rows, k), np.float32)
        _check(self.L.cfo_int4_dequantize(_p(packed), _p(scales), rows, k, _p(x)),
               "int4_dequantize")
        return x

    def lowrank_compress(self, a, ahat, err, q_state, rank, iters, factor_bits=4):
        """One low-rank sender step on an m x n tensor; q_state (n x rank) is updated."""
        m, n = a.shape
        u, us, v, vs = lowrank_payload(m, n, rank, factor_bits)
        _check(self.L.cfo_lowrank_compress(_dtype_code(a), _p(a), _p(ahat), _p(err), m, n, rank,
                                           iters, factor_bits, _p(q_state), _p(u), _p(us), _p(v),
                                           _p(vs)), "lowrank_compress")
        return u, us, v, vs

    def lowrank_decompress(self, factor_bits, u, us, v, vs, ahat, rank):
        m, n = ahat.shape
        _check(self.L.cfo_lowrank_decompress(factor_bits, _p(u), _p(us), _p(v), _p(vs), _p(ahat),
                                             m, n, rank), "lowrank_decompress")

    def topk_compress(self, k, a, ahat, err):
        """One top-k sender step; returns (idx uint8[G*k], vals uint16 bf16 bits[G*k])."""
        n = a.size
        idx = np.zeros(n // GROUP * k, np.uint8)
        vals = np.zeros(n // GROUP * k, np.uint16)
        _check(self.L.cfo_topk_compress(k, _dtype_code(a), _p(a), _p(ahat), _p(err), _p(idx),
                                        _p(vals), n), "topk_compress")
        return idx, vals

    def topk_decompress(self, k, idx, vals, ahat):
        _check(self.L.cfo_topk_decompress(k, _p(idx), _p(vals), _p(ahat), ahat.size),
               "topk_decompress")


def lowrank_payload(m, n, rank, factor_bits):
    """Zeroed factor/scale buffers for one tensor: (u, u_scales, v, v_scales)."""
    if factor_bits == 4:
        return (np.zeros(m * rank // 2, np.uint8), np.zeros(rank, np.float32),
                np.zeros(n * rank // 2, np.uint8), np.zeros(rank, np.float32))
    if factor_bits == 16:
        return (np.zeros((m, rank), np.uint16), np.zeros(rank, np.float32),
                np.zeros((n, rank), np.uint16), np.zeros(rank, np.float32))
    return (np.zeros((m, rank), np.float32), np.zeros(rank, np.float32),
            np.zeros((n, rank), np.float32), np.zeros(rank, np.float32))


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(LIB_PATH)
    return _default
