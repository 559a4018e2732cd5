"""Seeded synthetic activation trajectories (inputs only; no compression arithmetic).

The C library ``libcfgen.so`` (built from ``cfgen.c`` by ``__graft_entry__.build()``)
draws every random number with one counter-based generator (SplitMix64 output
function over (seed, kind, slot, step, index)), so a tensor of any slot and step can
be regenerated on its own, bit for bit, by any caller.

Workloads (stand-ins for the FLUX.1-dev and CogVideoX-2b activations the CompactFusion
paper measures on, which are not available here):

* ``tiny``   -- one 256x128 fp32 tensor, A_0 ~ N(0,1), A_t = A_{t-1} + N(0, 0.05^2).
* ``flux``   -- 114 tensors (57 layers x K,V) of 1024 tokens x 3072 channels, bf16,
  per-channel lognormal(0, 0.5) scales with 1% of channels x20, drift 0.05*c_j*N(0,1),
  28 denoising steps.
* ``cogvideo`` -- 60 tensors (30 layers x K,V) of 2925 tokens x 1920 channels, bf16,
  same distribution, 50 steps.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcfgen.so")

KIND_BASIS = 4  # stream kind used for the low-rank variant's start basis

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        i64, u64, p = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
        L.cfgen_key.argtypes = [u64, i64, i64, i64]
        L.cfgen_key.restype = u64
        L.cfgen_value.argtypes = [u64, i64]
        L.cfgen_value.restype = u64
        L.cfgen_normals.argtypes = [u64, i64, i64, i64, i64, p]
        L.cfgen_channel_scales.argtypes = [u64, i64, i64, ctypes.c_double, ctypes.c_double,
                                           ctypes.c_double, p]
        L.cfgen_start.argtypes = [u64, i64, i64, i64, i64, p, p, p, p, ctypes.c_int]
        L.cfgen_advance.argtypes = [u64, i64, i64, i64, i64, i64, p, ctypes.c_double, p, p, p,
                                    ctypes.c_int]
        L.cfgen_to_bf16.argtypes = [p, p, i64]
        for f in ("cfgen_normals", "cfgen_channel_scales", "cfgen_start", "cfgen_advance",
                  "cfgen_to_bf16"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# Worker threads for host-side work: at most the CPU share one GPU's host gives a job.
THREAD_CAP = 16


def affinity_cores() -> int:
    """CPU cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def default_threads() -> int:
    return max(1, min(affinity_cores(), THREAD_CAP))


@dataclass(frozen=True)
class Workload:
    name: str
    m: int            # tokens per shard
    n: int            # channels
    slots: int        # tensors per step (layers x K,V)
    steps: int        # denoising steps
    dtype: str        # "bf16" or "f32"
    scaled: bool      # per-channel lognormal scales with outlier channels
    drift: float = 0.05
    sigma: float = 0.5
    outlier_frac: float = 0.01
    outlier_mult: float = 20.0

    @property
    def numel(self) -> int:
        return self.m * self.n


WORKLOADS = {
    "tiny": Workload("tiny", 256, 128, 1, 4, "f32", False),
    "flux": Workload("flux", 1024, 3072, 114, 28, "bf16", True),
    "cogvideo": Workload("cogvideo", 2925, 1920, 60, 50, "bf16", True),
}


def bf16_to_f32(x16: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits (uint16) to float32."""
    return (x16.astype(np.uint32) << 16).view(np.float32)


def normals(seed: int, kind: int, slot: int, step: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    rc = lib().cfgen_normals(seed, kind, slot, step, count, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"cfgen_normals failed: {rc}")
    return out


def start_basis(seed: int, slot: int, n: int, rank: int) -> np.ndarray:
    """N(0,1) n x rank fp32 start basis for the low-rank variant of one slot."""
    return normals(seed, KIND_BASIS, slot, 0, n * rank).reshape(n, rank)


class Trajectory:
    """Step-by-step generator for slots [slot0, slot0+nslots) of a workload.

    ``next()`` returns step t's activations as a contiguous array of shape
    (nslots, m, n): uint16 raw bf16 bits for bf16 workloads, float32 otherwise.
    """

    def __init__(self, wl: Workload, seed: int = 0, slot0: int = 0, nslots: int | None = None,
                 threads: int | None = None):
        self.wl, self.seed, self.slot0 = wl, seed, slot0
        self.nslots = wl.slots - slot0 if nslots is None else nslots
        self.threads = threads or default_threads()
        self.step = -1
        self.state = np.empty((self.nslots, wl.m, wl.n), dtype=np.float32)
        if wl.scaled:
            self.c = np.empty((self.nslots, wl.n), dtype=np.float32)
            for s in range(self.nslots):
                rc = lib().cfgen_channel_scales(seed, slot0 + s, wl.n, wl.sigma, wl.outlier_frac,
                                                wl.outlier_mult, _ptr(self.c[s]))
                if rc != 0:
                    raise RuntimeError("cfgen_channel_scales failed")
        else:
            self.c = None

    def next(self, out: np.ndarray | None = None) -> np.ndarray:
        wl = self.wl
        if out is None:
            out = np.empty((self.nslots, wl.m, wl.n),
                           dtype=np.uint16 if wl.dtype == "bf16" else np.float32)
        o16 = out if wl.dtype == "bf16" else None
        o32 = out if wl.dtype == "f32" else None
        self.step += 1
        if self.step == 0:
            rc = lib().cfgen_start(self.seed, self.slot0, self.nslots, wl.m, wl.n, _ptr(self.c),
                                   _ptr(self.state), _ptr(o16), _ptr(o32), self.threads)
        else:
            rc = lib().cfgen_advance(self.seed, self.slot0, self.nslots, self.step, wl.m, wl.n,
                                     _ptr(self.c), wl.drift, _ptr(self.state), _ptr(o16),
                                     _ptr(o32), self.threads)
        if rc != 0:
            raise RuntimeError(f"trajectory generation failed: {rc}")
        return out


def as_f32(x: np.ndarray) -> np.ndarray:
    """Activation array (uint16 bf16 bits or float32) as float32."""
    return bf16_to_f32(x) if x.dtype == np.uint16 else x
