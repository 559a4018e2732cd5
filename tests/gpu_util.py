"""Helpers shared by the GPU tests (host <-> device copies, labelled progress)."""
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
