"""Python binding of libcf (argument marshalling only).

Every function here forwards to the C ABI declared in ``include/cf.h``; all
arithmetic runs in the HIP kernels of ``libcf.so``.  PyTorch supplies device memory
and streams.  Importing this module fails loudly when ``libcf.so`` is missing: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcf.so")

CF_BF16, CF_F32 = 0, 1
CF_MODE_NOEF, CF_MODE_NAIVE = 1, 2
GROUP = 128

STATUS = {0: "CF_OK", -1: "CF_E_NULL", -2: "CF_E_SHAPE", -3: "CF_E_ALIGN", -4: "CF_E_ARG",
          -5: "CF_E_ALIAS", -6: "CF_E_WORKSPACE", -7: "CF_E_DEVICE", -8: "CF_E_HIP", -9: "CF_E_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20  # CF_NOALLOC_SCRATCH_BYTES

# name -> (restype, argtypes) ; i=int, l=int64, p=pointer, z=size_t
_SIG = {
    "cf_init_state": ("i", "ippplp"),
    "cf_compress": ("i", "iippppplp"),
    "cf_decompress": ("i", "ippplp"),
    "cf_decompress_bf16": ("i", "ipppplp"),
    "cf_compress_ablation": ("i", "iiipppppl" "p"),
    "cf_topk_compress": ("i", "iippppplp"),
    "cf_topk_decompress": ("i", "ippplp"),
    "cf_lowrank_compress": ("i", "ipppllii" "iipppppp" "zp"),
    "cf_lowrank_compress_noalloc": ("i", "ipppllii" "iippppp" "p"),
    "cf_lowrank_decompress": ("i", "ipppp" "pllii" "p"),
    "cf_lowrank_workspace_bytes": ("z", "llii"),
    "cf_codes_bytes": ("l", "li"),
    "cf_strerror": ("s", "i"),
    "cf_abi_version": ("i", ""),
}
_CT = {"i": ctypes.c_int, "l": ctypes.c_int64, "p": ctypes.c_void_p, "z": ctypes.c_size_t,
       "s": ctypes.c_char_p}


class CFError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({strerror(status)})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(the HIP library is required; there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIG.items():
        f = getattr(lib, name)
        f.restype = _CT[res]
        f.argtypes = [_CT[c] for c in args]
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.cf_strerror(status).decode()


def _check(fn: str, rc: int):
    if rc != 0:
        raise CFError(fn, rc)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libcf takes device tensors (a host pointer would fault the kernel)")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensor on {t.device}, but the current device is cuda:{torch.cuda.current_device()} "
                         "(libcf launches on the current device)")
    if not t.is_contiguous():
        raise ValueError("libcf needs contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _need(name: str, t: torch.Tensor | None, nbytes: int, valid: bool = True):
    """The C ABI cannot see buffer sizes: refuse a buffer smaller than the call uses.
    With ``valid`` False (an argument the C ABI rejects anyway) nothing is checked, so
    the call reports the library's own status."""
    if valid and t is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} B, the call needs {nbytes} B")


_F32, _U8 = torch.float32, torch.uint8
_BITS16 = (torch.int16, torch.uint16, torch.bfloat16)  # raw 16-bit (bf16) storage


def _dtype(name: str, t: torch.Tensor | None, *allowed):
    """The C ABI takes untyped pointers: refuse a buffer whose element type the kernel
    would misread (state and scales are fp32, codes and index bytes uint8)."""
    if t is not None and t.dtype not in allowed:
        raise TypeError(f"{name} is {t.dtype}; libcf wants {' or '.join(map(str, allowed))}")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _keep_for(t: torch.Tensor | None, stream) -> torch.Tensor | None:
    """Tie a buffer this module allocated (on the current stream) to the launch stream.
    PyTorch's caching allocator may hand a freed block to new work on the stream it was
    allocated on at once; when the kernels run on another stream, record_stream makes it
    wait for that stream's work first."""
    if t is None or stream is None:
        return t
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    if stream.cuda_stream != torch.cuda.current_stream().cuda_stream:
        t.record_stream(stream)
    return t


def _act_dtype(a: torch.Tensor) -> int:
    if a.dtype == torch.bfloat16:
        return CF_BF16
    if a.dtype == torch.float32:
        return CF_F32
    raise TypeError(f"activation dtype {a.dtype}: want torch.bfloat16 or torch.float32")


def require_device() -> torch.device:
    """cuda:0 if it is an MI355X (gfx950); raises otherwise."""
    if not torch.cuda.is_available():
        raise RuntimeError("no HIP device visible")
    arch = torch.cuda.get_device_properties(0).gcnArchName
    if not arch.startswith("gfx950"):
        raise RuntimeError(f"device 0 is {arch}, libcf is built for gfx950 only")
    return torch.device("cuda", 0)


def codes_bytes(numel: int, bits: int) -> int:
    n = lib.cf_codes_bytes(numel, bits)
    if n < 0:
        raise CFError("cf_codes_bytes", n)
    return n


@dataclass
class SenderState:
    """Sender-side state of one tensor (or slab): reconstruction and error buffer."""
    ahat: torch.Tensor
    err: torch.Tensor

    @staticmethod
    def create(numel: int, device=None) -> "SenderState":
        device = device or require_device()
        return SenderState(torch.empty(numel, dtype=torch.float32, device=device),
                           torch.empty(numel, dtype=torch.float32, device=device))


def init_state(a: torch.Tensor, ahat: torch.Tensor, err: torch.Tensor | None = None, stream=None):
    """Warmup: ahat = a, err = 0 (err None on the receiver)."""
    _dtype("ahat", ahat, _F32)
    _dtype("err", err, _F32)
    _need("ahat", ahat, 4 * a.numel())
    _need("err", err, 4 * a.numel())
    _check("cf_init_state", lib.cf_init_state(_act_dtype(a), _ptr(a), _ptr(ahat), _ptr(err),
                                              a.numel(), _stream(stream)))


def compress(bits: int, a: torch.Tensor, ahat: torch.Tensor, err: torch.Tensor | None,
             codes: torch.Tensor | None = None, scales: torch.Tensor | None = None, stream=None):
    """One sender step; returns (codes uint8[numel*bits/8], scales fp32[numel/128]).
    err None skips the (diagnostic) error buffer."""
    n = a.numel()
    if codes is None:
        codes = _keep_for(torch.empty(max(n * bits // 8, 0), dtype=torch.uint8, device=a.device), stream)
    if scales is None:
        scales = _keep_for(torch.empty(max(n // GROUP, 0), dtype=torch.float32, device=a.device), stream)
    for nm, t, dt in (("ahat", ahat, _F32), ("err", err, _F32), ("codes", codes, _U8), ("scales", scales, _F32)):
        _dtype(nm, t, dt)
    for nm, t, nb in (("ahat", ahat, 4 * n), ("err", err, 4 * n), ("codes", codes, n * bits // 8),
                      ("scales", scales, 4 * (n // GROUP))):
        _need(nm, t, nb, bits in (1, 2))
    _check("cf_compress", lib.cf_compress(bits, _act_dtype(a), _ptr(a), _ptr(ahat), _ptr(err),
                                          _ptr(codes), _ptr(scales), n, _stream(stream)))
    return codes, scales


def decompress(bits: int, codes: torch.Tensor, scales: torch.Tensor, ahat: torch.Tensor,
               stream=None, out_bf16: torch.Tensor | None = None):
    """Receiver step: ahat += decoded residual; with out_bf16 (a bfloat16 tensor of the
    same size) also writes the updated reconstruction rounded to bf16."""
    n = ahat.numel()
    for nm, t, dt in (("codes", codes, _U8), ("scales", scales, _F32), ("ahat", ahat, _F32)):
        _dtype(nm, t, dt)
    _need("codes", codes, n * bits // 8, bits in (1, 2))
    _need("scales", scales, 4 * (n // GROUP), bits in (1, 2))
    if out_bf16 is None:
        _check("cf_decompress", lib.cf_decompress(bits, _ptr(codes), _ptr(scales), _ptr(ahat),
                                                  ahat.numel(), _stream(stream)))
        return
    if out_bf16.dtype != torch.bfloat16 or out_bf16.numel() != ahat.numel():
        raise ValueError("out_bf16 must be a bfloat16 tensor of ahat's size")
    _check("cf_decompress_bf16", lib.cf_decompress_bf16(bits, _ptr(codes), _ptr(scales), _ptr(ahat),
                                                        _ptr(out_bf16), ahat.numel(), _stream(stream)))


def compress_ablation(mode: int, bits: int, a: torch.Tensor, ahat: torch.Tensor,
                      a_prev: torch.Tensor | None = None, codes: torch.Tensor | None = None,
                      scales: torch.Tensor | None = None, stream=None):
    """Ablation sender step (CF_MODE_NOEF needs a_prev); returns (codes, scales)."""
    n = a.numel()
    if codes is None:
        codes = _keep_for(torch.empty(n * bits // 8, dtype=torch.uint8, device=a.device), stream)
    if scales is None:
        scales = _keep_for(torch.empty(n // GROUP, dtype=torch.float32, device=a.device), stream)
    for nm, t, dt in (("ahat", ahat, _F32), ("a_prev", a_prev, a.dtype), ("codes", codes, _U8),
                      ("scales", scales, _F32)):
        _dtype(nm, t, dt)
    for nm, t, nb in (("ahat", ahat, 4 * n), ("a_prev", a_prev, n * a.element_size()),
                      ("codes", codes, n * bits // 8), ("scales", scales, 4 * (n // GROUP))):
        _need(nm, t, nb, bits in (1, 2))
    _check("cf_compress_ablation", lib.cf_compress_ablation(
        mode, bits, _act_dtype(a), _ptr(a), _ptr(a_prev), _ptr(ahat), _ptr(codes), _ptr(scales), n,
        _stream(stream)))
    return codes, scales


def topk_compress(k: int, a: torch.Tensor, ahat: torch.Tensor, err: torch.Tensor | None,
                  idx: torch.Tensor | None = None, vals: torch.Tensor | None = None, stream=None):
    """One top-k sender step; returns (idx uint8[numel/128*k], vals bf16 bits int16[numel/128*k])."""
    slots = max(a.numel() // GROUP * k, 0)
    if idx is None:
        idx = _keep_for(torch.empty(slots, dtype=torch.uint8, device=a.device), stream)
    if vals is None:
        vals = _keep_for(torch.empty(slots, dtype=torch.int16, device=a.device), stream)
    n = a.numel()
    for nm, t, dts in (("ahat", ahat, (_F32,)), ("err", err, (_F32,)), ("idx", idx, (_U8,)), ("vals", vals, _BITS16)):
        _dtype(nm, t, *dts)
    for nm, t, nb in (("ahat", ahat, 4 * n), ("err", err, 4 * n), ("idx", idx, slots), ("vals", vals, 2 * slots)):
        _need(nm, t, nb, 1 <= k <= GROUP)
    _check("cf_topk_compress", lib.cf_topk_compress(k, _act_dtype(a), _ptr(a), _ptr(ahat), _ptr(err),
                                                    _ptr(idx), _ptr(vals), a.numel(), _stream(stream)))
    return idx, vals


def topk_decompress(k: int, idx: torch.Tensor, vals: torch.Tensor, ahat: torch.Tensor, stream=None):
    """Receiver step: ahat[group, idx] += bf16 value, for every sent slot."""
    slots = max(ahat.numel() // GROUP * k, 0)
    _dtype("idx", idx, _U8)
    _dtype("vals", vals, *_BITS16)
    _dtype("ahat", ahat, _F32)
    _need("idx", idx, slots, 1 <= k <= GROUP)
    _need("vals", vals, 2 * slots, 1 <= k <= GROUP)
    _check("cf_topk_decompress", lib.cf_topk_decompress(k, _ptr(idx), _ptr(vals), _ptr(ahat), ahat.numel(),
                                                        _stream(stream)))


def _dev_ptr(t: torch.Tensor) -> int:
    return _ptr(t).value


class Slab:
    """1/2-bit state of ``count`` tensors of ``numel`` elements laid out back to back
    (e.g. the K and V activations of every layer of one sequence-parallel shard).

    ``compress``/``decompress``/``init`` issue one C-ABI call per ``per_call``
    consecutive tensors (2 = one layer's K and V, the serving pattern; ``count`` = one
    call for the whole step).  Pointers are computed once; each call only forwards
    integers to libcf.
    """

    def __init__(self, count: int, numel: int, bits: int, device=None, receiver: bool = False):
        if numel % GROUP:
            raise ValueError("numel must be a multiple of 128")
        device = device or require_device()
        self.count, self.numel, self.bits = count, numel, bits
        f32 = torch.float32
        self.ahat = torch.empty((count, numel), dtype=f32, device=device)
        self.err = None if receiver else torch.empty((count, numel), dtype=f32, device=device)
        self.codes = torch.empty((count, numel * bits // 8), dtype=torch.uint8, device=device)
        self.scales = torch.empty((count, numel // GROUP), dtype=f32, device=device)

    def _chunks(self, per_call: int):
        per_call = max(1, min(per_call, self.count))
        for i in range(0, self.count, per_call):
            yield i, min(per_call, self.count - i)

    def init(self, a: torch.Tensor, per_call: int = 2, stream=None):
        if a.numel() != self.count * self.numel:
            raise ValueError("activation slab has the wrong size")
        dt, s = _act_dtype(a), _stream(stream)
        ab, esz = _dev_ptr(a), a.element_size()
        hb = _dev_ptr(self.ahat)
        eb = _dev_ptr(self.err) if self.err is not None else None
        n = self.numel
        for i, c in self._chunks(per_call):
            _check("cf_init_state", lib.cf_init_state(
                dt, ab + i * n * esz, hb + i * n * 4, None if eb is None else eb + i * n * 4,
                c * n, s))

    def compress(self, a: torch.Tensor, per_call: int = 2, stream=None, timer: list | None = None,
                 streams: list | None = None):
        """Compress one step.  With ``timer`` a list, a pair of timing events recorded on
        the launch stream just before and after every call is appended to it.  With
        ``streams`` a list of streams, call i goes to streams[i % len(streams)] instead (the
        calls touch disjoint tensors, so they may overlap); ordering those streams against
        the inputs and the later consumers is the caller's."""
        if self.err is None:
            raise RuntimeError("receiver slab has no error buffer")
        if a.numel() != self.count * self.numel:
            raise ValueError("activation slab has the wrong size")
        dt, s, bits, n = _act_dtype(a), _stream(stream), self.bits, self.numel
        ab, esz = _dev_ptr(a), a.element_size()
        hb, eb = _dev_ptr(self.ahat), _dev_ptr(self.err)
        cb, sb = _dev_ptr(self.codes), _dev_ptr(self.scales)
        cbytes, ng = n * bits // 8, n // GROUP
        f = lib.cf_compress
        ts = None if timer is None else (torch.cuda.current_stream() if stream is None else stream)
        rr = [_stream(x) for x in streams] if streams else None
        for j, (i, c) in enumerate(self._chunks(per_call)):
            if ts is not None:
                ev0 = torch.cuda.Event(enable_timing=True)
                ev0.record(ts)
            rc = f(bits, dt, ab + i * n * esz, hb + i * n * 4, eb + i * n * 4, cb + i * cbytes,
                   sb + i * ng * 4, c * n, s if rr is None else rr[j % len(rr)])
            if rc:
                raise CFError("cf_compress", rc)
            if ts is not None:
                ev1 = torch.cuda.Event(enable_timing=True)
                ev1.record(ts)
                timer.append((ev0, ev1))

    def decompress(self, codes: torch.Tensor, scales: torch.Tensor, per_call: int = 2, stream=None):
        s, bits, n = _stream(stream), self.bits, self.numel
        _dtype("codes", codes, _U8)
        _dtype("scales", scales, _F32)
        _need("codes", codes, self.count * n * bits // 8)
        _need("scales", scales, 4 * self.count * (n // GROUP))
        cb, sb, hb = _dev_ptr(codes), _dev_ptr(scales), _dev_ptr(self.ahat)
        cbytes, ng = n * bits // 8, n // GROUP
        f = lib.cf_decompress
        for i, c in self._chunks(per_call):
            rc = f(bits, cb + i * cbytes, sb + i * ng * 4, hb + i * n * 4, c * n, s)
            if rc:
                raise CFError("cf_decompress", rc)


def lowrank_workspace_bytes(m: int, n: int, rank: int, batch: int = 1) -> int:
    nb = lib.cf_lowrank_workspace_bytes(m, n, rank, batch)
    if nb == 0:
        raise CFError("cf_lowrank_workspace_bytes", -2)
    return nb


def lowrank_payload(batch: int, m: int, n: int, rank: int, factor_bits: int, device):
    """Empty payload buffers (u, u_scales, v, v_scales) for `batch` tensors."""
    if factor_bits == 4:
        return (torch.empty(batch * m * rank // 2, dtype=torch.uint8, device=device),
                torch.empty(batch * rank, dtype=torch.float32, device=device),
                torch.empty(batch * n * rank // 2, dtype=torch.uint8, device=device),
                torch.empty(batch * rank, dtype=torch.float32, device=device))
    dt = torch.int16 if factor_bits == 16 else torch.float32  # bf16 bits or fp32
    return (torch.empty(batch * m * rank, dtype=dt, device=device), None,
            torch.empty(batch * n * rank, dtype=dt, device=device), None)


def _check_lowrank_buffers(batch, m, n, rank, factor_bits, payload):
    u, us, v, vs = payload
    esz = {4: 0.5, 16: 2, 32: 4}.get(factor_bits)
    if esz is None or rank < 1:
        return  # the C ABI rejects these arguments itself
    fdt = {4: (_U8,), 16: _BITS16, 32: (_F32,)}[factor_bits]
    _dtype("u", u, *fdt)
    _dtype("v", v, *fdt)
    _dtype("u_scales", us, _F32)
    _dtype("v_scales", vs, _F32)
    _need("u", u, int(batch * m * rank * esz))
    _need("v", v, int(batch * n * rank * esz))
    if factor_bits == 4:
        _need("u_scales", us, 4 * batch * rank)
        _need("v_scales", vs, 4 * batch * rank)


def lowrank_compress(a: torch.Tensor, ahat: torch.Tensor, err: torch.Tensor | None,
                     q_state: torch.Tensor, rank: int, iters: int, factor_bits: int = 4,
                     payload=None, workspace: torch.Tensor | None = None, stream=None):
    """One low-rank sender step on a (batch, m, n) activation; returns the payload
    (u, u_scales, v, v_scales).  q_state is (batch, n, rank) fp32, updated in place."""
    batch, m, n = a.shape
    if payload is None:
        payload = tuple(_keep_for(t, stream) for t in lowrank_payload(batch, m, n, rank, factor_bits, a.device))
    u, us, v, vs = payload
    need = lowrank_workspace_bytes(m, n, rank, batch)
    if workspace is None:
        # freed when this call returns, possibly before the launch stream has used it
        workspace = _keep_for(torch.empty(need, dtype=torch.uint8, device=a.device), stream)
    _check_lowrank_buffers(batch, m, n, rank, factor_bits, payload)
    numel = batch * m * n
    for nm, t in (("ahat", ahat), ("err", err), ("q_state", q_state)):
        _dtype(nm, t, _F32)
    for nm, t, nb in (("ahat", ahat, 4 * numel), ("err", err, 4 * numel), ("q_state", q_state, 4 * batch * n * rank)):
        _need(nm, t, nb, rank >= 1)
    _check("cf_lowrank_compress", lib.cf_lowrank_compress(
        _act_dtype(a), _ptr(a), _ptr(ahat), _ptr(err), m, n, rank, iters, factor_bits, batch,
        _ptr(q_state), _ptr(u), _ptr(us), _ptr(v), _ptr(vs), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return u, us, v, vs


def lowrank_compress_noalloc(a: torch.Tensor, ahat: torch.Tensor, err: torch.Tensor | None,
                             q_state: torch.Tensor, rank: int, iters: int, factor_bits: int, payload,
                             stream=None):
    """cf_lowrank_compress_noalloc: one low-rank sender step that uses the library's fixed
    device scratch instead of a workspace, for callers that cannot allocate.  Every buffer,
    the payload (u, u_scales, v, v_scales) included, comes from the caller; nothing is
    allocated here.  Calls that may overlap on one GPU race on that scratch."""
    batch, m, n = a.shape
    u, us, v, vs = payload
    _check_lowrank_buffers(batch, m, n, rank, factor_bits, payload)
    numel = batch * m * n
    for nm, t in (("ahat", ahat), ("err", err), ("q_state", q_state)):
        _dtype(nm, t, _F32)
    for nm, t, nb in (("ahat", ahat, 4 * numel), ("err", err, 4 * numel), ("q_state", q_state, 4 * batch * n * rank)):
        _need(nm, t, nb, rank >= 1)
    _check("cf_lowrank_compress_noalloc", lib.cf_lowrank_compress_noalloc(
        _act_dtype(a), _ptr(a), _ptr(ahat), _ptr(err), m, n, rank, iters, factor_bits, batch,
        _ptr(q_state), _ptr(u), _ptr(us), _ptr(v), _ptr(vs), _stream(stream)))
    return u, us, v, vs


def lowrank_decompress(factor_bits: int, payload, ahat: torch.Tensor, rank: int, stream=None):
    """Receiver step on a (batch, m, n) reconstruction: ahat += U^ V^^T."""
    batch, m, n = ahat.shape
    u, us, v, vs = payload
    _dtype("ahat", ahat, _F32)
    _check_lowrank_buffers(batch, m, n, rank, factor_bits, payload)
    _check("cf_lowrank_decompress", lib.cf_lowrank_decompress(
        factor_bits, _ptr(u), _ptr(us), _ptr(v), _ptr(vs), _ptr(ahat), m, n, rank, batch,
        _stream(stream)))
