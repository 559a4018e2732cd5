"""The C ABI library: it loads, exports every symbol the headers declare, and its
validation (which runs before any HIP call) rejects bad arguments.  No compute call
is made here: pointers are fake addresses that are never dereferenced, and a fully
valid call stops at the device check where there is no gfx950.  On a machine with a
GPU driver those valid calls would be launched, so the validation tests are skipped
there (the GPU tests cover the same entry points with real buffers)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "activation_residual_compression_cf_amd", "libcf.so")

CF_OK, CF_E_NULL, CF_E_SHAPE, CF_E_ALIGN, CF_E_ARG, CF_E_ALIAS, CF_E_WORKSPACE, CF_E_DEVICE = (
    0, -1, -2, -3, -4, -5, -6, -7)


def declared_symbols():
    syms = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        syms |= set(re.findall(r"^\s*[a-z_][\w\s\*]*?\b(cf_\w+)\s*\(", text, flags=re.M))
    return sorted(syms)


@pytest.fixture(scope="module")
def lib():
    """The library, for calls that never reach the device check."""
    if not os.path.exists(LIB):
        pytest.fail("libcf.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


@pytest.fixture(scope="module")
def L(lib):
    """The library, for validation calls whose valid cases stop at the device check."""
    if os.path.exists("/dev/kfd"):
        pytest.skip("valid calls with placeholder pointers would launch on a present GPU")
    return lib


def P(x):
    return ctypes.c_void_p(x)


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for want in ("cf_init_state", "cf_compress", "cf_decompress", "cf_strerror"):
        assert want in syms


def test_every_declared_symbol_is_exported(lib):
    for s in declared_symbols():
        assert hasattr(lib, s), f"{s} declared in include/ but not exported by libcf.so"


def test_no_torch_in_the_library():
    # the boundary carries plain pointers and sizes only
    out = os.popen(f"nm -D --defined-only {LIB}").read()
    assert "torch" not in out and "at::" not in out


def test_strerror_and_version(lib):
    lib.cf_strerror.restype = ctypes.c_char_p
    for code in range(0, -10, -1):
        assert lib.cf_strerror(code) and lib.cf_strerror(code) != b"unknown status" and lib.cf_strerror(code) != b"unknown status"
    assert lib.cf_abi_version() == 1


def test_codes_bytes(lib):
    lib.cf_codes_bytes.restype = ctypes.c_int64
    lib.cf_codes_bytes.argtypes = [ctypes.c_int64, ctypes.c_int]
    assert lib.cf_codes_bytes(1024 * 3072, 1) == 393216
    assert lib.cf_codes_bytes(1024 * 3072, 2) == 786432
    assert lib.cf_codes_bytes(2925 * 1920, 2) == 1404000
    assert lib.cf_codes_bytes(100, 1) == CF_E_SHAPE
    assert lib.cf_codes_bytes(128, 3) == CF_E_ARG


def _compress(L, bits=1, dt=0, a=0x10000, ah=0x1000000, e=0x2000000, c=0x3000000, s=0x4000000,
              n=1280):
    L.cf_compress.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 5 + [
        ctypes.c_int64, ctypes.c_void_p]
    return L.cf_compress(bits, dt, P(a) if a else None, P(ah) if ah else None,
                         P(e) if e else None, P(c) if c else None, P(s) if s else None, n, None)


def test_compress_validation(L):
    assert _compress(L, bits=3) == CF_E_ARG
    assert _compress(L, dt=2) == CF_E_ARG
    assert _compress(L, a=0) == CF_E_NULL
    assert _compress(L, s=0) == CF_E_NULL
    assert _compress(L, n=0) == CF_E_SHAPE
    assert _compress(L, n=-128) == CF_E_SHAPE
    assert _compress(L, n=1000) == CF_E_SHAPE
    assert _compress(L, n=(1 << 40) + 128) == CF_E_SHAPE
    # the largest call: 2^33 elements (every grid stays inside a dispatch's 2^32 - 1
    # work-items); fake buffers 2^40 bytes apart so that none overlaps
    T = 1 << 40
    assert _compress(L, a=T, ah=2 * T, e=3 * T, c=4 * T, s=5 * T, n=(1 << 33) + 128) == CF_E_SHAPE
    assert _compress(L, a=T, ah=2 * T, e=3 * T, c=4 * T, s=5 * T, n=1 << 33) == CF_E_DEVICE
    assert _compress(L, a=0x10008) == CF_E_ALIGN
    assert _compress(L, c=0x3000004) == CF_E_ALIGN
    assert _compress(L, s=0x4000002) == CF_E_ALIGN
    assert _compress(L, s=0x4000004) == CF_E_DEVICE  # scales need 4-byte alignment only
    assert _compress(L, e=0x1000000 + 1280 * 4 - 16) == CF_E_ALIAS     # err overlaps ahat's tail
    assert _compress(L, a=0x1000000 - 16) == CF_E_ALIAS               # a runs into ahat
    assert _compress(L, c=0x4000000) == CF_E_ALIAS                    # codes == scales
    assert _compress(L, e=0x1000000 + 1280 * 4) == CF_E_DEVICE        # adjacent is fine
    assert _compress(L) == CF_E_DEVICE  # valid: stops at the device check (no gfx950 here)


def test_init_and_decompress_validation(L):
    L.cf_init_state.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 3 + [ctypes.c_int64,
                                                                          ctypes.c_void_p]
    L.cf_decompress.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 3 + [ctypes.c_int64,
                                                                          ctypes.c_void_p]
    assert L.cf_init_state(5, P(0x10000), P(0x100000), None, 128, None) == CF_E_ARG
    assert L.cf_init_state(0, None, P(0x100000), None, 128, None) == CF_E_NULL
    assert L.cf_init_state(0, P(0x10000), P(0x100000), None, 64, None) == CF_E_SHAPE
    assert L.cf_init_state(0, P(0x10000), P(0x100004), None, 128, None) == CF_E_ALIGN
    assert L.cf_init_state(1, P(0x10000), P(0x10000 + 256), None, 128, None) == CF_E_ALIAS
    assert L.cf_init_state(0, P(0x10000), P(0x100000), None, 128, None) == CF_E_DEVICE
    assert L.cf_decompress(0, P(0x10000), P(0x20000), P(0x30000), 128, None) == CF_E_ARG
    assert L.cf_decompress(1, None, P(0x20000), P(0x30000), 128, None) == CF_E_NULL
    assert L.cf_decompress(1, P(0x10000), P(0x20000), P(0x30000), 129, None) == CF_E_SHAPE
    assert L.cf_decompress(2, P(0x10000), P(0x20000), P(0x20000), 128, None) == CF_E_ALIAS
    assert L.cf_decompress(2, P(0x10000), P(0x20000), P(0x30000), 128, None) == CF_E_DEVICE


def test_lowrank_validation(L):
    L.cf_lowrank_workspace_bytes.restype = ctypes.c_size_t
    L.cf_lowrank_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    assert L.cf_lowrank_workspace_bytes(1024, 3072, 32, 114) > 114 * 1024 * 3072 * 4
    assert L.cf_lowrank_workspace_bytes(1000, 3072, 32, 1) == 0   # m not a multiple of 16
    assert L.cf_lowrank_workspace_bytes(1024, 3072, 65, 1) == 0   # rank above 64
    assert L.cf_lowrank_workspace_bytes(32, 64, 48, 1) == 0       # rank above min(m, n)
    assert L.cf_lowrank_workspace_bytes(1024, 3072, 32, 2731) == 0  # batch*m*n above 2^33
    # 2^23 tensors of 16 x 16: the factor quantization would need 2^32 work-items in
    # one dispatch (two 256-thread workgroups per tensor)
    assert L.cf_lowrank_workspace_bytes(16, 16, 16, 1 << 23) == 0
    assert L.cf_lowrank_workspace_bytes(16, 16, 16, 1 << 22) > 0
    assert L.cf_lowrank_workspace_bytes(16, 1 << 28, 16, 1) > 0
    L.cf_lowrank_compress.argtypes = ([ctypes.c_int] + [ctypes.c_void_p] * 3 +
                                      [ctypes.c_int64] * 2 + [ctypes.c_int] * 4 +
                                      [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p])
    ws = L.cf_lowrank_workspace_bytes(64, 128, 8, 1)

    def call(dt=0, a=0x100000, ah=0x200000, e=0x300000, m=64, n=128, k=8, it=2, fb=4, b=1,
             q=0x400000, u=0x500000, us=0x600000, v=0x700000, vs=0x800000, w=0x1000000, wsb=ws):
        P_ = lambda x: P(x) if x else None
        return L.cf_lowrank_compress(dt, P_(a), P_(ah), P_(e), m, n, k, it, fb, b, P_(q), P_(u),
                                     P_(us), P_(v), P_(vs), P_(w), wsb, None)

    assert call(fb=8) == CF_E_ARG
    assert call(it=0) == CF_E_ARG
    assert call(it=65) == CF_E_ARG
    assert call(w=0) == CF_E_NULL
    assert call(us=0) == CF_E_NULL
    assert call(fb=32, us=0, vs=0) == CF_E_DEVICE     # scales optional with fp32 factors
    assert call(k=7) == CF_E_SHAPE                   # odd rank with INT4
    assert call(k=0) == CF_E_SHAPE
    assert call(m=60) == CF_E_SHAPE
    assert call(b=0) == CF_E_SHAPE
    assert call(a=0x100008) == CF_E_ALIGN
    assert call(w=0x1000010) == CF_E_ALIGN           # workspace is 256-byte aligned
    assert call(wsb=ws - 1) == CF_E_WORKSPACE
    # a too-small workspace is reported as such, even where the size the call needs
    # would run into another operand (the size check comes before the overlap check)
    assert call(w=0x200000 - 1024, wsb=1024) == CF_E_WORKSPACE
    assert call(e=0x200000 + 64 * 128 * 4 - 16) == CF_E_ALIAS
    assert call(w=0x200000) == CF_E_ALIAS
    assert call() == CF_E_DEVICE
    L.cf_lowrank_decompress.argtypes = ([ctypes.c_int] + [ctypes.c_void_p] * 5 +
                                        [ctypes.c_int64] * 2 + [ctypes.c_int] * 2 + [ctypes.c_void_p])
    assert L.cf_lowrank_decompress(5, P(0x500000), P(0x600000), P(0x700000), P(0x800000),
                                   P(0x200000), 64, 128, 8, 1, None) == CF_E_ARG
    assert L.cf_lowrank_decompress(4, P(0x500000), None, P(0x700000), P(0x800000),
                                   P(0x200000), 64, 128, 8, 1, None) == CF_E_NULL
    assert L.cf_lowrank_decompress(4, P(0x500000), P(0x600000), P(0x700000), P(0x800000),
                                   P(0x200000), 64, 100, 8, 1, None) == CF_E_SHAPE
    assert L.cf_lowrank_decompress(4, P(0x500000), P(0x600000), P(0x700000), P(0x800000),
                                   P(0x500000), 64, 128, 8, 1, None) == CF_E_ALIAS
    assert L.cf_lowrank_decompress(4, P(0x500000), P(0x600000), P(0x700000), P(0x800000),
                                   P(0x200000), 64, 128, 8, 1, None) == CF_E_DEVICE


def test_lowrank_noalloc_validation(L):
    """The no-allocation variant validates like cf_lowrank_compress and refuses, before
    anything is enqueued, a call whose workspace would not fit its fixed scratch."""
    CF_E_SCRATCH = -9
    L.cf_lowrank_compress_noalloc.argtypes = ([ctypes.c_int] + [ctypes.c_void_p] * 3 +
                                              [ctypes.c_int64] * 2 + [ctypes.c_int] * 4 +
                                              [ctypes.c_void_p] * 6)
    G = 1 << 40  # placeholder buffers far apart, so no two of them overlap

    def call(dt=0, m=64, n=128, k=8, it=2, fb=4, b=1, a=1 * G, us=6 * G):
        return L.cf_lowrank_compress_noalloc(dt, P(a), P(2 * G), P(3 * G), m, n, k, it, fb, b, P(4 * G),
                                             P(5 * G), P(us) if us else None, P(7 * G), P(8 * G), None)

    assert call(fb=8) == CF_E_ARG
    assert call(us=0) == CF_E_NULL
    assert call(k=7) == CF_E_SHAPE
    assert call(a=G + 8) == CF_E_ALIGN
    assert call(m=1024, n=3072, k=32, b=5) == CF_E_SCRATCH   # 70.4 MiB of workspace
    assert call(m=1024, n=3072, k=32, b=4) == CF_E_DEVICE    # 56.3 MiB: fits
    assert call() == CF_E_DEVICE


def test_ablation_and_bf16_decode_validation(L):
    L.cf_compress_ablation.argtypes = ([ctypes.c_int] * 3 + [ctypes.c_void_p] * 5 +
                                       [ctypes.c_int64, ctypes.c_void_p])
    call = lambda mode, ap=0x200000, n=1280, bits=1: L.cf_compress_ablation(
        mode, bits, 0, P(0x100000), P(ap) if ap else None, P(0x300000), P(0x400000),
        P(0x500000), n, None)
    assert call(0) == CF_E_ARG                 # mode 0 is cf_compress itself
    assert call(3) == CF_E_ARG
    assert call(1, bits=4) == CF_E_ARG
    assert call(1, ap=0) == CF_E_NULL          # no-EF needs the previous activation
    assert call(2, ap=0) == CF_E_DEVICE        # naive does not
    assert call(1, n=100) == CF_E_SHAPE
    assert call(1, ap=0x200008) == CF_E_ALIGN
    assert call(1, ap=0x300000) == CF_E_ALIAS   # a_prev (input) overlapping ahat (output)
    L.cf_decompress_bf16.argtypes = ([ctypes.c_int] + [ctypes.c_void_p] * 4 + [ctypes.c_int64,
                                                                               ctypes.c_void_p])
    assert L.cf_decompress_bf16(1, P(0x10000), P(0x20000), P(0x30000), None, 128, None) == CF_E_NULL
    assert L.cf_decompress_bf16(1, P(0x10000), P(0x20000), P(0x30000), P(0x40008), 128, None) == CF_E_ALIGN
    assert L.cf_decompress_bf16(1, P(0x10000), P(0x20000), P(0x30000), P(0x30000), 128, None) == CF_E_ALIAS
    assert L.cf_decompress_bf16(1, P(0x10000), P(0x20000), P(0x30000), P(0x40000), 128, None) == CF_E_DEVICE


def test_topk_validation(L):
    L.cf_topk_compress.argtypes = ([ctypes.c_int] * 2 + [ctypes.c_void_p] * 5 +
                                   [ctypes.c_int64, ctypes.c_void_p])
    L.cf_topk_decompress.argtypes = ([ctypes.c_int] + [ctypes.c_void_p] * 3 +
                                     [ctypes.c_int64, ctypes.c_void_p])

    def call(k=12, dt=0, a=0x100000, ah=0x200000, e=0x300000, i=0x400000, v=0x500000, n=1280):
        return L.cf_topk_compress(k, dt, P(a) if a else None, P(ah) if ah else None,
                                  P(e) if e else None, P(i) if i else None, P(v) if v else None,
                                  n, None)

    assert call(k=0) == CF_E_ARG
    assert call(k=129) == CF_E_ARG
    assert call(dt=2) == CF_E_ARG
    assert call(i=0) == CF_E_NULL
    assert call(v=0) == CF_E_NULL
    assert call(n=1000) == CF_E_SHAPE
    assert call(e=0x300008) == CF_E_ALIGN
    assert call(v=0x500001) == CF_E_ALIGN
    assert call(i=0x400001, v=0x500002) == CF_E_DEVICE     # idx bytes need no alignment
    assert call(i=0x500000 - 10 * 12 + 1) == CF_E_ALIAS       # idx runs into vals
    assert call(i=0x500000 - 10 * 12) == CF_E_DEVICE          # adjacent is fine
    assert call(v=0x300000 + 1280 * 4 - 2) == CF_E_ALIAS      # vals overlaps err's tail
    assert call(k=128) == CF_E_DEVICE
    assert call() == CF_E_DEVICE
    dec = lambda k=12, i=0x400000, v=0x500000, ah=0x200000, n=1280: L.cf_topk_decompress(
        k, P(i) if i else None, P(v) if v else None, P(ah) if ah else None, n, None)
    assert dec(k=0) == CF_E_ARG
    assert dec(v=0) == CF_E_NULL
    assert dec(n=0) == CF_E_SHAPE
    assert dec(ah=0x200004) == CF_E_ALIGN
    assert dec(v=0x500001) == CF_E_ALIGN
    assert dec(i=0x200000 + 1280 * 4 - 1) == CF_E_ALIAS       # idx overlapping the output mirror
    assert dec() == CF_E_DEVICE


def test_binding_refuses_host_tensors():
    """The binding passes device pointers only: a host tensor is refused before any call
    (its address would fault a kernel)."""
    import torch

    from activation_residual_compression_cf_amd import cf

    a = torch.zeros(256, dtype=torch.bfloat16)
    ah = torch.zeros(256)
    er = torch.zeros(256)
    with pytest.raises(ValueError, match="device tensors"):
        cf.compress(1, a, ah, er, torch.zeros(32, dtype=torch.uint8), torch.zeros(2))
    with pytest.raises(ValueError, match="device tensors"):
        cf.topk_compress(4, a, ah, er, torch.zeros(8, dtype=torch.uint8), torch.zeros(8, dtype=torch.int16))


def test_binding_refuses_short_state_buffers():
    """Buffer sizes are invisible to the C ABI, so the binding compares them with what the
    call writes before any call (here before it even looks at the device)."""
    import torch

    from activation_residual_compression_cf_amd import cf

    a = torch.zeros(256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="ahat holds"):
        cf.init_state(a, torch.zeros(128), torch.zeros(256))
    with pytest.raises(ValueError, match="err holds"):
        cf.init_state(a, torch.zeros(256), torch.zeros(255))
    with pytest.raises(ValueError, match="codes holds"):
        cf.compress(2, a, torch.zeros(256), torch.zeros(256), torch.zeros(32, dtype=torch.uint8), torch.zeros(2))


def test_binding_refuses_wrong_element_types():
    """State and scales must be fp32, codes and index bytes uint8: the C ABI takes untyped
    pointers, so the binding refuses other element types before any call."""
    import torch

    from activation_residual_compression_cf_amd import cf

    a = torch.zeros(256, dtype=torch.bfloat16)
    f32, f64 = torch.zeros(256), torch.zeros(256, dtype=torch.float64)
    u8 = torch.zeros(32, dtype=torch.uint8)
    with pytest.raises(TypeError, match="ahat"):
        cf.compress(1, a, f64, f32, u8, torch.zeros(2))
    with pytest.raises(TypeError, match="codes"):
        cf.compress(1, a, f32, f32, torch.zeros(32, dtype=torch.int8), torch.zeros(2))
    with pytest.raises(TypeError, match="scales"):
        cf.decompress(1, u8, torch.zeros(2, dtype=torch.float16), f32)
    with pytest.raises(TypeError, match="vals"):
        cf.topk_compress(4, a, f32, f32, torch.zeros(8, dtype=torch.uint8), torch.zeros(8, dtype=torch.float32))
    with pytest.raises(TypeError, match="q_state"):
        cf.lowrank_compress(torch.zeros((1, 16, 16), dtype=torch.bfloat16), torch.zeros((1, 16, 16)), None,
                            torch.zeros((1, 16, 2), dtype=torch.float64), 2, 1, 4,
                            payload=(torch.zeros(16, dtype=torch.uint8), torch.zeros(2),
                                     torch.zeros(16, dtype=torch.uint8), torch.zeros(2)),
                            workspace=torch.zeros(1, dtype=torch.uint8))


def test_error_buffer_is_optional_for_senders(L):
    """err = NULL is accepted by every sender (the error feedback lives in ahat); the
    valid calls stop at the device check."""
    L.cf_compress.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_void_p]
    assert L.cf_compress(1, 0, P(0x100000), P(0x200000), None, P(0x300000), P(0x400000), 1280, None) == CF_E_DEVICE
    L.cf_topk_compress.argtypes = ([ctypes.c_int] * 2 + [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_void_p])
    assert L.cf_topk_compress(12, 0, P(0x100000), P(0x200000), None, P(0x400000), P(0x500000), 1280,
                              None) == CF_E_DEVICE
    L.cf_lowrank_workspace_bytes.restype = ctypes.c_size_t
    L.cf_lowrank_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    need = L.cf_lowrank_workspace_bytes(64, 128, 8, 1)
    L.cf_lowrank_compress.argtypes = ([ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int64] + [ctypes.c_int] * 4 +
                                      [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p])
    assert L.cf_lowrank_compress(0, P(0x1000000), P(0x2000000), None, 64, 128, 8, 2, 4, 1, P(0x3000000),
                                 P(0x4000000), P(0x5000000), P(0x6000000), P(0x7000000), P(0x8000000),
                                 need, None) == CF_E_DEVICE
