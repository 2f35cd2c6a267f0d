"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/tern.h declares, and rejects bad arguments on the host with
the documented status before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tern():
    import ternary_weight_g128_amd as t
    return t


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "tern.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tern_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ["tern_pack", "tern_fwht", "tern_gemv", "tern_gemm"]:
        assert required in names


def test_library_exports_every_declared_function(tern):
    lib = ctypes.CDLL(tern.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(tern.EXPORTED) == _declared_functions()


def test_abi_version_and_status_strings(tern):
    assert tern.tern_abi_version() == 1
    assert tern.tern_status_str(0) == "TERN_OK"
    assert tern.tern_status_str(5) == "TERN_EDEVICE"
    assert tern.tern_status_str(99) == "unknown"


def test_accounting_functions(tern):
    assert tern.tern_codes_bytes(17408, 5120) == 17408 * 5120 // 4
    assert tern.tern_scales_bytes(17408, 5120) == 2 * 17408 * 5120 // 128
    for N, K in [(1, 128), (1024, 1024), (12288, 4096)]:
        b = tern.tern_codes_bytes(N, K) + tern.tern_scales_bytes(N, K)
        assert 8 * b / (N * K) == 2.125
    assert tern.tern_codes_bytes(4, 100) == 0 and tern.tern_scales_bytes(-1, 128) == 0


# Fake, never-dereferenced device addresses: validation must fail before any
# HIP call, so these calls are safe without a GPU.
A16 = ctypes.c_void_p(0x10000)
A2 = ctypes.c_void_p(0x10002)
NULL = None


def _gemv(tern, x=A16, xdt=1, M=1, K=128, codes=A16, scales=A16, N=16, y=A16, ydt=0):
    return tern.lib().tern_gemv(x, xdt, M, K, codes, scales, N, y, ydt, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(M=17), 1), (dict(M=-1), 1), (dict(N=-3), 1), (dict(K=100), 1), (dict(K=-128), 1),
    (dict(xdt=2), 4), (dict(ydt=7), 4), (dict(x=NULL), 1), (dict(codes=NULL), 1),
    (dict(scales=NULL), 1), (dict(y=NULL), 1), (dict(x=A2), 1), (dict(codes=A2), 1),
])
def test_gemv_rejects(tern, kw, status):
    assert _gemv(tern, **kw) == status
    assert tern.tern_last_error().startswith("tern_gemv")


def test_gemv_empty_is_noop(tern):
    # M == 0 or N == 0 writes nothing and launches nothing
    assert _gemv(tern, M=0, x=NULL, codes=NULL, scales=NULL, y=NULL) == 0
    assert _gemv(tern, N=0, x=NULL, codes=NULL, scales=NULL, y=NULL) == 0


def _gemv_t5(tern, x=A16, xdt=1, M=1, K=640, data=A16, scales=A16, N=16, y=A16, ydt=0):
    return tern.lib().tern_gemv_t5(x, xdt, M, K, data, scales, N, y, ydt, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(M=17), 1), (dict(M=-1), 1), (dict(N=-3), 1), (dict(K=100), 1), (dict(xdt=0), 4),
    (dict(ydt=2), 4), (dict(x=NULL), 1), (dict(data=NULL), 1), (dict(scales=NULL), 1),
    (dict(y=NULL), 1), (dict(x=A2), 1), (dict(data=A2), 1), (dict(K=1 << 25), 1),
])
def test_gemv_t5_rejects(tern, kw, status):
    assert _gemv_t5(tern, **kw) == status
    assert tern.tern_last_error().startswith("tern_gemv_t5")


def test_gemv_t5_empty_is_noop(tern):
    assert _gemv_t5(tern, M=0, x=NULL, data=NULL, scales=NULL, y=NULL) == 0
    assert _gemv_t5(tern, N=0, x=NULL, data=NULL, scales=NULL, y=NULL) == 0


def _gemv_b1(tern, x=A16, xdt=1, M=1, K=1024, bits=A16, scales=A16, N=16, y=A16, ydt=0):
    return tern.lib().tern_gemv_b1(x, xdt, M, K, bits, scales, N, y, ydt, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(M=5), 4), (dict(M=-1), 1), (dict(N=-3), 1), (dict(K=100), 1), (dict(K=640), 4),
    (dict(xdt=0), 4), (dict(ydt=2), 4), (dict(x=NULL), 1), (dict(bits=NULL), 1),
    (dict(scales=NULL), 1), (dict(y=NULL), 1), (dict(x=A2), 1), (dict(bits=A2), 1),
    (dict(K=1 << 31), 1), (dict(K=0), 4),
])
def test_gemv_b1_rejects(tern, kw, status):
    assert _gemv_b1(tern, **kw) == status
    assert tern.tern_last_error().startswith("tern_gemv_b1")


def test_gemv_b1_empty_is_noop(tern):
    assert _gemv_b1(tern, M=0, x=NULL, bits=NULL, scales=NULL, y=NULL) == 0
    assert _gemv_b1(tern, N=0, x=NULL, bits=NULL, scales=NULL, y=NULL) == 0


def _gemm(tern, x=A16, xdt=1, M=64, K=128, codes=A16, scales=A16, N=16, y=A16, ws=NULL, wsb=0):
    return tern.lib().tern_gemm(x, xdt, M, K, codes, scales, N, y, ws, wsb, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(xdt=0), 4), (dict(xdt=3), 4), (dict(K=64), 1), (dict(M=-2), 1),
    (dict(x=NULL), 1), (dict(y=A2), 1), (dict(codes=A2), 1), (dict(K=1 << 22), 1),
])
def test_gemm_rejects(tern, kw, status):
    assert _gemm(tern, **kw) == status


def test_gemm_empty_is_noop(tern):
    assert _gemm(tern, M=0, x=NULL, codes=NULL, scales=NULL, y=NULL) == 0


def _gemm_noalloc(tern, x=A16, xdt=1, M=64, K=128, codes=A16, scales=A16, N=16, y=A16):
    return tern.lib().tern_gemm_noalloc(x, xdt, M, K, codes, scales, N, y, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(xdt=0), 4), (dict(xdt=3), 4), (dict(K=64), 1), (dict(M=-2), 1), (dict(K=1 << 31), 1),
    (dict(x=NULL), 1), (dict(y=A2), 1), (dict(codes=A2), 1),
])
def test_gemm_noalloc_rejects(tern, kw, status):
    # the same host checks as tern_gemm, before any device call
    assert _gemm_noalloc(tern, **kw) == status


def test_gemm_noalloc_empty_is_noop(tern):
    assert _gemm_noalloc(tern, M=0, x=NULL, codes=NULL, scales=NULL, y=NULL) == 0
    assert _gemm_noalloc(tern, N=0, x=NULL, codes=NULL, scales=NULL, y=NULL) == 0


def test_gemm_scratch_constant_matches_header(tern):
    src = open(os.path.join(ROOT, "include", "tern.h")).read()
    m = re.search(r"#define TERN_GEMM_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == tern.TERN_GEMM_SCRATCH_BYTES


def _fwht(tern, x=A16, xdt=0, signs=NULL, M=1, K=4096, block=4096, inverse=0, y=A16):
    return tern.lib().tern_fwht(x, xdt, signs, M, K, block, inverse, y, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(block=3), 1), (dict(block=0), 1), (dict(block=8192, K=8192), 1), (dict(K=6144), 1),
    (dict(xdt=5), 4), (dict(x=NULL), 1), (dict(y=NULL), 1), (dict(y=A2), 1), (dict(M=-1), 1),
    (dict(xdt=1), 1),  # bf16 in place (y == x) is rejected
])
def test_fwht_rejects(tern, kw, status):
    assert _fwht(tern, **kw) == status


def test_fwht_empty_is_noop(tern):
    assert _fwht(tern, M=0, x=NULL, y=NULL) == 0


def _rot(tern, x=A16, xdt=1, signs=NULL, block=4096, M=1, K=4096, codes=A16, scales=A16, N=16,
         y=A16, ydt=0):
    return tern.lib().tern_rotate_gemv(x, xdt, signs, block, M, K, codes, scales, N, y, ydt, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(block=8), 1), (dict(block=8192, K=8192), 1), (dict(block=1000), 1), (dict(K=6144), 1),
    (dict(M=17), 1), (dict(xdt=4), 4), (dict(ydt=3), 4), (dict(signs=A2), 1), (dict(x=NULL), 1),
    (dict(M=16, K=65536, block=4096), 4),   # staged activations exceed LDS
])
def test_rotate_gemv_rejects(tern, kw, status):
    assert _rot(tern, **kw) == status


def _packd(tern, t=A16, N=4, K=128, codes=A16):
    return tern.lib().tern_pack_device(t, N, K, codes, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(K=100), 1), (dict(N=-1), 1), (dict(t=NULL), 1), (dict(codes=NULL), 1),
    (dict(t=A2), 1), (dict(codes=A2), 1),
])
def test_pack_device_rejects(tern, kw, status):
    assert _packd(tern, **kw) == status
    assert tern.tern_last_error().startswith("tern_pack_device")


def test_pack_device_empty_is_noop(tern):
    assert _packd(tern, N=0, t=NULL, codes=NULL) == 0
    assert _packd(tern, K=0, t=NULL, codes=NULL) == 0


def test_codec_rejects(tern):
    t = np.zeros((2, 128), dtype=np.int8)
    t[1, 5] = 2
    s = np.zeros((2, 1), dtype=np.uint16)
    with pytest.raises(tern.TernError) as e:
        tern.tern_pack(t, s)
    assert e.value.status == tern.TERN_ENOTTERNARY
    t[1, 5] = 1
    s[0, 0] = 0x7C00  # +inf scale
    with pytest.raises(tern.TernError) as e:
        tern.tern_pack(t, s)
    assert e.value.status == tern.TERN_EINVAL
    codes = np.full((1, 8), 0x55555555, dtype=np.uint32)
    codes[0, 7] = 0xD5555555  # slot 15 of word 7 holds 3
    with pytest.raises(tern.TernError) as e:
        tern.tern_unpack(codes, 128)
    assert e.value.status == tern.TERN_EBADCODE
    with pytest.raises(tern.TernError) as e:
        tern.tern_dequant_f32(codes, np.zeros((1, 1), np.uint16), 128)
    assert e.value.status == tern.TERN_EBADCODE
    lib = tern.lib()
    assert lib.tern_pack(None, None, 1, 100, None, None) == tern.TERN_EINVAL
    assert lib.tern_pack(None, None, 0, 128, None, None) == tern.TERN_OK


# K above TERN_MAX_K (INT32_MAX - 127) is rejected before any launch: the
# kernels index K in 32-bit integers.  N = 1 keeps N * K / 16 below the
# separate size cap, so only the K bound can fire.
BIG_K = 1 << 31


def test_k_bound_constant(tern):
    assert tern.TERN_MAX_K == 2 ** 31 - 1 - 127
    assert tern.TERN_MAX_K % 128 == 0


@pytest.mark.parametrize("call", ["gemv", "rotate_gemv", "gemm"])
def test_matmul_rejects_k_above_int32(tern, call):
    if call == "gemv":
        st = _gemv(tern, K=BIG_K, N=1)
        ok = _gemv(tern, K=tern.TERN_MAX_K + 128, N=1)
    elif call == "rotate_gemv":
        st = _rot(tern, K=BIG_K, N=1)
        ok = _rot(tern, K=tern.TERN_MAX_K + 128, N=1)
    else:
        st = _gemm(tern, K=BIG_K, N=1)
        ok = _gemm(tern, K=tern.TERN_MAX_K + 128, N=1)
    assert st == tern.TERN_EINVAL and ok == tern.TERN_EINVAL
    assert "K" in tern.tern_last_error()


def test_f16_dtype_is_named_and_unsupported(tern):
    assert tern.TERN_F16 == 2
    assert _gemv(tern, xdt=tern.TERN_F16) == tern.TERN_EUNSUPPORTED
    assert _gemv(tern, ydt=tern.TERN_F16) == tern.TERN_EUNSUPPORTED
    assert _fwht(tern, xdt=tern.TERN_F16) == tern.TERN_EUNSUPPORTED
    assert _rot(tern, xdt=tern.TERN_F16) == tern.TERN_EUNSUPPORTED
    assert _gemm(tern, xdt=tern.TERN_F16) == tern.TERN_EUNSUPPORTED


# The Python wrappers check shapes, element sizes and devices before the C
# call (argument marshalling; a mismatch would otherwise reach the kernels as
# out-of-bounds addresses).  CPU tensors suffice: the check fires first.

def _torch():
    import torch
    return torch


def _w(N, K):
    T = _torch()
    return T.zeros((N, K // 16), dtype=T.int32), T.zeros((N, K // 128), dtype=T.int16)


@pytest.mark.parametrize("bad", ["codes_rows", "codes_cols", "scales", "out", "codes_dtype", "x_3d", "k"])
def test_gemv_wrapper_checks_shapes(tern, bad):
    T = _torch()
    M, K, N = 2, 256, 32
    x = T.zeros((M, K), dtype=T.bfloat16)
    codes, scales = _w(N, K)
    out = T.zeros((M, N), dtype=T.float32)
    if bad == "codes_rows":
        scales = T.zeros((N + 1, K // 128), dtype=T.int16)
        codes = T.zeros((N + 1, K // 16 + 1), dtype=T.int32)
    elif bad == "codes_cols":
        codes = T.zeros((N, K // 16 - 1), dtype=T.int32)
    elif bad == "scales":
        scales = T.zeros((N, K // 128 + 1), dtype=T.int16)
    elif bad == "out":
        out = T.zeros((M, N + 1), dtype=T.float32)
    elif bad == "codes_dtype":
        codes = T.zeros((N, K // 16), dtype=T.int16)
    elif bad == "x_3d":
        x = T.zeros((1, M, K), dtype=T.bfloat16)
    elif bad == "k":
        x = T.zeros((M, 200), dtype=T.bfloat16)
    with pytest.raises(ValueError):
        tern.tern_gemv(x, codes, scales, out=out)


def test_other_wrappers_check_shapes(tern):
    T = _torch()
    M, K, N = 2, 4096, 16
    x = T.zeros((M, K), dtype=T.bfloat16)
    codes, scales = _w(N, K)
    with pytest.raises(ValueError, match="signs"):
        tern.tern_rotate_gemv(x, T.ones(K - 1, dtype=T.int8), 4096, codes, scales)
    with pytest.raises(ValueError, match="scales"):
        tern.tern_rotate_gemv(x, None, 4096, codes, scales[:, :-1])
    with pytest.raises(ValueError, match="signs"):
        tern.tern_fwht(x, T.ones(K, dtype=T.int16), 4096)
    with pytest.raises(ValueError, match="out"):
        tern.tern_fwht(x, None, 4096, out=T.zeros((M, K), dtype=T.bfloat16))
    with pytest.raises(ValueError, match="out"):
        tern.tern_gemm(x, codes, scales, out=T.zeros((M, N), dtype=T.bfloat16))
    with pytest.raises(ValueError, match="codes"):
        tern.tern_gemm(x, codes[:, 1:], scales)
    with pytest.raises(ValueError, match="data"):
        tern.tern_gemv_t5(x, T.zeros((N, 100), dtype=T.uint8), scales)
    with pytest.raises(ValueError, match="out"):
        tern.tern_pack_device(T.zeros((N, K), dtype=T.int8), out=T.zeros((N, K // 8), dtype=T.int32))
