"""Python binding of libtern (ternary-g128 matmul and signed Walsh-Hadamard
rotation for AMD MI355X).

Argument marshalling only: every computation runs in libtern.so (host codec
in C++, device operations in HIP kernels).  Host-codec functions take numpy
arrays; device functions take torch tensors on the current HIP device and
enqueue on torch's current stream.  The names are the C ABI names of
include/tern.h.  A missing or unloadable libtern.so raises at import.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtern.so")

TERN_OK, TERN_EINVAL, TERN_ENOTTERNARY, TERN_EBADCODE, TERN_EUNSUPPORTED, TERN_EDEVICE = range(6)
TERN_F32, TERN_BF16, TERN_F16 = 0, 1, 2
TERN_MAX_K = 2147483520
TERN_GROUP = 128
TERN_GEMV_MAX_M = 16
TERN_FWHT_MAX_BLOCK = 4096
TERN_GEMM_SCRATCH_BYTES = 32 << 20

EXPORTED = [
    "tern_abi_version", "tern_status_str", "tern_last_error", "tern_codes_bytes",
    "tern_scales_bytes", "tern_pack", "tern_pack_f32", "tern_unpack", "tern_dequant_f32",
    "tern_pack_device", "tern_fwht", "tern_gemv", "tern_rotate_gemv", "tern_gemm_workspace_bytes",
    "tern_gemm", "tern_scales_g64_bytes", "tern_scales_to_g64", "tern_scales_from_g64",
    "tern_mlx_export", "tern_mlx_import", "tern_b1_bytes", "tern_pack_b1", "tern_unpack_b1",
    "tern_b1_to_codes", "tern_codes_to_b1", "tern_mlx_export_b1", "tern_mlx_import_b1",
    "tern_t5_bytes", "tern_pack_t5", "tern_unpack_t5", "tern_gemv_t5", "tern_gemm_noalloc",
    "tern_gemv_b1",
]
_SIZE_FNS = ("tern_codes_bytes", "tern_scales_bytes", "tern_gemm_workspace_bytes",
             "tern_scales_g64_bytes", "tern_b1_bytes", "tern_t5_bytes")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libtern.so is not built ({LIB_PATH}); run __graft_entry__.build()")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_lib.tern_abi_version.restype = _I
_lib.tern_status_str.argtypes = [_I]
_lib.tern_status_str.restype = ctypes.c_char_p
_lib.tern_last_error.restype = ctypes.c_char_p
_lib.tern_codes_bytes.argtypes = [_I64, _I64]
_lib.tern_codes_bytes.restype = _SZ
_lib.tern_scales_bytes.argtypes = [_I64, _I64]
_lib.tern_scales_bytes.restype = _SZ
_lib.tern_pack.argtypes = [_P, _P, _I64, _I64, _P, _P]
_lib.tern_pack_f32.argtypes = [_P, _I64, _I64, _P, _P]
_lib.tern_unpack.argtypes = [_P, _I64, _I64, _P]
_lib.tern_dequant_f32.argtypes = [_P, _P, _I64, _I64, _P]
_lib.tern_pack_device.argtypes = [_P, _I64, _I64, _P, _P]
_lib.tern_fwht.argtypes = [_P, _I, _P, _I64, _I64, _I64, _I, _P, _P]
_lib.tern_gemv.argtypes = [_P, _I, _I64, _I64, _P, _P, _I64, _P, _I, _P]
_lib.tern_rotate_gemv.argtypes = [_P, _I, _P, _I64, _I64, _I64, _P, _P, _I64, _P, _I, _P]
_lib.tern_gemm_workspace_bytes.argtypes = [_I64, _I64, _I64]
_lib.tern_gemm_workspace_bytes.restype = _SZ
_lib.tern_gemm.argtypes = [_P, _I, _I64, _I64, _P, _P, _I64, _P, _P, _SZ, _P]
_lib.tern_gemm_noalloc.argtypes = [_P, _I, _I64, _I64, _P, _P, _I64, _P, _P]
_lib.tern_gemv_t5.argtypes = [_P, _I, _I64, _I64, _P, _P, _I64, _P, _I, _P]
_lib.tern_gemv_b1.argtypes = [_P, _I, _I64, _I64, _P, _P, _I64, _P, _I, _P]
for _name in ("tern_scales_g64_bytes", "tern_b1_bytes", "tern_t5_bytes"):
    getattr(_lib, _name).argtypes = [_I64, _I64]
    getattr(_lib, _name).restype = _SZ
for _name in ("tern_scales_to_g64", "tern_scales_from_g64", "tern_pack_b1", "tern_unpack_b1",
              "tern_b1_to_codes", "tern_codes_to_b1", "tern_pack_t5", "tern_unpack_t5"):
    getattr(_lib, _name).argtypes = [_P, _I64, _I64, _P]
for _name in ("tern_mlx_export", "tern_mlx_export_b1"):
    getattr(_lib, _name).argtypes = [_P, _I64, _I64, _P, _P]
for _name in ("tern_mlx_import", "tern_mlx_import_b1"):
    getattr(_lib, _name).argtypes = [_P, _P, _I64, _I64, _P]
for _name in EXPORTED:
    if _name not in ("tern_abi_version", "tern_status_str", "tern_last_error") + _SIZE_FNS:
        getattr(_lib, _name).restype = _I


class TernError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.tern_last_error().decode()
        super().__init__(f"{where}: {_lib.tern_status_str(status).decode()}: {msg}")


def _check(status: int, where: str):
    if status != TERN_OK:
        raise TernError(status, where)


def lib():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib


def tern_abi_version() -> int:
    return _lib.tern_abi_version()


def tern_status_str(status: int) -> str:
    return _lib.tern_status_str(status).decode()


def tern_last_error() -> str:
    return _lib.tern_last_error().decode()


def tern_codes_bytes(N: int, K: int) -> int:
    return _lib.tern_codes_bytes(N, K)


def tern_scales_bytes(N: int, K: int) -> int:
    return _lib.tern_scales_bytes(N, K)


# --------------------------------------------------------------------------
# host codec (numpy in, numpy out)
# --------------------------------------------------------------------------

def _np_ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def tern_pack(t: np.ndarray, s_f16: np.ndarray):
    """t int8 [N, K], binary16 scale bits uint16 [N, K/128] ->
    (codes uint32 [N, K/16], scales uint16 [N, K/128])."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    N, K = t.shape
    s = np.ascontiguousarray(s_f16, dtype=np.uint16)
    if K % TERN_GROUP or s.shape != (N, K // TERN_GROUP):
        raise ValueError("tern_pack: need K % 128 == 0 and scales of shape [N, K/128]")
    codes = np.empty((N, K // 16), dtype=np.uint32)
    s_out = np.empty_like(s)
    _check(_lib.tern_pack(_np_ptr(t), _np_ptr(s), N, K, _np_ptr(codes), _np_ptr(s_out)), "tern_pack")
    return codes, s_out


def tern_pack_f32(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if K % TERN_GROUP:
        raise ValueError("tern_pack_f32: K % 128 != 0")
    codes = np.empty((N, K // 16), dtype=np.uint32)
    s = np.empty((N, K // TERN_GROUP), dtype=np.uint16)
    _check(_lib.tern_pack_f32(_np_ptr(w), N, K, _np_ptr(codes), _np_ptr(s)), "tern_pack_f32")
    return codes, s


def tern_unpack(codes: np.ndarray, K: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    N = codes.shape[0]
    t = np.empty((N, K), dtype=np.int8)
    _check(_lib.tern_unpack(_np_ptr(codes), N, K, _np_ptr(t)), "tern_unpack")
    return t


def tern_dequant_f32(codes: np.ndarray, s_f16: np.ndarray, K: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    s = np.ascontiguousarray(s_f16, dtype=np.uint16)
    N = codes.shape[0]
    w = np.empty((N, K), dtype=np.float32)
    _check(_lib.tern_dequant_f32(_np_ptr(codes), _np_ptr(s), N, K, _np_ptr(w)), "tern_dequant_f32")
    return w


# --------------------------------------------------------------------------
# format variants (host)
# --------------------------------------------------------------------------

def tern_scales_g64_bytes(N: int, K: int) -> int:
    return _lib.tern_scales_g64_bytes(N, K)


def tern_b1_bytes(N: int, K: int) -> int:
    return _lib.tern_b1_bytes(N, K)


def _scales_arg(s: np.ndarray, per_group: int, name: str):
    s = np.ascontiguousarray(s, dtype=np.uint16)
    if s.ndim != 2:
        raise ValueError(f"{name}: scales must be 2-D")
    return s, s.shape[0], s.shape[1] * TERN_GROUP // per_group


def tern_scales_to_g64(s: np.ndarray) -> np.ndarray:
    """binary16 scale bits [N, K/128] -> [N, K/64], each scale repeated."""
    s, N, K = _scales_arg(s, 1, "tern_scales_to_g64")
    out = np.empty((N, K // 64), dtype=np.uint16)
    _check(_lib.tern_scales_to_g64(_np_ptr(s), N, K, _np_ptr(out)), "tern_scales_to_g64")
    return out


def tern_scales_from_g64(s64: np.ndarray) -> np.ndarray:
    """binary16 scale bits [N, K/64] with equal halves -> [N, K/128]."""
    s64 = np.ascontiguousarray(s64, dtype=np.uint16)
    N, K = s64.shape[0], s64.shape[1] * 64
    if K % TERN_GROUP:
        raise ValueError("tern_scales_from_g64: need an even number of 64-blocks per row")
    out = np.empty((N, K // TERN_GROUP), dtype=np.uint16)
    _check(_lib.tern_scales_from_g64(_np_ptr(s64), N, K, _np_ptr(out)), "tern_scales_from_g64")
    return out


def _mlx_export(fn, s, where):
    s, N, K = _scales_arg(s, 1, where)
    sc = np.empty_like(s)
    bi = np.empty_like(s)
    _check(fn(_np_ptr(s), N, K, _np_ptr(sc), _np_ptr(bi)), where)
    return sc, bi


def _mlx_import(fn, sc, bi, where):
    sc, N, K = _scales_arg(sc, 1, where)
    bi = np.ascontiguousarray(bi, dtype=np.uint16)
    if bi.shape != sc.shape:
        raise ValueError(f"{where}: scales and biases differ in shape")
    s = np.empty_like(sc)
    _check(fn(_np_ptr(sc), _np_ptr(bi), N, K, _np_ptr(s)), where)
    return s


def tern_mlx_export(s: np.ndarray):
    """g128 scales -> (mlx_scales, mlx_biases) = (s, -s) for the 2-bit slots."""
    return _mlx_export(_lib.tern_mlx_export, s, "tern_mlx_export")


def tern_mlx_import(mlx_scales: np.ndarray, mlx_biases: np.ndarray) -> np.ndarray:
    return _mlx_import(_lib.tern_mlx_import, mlx_scales, mlx_biases, "tern_mlx_import")


def tern_mlx_export_b1(s: np.ndarray):
    """binary-variant scales -> (mlx_scales, mlx_biases) = (2s, -s) for 1-bit fields."""
    return _mlx_export(_lib.tern_mlx_export_b1, s, "tern_mlx_export_b1")


def tern_mlx_import_b1(mlx_scales: np.ndarray, mlx_biases: np.ndarray) -> np.ndarray:
    return _mlx_import(_lib.tern_mlx_import_b1, mlx_scales, mlx_biases, "tern_mlx_import_b1")


def tern_pack_b1(b: np.ndarray) -> np.ndarray:
    """int8 b [N, K] in {-1, +1} -> uint32 bit words [N, K/32]."""
    b = np.ascontiguousarray(b, dtype=np.int8)
    N, K = b.shape
    if K % TERN_GROUP:
        raise ValueError("tern_pack_b1: K % 128 != 0")
    bits = np.empty((N, K // 32), dtype=np.uint32)
    _check(_lib.tern_pack_b1(_np_ptr(b), N, K, _np_ptr(bits)), "tern_pack_b1")
    return bits


def tern_unpack_b1(bits: np.ndarray, K: int) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    N = bits.shape[0]
    b = np.empty((N, K), dtype=np.int8)
    _check(_lib.tern_unpack_b1(_np_ptr(bits), N, K, _np_ptr(b)), "tern_unpack_b1")
    return b


def tern_b1_to_codes(bits: np.ndarray, K: int) -> np.ndarray:
    """Binary bit words [N, K/32] -> ternary slot codes [N, K/16] (t = b)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    N = bits.shape[0]
    if bits.shape != (N, K // 32):
        raise ValueError("tern_b1_to_codes: bits must be [N, K/32]")
    codes = np.empty((N, K // 16), dtype=np.uint32)
    _check(_lib.tern_b1_to_codes(_np_ptr(bits), N, K, _np_ptr(codes)), "tern_b1_to_codes")
    return codes


def tern_codes_to_b1(codes: np.ndarray, K: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    N = codes.shape[0]
    if codes.shape != (N, K // 16):
        raise ValueError("tern_codes_to_b1: codes must be [N, K/16]")
    bits = np.empty((N, K // 32), dtype=np.uint32)
    _check(_lib.tern_codes_to_b1(_np_ptr(codes), N, K, _np_ptr(bits)), "tern_codes_to_b1")
    return bits


def tern_t5_bytes(N: int, K: int) -> int:
    return _lib.tern_t5_bytes(N, K)


def tern_pack_t5(codes: np.ndarray, K: int) -> np.ndarray:
    """2-bit slot codes [N, K/16] -> base-3 data uint8 [N, ceil(K/640) * 128]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    N = codes.shape[0]
    if K % TERN_GROUP or codes.shape != (N, K // 16):
        raise ValueError("tern_pack_t5: codes must be [N, K/16] with K % 128 == 0")
    data = np.empty((N, ((K // TERN_GROUP) + 4) // 5 * 128), dtype=np.uint8)
    _check(_lib.tern_pack_t5(_np_ptr(codes), N, K, _np_ptr(data)), "tern_pack_t5")
    return data


def tern_unpack_t5(data: np.ndarray, K: int) -> np.ndarray:
    data = np.ascontiguousarray(data, dtype=np.uint8)
    N = data.shape[0]
    if K % TERN_GROUP or data.shape != (N, ((K // TERN_GROUP) + 4) // 5 * 128):
        raise ValueError("tern_unpack_t5: data must be [N, ceil(K/640) * 128]")
    codes = np.empty((N, K // 16), dtype=np.uint32)
    _check(_lib.tern_unpack_t5(_np_ptr(data), N, K, _np_ptr(codes)), "tern_unpack_t5")
    return codes


# --------------------------------------------------------------------------
# device operations (torch tensors on the current HIP device)
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_ptr(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TERN_F32
    if t.dtype == torch.bfloat16:
        return TERN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev_ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device operations take tensors on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _shape_check(where, name, t, shape, sizes, device):
    """Raise ValueError unless tensor t has the given shape, an element size
    in `sizes` and lives on `device` (marshalling only: nothing is computed)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{where}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.element_size() not in sizes:
        raise ValueError(f"{where}: {name} has dtype {t.dtype} (element size {t.element_size()}), "
                         f"expected element size {sizes}")
    if t.device != device:
        raise ValueError(f"{where}: {name} is on {t.device}, expected {device}")


def _matrix_shapes(where, x, K, codes, scales, out, M, N, out_sizes=(2, 4)):
    """Check packed weights [N, K/16] (4-byte words), scales [N, K/128]
    (2-byte binary16 bits) and the output [M, N] against x [M, K]."""
    if K % TERN_GROUP:
        raise ValueError(f"{where}: K = {K} is not a multiple of {TERN_GROUP}")
    _shape_check(where, "codes", codes, (N, K // 16), (4,), x.device)
    _shape_check(where, "scales", scales, (N, K // TERN_GROUP), (2,), x.device)
    _shape_check(where, "out", out, (M, N), out_sizes, x.device)


def _dims2(where, x):
    if x.dim() != 2:
        raise ValueError(f"{where}: x must be 2-D [M, K], got {tuple(x.shape)}")
    return x.shape


def tern_pack_device(t, out=None, stream=None):
    """t: int8 [N, K] on the GPU, values in {-1, 0, 1} (not checked) ->
    codes int32 [N, K/16] (bit patterns of the uint32 words)."""
    torch = _torch()
    N, K = _dims2("tern_pack_device", t)
    if K % TERN_GROUP:
        raise ValueError(f"tern_pack_device: K = {K} is not a multiple of {TERN_GROUP}")
    if t.element_size() != 1:
        raise ValueError("tern_pack_device: t must be int8")
    if out is None:
        out = torch.empty((N, K // 16), dtype=torch.int32, device=t.device)
    _shape_check("tern_pack_device", "out", out, (N, K // 16), (4,), t.device)
    _check(_lib.tern_pack_device(_dev_ptr(t), N, K, _dev_ptr(out), _stream_ptr(stream)), "tern_pack_device")
    return out


def tern_fwht(x, signs, block: int, inverse: bool = False, out=None, stream=None):
    """Signed normalized Walsh-Hadamard transform along the last dim.
    x: [M, K] float32 or bfloat16; signs: int8 [K] or None; returns float32
    [M, K] (out may be x itself when x is float32)."""
    torch = _torch()
    M, K = _dims2("tern_fwht", x)
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=x.device)
    _shape_check("tern_fwht", "out", out, (M, K), (4,), x.device)
    if signs is not None:
        _shape_check("tern_fwht", "signs", signs, (K,), (1,), x.device)
    _check(_lib.tern_fwht(_dev_ptr(x), _dt(x), _dev_ptr(signs), M, K, block, int(bool(inverse)),
                          _dev_ptr(out), _stream_ptr(stream)), "tern_fwht")
    return out


def tern_gemv(x, codes, scales, out=None, out_dtype=None, stream=None):
    """y[M, N] = x[M, K] (s_g t)^T for M <= 16.  codes int32 [N, K/16] (bit
    patterns of the uint32 words), scales int16 [N, K/128] (binary16 bits)."""
    torch = _torch()
    M, K = _dims2("tern_gemv", x)
    N = codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=x.device)
    _matrix_shapes("tern_gemv", x, K, codes, scales, out, M, N)
    _check(_lib.tern_gemv(_dev_ptr(x), _dt(x), M, K, _dev_ptr(codes), _dev_ptr(scales), N,
                          _dev_ptr(out), _dt(out), _stream_ptr(stream)), "tern_gemv")
    return out


def tern_rotate_gemv(x, signs, block: int, codes, scales, out=None, out_dtype=None, stream=None):
    """y = rot(x) (s_g t)^T in one launch, rot = signed normalized WHT over
    blocks of `block` along K (forward).  x: [M, K] float32 or bfloat16,
    M <= 16; signs int8 [K] or None."""
    torch = _torch()
    M, K = _dims2("tern_rotate_gemv", x)
    N = codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=x.device)
    _matrix_shapes("tern_rotate_gemv", x, K, codes, scales, out, M, N)
    if signs is not None:
        _shape_check("tern_rotate_gemv", "signs", signs, (K,), (1,), x.device)
    _check(_lib.tern_rotate_gemv(_dev_ptr(x), _dt(x), _dev_ptr(signs), block, M, K, _dev_ptr(codes),
                                 _dev_ptr(scales), N, _dev_ptr(out), _dt(out), _stream_ptr(stream)),
           "tern_rotate_gemv")
    return out


def tern_gemv_t5(x, data, scales, out=None, out_dtype=None, stream=None):
    """y [M, N] = x [M, K] (bfloat16, M <= 16) times the base-3 weights (data
    uint8 [N, ceil(K/640) * 128] on the device) with their group scales."""
    T = _torch()
    M, K = _dims2("tern_gemv_t5", x)
    N = data.shape[0]
    if K % TERN_GROUP:
        raise ValueError(f"tern_gemv_t5: K = {K} is not a multiple of {TERN_GROUP}")
    if out is None:
        out = T.empty((M, N), dtype=out_dtype or T.float32, device=x.device)
    _shape_check("tern_gemv_t5", "data", data, (N, ((K // TERN_GROUP) + 4) // 5 * 128), (1,), x.device)
    _shape_check("tern_gemv_t5", "scales", scales, (N, K // TERN_GROUP), (2,), x.device)
    _shape_check("tern_gemv_t5", "out", out, (M, N), (2, 4), x.device)
    _check(_lib.tern_gemv_t5(_dev_ptr(x), _dt(x), M, K, _dev_ptr(data), _dev_ptr(scales), N,
                             _dev_ptr(out), _dt(out), _stream_ptr(stream)), "tern_gemv_t5")
    return out


def tern_gemv_b1(x, bits, scales, out=None, out_dtype=None, stream=None):
    """y [M, N] = x [M, K] (bfloat16, M <= 4, K a multiple of 1024) times the
    binary variant's weights (bits int32 [N, K/32] on the device, as
    tern_pack_b1 writes them) with their group scales."""
    T = _torch()
    M, K = _dims2("tern_gemv_b1", x)
    N = bits.shape[0]
    if K % TERN_GROUP:
        raise ValueError(f"tern_gemv_b1: K = {K} is not a multiple of {TERN_GROUP}")
    if out is None:
        out = T.empty((M, N), dtype=out_dtype or T.float32, device=x.device)
    _shape_check("tern_gemv_b1", "bits", bits, (N, K // 32), (4,), x.device)
    _shape_check("tern_gemv_b1", "scales", scales, (N, K // TERN_GROUP), (2,), x.device)
    _shape_check("tern_gemv_b1", "out", out, (M, N), (2, 4), x.device)
    _check(_lib.tern_gemv_b1(_dev_ptr(x), _dt(x), M, K, _dev_ptr(bits), _dev_ptr(scales), N,
                             _dev_ptr(out), _dt(out), _stream_ptr(stream)), "tern_gemv_b1")
    return out


def tern_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return _lib.tern_gemm_workspace_bytes(M, N, K)


def tern_gemm(x, codes, scales, out=None, workspace=None, stream=None):
    """y[M, N] = x[M, K] (s_g t)^T, bfloat16 x, any M."""
    torch = _torch()
    M, K = _dims2("tern_gemm", x)
    N = codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _matrix_shapes("tern_gemm", x, K, codes, scales, out, M, N, out_sizes=(4,))
    need = tern_gemm_workspace_bytes(M, N, K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None and workspace.device != x.device:
        raise ValueError(f"tern_gemm: workspace is on {workspace.device}, expected {x.device}")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.tern_gemm(_dev_ptr(x), _dt(x), M, K, _dev_ptr(codes), _dev_ptr(scales), N,
                          _dev_ptr(out), _dev_ptr(workspace), ws_bytes, _stream_ptr(stream)),
           "tern_gemm")
    return out


def tern_gemm_noalloc(x, codes, scales, out, stream=None):
    """tern_gemm with the library's static device scratch instead of a
    workspace: allocates nothing (the caller passes `out`)."""
    M, K = _dims2("tern_gemm_noalloc", x)
    N = codes.shape[0]
    _matrix_shapes("tern_gemm_noalloc", x, K, codes, scales, out, M, N, out_sizes=(4,))
    _check(_lib.tern_gemm_noalloc(_dev_ptr(x), _dt(x), M, K, _dev_ptr(codes), _dev_ptr(scales), N,
                                  _dev_ptr(out), _stream_ptr(stream)),
           "tern_gemm_noalloc")
    return out


def to_device(codes: np.ndarray, scales: np.ndarray, device="cuda"):
    """Upload packed weights as int32 / int16 tensors (same bits)."""
    torch = _torch()
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint32).view(np.int32)).to(device)
    s = torch.from_numpy(np.ascontiguousarray(scales, dtype=np.uint16).view(np.int16)).to(device)
    return c, s
