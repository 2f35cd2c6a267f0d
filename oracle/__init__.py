"""FP64 CPU oracle for the ternary-g128 matmul and the signed normalized
Walsh-Hadamard rotation.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark are the only callers.  The product path never imports this
package, and this package imports nothing from the product package.

The arithmetic lives in ``tern_oracle.c`` (plain C, double precision); this
module builds it with gcc, loads it with ctypes and converts numpy arrays.
Each wrapper names the definition it follows; see the C file for the source
passages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tern_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# dtype codes understood by the C oracle for activations
XDT_F32, XDT_BF16, XDT_F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile tern_oracle.c into liboracle.so with gcc (no fast-math, so the
    C evaluation order is the order the additions happen in)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", "-fopenmp", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_decode.argtypes = [P, I64, I64, P]
        L.oracle_encode.argtypes = [P, I64, I64, P]
        L.oracle_matmul.argtypes = [P, ctypes.c_int, I64, I64, P, P, I64, P, P]
        L.oracle_matmul_threaded.argtypes = [P, ctypes.c_int, I64, I64, P, P, I64, P, P, ctypes.c_int]
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_matmul_at.argtypes = [P, ctypes.c_int, I64, P, P, P, P, I64, P, P]
        L.oracle_hadamard_entry.argtypes = [I64, I64]
        L.oracle_hadamard_entry.restype = ctypes.c_double
        L.oracle_fwht.argtypes = [P, P, I64, I64, I64, ctypes.c_int, P]
        L.oracle_ternary_from_f32.argtypes = [P, I64, I64, P, P]
        L.oracle_bits_per_weight.argtypes = [I64, I64]
        L.oracle_bits_per_weight.restype = ctypes.c_double
        L.oracle_dequant_g64.argtypes = [P, P, I64, I64, P]
        L.oracle_dequant_affine.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, I64, I64, P]
        L.oracle_b1_decode.argtypes = [P, I64, I64, P]
        L.oracle_b1_decode.restype = None
        L.oracle_b1_encode.argtypes = [P, I64, I64, P]
        L.oracle_format_bits_per_weight.argtypes = [ctypes.c_int, I64, I64]
        L.oracle_format_bits_per_weight.restype = ctypes.c_double
        L.oracle_t5_decode.argtypes = [P, I64, I64, P]
        L.oracle_t5_encode.argtypes = [P, I64, I64, P]
        L.oracle_t5_bits_per_weight.argtypes = [I64, I64]
        L.oracle_t5_bits_per_weight.restype = ctypes.c_double
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def half_to_double(h: int) -> float:
    """IEEE binary16 bit pattern -> value (from the format definition)."""
    return lib().oracle_half_to_double(int(h))


def bf16_to_double(b: int) -> float:
    """bfloat16 bit pattern -> value (upper half of a binary32)."""
    return lib().oracle_bf16_to_double(int(b))


def encode(t: np.ndarray) -> np.ndarray:
    """t int8 [N, K] in {-1,0,1} -> uint32 codes [N, K/16]; slot q = t + 1."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    N, K = t.shape
    assert K % 16 == 0
    codes = np.zeros((N, K // 16), dtype=np.uint32)
    rc = lib().oracle_encode(_ptr(t), N, K, _ptr(codes))
    if rc:
        raise ValueError("not ternary")
    return codes


def decode(codes: np.ndarray, K: int) -> np.ndarray:
    """uint32 codes [N, K/16] -> int8 t [N, K]; raises on the unused slot 3."""
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    N = codes.shape[0]
    t = np.zeros((N, K), dtype=np.int8)
    rc = lib().oracle_decode(_ptr(codes), N, K, _ptr(t))
    if rc:
        raise ValueError("slot value 3 is not a ternary code")
    return t


def _x_and_code(x: np.ndarray):
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), XDT_F32
    if x.dtype == np.uint16:  # bfloat16 bit patterns
        return np.ascontiguousarray(x), XDT_BF16
    if x.dtype == np.float64:
        return np.ascontiguousarray(x), XDT_F64
    raise TypeError(f"unsupported activation dtype {x.dtype}")


def max_threads() -> int:
    """Host threads the threaded oracle may use (OpenMP's default)."""
    return lib().oracle_max_threads()


def matmul(x: np.ndarray, codes: np.ndarray, scales: np.ndarray, K: int, threads: int = 1):
    """y[m, n] = sum_k s_g t[n, k] x[m, k] in double, and the error scale
    B[m, n] = sum_k |s_g t[n, k] x[m, k]|.

    x: float32 [M, K], uint16 bfloat16 bits [M, K] or float64 [M, K];
    codes: uint32 [N, K/16]; scales: uint16 binary16 bits [N, K/128].
    threads > 1 shares the outputs over host threads; every output is the
    same k-ordered sum, so the result is bit-identical to threads = 1.
    """
    x, xdt = _x_and_code(x)
    M = x.shape[0]
    assert x.shape[1] == K
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    N = codes.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    b = np.zeros((M, N), dtype=np.float64)
    if threads > 1:
        rc = lib().oracle_matmul_threaded(_ptr(x), xdt, M, K, _ptr(codes), _ptr(scales), N,
                                          _ptr(y), _ptr(b), int(threads))
    else:
        rc = lib().oracle_matmul(_ptr(x), xdt, M, K, _ptr(codes), _ptr(scales), N,
                                 _ptr(y), _ptr(b))
    if rc:
        raise ValueError("slot value 3 is not a ternary code")
    return y, b


def matmul_at(x: np.ndarray, codes: np.ndarray, scales: np.ndarray, K: int,
              ms: np.ndarray, ns: np.ndarray):
    """The matmul definition evaluated only at outputs (ms[i], ns[i])."""
    x, xdt = _x_and_code(x)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    y = np.zeros(len(ms), dtype=np.float64)
    b = np.zeros(len(ms), dtype=np.float64)
    rc = lib().oracle_matmul_at(_ptr(x), xdt, K, _ptr(codes), _ptr(scales),
                                _ptr(ms), _ptr(ns), len(ms), _ptr(y), _ptr(b))
    if rc:
        raise ValueError("slot value 3 is not a ternary code")
    return y, b


def hadamard_entry(i: int, l: int) -> float:
    return lib().oracle_hadamard_entry(i, l)


def fwht(x: np.ndarray, signs, block: int, inverse: bool = False) -> np.ndarray:
    """Signed normalized Walsh-Hadamard transform over contiguous blocks of
    the last dimension; x float64 [M, K] (other float dtypes are widened
    exactly); signs int8 [K] of +-1 or None."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if x.ndim == 1:
        x = x[None, :]
    M, K = x.shape
    y = np.zeros_like(x)
    sp = None
    if signs is not None:
        signs = np.ascontiguousarray(signs, dtype=np.int8)
        assert signs.shape == (K,)
        sp = _ptr(signs)
    rc = lib().oracle_fwht(_ptr(x), sp, M, K, block, int(bool(inverse)), _ptr(y))
    if rc:
        raise ValueError("K must be a multiple of the block")
    return y


def ternary_from_f32(w: np.ndarray):
    """Lossless FP32 -> (t int8 [N,K], scale bits uint16 [N,K/128]) or None
    when some group is not of the form s * {-1,0,1} with an FP16-exact s."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    t = np.zeros((N, K), dtype=np.int8)
    s = np.zeros((N, K // 128), dtype=np.uint16)
    rc = lib().oracle_ternary_from_f32(_ptr(w), N, K, _ptr(t), _ptr(s))
    if rc:
        return None
    return t, s


def bits_per_weight(N: int, K: int) -> float:
    return lib().oracle_bits_per_weight(N, K)


def bf16_bits_to_f64(xb: np.ndarray) -> np.ndarray:
    """Vectorized bfloat16 -> float64 (upper half of binary32), for callers
    that need activations as doubles."""
    xb = np.asarray(xb, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def half_bits_to_f64(hb: np.ndarray) -> np.ndarray:
    """Vectorized binary16 -> float64 by the format definition."""
    hb = np.asarray(hb, dtype=np.uint16).astype(np.int64)
    sign = np.where((hb >> 15) & 1, -1.0, 1.0)
    e = (hb >> 10) & 0x1F
    f = (hb & 0x3FF).astype(np.float64)
    normal = np.ldexp(1.0 + f / 1024.0, (e - 15).astype(np.int32))
    sub = np.ldexp(f, -24)
    v = np.where(e == 0, sub, normal)
    v = np.where(e == 31, np.where(f == 0, np.inf, np.nan), v)
    return sign * v


def dequant(codes: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """Dense w = s_g * t in float64 (only for small matrices)."""
    t = decode(codes, K).astype(np.float64)
    s = half_bits_to_f64(scales)
    return t * np.repeat(s, 128, axis=1)


# ---------------------------------------------------------------------------
# format variants (group-64 scales, affine scale+bias container, binary g128)
# ---------------------------------------------------------------------------

FMT_G128, FMT_G64, FMT_AFFINE2, FMT_B1, FMT_AFFINE1 = 0, 1, 2, 3, 4


def format_bits_per_weight(fmt: int, N: int, K: int) -> float:
    return lib().oracle_format_bits_per_weight(fmt, N, K)


def dequant_g64(codes: np.ndarray, s64: np.ndarray, K: int) -> np.ndarray:
    """Dense float64 weights of the group-64 variant: same slot codes, the
    scale of weight k is s64[n][k / 64]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    s64 = np.ascontiguousarray(s64, dtype=np.uint16)
    N = codes.shape[0]
    assert s64.shape == (N, K // 64)
    w = np.zeros((N, K), dtype=np.float64)
    if lib().oracle_dequant_g64(_ptr(codes), _ptr(s64), N, K, _ptr(w)):
        raise ValueError("slot value 3 is not a ternary code")
    return w


def dequant_affine(words: np.ndarray, bits: int, group: int, scales: np.ndarray,
                   biases: np.ndarray, K: int) -> np.ndarray:
    """Dense float64 weights scale * q + bias of the affine group format with
    `bits`-bit fields (1 or 2), lowest field first in each uint32."""
    words = np.ascontiguousarray(words, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    biases = np.ascontiguousarray(biases, dtype=np.uint16)
    N = words.shape[0]
    assert words.shape == (N, K * bits // 32)
    assert scales.shape == biases.shape == (N, K // group)
    w = np.zeros((N, K), dtype=np.float64)
    if lib().oracle_dequant_affine(_ptr(words), bits, group, _ptr(scales), _ptr(biases), N, K, _ptr(w)):
        raise ValueError("unsupported affine format")
    return w


def b1_decode(bits: np.ndarray, K: int) -> np.ndarray:
    """uint32 bit words [N, K/32] -> int8 b [N, K] in {-1, +1} (bit 1 is +1)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    N = bits.shape[0]
    b = np.zeros((N, K), dtype=np.int8)
    lib().oracle_b1_decode(_ptr(bits), N, K, _ptr(b))
    return b


def b1_encode(b: np.ndarray) -> np.ndarray:
    """int8 b [N, K] in {-1, +1} -> uint32 bit words [N, K/32]."""
    b = np.ascontiguousarray(b, dtype=np.int8)
    N, K = b.shape
    assert K % 32 == 0
    bits = np.zeros((N, K // 32), dtype=np.uint32)
    if lib().oracle_b1_encode(_ptr(b), N, K, _ptr(bits)):
        raise ValueError("not binary")
    return bits


# ---------------------------------------------------------------------------
# base-3 layout: five ternary values per byte, groups taken five at a time
# ---------------------------------------------------------------------------

def t5_row_bytes(K: int) -> int:
    return ((K // 128 + 4) // 5) * 128


def t5_encode(t: np.ndarray) -> np.ndarray:
    """int8 t [N, K] in {-1,0,1} -> uint8 [N, ceil(K/640) * 128]."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    N, K = t.shape
    assert K % 128 == 0
    d = np.zeros((N, t5_row_bytes(K)), dtype=np.uint8)
    if lib().oracle_t5_encode(_ptr(t), N, K, _ptr(d)):
        raise ValueError("not ternary")
    return d


def t5_decode(d: np.ndarray, K: int) -> np.ndarray:
    d = np.ascontiguousarray(d, dtype=np.uint8)
    N = d.shape[0]
    assert d.shape == (N, t5_row_bytes(K))
    t = np.zeros((N, K), dtype=np.int8)
    if lib().oracle_t5_decode(_ptr(d), N, K, _ptr(t)):
        raise ValueError("byte out of range for its superblock")
    return t


def t5_bits_per_weight(N: int, K: int) -> float:
    return lib().oracle_t5_bits_per_weight(N, K)
