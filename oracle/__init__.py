"""CPU oracle for the MXFP4 GEMM with on-the-fly bf16 A quantization.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library.  The arithmetic lives in
``mxfp4_oracle.c`` (plain C, exact integer quantization, a GEMM in fp64 and
in fp32 group accumulation, OpenMP over independent outputs); this module
only marshals numpy arrays through ctypes.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, exhaustive brute force, page constants and library special cases.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxfp4_oracle.c")
_LIB = os.environ.get("MXFP4_ORACLE_LIB") or os.path.join(_HERE, "liboracle_mxfp4.so")


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (no HIP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
             "-fvisibility=hidden", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.oracle_e8m0_value.restype = ctypes.c_double
        L.oracle_e8m0_value.argtypes = [ctypes.c_int]
        L.oracle_scale_byte.restype = ctypes.c_int
        L.oracle_scale_byte.argtypes = [P, ctypes.c_int]
        L.oracle_encode.restype = ctypes.c_int
        L.oracle_encode.argtypes = [ctypes.c_uint16, ctypes.c_int]
        L.oracle_encode_nearest.restype = ctypes.c_int
        L.oracle_encode_nearest.argtypes = [ctypes.c_uint16, ctypes.c_int]
        L.oracle_encode_many.restype = None
        L.oracle_encode_many.argtypes = [P, P, I64, P]
        L.oracle_encode_nearest_many.restype = None
        L.oracle_encode_nearest_many.argtypes = [P, P, I64, P]
        L.oracle_quantize.restype = ctypes.c_int
        L.oracle_quantize.argtypes = [P, I64, I64, P, P]
        L.oracle_dequantize.restype = None
        L.oracle_dequantize.argtypes = [P, P, I64, I64, P]
        L.oracle_shuffled_scale_bytes.restype = I64
        L.oracle_shuffled_scale_bytes.argtypes = [I64, I64]
        L.oracle_shuffle_scales.restype = None
        L.oracle_shuffle_scales.argtypes = [P, I64, I64, P]
        L.oracle_unshuffle_scales.restype = None
        L.oracle_unshuffle_scales.argtypes = [P, I64, I64, P]
        L.oracle_preshuffle_b.restype = None
        L.oracle_preshuffle_b.argtypes = [P, I64, I64, P]
        L.oracle_unpreshuffle_b.restype = None
        L.oracle_unpreshuffle_b.argtypes = [P, I64, I64, P]
        L.oracle_gemm_f64.restype = None
        L.oracle_gemm_f64.argtypes = [P, P, P, P, I64, I64, I64, P]
        L.oracle_gemm_f32.restype = None
        L.oracle_gemm_f32.argtypes = [P, P, P, P, I64, I64, I64, P]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_gemm_f64_sampled.restype = None
        L.oracle_gemm_f64_sampled.argtypes = [P, P, P, P, I64, I64, I64, P, P, I64, P]
        L.oracle_bf16_from_f64.restype = ctypes.c_uint16
        L.oracle_bf16_from_f64.argtypes = [ctypes.c_double]
        L.oracle_bf16_from_f64_many.restype = None
        L.oracle_bf16_from_f64_many.argtypes = [P, I64, P]
        L.oracle_mxfp4_gemm_bf16.restype = ctypes.c_int
        L.oracle_mxfp4_gemm_bf16.argtypes = [P, P, P, I64, I64, I64, P, ctypes.c_int]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, "bf16 inputs are passed as their uint16 bit patterns"
    return a


# ---- scalar helpers -------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def e8m0_value(b: int) -> float:
    return lib().oracle_e8m0_value(int(b))


def scale_byte(group_bits) -> int:
    g = _u16(group_bits)
    return lib().oracle_scale_byte(_p(g), int(g.size))


def encode(x_bits: int, s: int) -> int:
    return lib().oracle_encode(int(x_bits), int(s))


def encode_nearest(x_bits: int, s: int) -> int:
    return lib().oracle_encode_nearest(int(x_bits), int(s))


def encode_many(x_bits, s) -> np.ndarray:
    x = _u16(x_bits).ravel()
    sc = np.ascontiguousarray(np.broadcast_to(np.asarray(s, dtype=np.uint8), x.shape))
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_encode_many(_p(x), _p(sc), x.size, _p(out))
    return out


def encode_nearest_many(x_bits, s) -> np.ndarray:
    x = _u16(x_bits).ravel()
    sc = np.ascontiguousarray(np.broadcast_to(np.asarray(s, dtype=np.uint8), x.shape))
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_encode_nearest_many(_p(x), _p(sc), x.size, _p(out))
    return out


# ---- array operations -----------------------------------------------------

def quantize(x_bits: np.ndarray):
    """bf16 bits [rows, K] -> (q uint8 [rows, K/2], raw scales uint8 [rows, K/32])."""
    x = _u16(x_bits)
    rows, K = x.shape
    q = np.empty((rows, K // 2), dtype=np.uint8)
    s = np.empty((rows, K // 32), dtype=np.uint8)
    rc = lib().oracle_quantize(_p(x), rows, K, _p(q), _p(s))
    if rc != 0:
        raise ValueError("oracle_quantize: non-finite input or K % 32 != 0")
    return q, s


def dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    rows, KB = q.shape
    out = np.empty((rows, KB * 2), dtype=np.float64)
    lib().oracle_dequantize(_p(q), _p(s), rows, KB * 2, _p(out))
    return out


def shuffled_scale_bytes(rows: int, K: int) -> int:
    return int(lib().oracle_shuffled_scale_bytes(rows, K))


def shuffle_scales(raw: np.ndarray, rows: int, K: int) -> np.ndarray:
    """raw [rows, K/32] -> shuffled, padded buffer viewed [pad256(rows)/32, pad8(K/32)*32]."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    assert raw.shape == (rows, K // 32)
    gp = (K // 32 + 7) // 8 * 8
    rp = (rows + 255) // 256 * 256
    out = np.empty((rp // 32, gp * 32), dtype=np.uint8)
    lib().oracle_shuffle_scales(_p(raw), rows, K, _p(out))
    return out


def unshuffle_scales(sh: np.ndarray, rows: int, K: int) -> np.ndarray:
    sh = np.ascontiguousarray(sh, dtype=np.uint8)
    raw = np.empty((rows, K // 32), dtype=np.uint8)
    lib().oracle_unshuffle_scales(_p(sh), rows, K, _p(raw))
    return raw


def preshuffle_b(bq: np.ndarray) -> np.ndarray:
    """bq [N, K/2] -> preshuffled bytes viewed [N/16, (K/2)*16]."""
    bq = np.ascontiguousarray(bq, dtype=np.uint8)
    N, KB = bq.shape
    out = np.empty((N // 16, KB * 16), dtype=np.uint8)
    lib().oracle_preshuffle_b(_p(bq), N, KB * 2, _p(out))
    return out


def unpreshuffle_b(sh: np.ndarray, N: int, K: int) -> np.ndarray:
    sh = np.ascontiguousarray(sh, dtype=np.uint8)
    out = np.empty((N, K // 2), dtype=np.uint8)
    lib().oracle_unpreshuffle_b(_p(sh), N, K, _p(out))
    return out


def gemm_f64(qa, sa, qb, sb) -> np.ndarray:
    """Exact-as-fp64 C = deq(A) @ deq(B)^T from natural-layout quantized operands."""
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    qb = np.ascontiguousarray(qb, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    M, N, K = qa.shape[0], qb.shape[0], qa.shape[1] * 2
    C = np.empty((M, N), dtype=np.float64)
    lib().oracle_gemm_f64(_p(qa), _p(sa), _p(qb), _p(sb), M, N, K, _p(C))
    return C


def gemm_f32(qa, sa, qb, sb) -> np.ndarray:
    """C = deq(A) @ deq(B)^T with the matrix unit's accumulation: per 32-group
    an exact integer dot times both scales, rounded to fp32, the groups summed
    in fp32 in ascending order.  Returns float32 [M, N]."""
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    qb = np.ascontiguousarray(qb, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    M, N, K = qa.shape[0], qb.shape[0], qa.shape[1] * 2
    C = np.empty((M, N), dtype=np.float32)
    lib().oracle_gemm_f32(_p(qa), _p(sa), _p(qb), _p(sb), M, N, K, _p(C))
    return C


def num_threads() -> int:
    """Threads the oracle's parallel loops use (OpenMP; OMP_NUM_THREADS)."""
    return int(lib().oracle_num_threads())


def gemm_f64_sampled(qa, sa, qb, sb, ms, ns) -> np.ndarray:
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    qb = np.ascontiguousarray(qb, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    M, N, K = qa.shape[0], qb.shape[0], qa.shape[1] * 2
    out = np.empty(ms.shape, dtype=np.float64)
    lib().oracle_gemm_f64_sampled(_p(qa), _p(sa), _p(qb), _p(sb), M, N, K, _p(ms), _p(ns), ms.size, _p(out))
    return out


def bf16_from_f64(d: np.ndarray) -> np.ndarray:
    d = np.ascontiguousarray(d, dtype=np.float64)
    out = np.empty(d.shape, dtype=np.uint16)
    lib().oracle_bf16_from_f64_many(_p(d), d.size, _p(out))
    return out


def mxfp4_gemm_bf16(a_bits: np.ndarray, qb: np.ndarray, sb: np.ndarray, f32acc: bool = False) -> np.ndarray:
    """The whole per-call path: quantize bf16 A, multiply by quantized B (fp64,
    or fp32 group accumulation), round to bf16 bits."""
    a = _u16(a_bits)
    qb = np.ascontiguousarray(qb, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    M, K = a.shape
    N = qb.shape[0]
    C = np.empty((M, N), dtype=np.uint16)
    rc = lib().oracle_mxfp4_gemm_bf16(_p(a), _p(qb), _p(sb), M, N, K, _p(C), 1 if f32acc else 0)
    if rc != 0:
        raise ValueError("oracle_mxfp4_gemm_bf16: non-finite input")
    return C
