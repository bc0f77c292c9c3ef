"""Python binding of libmxfp4.so, the MI355X (gfx950) MXFP4 GEMM library.

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the C ABI declared in ``include/mxfp4.h`` and
raises ``RuntimeError`` with the library's status string on failure.  All
computation happens in the library's HIP kernels; torch provides device
memory and streams.  If the library is not built, importing the binding's
functions raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# MXFP4_LIB may point at another build of the same library (e.g. a debug build).
LIB_PATH = os.environ.get("MXFP4_LIB") or os.path.join(_PKG, "libmxfp4.so")

MXFP4_OK = 0

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # PyTorch ships its own HIP runtime and asks for it as "libamdhip64.so";
    # this library asks for "libamdhip64.so.7", the soname that copy carries.
    # Loaded after torch, this library therefore binds to torch's runtime.
    # Loaded first, it would bring in /opt/rocm's copy and torch would then
    # load a second one, and the two runtimes in one process do not share
    # the device.  So torch goes first whenever it is installed.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libmxfp4.so is not built (expected at %s); run __graft_entry__.build() or "
            "python block_scaled_mxfp4_bf16_amd/build.py" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sigs = {
        "mxfp4_packed_bytes": (SZ, [I64, I64]),
        "mxfp4_raw_scale_bytes": (SZ, [I64, I64]),
        "mxfp4_shuffled_scale_bytes": (SZ, [I64, I64]),
        "mxfp4_gemm_workspace_bytes": (SZ, [I64, I64, I64]),
        "mxfp4_quantize": (I, [P, I64, I64, P, P, I, P]),
        "mxfp4_preshuffle_b": (I, [P, P, I64, I64, P, P, P]),
        "mxfp4_prepare_b": (I, [P, I64, I64, P, P, P]),
        "mxfp4_gemm": (I, [P, P, P, P, I64, I64, I64, P]),
        "mxfp4_gemm_ex": (I, [P, P, P, P, I64, I64, I64, P, SZ, P]),
        "mxfp4_gemm_noalloc": (I, [P, P, P, P, I64, I64, I64, P]),
        "mxfp4_gemm_q": (I, [P, P, P, P, P, I64, I64, I64, P]),
        "mxfp4_gemm_q_schedule_name": (ctypes.c_char_p, [I64, I64, I64]),
        "mxfp4_reserve": (I, [I64, I64, I64, P]),
        "mxfp4_status_string": (ctypes.c_char_p, [I]),
        "mxfp4_last_hip_error": (ctypes.c_char_p, []),
        "mxfp4_gemm_schedule_name": (ctypes.c_char_p, [I64, I64, I64]),
        "mxfp4_set_quant_mode": (I, [I]),
        "mxfp4_set_schedule_override": (I, [ctypes.c_char_p]),
        "mxfp4_list_schedules": (SZ, [I64, I64, I64, I, ctypes.c_char_p, SZ]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def lib():
    return _load()


def exported_symbols():
    """Names every entry point the header declares (used by the ABI test)."""
    return ["mxfp4_packed_bytes", "mxfp4_raw_scale_bytes", "mxfp4_shuffled_scale_bytes",
            "mxfp4_gemm_workspace_bytes", "mxfp4_quantize", "mxfp4_preshuffle_b", "mxfp4_prepare_b", "mxfp4_gemm",
            "mxfp4_gemm_ex", "mxfp4_gemm_noalloc", "mxfp4_gemm_q", "mxfp4_gemm_q_schedule_name", "mxfp4_reserve", "mxfp4_status_string", "mxfp4_last_hip_error", "mxfp4_gemm_schedule_name",
            "mxfp4_set_quant_mode", "mxfp4_set_schedule_override", "mxfp4_list_schedules"]


def _check(rc: int, what: str):
    if rc != MXFP4_OK:
        L = _load()
        msg = L.mxfp4_status_string(rc).decode()
        if rc == 4:  # MXFP4_ERR_HIP: name the HIP error
            msg += " (%s)" % L.mxfp4_last_hip_error().decode()
        raise RuntimeError("%s failed: %s" % (what, msg))


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---- sizes -----------------------------------------------------------------

def mxfp4_packed_bytes(rows: int, K: int) -> int:
    return _load().mxfp4_packed_bytes(rows, K)


def mxfp4_raw_scale_bytes(rows: int, K: int) -> int:
    return _load().mxfp4_raw_scale_bytes(rows, K)


def mxfp4_shuffled_scale_bytes(rows: int, K: int) -> int:
    return _load().mxfp4_shuffled_scale_bytes(rows, K)


def mxfp4_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return _load().mxfp4_gemm_workspace_bytes(M, N, K)


def mxfp4_gemm_schedule_name(M: int, N: int, K: int):
    r = _load().mxfp4_gemm_schedule_name(M, N, K)
    return r.decode() if r is not None else None


# ---- operations (raw: caller passes every buffer) --------------------------

def mxfp4_quantize(x, rows: int, K: int, q, scales, shuffled_scales: bool = False, stream=None):
    _check(_load().mxfp4_quantize(_ptr(x), rows, K, _ptr(q), _ptr(scales), int(bool(shuffled_scales)),
                                  _stream(stream)), "mxfp4_quantize")


def mxfp4_preshuffle_b(bq, bs_raw, N: int, K: int, bq_shuffled, bs_shuffled, stream=None):
    _check(_load().mxfp4_preshuffle_b(_ptr(bq), _ptr(bs_raw), N, K, _ptr(bq_shuffled), _ptr(bs_shuffled),
                                      _stream(stream)), "mxfp4_preshuffle_b")


def mxfp4_prepare_b(b, N: int, K: int, bq_shuffled, bs_shuffled, stream=None):
    _check(_load().mxfp4_prepare_b(_ptr(b), N, K, _ptr(bq_shuffled), _ptr(bs_shuffled), _stream(stream)),
           "mxfp4_prepare_b")


def mxfp4_gemm(A, Bq_sh, Bs_sh, C, M: int, N: int, K: int, stream=None):
    _check(_load().mxfp4_gemm(_ptr(A), _ptr(Bq_sh), _ptr(Bs_sh), _ptr(C), M, N, K, _stream(stream)), "mxfp4_gemm")


def mxfp4_gemm_ex(A, Bq_sh, Bs_sh, C, M: int, N: int, K: int, workspace, workspace_bytes: int, stream=None):
    _check(_load().mxfp4_gemm_ex(_ptr(A), _ptr(Bq_sh), _ptr(Bs_sh), _ptr(C), M, N, K, _ptr(workspace),
                                 workspace_bytes, _stream(stream)), "mxfp4_gemm_ex")


def mxfp4_gemm_noalloc(A, Bq_sh, Bs_sh, C, M: int, N: int, K: int, stream=None):
    _check(_load().mxfp4_gemm_noalloc(_ptr(A), _ptr(Bq_sh), _ptr(Bs_sh), _ptr(C), M, N, K, _stream(stream)),
           "mxfp4_gemm_noalloc")


def mxfp4_gemm_q(Aq, As, Bq_sh, Bs_sh, C, M: int, N: int, K: int, stream=None):
    _check(_load().mxfp4_gemm_q(_ptr(Aq), _ptr(As), _ptr(Bq_sh), _ptr(Bs_sh), _ptr(C), M, N, K, _stream(stream)),
           "mxfp4_gemm_q")


def mxfp4_gemm_q_schedule_name(M: int, N: int, K: int):
    r = _load().mxfp4_gemm_q_schedule_name(M, N, K)
    return r.decode() if r is not None else None


def mxfp4_reserve(M: int, N: int, K: int, stream=None):
    _check(_load().mxfp4_reserve(M, N, K, _stream(stream)), "mxfp4_reserve")


def mxfp4_set_quant_mode(mode: int):
    _check(_load().mxfp4_set_quant_mode(mode), "mxfp4_set_quant_mode")


def mxfp4_set_schedule_override(name):
    _check(_load().mxfp4_set_schedule_override(name.encode() if name else None), "mxfp4_set_schedule_override")


def mxfp4_list_schedules(M: int, N: int, K: int, quantized_a: bool = False):
    """Names of every compiled schedule that can serve (M, N, K) (empty for a
    shape outside the ABI); each is accepted by mxfp4_set_schedule_override."""
    L = _load()
    need = L.mxfp4_list_schedules(M, N, K, int(quantized_a), None, 0)
    if need == 0:
        return []
    buf = ctypes.create_string_buffer(need + 1)
    L.mxfp4_list_schedules(M, N, K, int(quantized_a), buf, need + 1)
    return buf.value.decode().split()


# ---- tensor conveniences (allocate outputs with torch, then call the above) --

def quantize(x, shuffled_scales: bool = False, stream=None):
    """bf16 [rows, K] cuda tensor -> (q uint8 [rows, K/2], scales uint8)."""
    import torch
    rows, K = x.shape
    assert x.dtype == torch.bfloat16 and x.is_contiguous()
    q = torch.empty((rows, K // 2), dtype=torch.uint8, device=x.device)
    if shuffled_scales:
        s = torch.empty(mxfp4_shuffled_scale_bytes(rows, K), dtype=torch.uint8, device=x.device)
        s = s.view(-1, ((K // 32 + 7) // 8) * 32)
    else:
        s = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    mxfp4_quantize(x, rows, K, q, s, shuffled_scales, stream)
    return q, s


def preshuffle_b(bq, bs_raw, stream=None):
    """Quantized B (natural layouts) -> (Bw [N/16, (K/2)*16], Bs shuffled)."""
    import torch
    N, KB = bq.shape
    K = KB * 2
    bw = torch.empty((N // 16, KB * 16), dtype=torch.uint8, device=bq.device)
    bs = torch.empty(mxfp4_shuffled_scale_bytes(N, K), dtype=torch.uint8, device=bq.device)
    bs = bs.view(-1, ((K // 32 + 7) // 8) * 32)
    mxfp4_preshuffle_b(bq, bs_raw, N, K, bw, bs, stream)
    return bw, bs


def prepare_b(b, stream=None):
    """bf16 [N, K] cuda tensor -> (Bw [N/16, (K/2)*16], Bs shuffled), in one launch."""
    import torch
    N, K = b.shape
    assert b.dtype == torch.bfloat16 and b.is_contiguous()
    bw = torch.empty((N // 16, (K // 2) * 16), dtype=torch.uint8, device=b.device)
    bs = torch.empty(mxfp4_shuffled_scale_bytes(N, K), dtype=torch.uint8, device=b.device)
    bs = bs.view(-1, ((K // 32 + 7) // 8) * 32)
    mxfp4_prepare_b(b, N, K, bw, bs, stream)
    return bw, bs


def gemm_q(Aq, As, Bw, Bs, N: int, out=None, stream=None):
    """C = dequant(Aq, As) * B^T as bf16 [M, N]; Aq uint8 [M, K/2], As shuffled scales."""
    import torch
    M, KB = Aq.shape
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=Aq.device)
    mxfp4_gemm_q(Aq, As, Bw, Bs, out, M, N, 2 * KB, stream)
    return out


def gemm(A, Bw, Bs, N: int, out=None, stream=None):
    """C = Q(A) * B^T as bf16 [M, N]; A bf16 [M, K] cuda tensor."""
    import torch
    M, K = A.shape
    assert A.dtype == torch.bfloat16 and A.is_contiguous()
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    mxfp4_gemm(A, Bw, Bs, out, M, N, K, stream)
    return out
