"""ctypes binding for libqgemv.so, with the names of the C ABI (include/qgemv.h).

Argument marshalling only: every step of the GEMV runs in the library's HIP
kernels.  Device buffers are torch tensors (torch supplies memory and the
stream); host buffers for the packer are numpy arrays.  If the library has
not been built this module raises on first use; there is no other path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# QG_LIBRARY names another build of the same library (the host-sanitizer
# build of the CPU tests); by default the in-tree libqgemv.so.
LIB_PATH = os.environ.get("QG_LIBRARY") or os.path.join(_PKG, "libqgemv.so")

QG_OK = 0
QG_ERR_INVALID_ARG = 1
QG_ERR_UNSUPPORTED = 2
QG_ERR_ALIGNMENT = 3
QG_ERR_HIP = 4

FMT_Q8G64 = 0
FMT_Q4G32 = 1
FMT_GROUPED_Q4G32 = 2
FMT_Q8G128 = 3
FMT_Q8PC = 4
FMT_GROUPED_Q4G32_SWIGLU = 5
FMT_Q8G64_ARGMAX = 6
FMT_Q8G128_ARGMAX = 7
FMT_Q8G64_MMA = 8
FMT_Q8G128_MMA = 9
FMT_Q8PC_MMA = 10
FMT_Q4G32_MMA = 11

_lib = None


class QGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        names = {QG_OK: "ok", QG_ERR_INVALID_ARG: "invalid argument", QG_ERR_UNSUPPORTED: "unsupported",
                 QG_ERR_ALIGNMENT: "misaligned pointer or stride", QG_ERR_HIP: "HIP runtime error"}
        super().__init__("%s failed: %s (status %d)" % (where, names.get(self.status, "unknown status"),
                                                        status))


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libqgemv.so is not built (run python -m weight_only_block_amd.build); "
                               "there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32, sz, st = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t,
                               ctypes.c_int)
        sig = {
            "qg_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "qg_abi_version": ([], ctypes.c_int),
            "qpack_q8g64_size": ([i64, i64], sz),
            "qpack_q8g64": ([p, p, i64, i64, p, sz], st),
            "qunpack_q8g64": ([p, sz, i64, i64, p, p], st),
            "qpack_q8g128_size": ([i64, i64], sz),
            "qpack_q8g128": ([p, p, i64, i64, p, sz], st),
            "qunpack_q8g128": ([p, sz, i64, i64, p, p], st),
            "qpack_q8pc_size": ([i64, i64], sz),
            "qpack_q8pc": ([p, p, i64, i64, p, sz], st),
            "qunpack_q8pc": ([p, sz, i64, i64, p, p], st),
            "qgemv_q8g128": ([p, p, p, i64, i64, i64, i64, i64, p], st),
            "qgemv_q8pc": ([p, p, p, i64, i64, i64, i64, i64, p], st),
            "qpack_q4g32_size": ([i64, i64], sz),
            "qpack_q4g32": ([p, p, p, i64, i64, p, sz], st),
            "qunpack_q4g32": ([p, sz, i64, i64, p, p, p], st),
            "qgemv_q8g64": ([p, p, p, i64, i64, i64, i64, i64, p], st),
            "qgemv_q4g32": ([p, p, p, i64, i64, i64, i64, i64, p], st),
            "qgemv_grouped_q4g32": ([p, i64, i32, p, i32, p, i64, p, i64, i64, i64, p], st),
            "qpack_q4g32_gate_up_size": ([i64, i64], sz),
            "qpack_q4g32_gate_up": ([p, p, p, p, p, p, i64, i64, p, sz], st),
            "qunpack_q4g32_gate_up": ([p, sz, i64, i64, p, p, p, p, p, p], st),
            "qgemv_grouped_q4g32_swiglu": ([p, i64, i32, p, i32, p, i64, p, i64, i64, i64, p], st),
            "qg_argmax_workspace_size": ([i64], sz),
            "qpack_q8g64_mma_size": ([i64, i64], sz),
            "qpack_q8g128_mma_size": ([i64, i64], sz),
            "qpack_q8pc_mma_size": ([i64, i64], sz),
            "qpack_q8g64_mma": ([p, p, i64, i64, p, sz], st),
            "qpack_q8g128_mma": ([p, p, i64, i64, p, sz], st),
            "qpack_q8pc_mma": ([p, p, i64, i64, p, sz], st),
            "qunpack_q8g64_mma": ([p, sz, i64, i64, p, p], st),
            "qunpack_q8g128_mma": ([p, sz, i64, i64, p, p], st),
            "qunpack_q8pc_mma": ([p, sz, i64, i64, p, p], st),
            "qgemv_q8g64_mma": ([p, p, p, i64, i64, i64, i64, i64, p], st),
            "qgemv_q8g128_mma": ([p, p, p, i64, i64, i64, i64, i64, p], st),
            "qgemv_q8pc_mma": ([p, p, p, i64, i64, i64, i64, i64, p], st),
            "qpack_q4g32_mma_size": ([i64, i64], sz),
            "qpack_q4g32_mma": ([p, p, p, i64, i64, p, sz], st),
            "qunpack_q4g32_mma": ([p, sz, i64, i64, p, p, p], st),
            "qgemv_q4g32_mma": ([p, p, p, i64, i64, i64, i64, i64, p], st),
            "qgemv_q8g64_argmax": ([p, p, p, p, i64, i64, i64, i64, i64, p, sz, p], st),
            "qgemv_q8g128_argmax": ([p, p, p, p, i64, i64, i64, i64, i64, p, sz, p], st),
            "qgemv_q8g64_argmax_noalloc": ([p, p, p, p, i64, i64, i64, i64, i64, p], st),
            "qg_argmax_f32": ([p, i64, i64, i64, p, p, sz, p], st),
            "qg_route_counts_reset": ([], None),
            "qg_route_count": ([ctypes.c_char_p], ctypes.c_uint64),
            "qg_variant_name": ([ctypes.c_int, i64, i64, i64, ctypes.c_char_p, sz], st),
            "qg_set_launch_override": ([i64, ctypes.c_int32, ctypes.c_int32], st),
            "qg_set_wave_trace": ([p, i64], st),
            "qg_wave_trace_state": ([p, p, p], st),
            "qg_read_stream": ([p, sz, p, ctypes.c_int32, p], st),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().qg_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != QG_OK:
        raise QGError(status, where)


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------- device-argument checks
# The C ABI sees only pointers, so a tensor on the wrong device, of the wrong
# element type or too short for the shape would be read or written out of
# bounds on the GPU.  Every torch-facing call below checks its tensors here
# first and raises QGError(QG_ERR_INVALID_ARG) instead of calling the library.

_W_DTYPES = ("uint8", "int8")
_X_DTYPES = ("bfloat16", "int16", "uint16")
_F32 = ("float32",)
_I32 = ("int32",)


def _extent(t) -> int:
    """Elements the view t spans from t.data_ptr(): one past its last element
    (for a row-strided view of m rows of K, (m - 1) * stride + K)."""
    if t.numel() == 0:
        return 0
    return 1 + sum((n - 1) * st for n, st in zip(t.shape, t.stride()))


def _need(t, where: str, what: str, dtypes, elems: int) -> None:
    """Element type and extent of one tensor (the device is checked by _on_gpu)."""
    dt = str(t.dtype).replace("torch.", "")
    if dt not in dtypes:
        raise QGError(QG_ERR_INVALID_ARG, "%s: %s has dtype %s, needs %s" % (where, what, dt, "/".join(dtypes)))
    if elems > 0 and _extent(t) < elems:
        raise QGError(QG_ERR_INVALID_ARG, "%s: %s holds %d elements from its start, the call reads or "
                      "writes %d" % (where, what, _extent(t), elems))


def _on_gpu(where: str, **tensors) -> None:
    for what, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise QGError(QG_ERR_INVALID_ARG, "%s: %s is not a GPU tensor" % (where, what))


_PACKED_SIZE = {
    "qgemv_q8g64": "qpack_q8g64_size", "qgemv_q4g32": "qpack_q4g32_size",
    "qgemv_q8g128": "qpack_q8g128_size", "qgemv_q8pc": "qpack_q8pc_size",
    "qgemv_q8g64_mma": "qpack_q8g64_mma_size", "qgemv_q8g128_mma": "qpack_q8g128_mma_size",
    "qgemv_q8pc_mma": "qpack_q8pc_mma_size", "qgemv_q4g32_mma": "qpack_q4g32_mma_size",
    "qgemv_q8g64_argmax": "qpack_q8g64_size", "qgemv_q8g128_argmax": "qpack_q8g128_size",
    "qgemv_q8g64_argmax_noalloc": "qpack_q8g64_size",
}


def _check_dense(fn_name, w_packed, x, y, m, N, K, ldx, ldy, idx_out=None):
    if m <= 0:
        return
    size = int(getattr(lib(), _PACKED_SIZE[fn_name])(N, K)) if N > 0 and K > 0 else 0
    _need(w_packed, fn_name, "w_packed", _W_DTYPES, size)
    _need(x, fn_name, "x", _X_DTYPES, (m - 1) * ldx + K)
    if y is not None:
        _need(y, fn_name, "y", _F32, (m - 1) * ldy + N)
    if idx_out is not None:
        _need(idx_out, fn_name, "idx_out", _I32, m)
    _on_gpu(fn_name, w_packed=w_packed, x=x, y=y, idx_out=idx_out)


def _check_grouped(fn_name, w, stride, n_experts, ids, n_slots, x, x_slot_stride, out, out_slot_stride,
                   N, K, out_dtypes, packed_size):
    if n_slots <= 0:
        return
    _need(w, fn_name, "w_experts", _W_DTYPES, (n_experts - 1) * stride + packed_size if n_experts > 0 else 0)
    _need(ids, fn_name, "expert_ids", _I32, n_slots)
    _need(x, fn_name, "x", _X_DTYPES, (n_slots - 1) * x_slot_stride + K)
    _need(out, fn_name, "y" if out_dtypes == _F32 else "act", out_dtypes, (n_slots - 1) * out_slot_stride + N)
    _on_gpu(fn_name, w_experts=w, expert_ids=ids, x=x, out=out)


def _stream_handle(stream):
    """A torch stream, a raw hipStream_t integer, or None for torch's current stream."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ packing

def qpack_q8g64_size(N: int, K: int) -> int:
    return int(lib().qpack_q8g64_size(N, K))


def qpack_q4g32_size(N: int, K: int) -> int:
    return int(lib().qpack_q4g32_size(N, K))


def _fp16_bits(a, where: str) -> np.ndarray:
    """fp16 scales or mins as their uint16 bit patterns: float16 arrays are
    reinterpreted, integer arrays taken as the bit patterns themselves, and
    other float arrays refused (converting them by value would pack wrong
    bits)."""
    a = np.asarray(a)
    if a.dtype == np.float16:
        return np.ascontiguousarray(a).view(np.uint16)
    if a.dtype.kind == "f":
        raise QGError(QG_ERR_INVALID_ARG, where + " (fp16 values must be float16 or uint16 bit patterns)")
    return np.ascontiguousarray(a, dtype=np.uint16)


def qpack_q8g64(q: np.ndarray, scales_f16: np.ndarray) -> np.ndarray:
    """Canonical q [N][K] int8 and scales [N][K/64] fp16 bits -> packed uint8 buffer."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = _fp16_bits(scales_f16, "qpack_q8g64")
    N, K = q.shape
    size = qpack_q8g64_size(N, K)
    if size == 0 or s.shape != (N, K // 64):
        raise QGError(QG_ERR_INVALID_ARG, "qpack_q8g64")
    out = np.empty(size, np.uint8)
    _check(lib().qpack_q8g64(_np_ptr(q), _np_ptr(s), N, K, _np_ptr(out), size), "qpack_q8g64")
    return out


def qunpack_q8g64(packed: np.ndarray, N: int, K: int):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    q = np.empty((N, K), np.int8)
    s = np.empty((N, K // 64), np.uint16)
    _check(lib().qunpack_q8g64(_np_ptr(packed), packed.nbytes, N, K, _np_ptr(q), _np_ptr(s)),
           "qunpack_q8g64")
    return q, s


def qpack_q8g128_size(N: int, K: int) -> int:
    return int(lib().qpack_q8g128_size(N, K))


def qpack_q8pc_size(N: int, K: int) -> int:
    return int(lib().qpack_q8pc_size(N, K))


def qpack_q8g128(q: np.ndarray, scales_f16: np.ndarray) -> np.ndarray:
    """Canonical q [N][K] int8 and scales [N][K/128] fp16 bits -> packed uint8 buffer."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = _fp16_bits(scales_f16, "qpack_q8g128")
    N, K = q.shape
    size = qpack_q8g128_size(N, K)
    if size == 0 or s.shape != (N, K // 128):
        raise QGError(QG_ERR_INVALID_ARG, "qpack_q8g128")
    out = np.empty(size, np.uint8)
    _check(lib().qpack_q8g128(_np_ptr(q), _np_ptr(s), N, K, _np_ptr(out), size), "qpack_q8g128")
    return out


def qunpack_q8g128(packed: np.ndarray, N: int, K: int):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    q = np.empty((N, K), np.int8)
    s = np.empty((N, K // 128), np.uint16)
    _check(lib().qunpack_q8g128(_np_ptr(packed), packed.nbytes, N, K, _np_ptr(q), _np_ptr(s)),
           "qunpack_q8g128")
    return q, s


def qpack_q8pc(q: np.ndarray, scales_f32: np.ndarray) -> np.ndarray:
    """Canonical q [N][K] int8 and one fp32 scale per row (float32 [N], or its
    bit patterns as uint32) -> packed uint8 buffer."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.asarray(scales_f32)
    s = np.ascontiguousarray(s, dtype=np.float32 if s.dtype.kind == "f" else np.uint32)
    N, K = q.shape
    size = qpack_q8pc_size(N, K)
    if size == 0 or s.shape != (N,):
        raise QGError(QG_ERR_INVALID_ARG, "qpack_q8pc")
    out = np.empty(size, np.uint8)
    _check(lib().qpack_q8pc(_np_ptr(q), _np_ptr(s), N, K, _np_ptr(out), size), "qpack_q8pc")
    return out


def qunpack_q8pc(packed: np.ndarray, N: int, K: int):
    """-> (q [N][K] int8, scales as fp32 bit patterns uint32 [N])."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    q = np.empty((N, K), np.int8)
    s = np.empty(N, np.uint32)
    _check(lib().qunpack_q8pc(_np_ptr(packed), packed.nbytes, N, K, _np_ptr(q), _np_ptr(s)),
           "qunpack_q8pc")
    return q, s


def qpack_q4g32(codes: np.ndarray, scales_f16: np.ndarray, mins_f16: np.ndarray) -> np.ndarray:
    """Canonical codes [N][K/2] (even k in the low nibble), scales and mins
    [N][K/32] fp16 bits -> packed uint8 buffer."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    s = _fp16_bits(scales_f16, "qpack_q4g32")
    mn = _fp16_bits(mins_f16, "qpack_q4g32")
    N, half_k = codes.shape
    K = 2 * half_k
    size = qpack_q4g32_size(N, K)
    if size == 0 or s.shape != (N, K // 32) or mn.shape != (N, K // 32):
        raise QGError(QG_ERR_INVALID_ARG, "qpack_q4g32")
    out = np.empty(size, np.uint8)
    _check(lib().qpack_q4g32(_np_ptr(codes), _np_ptr(s), _np_ptr(mn), N, K, _np_ptr(out), size),
           "qpack_q4g32")
    return out


def qunpack_q4g32(packed: np.ndarray, N: int, K: int):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    codes = np.empty((N, K // 2), np.uint8)
    s = np.empty((N, K // 32), np.uint16)
    mn = np.empty((N, K // 32), np.uint16)
    _check(lib().qunpack_q4g32(_np_ptr(packed), packed.nbytes, N, K, _np_ptr(codes), _np_ptr(s),
                               _np_ptr(mn)), "qunpack_q4g32")
    return codes, s, mn


def _mma_pack(fmt, q, scales, scale_dtype, scale_shape):
    q = np.ascontiguousarray(q, dtype=np.int8)
    if scale_dtype == np.uint16:
        s = _fp16_bits(scales, "qpack_%s_mma" % fmt)
    else:
        # Q8PC: float arrays by value (as float32), integer arrays as the
        # float32 bit patterns.
        s = np.asarray(scales)
        s = np.ascontiguousarray(s, dtype=np.float32 if s.dtype.kind == "f" else np.uint32)
    N, K = q.shape
    size = int(getattr(lib(), "qpack_%s_mma_size" % fmt)(N, K))
    if size == 0 or s.shape != scale_shape(N, K):
        raise QGError(QG_ERR_INVALID_ARG, "qpack_%s_mma" % fmt)
    out = np.empty(size, np.uint8)
    _check(getattr(lib(), "qpack_%s_mma" % fmt)(_np_ptr(q), _np_ptr(s), N, K, _np_ptr(out), size),
           "qpack_%s_mma" % fmt)
    return out


def qpack_q8g64_mma(q: np.ndarray, scales_f16: np.ndarray) -> np.ndarray:
    """Q8G64 weights in the matrix-core layout (for qgemv_q8g64_mma; K % 64 == 0)."""
    return _mma_pack("q8g64", q, scales_f16, np.uint16, lambda N, K: (N, K // 64))


def qpack_q8g128_mma(q: np.ndarray, scales_f16: np.ndarray) -> np.ndarray:
    """Q8G128 weights in the matrix-core layout (K % 128 == 0)."""
    return _mma_pack("q8g128", q, scales_f16, np.uint16, lambda N, K: (N, K // 128))


def qpack_q8pc_mma(q: np.ndarray, scales_f32: np.ndarray) -> np.ndarray:
    """Per-output-channel Q8 in the matrix-core layout (K % 64 == 0); scales
    float32 [N] or their uint32 bit patterns."""
    return _mma_pack("q8pc", q, scales_f32, np.uint32, lambda N, K: (N,))


def qpack_q4g32_mma(codes: np.ndarray, scales_f16: np.ndarray, mins_f16: np.ndarray) -> np.ndarray:
    """Q4G32 canonical arrays (as qpack_q4g32) in the matrix-core layout
    (for qgemv_q4g32_mma; K % 128 == 0)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    s = _fp16_bits(scales_f16, "qpack_q4g32_mma")
    mn = _fp16_bits(mins_f16, "qpack_q4g32_mma")
    N, half_k = codes.shape
    K = 2 * half_k
    size = qpack_mma_size("q4g32", N, K)
    if size == 0 or s.shape != (N, K // 32) or mn.shape != (N, K // 32):
        raise QGError(QG_ERR_INVALID_ARG, "qpack_q4g32_mma")
    out = np.empty(size, np.uint8)
    _check(lib().qpack_q4g32_mma(_np_ptr(codes), _np_ptr(s), _np_ptr(mn), N, K, _np_ptr(out), size),
           "qpack_q4g32_mma")
    return out


def qpack_mma_size(fmt: str, N: int, K: int) -> int:
    return int(getattr(lib(), "qpack_%s_mma_size" % fmt)(N, K))


def qunpack_mma(fmt: str, packed: np.ndarray, N: int, K: int):
    """-> (q int8 [N][K], scales) from a matrix-core buffer of format fmt
    ((codes, scales, mins) as qunpack_q4g32 for q4g32)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    if fmt == "q4g32":
        codes = np.empty((N, K // 2), np.uint8)
        sc = np.empty((N, K // 32), np.uint16)
        mn = np.empty((N, K // 32), np.uint16)
        _check(lib().qunpack_q4g32_mma(_np_ptr(packed), packed.nbytes, N, K, _np_ptr(codes), _np_ptr(sc),
                                       _np_ptr(mn)), "qunpack_q4g32_mma")
        return codes, sc, mn
    q = np.empty((N, K), np.int8)
    if fmt == "q8pc":
        s = np.empty(N, np.uint32)
    else:
        s = np.empty((N, K // (64 if fmt == "q8g64" else 128)), np.uint16)
    _check(getattr(lib(), "qunpack_%s_mma" % fmt)(_np_ptr(packed), packed.nbytes, N, K, _np_ptr(q),
                                                  _np_ptr(s)), "qunpack_%s_mma" % fmt)
    return q, s


def qpack_q4g32_gate_up_size(N: int, K: int) -> int:
    return int(lib().qpack_q4g32_gate_up_size(N, K))


def qpack_q4g32_gate_up(gate, up) -> np.ndarray:
    """gate and up: (codes [N][K/2], scales [N][K/32], mins [N][K/32]) of one
    expert's two projections -> one packed gate/up pair buffer (uint8) for
    qgemv_grouped_q4g32_swiglu."""
    g = [np.ascontiguousarray(a, dtype=t) for a, t in zip(gate, (np.uint8, np.uint16, np.uint16))]
    u = [np.ascontiguousarray(a, dtype=t) for a, t in zip(up, (np.uint8, np.uint16, np.uint16))]
    N, half_k = g[0].shape
    K = 2 * half_k
    size = qpack_q4g32_gate_up_size(N, K)
    shapes = [(N, half_k), (N, K // 32), (N, K // 32)]
    if size == 0 or [a.shape for a in g] != shapes or [a.shape for a in u] != shapes:
        raise QGError(QG_ERR_INVALID_ARG, "qpack_q4g32_gate_up")
    out = np.empty(size, np.uint8)
    _check(lib().qpack_q4g32_gate_up(*[_np_ptr(a) for a in g + u], N, K, _np_ptr(out), size),
           "qpack_q4g32_gate_up")
    return out


def qunpack_q4g32_gate_up(packed: np.ndarray, N: int, K: int):
    """-> (gate, up), each (codes, scales, mins) as qpack_q4g32_gate_up takes them."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    mats = [np.empty((N, K // 2), np.uint8), np.empty((N, K // 32), np.uint16),
            np.empty((N, K // 32), np.uint16), np.empty((N, K // 2), np.uint8),
            np.empty((N, K // 32), np.uint16), np.empty((N, K // 32), np.uint16)]
    _check(lib().qunpack_q4g32_gate_up(_np_ptr(packed), packed.nbytes, N, K,
                                       *[_np_ptr(a) for a in mats]), "qunpack_q4g32_gate_up")
    return tuple(mats[:3]), tuple(mats[3:])


# --------------------------------------------------------------------- GEMV

def _dense(fn_name, w_packed, x, y, N, K, m=None, ldx=None, ldy=None, stream=None, check=True):
    if m is None:
        m = 1 if x.dim() == 1 else x.shape[0]
    if ldx is None:
        ldx = x.stride(0) if x.dim() == 2 else K
    if ldy is None:
        ldy = y.stride(0) if y.dim() == 2 else N
    _check_dense(fn_name, w_packed, x, y, m, N, K, ldx, ldy)
    st = getattr(lib(), fn_name)(w_packed.data_ptr(), x.data_ptr(), y.data_ptr(), m, N, K, ldx, ldy,
                                 _stream_handle(stream))
    if check:
        _check(st, fn_name)
    return st


def qgemv_q8g64(w_packed, x, y, N: int, K: int, m=None, ldx=None, ldy=None, stream=None,
                check=True):
    """y[i*ldy + n] = sum_k W[n][k] x[i*ldx + k] with W packed Q8G64.

    w_packed: device uint8 tensor from qpack_q8g64; x: device bf16 (or 16-bit
    integer) tensor [m][>=K] or [K]; y: device float32 tensor [m][>=N] or [N].
    Enqueued on ``stream`` (default: torch's current stream); returns the
    status (raises on error when ``check``)."""
    return _dense("qgemv_q8g64", w_packed, x, y, N, K, m, ldx, ldy, stream, check)


def qgemv_q4g32(w_packed, x, y, N: int, K: int, m=None, ldx=None, ldy=None, stream=None,
                check=True):
    """As qgemv_q8g64 for Q4G32 weights packed by qpack_q4g32."""
    return _dense("qgemv_q4g32", w_packed, x, y, N, K, m, ldx, ldy, stream, check)


def qgemv_q8g128(w_packed, x, y, N: int, K: int, m=None, ldx=None, ldy=None, stream=None,
                 check=True):
    """As qgemv_q8g64 for Q8G128 weights packed by qpack_q8g128."""
    return _dense("qgemv_q8g128", w_packed, x, y, N, K, m, ldx, ldy, stream, check)


def qgemv_q8pc(w_packed, x, y, N: int, K: int, m=None, ldx=None, ldy=None, stream=None,
               check=True):
    """As qgemv_q8g64 for per-output-channel Q8 weights packed by qpack_q8pc."""
    return _dense("qgemv_q8pc", w_packed, x, y, N, K, m, ldx, ldy, stream, check)


def qgemv_q8g64_mma(w_packed, x, y, N: int, K: int, m=None, ldx=None, ldy=None, stream=None,
                    check=True):
    """Batched decode on the matrix cores, m = 2..16: as qgemv_q8g64 with W
    packed by qpack_q8g64_mma."""
    return _dense("qgemv_q8g64_mma", w_packed, x, y, N, K, m, ldx, ldy, stream, check)


def qgemv_q8g128_mma(w_packed, x, y, N: int, K: int, m=None, ldx=None, ldy=None, stream=None,
                     check=True):
    """As qgemv_q8g64_mma for qpack_q8g128_mma buffers."""
    return _dense("qgemv_q8g128_mma", w_packed, x, y, N, K, m, ldx, ldy, stream, check)


def qgemv_q4g32_mma(w_packed, x, y, N: int, K: int, m=None, ldx=None, ldy=None, stream=None,
                    check=True):
    """As qgemv_q8g64_mma for qpack_q4g32_mma buffers."""
    return _dense("qgemv_q4g32_mma", w_packed, x, y, N, K, m, ldx, ldy, stream, check)


def qgemv_q8pc_mma(w_packed, x, y, N: int, K: int, m=None, ldx=None, ldy=None, stream=None,
                   check=True):
    """As qgemv_q8g64_mma for qpack_q8pc_mma buffers."""
    return _dense("qgemv_q8pc_mma", w_packed, x, y, N, K, m, ldx, ldy, stream, check)


def qgemv_grouped_q4g32(w_experts, expert_stride_bytes: int, n_experts: int, expert_ids, x,
                        x_slot_stride: int, y, y_slot_stride: int, N: int, K: int,
                        n_slots=None, stream=None, check=True):
    """Routed-expert decode: y[j*y_slot_stride + n] = W_{ids[j]}[n] . x[j*x_slot_stride:].

    w_experts: device uint8 tensor holding n_experts packed matrices at
    expert_stride_bytes; expert_ids: device int32 tensor [n_slots]."""
    if n_slots is None:
        n_slots = expert_ids.numel()
    _check_grouped("qgemv_grouped_q4g32", w_experts, expert_stride_bytes, n_experts, expert_ids, n_slots,
                   x, x_slot_stride, y, y_slot_stride, N, K, _F32, qpack_q4g32_size(N, K))
    st = lib().qgemv_grouped_q4g32(w_experts.data_ptr(), expert_stride_bytes, n_experts,
                                   expert_ids.data_ptr(), n_slots, x.data_ptr(), x_slot_stride,
                                   y.data_ptr(), y_slot_stride, N, K, _stream_handle(stream))
    if check:
        _check(st, "qgemv_grouped_q4g32")
    return st


def qgemv_grouped_q4g32_swiglu(w_gate_up, expert_stride_bytes: int, n_experts: int, expert_ids,
                               x, x_slot_stride: int, act, act_slot_stride: int, N: int, K: int,
                               n_slots=None, stream=None, check=True):
    """Routed-expert gate+up with the SwiGLU epilogue:
    act[j*act_slot_stride + n] = bf16(silu(g[n]) * u[n]) with g, u the gate
    and up projections of expert ids[j] applied to x[j*x_slot_stride:].

    w_gate_up: device uint8 tensor of n_experts buffers from
    qpack_q4g32_gate_up at expert_stride_bytes; act: device 16-bit tensor."""
    if n_slots is None:
        n_slots = expert_ids.numel()
    _check_grouped("qgemv_grouped_q4g32_swiglu", w_gate_up, expert_stride_bytes, n_experts, expert_ids,
                   n_slots, x, x_slot_stride, act, act_slot_stride, N, K, _X_DTYPES,
                   qpack_q4g32_gate_up_size(N, K))
    st = lib().qgemv_grouped_q4g32_swiglu(w_gate_up.data_ptr(), expert_stride_bytes, n_experts,
                                          expert_ids.data_ptr(), n_slots, x.data_ptr(),
                                          x_slot_stride, act.data_ptr(), act_slot_stride, N, K,
                                          _stream_handle(stream))
    if check:
        _check(st, "qgemv_grouped_q4g32_swiglu")
    return st


def argmax_workspace_size(m: int) -> int:
    return int(lib().qg_argmax_workspace_size(m))


def argmax_f32(x, idx_out, workspace, N=None, m=None, ldx=None, stream=None, check=True):
    """Greedy choice per row of device fp32 logits x [m][>=N]: idx_out[i] =
    index of the largest value (lowest on ties, first NaN wins).

    idx_out: device int32 tensor [m]; workspace: device tensor of at least
    argmax_workspace_size(m) bytes, zero before the first call and left zero
    by every call."""
    if m is None:
        m = 1 if x.dim() == 1 else x.shape[0]
    if N is None:
        N = x.shape[-1]
    if ldx is None:
        ldx = x.stride(0) if x.dim() == 2 else N
    nbytes = workspace.numel() * workspace.element_size()
    _check_argmax(x, idx_out, workspace, m, N, ldx)
    st = lib().qg_argmax_f32(x.data_ptr(), m, N, ldx, idx_out.data_ptr(), workspace.data_ptr(),
                             nbytes, _stream_handle(stream))
    if check:
        _check(st, "qg_argmax_f32")
    return st


def _check_argmax(x, idx_out, workspace, m, N, ldx):
    if m <= 0:
        return
    _need(x, "qg_argmax_f32", "x", _F32, (m - 1) * ldx + N)
    _need(idx_out, "qg_argmax_f32", "idx_out", _I32, m)
    _on_gpu("qg_argmax_f32", x=x, idx_out=idx_out, workspace=workspace)


def _argmax_gemv_args(w_packed, x, logits, idx_out, workspace, N, K, m, ldx, ldy, stream,
                      fn_name="qgemv_q8g64_argmax"):
    if m is None:
        m = 1 if x.dim() == 1 else x.shape[0]
    if ldx is None:
        ldx = x.stride(0) if x.dim() == 2 else K
    if ldy is None:
        ldy = logits.stride(0) if logits is not None and logits.dim() == 2 else N
    _check_dense(fn_name, w_packed, x, logits, m, N, K, ldx, ldy, idx_out)
    _on_gpu(fn_name, workspace=workspace)
    nbytes = workspace.numel() * workspace.element_size()
    return (w_packed.data_ptr(), x.data_ptr(), None if logits is None else logits.data_ptr(),
            idx_out.data_ptr(), m, N, K, ldx, ldy, workspace.data_ptr(), nbytes,
            _stream_handle(stream))


def qgemv_q8g64_argmax(w_packed, x, logits, idx_out, workspace, N: int, K: int, m=None, ldx=None,
                       ldy=None, stream=None, check=True):
    """LM head and greedy choice in one launch: as qgemv_q8g64 (logits may be
    None to skip writing them) plus idx_out[i] = argmax of output row i.
    workspace: as argmax_f32 (argmax_workspace_size(m) bytes, zero before
    the first call, left zero by every call)."""
    st = lib().qgemv_q8g64_argmax(*_argmax_gemv_args(w_packed, x, logits, idx_out, workspace, N,
                                                      K, m, ldx, ldy, stream))
    if check:
        _check(st, "qgemv_q8g64_argmax")
    return st


def qgemv_q8g64_argmax_noalloc(w_packed, x, logits, idx_out, N: int, K: int, m=None, ldx=None,
                               ldy=None, stream=None, check=True):
    """As qgemv_q8g64_argmax with the library's own per-GPU scratch in place
    of a workspace (m = 1..4; calls that overlap on one GPU race)."""
    if m is None:
        m = 1 if x.dim() == 1 else x.shape[0]
    if ldx is None:
        ldx = x.stride(0) if x.dim() == 2 else K
    if ldy is None:
        ldy = logits.stride(0) if logits is not None and logits.dim() == 2 else N
    _check_dense("qgemv_q8g64_argmax_noalloc", w_packed, x, logits, m, N, K, ldx, ldy, idx_out)
    st = lib().qgemv_q8g64_argmax_noalloc(w_packed.data_ptr(), x.data_ptr(),
                                          None if logits is None else logits.data_ptr(),
                                          idx_out.data_ptr(), m, N, K, ldx, ldy, _stream_handle(stream))
    if check:
        _check(st, "qgemv_q8g64_argmax_noalloc")
    return st


def qgemv_q8g128_argmax(w_packed, x, logits, idx_out, workspace, N: int, K: int, m=None, ldx=None,
                        ldy=None, stream=None, check=True):
    """As qgemv_q8g64_argmax for Q8G128 weights."""
    st = lib().qgemv_q8g128_argmax(*_argmax_gemv_args(w_packed, x, logits, idx_out, workspace, N,
                                                       K, m, ldx, ldy, stream, "qgemv_q8g128_argmax"))
    if check:
        _check(st, "qgemv_q8g128_argmax")
    return st


# ------------------------------------------------------- prepared launches

class BoundCall:
    """One library call with its arguments marshalled once.

    It holds references to every tensor whose device address it passes, so
    the memory cannot be released (for example by torch's empty_cache, which
    graph capture runs) while the call can still be issued."""

    __slots__ = ("fn", "args", "name", "tensors")

    def __init__(self, fn, args, name, tensors):
        self.fn = fn
        self.args = args
        self.name = name
        self.tensors = tuple(tensors)

    def __call__(self):
        st = self.fn(*self.args)
        if st != QG_OK:
            raise QGError(st, self.name)


def bound_q8g64(w_packed, x, y, N: int, K: int, m: int = 1, ldx=None, ldy=None, stream=None):
    """Marshal the arguments of one qgemv_q8g64 call once; the returned
    BoundCall re-issues exactly that call (for decode loops that repeat the
    same launch, and for graph capture).  Each call checks the status."""
    return _bind("qgemv_q8g64", w_packed, x, y, N, K, m, ldx, ldy, stream)


def bound_q4g32(w_packed, x, y, N: int, K: int, m: int = 1, ldx=None, ldy=None, stream=None):
    """As bound_q8g64 for qgemv_q4g32."""
    return _bind("qgemv_q4g32", w_packed, x, y, N, K, m, ldx, ldy, stream)


def bound_q8g128(w_packed, x, y, N: int, K: int, m: int = 1, ldx=None, ldy=None, stream=None):
    """As bound_q8g64 for qgemv_q8g128."""
    return _bind("qgemv_q8g128", w_packed, x, y, N, K, m, ldx, ldy, stream)


def bound_q8pc(w_packed, x, y, N: int, K: int, m: int = 1, ldx=None, ldy=None, stream=None):
    """As bound_q8g64 for qgemv_q8pc."""
    return _bind("qgemv_q8pc", w_packed, x, y, N, K, m, ldx, ldy, stream)


def _bind(fn_name, w_packed, x, y, N, K, m, ldx, ldy, stream):
    ldx = K if ldx is None else ldx
    ldy = N if ldy is None else ldy
    _check_dense(fn_name, w_packed, x, y, m, N, K, ldx, ldy)
    args = (w_packed.data_ptr(), x.data_ptr(), y.data_ptr(), m, N, K, ldx, ldy,
            _stream_handle(stream))
    return BoundCall(getattr(lib(), fn_name), args, fn_name, (w_packed, x, y))


def bound_grouped_q4g32(w_experts, expert_stride_bytes: int, n_experts: int, expert_ids, x,
                        x_slot_stride: int, y, y_slot_stride: int, N: int, K: int,
                        n_slots=None, stream=None):
    """As bound_q8g64 for qgemv_grouped_q4g32."""
    if n_slots is None:
        n_slots = expert_ids.numel()
    _check_grouped("qgemv_grouped_q4g32", w_experts, expert_stride_bytes, n_experts, expert_ids, n_slots,
                   x, x_slot_stride, y, y_slot_stride, N, K, _F32, qpack_q4g32_size(N, K))
    args = (w_experts.data_ptr(), expert_stride_bytes, n_experts, expert_ids.data_ptr(), n_slots,
            x.data_ptr(), x_slot_stride, y.data_ptr(), y_slot_stride, N, K, _stream_handle(stream))
    return BoundCall(lib().qgemv_grouped_q4g32, args, "qgemv_grouped_q4g32",
                     (w_experts, expert_ids, x, y))


def bound_grouped_q4g32_swiglu(w_gate_up, expert_stride_bytes: int, n_experts: int, expert_ids,
                               x, x_slot_stride: int, act, act_slot_stride: int, N: int, K: int,
                               n_slots=None, stream=None):
    """As bound_q8g64 for qgemv_grouped_q4g32_swiglu."""
    if n_slots is None:
        n_slots = expert_ids.numel()
    _check_grouped("qgemv_grouped_q4g32_swiglu", w_gate_up, expert_stride_bytes, n_experts, expert_ids,
                   n_slots, x, x_slot_stride, act, act_slot_stride, N, K, _X_DTYPES,
                   qpack_q4g32_gate_up_size(N, K))
    args = (w_gate_up.data_ptr(), expert_stride_bytes, n_experts, expert_ids.data_ptr(), n_slots,
            x.data_ptr(), x_slot_stride, act.data_ptr(), act_slot_stride, N, K,
            _stream_handle(stream))
    return BoundCall(lib().qgemv_grouped_q4g32_swiglu, args, "qgemv_grouped_q4g32_swiglu",
                     (w_gate_up, expert_ids, x, act))


def bound_argmax_f32(x, idx_out, workspace, N: int, m: int = 1, ldx=None, stream=None):
    """As bound_q8g64 for qg_argmax_f32."""
    ldx = N if ldx is None else ldx
    nbytes = workspace.numel() * workspace.element_size()
    _check_argmax(x, idx_out, workspace, m, N, ldx)
    args = (x.data_ptr(), m, N, ldx, idx_out.data_ptr(), workspace.data_ptr(), nbytes,
            _stream_handle(stream))
    return BoundCall(lib().qg_argmax_f32, args, "qg_argmax_f32", (x, idx_out, workspace))


def bound_mma(fmt: str, w_packed, x, y, N: int, K: int, m: int = 1, ldx=None, ldy=None, stream=None):
    """As bound_q8g64 for qgemv_<fmt>_mma."""
    return _bind("qgemv_%s_mma" % fmt, w_packed, x, y, N, K, m, ldx, ldy, stream)


def bound_q8g64_argmax(w_packed, x, logits, idx_out, workspace, N: int, K: int, m: int = 1,
                       ldx=None, ldy=None, stream=None):
    """As bound_q8g64 for qgemv_q8g64_argmax (logits may be None)."""
    args = _argmax_gemv_args(w_packed, x, logits, idx_out, workspace, N, K, m, ldx, ldy, stream)
    keep = [t for t in (w_packed, x, logits, idx_out, workspace) if t is not None]
    return BoundCall(lib().qgemv_q8g64_argmax, args, "qgemv_q8g64_argmax", keep)


# --------------------------------------------------------------- test hooks

def route_counts_reset() -> None:
    lib().qg_route_counts_reset()


def route_count(variant: str) -> int:
    return int(lib().qg_route_count(variant.encode()))


def variant_name(fmt: int, m: int, N: int, K: int) -> str:
    buf = ctypes.create_string_buffer(64)
    _check(lib().qg_variant_name(fmt, m, N, K, buf, 64), "qg_variant_name")
    return buf.value.decode()


def read_stream(buf, sink, nbytes=None, waves_per_cu: int = 0, stream=None) -> None:
    """qg_read_stream over the first nbytes (default: all) of device tensor buf."""
    nbytes = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check(lib().qg_read_stream(buf.data_ptr(), nbytes, sink.data_ptr(), waves_per_cu,
                                _stream_handle(stream)), "qg_read_stream")


def set_launch_override(target_waves: int = 0, contig: int = -1, ring_depth: int = 0) -> None:
    """qg_set_launch_override; call with no arguments to restore the defaults."""
    _check(lib().qg_set_launch_override(target_waves, contig, ring_depth), "qg_set_launch_override")


_trace_records = None   # the traced buffer, held while the library may write it


def set_wave_trace(records=None) -> None:
    """qg_set_wave_trace over a device tensor of whole 64-byte records (eight
    int64 each); None turns tracing off.  The tensor is held here until the
    next call."""
    global _trace_records
    if records is None:
        _check(lib().qg_set_wave_trace(None, 0), "qg_set_wave_trace")
        _trace_records = None
        return
    nbytes = records.numel() * records.element_size()
    _on_gpu("qg_set_wave_trace", records=records)
    if not records.is_contiguous() or nbytes < 64:
        raise QGError(QG_ERR_INVALID_ARG, "qg_set_wave_trace: need a contiguous buffer of >= 64 bytes")
    _check(lib().qg_set_wave_trace(records.data_ptr(), nbytes // 64), "qg_set_wave_trace")
    _trace_records = records


def wave_trace_state():
    """(records reserved, launches traced, launches dropped) since the buffer was set."""
    vals = [ctypes.c_int64(0) for _ in range(3)]
    _check(lib().qg_wave_trace_state(*[ctypes.byref(v) for v in vals]), "qg_wave_trace_state")
    return tuple(int(v.value) for v in vals)


def expert_stride(N: int, K: int) -> int:
    """Smallest valid expert stride (packed size is already a multiple of 256)."""
    return qpack_q4g32_size(N, K)


def gate_up_expert_stride(N: int, K: int) -> int:
    """Smallest valid expert stride for gate/up pair buffers."""
    return qpack_q4g32_gate_up_size(N, K)
