"""CPU oracle for the block-quantized decode GEMV — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and it imports nothing from the product.

The GEMV arithmetic lives in ``oracle.c`` (plain C, fp64 decode and fp64
accumulation in ascending k).  This module marshals numpy arrays into it,
splits output rows across threads when asked (each thread runs the same
plain loop on its own rows, so the result does not depend on the split),
loops over expert slots for the routed-expert case, and applies the SwiGLU
activation (elementwise fp64 numpy, ``silu`` / ``swiglu`` below) to the
GEMV results for the fused gate+up call.  The routed-expert MLP rounds that
activation to bf16 (``bf16_round``) before the down projection.  The greedy
argmax over logits is a plain left-to-right scan in ``oracle.c``.

Every function is pinned by ``tests/test_oracle_pins.py``,
``tests/test_oracle_swiglu.py``, ``tests/test_oracle_argmax.py`` and
``tests/test_oracle_mlp.py``; ``tests/test_oracle_mutations.py`` plants
mistakes in a copy of ``oracle.c`` and checks that the pins catch them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math); also when
    the source is newer than the built library."""
    stale = not os.path.exists(_LIB) or os.path.getmtime(_SRC) > os.path.getmtime(_LIB)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c99",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out_path: str, clang: str = "/opt/rocm/llvm/bin/clang") -> str:
    """oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer, linked
    against clang's shared ASan runtime (for the host-sanitizer CPU tests,
    which load it through ORACLE_LIBRARY)."""
    cmd = [clang, "-O1", "-g", "-fPIC", "-shared", "-std=c99", "-fno-fast-math",
           "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-shared-libasan",
           "-o", out_path, _SRC, "-lm"]
    subprocess.check_call(cmd)
    return out_path


def _load():
    global _lib
    if _lib is None:
        # ORACLE_LIBRARY names another build of oracle.c (the host-sanitizer
        # build of the CPU tests).
        lib = ctypes.CDLL(os.environ.get("ORACLE_LIBRARY") or build())
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_q8g64.argtypes = [p, p, i64, i64, p, i64, i64, i64, i64, p, p, i64]
        lib.oracle_q8g64.restype = ctypes.c_int
        lib.oracle_q4g32.argtypes = [p, p, p, i64, i64, p, i64, i64, i64, i64, p, p, i64]
        lib.oracle_q4g32.restype = ctypes.c_int
        lib.oracle_q8g128.argtypes = [p, p, i64, i64, p, i64, i64, i64, i64, p, p, i64]
        lib.oracle_q8g128.restype = ctypes.c_int
        lib.oracle_q8pc.argtypes = [p, p, i64, i64, p, i64, i64, i64, i64, p, p, i64]
        lib.oracle_q8pc.restype = ctypes.c_int
        lib.oracle_f32_to_double.argtypes = [ctypes.c_uint32]
        lib.oracle_f32_to_double.restype = ctypes.c_double
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_argmax_f32.argtypes = [p, i64, i64, i64, p]
        lib.oracle_argmax_f32.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def half_to_double(bits: int) -> float:
    return _load().oracle_half_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(int(bits))


def f32_to_double(bits: int) -> float:
    return _load().oracle_f32_to_double(int(bits))


def _row_splits(N: int, threads: int):
    threads = max(1, min(int(threads), N if N > 0 else 1))
    edges = [N * t // threads for t in range(threads + 1)]
    return [(edges[t], edges[t + 1]) for t in range(threads)]


def _check_x(x: np.ndarray, K: int):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    if x.ndim == 1:
        x = x[None, :]
    if x.shape[1] < K:
        raise ValueError("x rows shorter than K")
    return x


def q8g64(q: np.ndarray, scale: np.ndarray, x: np.ndarray, threads: int = 1):
    """y, a = oracle Q8G64 GEMV.

    q [N][K] int8, scale [N][K/64] uint16 (fp16 bits), x [m][>=K] uint16
    (bf16 bits).  Returns (y, a), each float64 [m][N]."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    scale = np.ascontiguousarray(scale, dtype=np.uint16)
    N, K = q.shape
    if K % 64 or scale.shape != (N, K // 64):
        raise ValueError("bad Q8G64 shapes")
    x = _check_x(x, K)
    m, ldx = x.shape
    y = np.zeros((m, N), np.float64)
    a = np.zeros((m, N), np.float64)
    lib = _load()

    def run(rng):
        rc = lib.oracle_q8g64(_ptr(q), _ptr(scale), N, K, _ptr(x), m, ldx,
                              rng[0], rng[1], _ptr(y), _ptr(a), N)
        if rc != 0:
            raise RuntimeError("oracle_q8g64 failed")

    splits = _row_splits(N, threads)
    if len(splits) == 1:
        run(splits[0])
    else:
        with ThreadPoolExecutor(len(splits)) as ex:
            list(ex.map(run, splits))
    return y, a


def _q8_generic(fn_name, q, scale, x, threads, scale_dtype, scale_shape):
    q = np.ascontiguousarray(q, dtype=np.int8)
    scale = np.ascontiguousarray(scale, dtype=scale_dtype)
    N, K = q.shape
    if scale.shape != scale_shape(N, K):
        raise ValueError("bad scale shape for " + fn_name)
    x = _check_x(x, K)
    m, ldx = x.shape
    y = np.zeros((m, N), np.float64)
    a = np.zeros((m, N), np.float64)
    fn = getattr(_load(), fn_name)

    def run(rng):
        if fn(_ptr(q), _ptr(scale), N, K, _ptr(x), m, ldx, rng[0], rng[1], _ptr(y), _ptr(a), N) != 0:
            raise RuntimeError(fn_name + " failed")

    splits = _row_splits(N, threads)
    if len(splits) == 1:
        run(splits[0])
    else:
        with ThreadPoolExecutor(len(splits)) as ex:
            list(ex.map(run, splits))
    return y, a


def q8g128(q: np.ndarray, scale: np.ndarray, x: np.ndarray, threads: int = 1):
    """Q8G128: q [N][K] int8, scale [N][K/128] fp16 bits, x [m][>=K] bf16 bits."""
    if q.shape[1] % 128:
        raise ValueError("K must be a multiple of 128")
    return _q8_generic("oracle_q8g128", q, scale, x, threads, np.uint16,
                       lambda N, K: (N, K // 128))


def q8pc(q: np.ndarray, scale_f32: np.ndarray, x: np.ndarray, threads: int = 1):
    """Q8 per output channel: q [N][K] int8, scale [N] fp32 bit patterns (uint32)
    or float32 values (taken bit for bit, never converted)."""
    scale_f32 = np.asarray(scale_f32)
    if scale_f32.dtype == np.float32:
        scale_f32 = scale_f32.view(np.uint32)
    return _q8_generic("oracle_q8pc", q, scale_f32, x, threads, np.uint32, lambda N, K: (N,))


def q4g32(codes: np.ndarray, scale: np.ndarray, minv: np.ndarray, x: np.ndarray,
          threads: int = 1):
    """y, a = oracle Q4G32 GEMV.

    codes [N][K/2] uint8 (even k in the low nibble), scale/minv [N][K/32]
    uint16 (fp16 bits), x [m][>=K] uint16 (bf16 bits)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.uint16)
    minv = np.ascontiguousarray(minv, dtype=np.uint16)
    N, half_k = codes.shape
    K = 2 * half_k
    if K % 32 or scale.shape != (N, K // 32) or minv.shape != (N, K // 32):
        raise ValueError("bad Q4G32 shapes")
    x = _check_x(x, K)
    m, ldx = x.shape
    y = np.zeros((m, N), np.float64)
    a = np.zeros((m, N), np.float64)
    lib = _load()

    def run(rng):
        rc = lib.oracle_q4g32(_ptr(codes), _ptr(scale), _ptr(minv), N, K, _ptr(x),
                              m, ldx, rng[0], rng[1], _ptr(y), _ptr(a), N)
        if rc != 0:
            raise RuntimeError("oracle_q4g32 failed")

    splits = _row_splits(N, threads)
    if len(splits) == 1:
        run(splits[0])
    else:
        with ThreadPoolExecutor(len(splits)) as ex:
            list(ex.map(run, splits))
    return y, a


def grouped_q4g32(experts, ids, x_slots, threads: int = 1):
    """Routed-expert decode: slot j uses expert ids[j] and its own x row.

    experts: sequence of (codes, scale, minv) canonical arrays, one per expert
    ids:     expert index per slot
    x_slots: [n_slots][>=K] bf16 bits (row j is slot j's activation)
    Returns (y, a), each float64 [n_slots][N]; each slot is computed and
    written separately, with no weighting across slots."""
    x_slots = np.ascontiguousarray(x_slots, dtype=np.uint16)
    ys, as_ = [], []
    for j, e in enumerate(ids):
        codes, scale, minv = experts[int(e)]
        y, a = q4g32(codes, scale, minv, x_slots[j:j + 1], threads=threads)
        ys.append(y[0])
        as_.append(a[0])
    return np.stack(ys), np.stack(as_)


def within_tolerance(y_test, y_ref, a_ref, rel: float = 2e-3):
    """The acceptance test: |y - y_ref| <= rel * sum_k |w x| per output,
    evaluated in fp64; y must be finite.  Returns a boolean mask."""
    y_test = np.asarray(y_test, np.float64)
    return np.isfinite(y_test) & (np.abs(y_test - y_ref) <= rel * a_ref)


# ------------------------------------------------------------------ argmax

def argmax_f32(x) -> np.ndarray:
    """Greedy choice per row of fp32 logits x [m][>=N] (float32 values or
    their uint32 bit patterns; rows of length N = x.shape[1]): the index of
    the largest value, the lowest index on ties, -0 == +0, and the first NaN
    of a row if it has one.  Returns int64 [m]."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        x = x.view(np.uint32)
    x = np.ascontiguousarray(x, dtype=np.uint32)
    if x.ndim == 1:
        x = x[None, :]
    m, N = x.shape
    out = np.zeros(m, np.int64)
    if m and _load().oracle_argmax_f32(_ptr(x), m, N, N, _ptr(out)) != 0:
        raise ValueError("bad argmax shape")
    return out


# ------------------------------------------------------------------ SwiGLU
#
# The merged gate+up projection of a routed expert is followed by SwiGLU,
# act = silu(gate) * up, which becomes the down projection's input (Qwen3
# C++ Reference Runtime (MetaInfer-cpp) README, milestone M6.5-D; the
# SiluAndMul step after the merged gate_up GEMM in the commit log of
# vllm.cpp pull request #1936).  Neither page spells out SiLU; the reading
# taken is the standard one, silu(z) = z * sigmoid(z) = z / (1 + e^-z).

# Upper bound of |silu'(z)| over all real z.  silu'(z) = s (1 + z (1 - s))
# with s = sigmoid(z) peaks at z ~= 2.3994 with value ~= 1.09984.
SILU_SLOPE_BOUND = 1.0999


def silu(z):
    """silu(z) = z / (1 + exp(-z)) in fp64, written so that exp never
    overflows: for z < 0 it is z e^z / (1 + e^z)."""
    z = np.asarray(z, np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def swiglu(gate, up):
    """act = silu(gate) * up, elementwise, fp64."""
    return silu(gate) * np.asarray(up, np.float64)


def grouped_q4g32_swiglu(gate_experts, up_experts, ids, x_slots, threads: int = 1):
    """Routed-expert gate+up with SwiGLU: for slot j with e = ids[j],
    g = Gate_e x_j and u = Up_e x_j (the Q4G32 GEMV above), act = swiglu(g, u).

    Returns (act, g, u, a_g, a_u), each float64 [n_slots][N]; a_g and a_u are
    the sum_k |w x| of the two GEMVs (their tolerance scale)."""
    g, a_g = grouped_q4g32(gate_experts, ids, x_slots, threads=threads)
    u, a_u = grouped_q4g32(up_experts, ids, x_slots, threads=threads)
    return swiglu(g, u), g, u, a_g, a_u


def swiglu_propagated_bound(g, u, a_g, a_u, rel: float = 2e-3):
    """How far silu(g') u' can move from silu(g) u when the fp32 gate/up sums
    each meet the GEMV bar (|g' - g| <= rel a_g, |u' - u| <= rel a_u).

    By the mean value theorem, with dg = rel a_g and du = rel a_u,
      |silu(g')u' - silu(g)u| <= B |u'| dg + |silu(g)| du
                               <= B dg (|u| + du) + |silu(g)| du =: E
    with B = SILU_SLOPE_BOUND."""
    dg = rel * np.asarray(a_g, np.float64)
    du = rel * np.asarray(a_u, np.float64)
    return SILU_SLOPE_BOUND * dg * (np.abs(u) + du) + np.abs(silu(g)) * du


def swiglu_tolerance(act_ref, g, u, a_g, a_u, rel: float = 2e-3):
    """Per-output bound on |act_test - act_ref| for a bf16 SwiGLU output built
    from fp32 gate/up sums that each meet the GEMV bar.

    The kernel forms t = silu(g') u' in fp32 (relative error below 2^-20 for
    the exp, add, divide and multiply) and rounds t to bf16 (8 significant
    bits: relative error up to 2^-8).  With E the propagated bound above,
      |act - act_ref| <= E + 2^-20 |a'| + 2^-8 |t|
                      <= (1 + 2^-7) E + (2^-8 + 2^-19) |act_ref|.
    Results below the smallest normal bf16 may come out as zero (an fp32 exp
    that overflows for very negative g), so 2^-126 is added."""
    E = swiglu_propagated_bound(g, u, a_g, a_u, rel)
    return (1.0 + 2.0 ** -7) * E + (2.0 ** -8 + 2.0 ** -19) * np.abs(act_ref) + 2.0 ** -126


# ------------------------------------------------------- routed-expert MLP
#
# The SwiGLU output is written as the down projection's bf16 input (Qwen3
# C++ Reference Runtime (MetaInfer-cpp) README, milestone M6.5-D: the packed
# Gate/Up GEMM and SwiGLU write the down projection's input), so the MLP of
# one routed expert is y = Down_e bf16(silu(Gate_e x) * (Up_e x)).  The pages
# do not say how that input is rounded; the reading taken is IEEE
# round-to-nearest-even, the rounding of every other bf16 value here.

def _bf16_quantum_exp(v):
    # bf16 keeps 8 significant bits over binary32's exponent range: a value
    # m 2^e (0.5 <= |m| < 1) is a multiple of 2^(e-8) when normal
    # (e >= -125), and of 2^-133 below that.
    _, e = np.frexp(v)
    return np.maximum(e, -125) - 8


def _bf16_bits_of_exact(val):
    # val holds bf16-representable fp64 values (or +-inf, NaN).
    out = (val.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out[np.isnan(val)] = 0x7FC0
    return out


def bf16_round(v) -> np.ndarray:
    """fp64 values -> bf16 bit patterns, rounded to nearest with ties to
    even (8 significant bits, binary32 exponent range); past the largest
    finite bf16 the result is +-inf, NaN gives 0x7FC0."""
    v = np.asarray(v, np.float64)
    q = _bf16_quantum_exp(v)
    with np.errstate(invalid="ignore", over="ignore"):
        # Scaling by a power of two is exact; rint rounds half to even.
        val = np.ldexp(np.rint(np.ldexp(v, -q)), q)
        val = np.where(np.abs(val) >= 2.0 ** 128, np.copysign(np.inf, v), val)
    return _bf16_bits_of_exact(np.where(np.isfinite(v), val, v))


def bf16_round_up_abs(v) -> np.ndarray:
    """The smallest bf16 >= |v| for finite fp64 v (bit patterns), for bounds
    that a bf16-input GEMV evaluates."""
    v = np.abs(np.asarray(v, np.float64))
    if not np.all(np.isfinite(v)):
        raise ValueError("bf16_round_up_abs needs finite values")
    q = _bf16_quantum_exp(v)
    with np.errstate(over="ignore"):
        val = np.ldexp(np.ceil(np.ldexp(v, -q)), q)
    return _bf16_bits_of_exact(val)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values (vectorised)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


class MlpRef:
    """Reference values of the routed-expert MLP, each float64 [n_slots][.]:
    act (fp64 silu(g) u), act_bits (its bf16 rounding, the down projection's
    input), y (Down act_bits), a_y (sum |w act_bits| of the down GEMV), and
    the gate/up sums g, u with their sum |w x| a_g, a_u."""

    def __init__(self, act, act_bits, y, a_y, g, u, a_g, a_u):
        self.act, self.act_bits, self.y, self.a_y = act, act_bits, y, a_y
        self.g, self.u, self.a_g, self.a_u = g, u, a_g, a_u


def expert_mlp(gate_experts, up_experts, down_experts, ids, x_slots, threads: int = 1) -> MlpRef:
    """Routed-expert MLP: for slot j with e = ids[j],
      act_j = silu(Gate_e x_j) * (Up_e x_j)      (grouped_q4g32_swiglu)
      y_j   = Down_e bf16(act_j)                 (grouped_q4g32)."""
    act, g, u, a_g, a_u = grouped_q4g32_swiglu(gate_experts, up_experts, ids, x_slots,
                                               threads=threads)
    act_bits = bf16_round(act)
    y, a_y = grouped_q4g32(down_experts, ids, act_bits, threads=threads)
    return MlpRef(act, act_bits, y, a_y, g, u, a_g, a_u)


def expert_mlp_tolerance(ref: MlpRef, down_experts, ids, rel: float = 2e-3, threads: int = 1):
    """Per-output bounds (tol_act, tol_y) for an MLP whose gate/up sums and
    down sums each meet the GEMV bar (rel sum |w x| of their own inputs).

    tol_act is swiglu_tolerance.  For y: a kernel's bf16 activation a_k is
    within tol_act of act, so |a_k - a_r| <= d := tol_act + |act - a_r| with
    a_r = bf16(act).  The down GEMV meets the bar on a_k:
      |y_k - Down a_k| <= rel sum |w| |a_k| <= rel (a_y + sum |w| d),
    and |Down a_k - Down a_r| <= sum |w| d, so
      |y_k - y| <= rel a_y + (1 + rel) sum |w| d.
    sum |w| d is taken from the oracle GEMV's sum |w x| with d rounded up to
    bf16, which only enlarges it."""
    tol_act = swiglu_tolerance(ref.act, ref.g, ref.u, ref.a_g, ref.a_u, rel)
    d = tol_act + np.abs(ref.act - bf16_to_f64(ref.act_bits))
    _, wd = grouped_q4g32(down_experts, ids, bf16_round_up_abs(d), threads=threads)
    return tol_act, rel * ref.a_y + (1.0 + rel) * wd
