"""Host-side tests of the C-ABI library (no GPU needed).

* every function declared in include/qgemv.h is exported by libqgemv.so
* qpack/qunpack round-trip byte for byte, are deterministic, and use the
  documented sizes (every weight byte once, plus tail-tile padding)
* argument validation returns its status before anything is enqueued:
  only calls that must be rejected are made here, with fake device
  addresses that are never dereferenced
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from weight_only_block_amd import qgemv as Q
from weight_only_block_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "qgemv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    keywords = {"if", "sizeof", "defined"}
    return sorted({n for n in names if n not in keywords})


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert "qgemv_q8g64" in names and "qgemv_grouped_q4g32" in names
    out = subprocess.check_output(["nm", "-D", "--defined-only", Q.LIB_PATH]).decode()
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = Q.lib()
    for n in names:
        assert getattr(lib, n) is not None


def test_version_and_status_strings():
    assert Q.lib().qg_abi_version() == 2
    for s in range(5):
        assert Q.status_string(s)
    assert Q.status_string(99) == "unknown status"


@pytest.mark.parametrize("N,K", [(1, 64), (7, 192), (129, 64), (1024, 1024), (3, 2560), (33, 3072)])
def test_q8_pack_roundtrip(N, K):
    rng = synth.rng_for(7, N, K)
    q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    s = rng.integers(0, 65536, size=(N, K // 64), dtype=np.uint16)
    packed = Q.qpack_q8g64(q, s)
    assert packed.nbytes == Q.qpack_q8g64_size(N, K)
    assert packed.nbytes % 256 == 0
    q2, s2 = Q.qunpack_q8g64(packed, N, K)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    assert np.array_equal(packed, Q.qpack_q8g64(q, s))      # deterministic


@pytest.mark.parametrize("N,K", [(1, 128), (7, 384), (129, 128), (3, 2560), (33, 5120)])
def test_q8g128_pack_roundtrip(N, K):
    rng = synth.rng_for(9, N, K)
    q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    s = rng.integers(0, 65536, size=(N, K // 128), dtype=np.uint16)
    packed = Q.qpack_q8g128(q, s)
    assert packed.nbytes == Q.qpack_q8g128_size(N, K)
    q2, s2 = Q.qunpack_q8g128(packed, N, K)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


@pytest.mark.parametrize("N,K", [(1, 16), (7, 48), (129, 16), (5, 4352), (33, 1280), (2, 5120)])
def test_q8pc_pack_roundtrip(N, K):
    rng = synth.rng_for(10, N, K)
    q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    s = rng.integers(0, 2**32, size=N, dtype=np.uint64).astype(np.uint32)
    packed = Q.qpack_q8pc(q, s)
    assert packed.nbytes == Q.qpack_q8pc_size(N, K)
    q2, s2 = Q.qunpack_q8pc(packed, N, K)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


@pytest.mark.parametrize("N,K", [(1, 32), (7, 96), (129, 32), (5, 1536), (9, 9216), (33, 2560)])
def test_q4_pack_roundtrip(N, K):
    rng = synth.rng_for(8, N, K)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = rng.integers(0, 65536, size=(N, K // 32), dtype=np.uint16)
    mn = rng.integers(0, 65536, size=(N, K // 32), dtype=np.uint16)
    packed = Q.qpack_q4g32(codes, s, mn)
    assert packed.nbytes == Q.qpack_q4g32_size(N, K)
    c2, s2, mn2 = Q.qunpack_q4g32(packed, N, K)
    assert np.array_equal(codes, c2) and np.array_equal(s, s2) and np.array_equal(mn, mn2)


def test_packed_size_is_algorithmic_bytes_plus_tail_padding():
    # lm_head: N = 151936 is a whole number of tiles, so no padding at all.
    N, K = 151936, 2560
    assert Q.qpack_q8g64_size(N, K) == synth.bytes_q8g64(N, K)
    for (N, K) in [(9216, 2560), (2560, 9216), (1536, 4096), (4096, 1536)]:
        assert Q.qpack_q4g32_size(N, K) == synth.bytes_q4g32(N, K)
    for (N, K) in [(2048, 1024), (1024, 2048), (3072, 1024), (1024, 3072)]:
        assert Q.qpack_q8g64_size(N, K) == synth.bytes_q8g64(N, K)
    assert Q.qpack_q8g128_size(151936, 2560) == synth.bytes_q8g128(151936, 2560)
    for (_, _, N, K) in synth.W8A16_QWEN3_14B_TP4:
        assert Q.qpack_q8pc_size(N, K) == synth.bytes_q8pc(N, K)
    # ragged N: at most one partial tile of padding, rounded to 256 bytes
    for N in (1, 7, 129, 1000):
        per_row = synth.bytes_q8g64(1, 1024)
        size = Q.qpack_q8g64_size(N, 1024)
        assert synth.bytes_q8g64(N, 1024) <= size <= per_row * (N + 128) + 256


def test_invalid_shapes_have_no_packed_size():
    assert Q.qpack_q8g64_size(0, 64) == 0
    assert Q.qpack_q8g64_size(4, 32) == 0      # not a whole 64-group
    assert Q.qpack_q8g64_size(4, 0) == 0
    assert Q.qpack_q4g32_size(4, 48) == 0      # not a whole 32-group
    assert Q.qpack_q4g32_size(-1, 32) == 0
    assert Q.qpack_q4g32_size(1 << 31, 32) == 0
    assert Q.qpack_q8g128_size(4, 64) == 0    # not a whole 128-group
    assert Q.qpack_q8pc_size(4, 24) == 0      # not a multiple of 16


def test_qpack_rejects_short_output_and_nulls():
    L = Q.lib()
    q = np.zeros((4, 64), np.int8)
    s = np.zeros((4, 1), np.uint16)
    out = np.zeros(Q.qpack_q8g64_size(4, 64), np.uint8)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert L.qpack_q8g64(p(q), p(s), 4, 64, p(out), out.nbytes - 1) == Q.QG_ERR_INVALID_ARG
    assert L.qpack_q8g64(None, p(s), 4, 64, p(out), out.nbytes) == Q.QG_ERR_INVALID_ARG
    assert L.qpack_q8g64(p(q), p(s), 4, 64, p(out), out.nbytes) == Q.QG_OK


# Fake device addresses: the library must reject each call below before it
# dereferences or launches anything.
W, X, Y, IDS = 1 << 20, 1 << 21, 1 << 22, 1 << 23


# (entry point, K granularity).  Every call below must fail validation: a
# call that passed would launch a kernel on the fake addresses.
DENSE = [("qgemv_q8g64", 64), ("qgemv_q4g32", 32), ("qgemv_q8g128", 128), ("qgemv_q8pc", 16)]


@pytest.mark.parametrize("fn,group", DENSE)
def test_dense_validation(fn, group):
    f = getattr(Q.lib(), fn)
    K = 128
    ragged = K + group // 2                    # not a whole number of groups
    assert f(None, X, Y, 1, 16, K, K, 16, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, None, Y, 1, 16, K, K, 16, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, X, None, 1, 16, K, K, 16, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, X, Y, 5, 16, K, K, 16, None) == Q.QG_ERR_UNSUPPORTED          # m gate
    assert f(W, X, Y, -1, 16, K, K, 16, None) == Q.QG_ERR_UNSUPPORTED
    assert f(W, X, Y, 1, 0, K, K, 16, None) == Q.QG_ERR_INVALID_ARG           # N < 1
    assert f(W, X, Y, 1, 16, 0, K, 16, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, X, Y, 1, 16, ragged, ragged, 16, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, X, Y, 2, 16, K, K - 2, 16, None) == Q.QG_ERR_INVALID_ARG      # ldx < K
    assert f(W, X, Y, 2, 16, K, K, 15, None) == Q.QG_ERR_INVALID_ARG          # ldy < N
    assert f(W + 16, X, Y, 1, 16, K, K, 16, None) == Q.QG_ERR_ALIGNMENT
    assert f(W, X + 2, Y, 1, 16, K, K, 16, None) == Q.QG_ERR_ALIGNMENT
    assert f(W, X, Y + 2, 1, 16, K, K, 16, None) == Q.QG_ERR_ALIGNMENT
    assert f(W, X, Y, 2, 16, K, K + 1, 16, None) == Q.QG_ERR_ALIGNMENT        # odd ldx
    assert f(W, X, Y, 4, 16, 32768, 32768, 16, None) == Q.QG_ERR_UNSUPPORTED  # LDS limit
    assert f(W, X, Y, 0, 16, K, K, 16, None) == Q.QG_OK                       # empty batch


def test_grouped_validation():
    f = Q.lib().qgemv_grouped_q4g32
    N, K = 64, 128
    stride = Q.qpack_q4g32_size(N, K)
    ok = dict(w=W, st=stride, ne=4, ids=IDS, ns=2, x=X, xs=0, y=Y, ys=N, N=N, K=K)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["w"], a["st"], a["ne"], a["ids"], a["ns"], a["x"], a["xs"], a["y"], a["ys"],
                 a["N"], a["K"], None)

    assert call(ids=None) == Q.QG_ERR_INVALID_ARG
    assert call(ns=65) == Q.QG_ERR_UNSUPPORTED
    assert call(ns=0) == Q.QG_OK
    assert call(ne=0) == Q.QG_ERR_INVALID_ARG
    assert call(st=stride - 256) == Q.QG_ERR_INVALID_ARG
    assert call(st=stride + 16) == Q.QG_ERR_ALIGNMENT
    assert call(ys=N - 1) == Q.QG_ERR_INVALID_ARG
    assert call(xs=-2) == Q.QG_ERR_INVALID_ARG
    assert call(xs=3) == Q.QG_ERR_ALIGNMENT
    assert call(K=48) == Q.QG_ERR_INVALID_ARG
    assert call(w=W + 128) == Q.QG_ERR_ALIGNMENT
    assert call(ids=IDS + 2) == Q.QG_ERR_ALIGNMENT


def test_variant_names_follow_layout():
    assert Q.variant_name(0, 1, 151936, 2560) == "q8g64_m1_g32_r2"
    assert Q.variant_name(0, 1, 1024, 1024) == "q8g64_m1_g32_r2"
    assert Q.variant_name(1, 4, 9216, 2560) == "q4g32_m4_g16_r2"
    assert Q.variant_name(1, 1, 2560, 9216) == "q4g32_m1_g32_r2"
    assert Q.variant_name(2, 1, 1536, 4096) == "q4g32_grouped_m1_g64_r2"
    assert Q.variant_name(2, 1, 4096, 1536) == "q4g32_grouped_m1_g16_r2"
    assert Q.variant_name(1, 1, 8, 96) == "q4g32_m1_g1_r2"     # 3 units: G = 1
    assert Q.variant_name(3, 1, 151936, 2560) == "q8g128_m1_g32_r2"
    assert Q.variant_name(3, 2, 7, 128) == "q8g128_m2_g8_r2"  # one group: G = 8
    assert Q.variant_name(4, 1, 1792, 5120) == "q8pc_m1_g64_r2"
    assert Q.variant_name(4, 4, 5120, 4352) == "q8pc_m4_g16_r2"
    assert Q.variant_name(4, 1, 3, 48) == "q8pc_m1_g1_r2"
    with pytest.raises(Q.QGError):
        Q.variant_name(0, 5, 16, 64)
    assert Q.route_count("no_such_variant") == 0


def test_bound_calls_keep_their_buffers_alive(monkeypatch):
    # A prepared call passes raw device addresses; it must own the tensors
    # behind them, or torch may release the memory (graph capture empties
    # torch's cache) while the call can still be replayed.  (Small host
    # tensors stand in for device ones here, so the binding's tensor checks
    # are switched off; the calls are never issued.)
    import gc
    import weakref

    import torch
    monkeypatch.setattr(Q, "_on_gpu", lambda *a, **k: None)
    monkeypatch.setattr(Q, "_need", lambda *a, **k: None)
    w = torch.zeros(4096, dtype=torch.uint8)
    x = torch.zeros(64, dtype=torch.int16)
    y = torch.zeros(16, dtype=torch.float32)
    ids = torch.zeros(2, dtype=torch.int32)
    refs = [weakref.ref(t) for t in (w, x, y, ids)]
    dense = Q.bound_q8g64(w, x, y, 16, 64, stream=0)
    grouped = Q.bound_grouped_q4g32(w, 256, 1, ids, x, 0, y, 16, 16, 32, stream=0)
    del w, x, y, ids
    gc.collect()
    assert all(r() is not None for r in refs)
    del dense, grouped
    gc.collect()
    assert all(r() is None for r in refs)


def test_argmax_validation_and_workspace_size():
    f = Q.lib().qg_argmax_f32
    ws_need = Q.argmax_workspace_size(4)
    assert ws_need >= 12 * 4 and ws_need % 256 == 0
    assert Q.argmax_workspace_size(0) == 0 and Q.argmax_workspace_size(-1) == 0
    WS, OUT = W, Y
    # Every call below must fail validation (no launch on fake addresses).
    assert f(None, 4, 100, 100, OUT, WS, ws_need, None) == Q.QG_ERR_INVALID_ARG
    assert f(X, 4, 100, 100, None, WS, ws_need, None) == Q.QG_ERR_INVALID_ARG
    assert f(X, 4, 100, 100, OUT, None, ws_need, None) == Q.QG_ERR_INVALID_ARG
    assert f(X, -1, 100, 100, OUT, WS, ws_need, None) == Q.QG_ERR_INVALID_ARG
    assert f(X, 65536, 100, 100, OUT, WS, 1 << 30, None) == Q.QG_ERR_INVALID_ARG
    assert f(X, 4, 0, 100, OUT, WS, ws_need, None) == Q.QG_ERR_INVALID_ARG
    assert f(X, 4, 1 << 31, 1 << 31, OUT, WS, ws_need, None) == Q.QG_ERR_INVALID_ARG
    assert f(X, 4, 100, 99, OUT, WS, ws_need, None) == Q.QG_ERR_INVALID_ARG
    assert f(X, 4, 100, 100, OUT, WS, ws_need - 1, None) == Q.QG_ERR_INVALID_ARG
    assert f(X + 2, 4, 100, 100, OUT, WS, ws_need, None) == Q.QG_ERR_ALIGNMENT
    assert f(X, 4, 100, 100, OUT + 2, WS, ws_need, None) == Q.QG_ERR_ALIGNMENT
    assert f(X, 4, 100, 100, OUT, WS + 4, ws_need, None) == Q.QG_ERR_ALIGNMENT
    assert f(X, 0, 100, 100, OUT, WS, ws_need, None) == Q.QG_OK      # no rows


def test_swiglu_validation():
    f = Q.lib().qgemv_grouped_q4g32_swiglu
    N, K = 64, 256
    st = Q.gate_up_expert_stride(N, K)
    assert st == Q.qpack_q4g32_gate_up_size(N, K) and st % 256 == 0
    A = Y
    # Every call below must fail validation (no launch on fake addresses).
    assert f(None, st, 4, IDS, 2, X, 0, A, N, N, K, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, st, 4, None, 2, X, 0, A, N, N, K, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, st, 4, IDS, 2, X, 0, None, N, N, K, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, st, 4, IDS, 65, X, 0, A, N, N, K, None) == Q.QG_ERR_UNSUPPORTED
    assert f(W, st, 0, IDS, 2, X, 0, A, N, N, K, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, st - 256, 4, IDS, 2, X, 0, A, N, N, K, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, st, 4, IDS, 2, X, 0, A, N - 1, N, K, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, st, 4, IDS, 2, X, 0, A, N, N, K + 16, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, st + 16, 4, IDS, 2, X, 0, A, N, N, K, None) == Q.QG_ERR_ALIGNMENT
    assert f(W, st, 4, IDS, 2, X, 3, A, N, N, K, None) == Q.QG_ERR_ALIGNMENT
    assert f(W, st, 4, IDS, 2, X, 0, A + 1, N, N, K, None) == Q.QG_ERR_ALIGNMENT
    assert f(W + 64, st, 4, IDS, 2, X, 0, A, N, N, K, None) == Q.QG_ERR_ALIGNMENT
    assert f(W, st, 4, IDS, 0, X, 0, A, N, N, K, None) == Q.QG_OK     # no slots


def test_gate_up_pack_roundtrip_and_interleave():
    for (N, K) in [(1, 32), (7, 96), (100, 2560), (1536, 4096), (129, 32)]:
        rng = synth.rng_for(11, N, K)
        g = synth.q4g32_weights(rng, N, K)
        u = synth.q4g32_weights(rng, N, K)
        buf = Q.qpack_q4g32_gate_up(g, u)
        assert buf.nbytes == Q.qpack_q4g32_gate_up_size(N, K)
        g2, u2 = Q.qunpack_q4g32_gate_up(buf, N, K)
        assert all(np.array_equal(a, b) for a, b in zip(g + u, g2 + u2))
        # The pair buffer is the plain packing of the rows interleaved in
        # blocks of RPS = 64 / G: gate rows of a tile, then its up rows.
        G = int(Q.variant_name(Q.FMT_GROUPED_Q4G32_SWIGLU, 1, N, K).split("_g")[-1].split("_")[0])
        rps = 64 // G
        Nv = 2 * (-(-N // rps)) * rps
        mats = [np.zeros((Nv,) + a.shape[1:], a.dtype) for a in g]
        for v in range(Nv):
            t, w = divmod(v, 2 * rps)
            n = t * rps + w % rps
            if n < N:
                for k in range(3):
                    mats[k][v] = (g if w < rps else u)[k][n]
        assert np.array_equal(Q.qpack_q4g32(*mats), buf)


def test_fused_argmax_validation():
    ws_need = Q.argmax_workspace_size(2)
    for name in ("qgemv_q8g64_argmax", "qgemv_q8g128_argmax"):
        f = getattr(Q.lib(), name)
        K = 256
        # Every call below must fail validation (no launch on fake addresses).
        assert f(W, X, Y, None, 2, 16, K, K, 16, IDS, ws_need, None) == Q.QG_ERR_INVALID_ARG
        assert f(W, X, Y, IDS, 2, 16, K, K, 16, None, ws_need, None) == Q.QG_ERR_INVALID_ARG
        assert f(W, X, Y, IDS, 2, 16, K, K, 16, IDS, ws_need - 1, None) == Q.QG_ERR_INVALID_ARG
        assert f(W, X, Y, IDS, 5, 16, K, K, 16, IDS, 1 << 20, None) == Q.QG_ERR_UNSUPPORTED
        assert f(W, X, Y, IDS, 2, 16, K, K, 15, IDS, ws_need, None) == Q.QG_ERR_INVALID_ARG
        assert f(W, X, Y, IDS + 2, 2, 16, K, K, 16, IDS, ws_need, None) == Q.QG_ERR_ALIGNMENT
        assert f(W, X, Y, IDS, 2, 16, K, K, 16, IDS + 4, ws_need, None) == Q.QG_ERR_ALIGNMENT
        assert f(W, X, Y, IDS, 0, 16, K, K, 16, IDS, ws_need, None) == Q.QG_OK   # empty batch
    assert Q.variant_name(Q.FMT_Q8G64_ARGMAX, 1, 151936, 2560) == "q8g64_argmax_m1_g32_r2"
    assert Q.variant_name(Q.FMT_Q8G128_ARGMAX, 3, 151936, 2560) == "q8g128_argmax_m3_g32_r2"


@pytest.mark.parametrize("fmt", ["q8g64", "q8g128", "q8pc"])
def test_mma_pack_roundtrip_sizes_and_validation(fmt):
    gen = {"q8g64": synth.q8g64_weights, "q8g128": synth.q8g128_weights,
           "q8pc": synth.q8pc_weights}[fmt]
    pack = getattr(Q, "qpack_%s_mma" % fmt)
    alg = {"q8g64": synth.bytes_q8g64, "q8g128": synth.bytes_q8g128, "q8pc": synth.bytes_q8pc}[fmt]
    for N, K in [(1, 128), (17, 256), (48, 1280), (5120, 1280)]:
        q, s = gen(synth.rng_for(12, N, K), N, K)
        packed = pack(q, s)
        assert packed.nbytes == Q.qpack_mma_size(fmt, N, K)
        q2, s2 = Q.qunpack_mma(fmt, packed, N, K)
        assert np.array_equal(q, q2) and np.array_equal(s, s2)
        if N % 16 == 0:
            assert packed.nbytes == -(-alg(N, K) // 256) * 256
    assert Q.qpack_mma_size(fmt, 4, 96) == 0            # K not a multiple of 64
    f = getattr(Q.lib(), "qgemv_%s_mma" % fmt)
    K = 1024
    # Every call below must fail validation (no launch on fake addresses).
    assert f(W, X, Y, 17, 16, K, K, 16, None) == Q.QG_ERR_UNSUPPORTED          # m > 16
    assert f(W, X, Y, 1, 16, K, K, 16, None) == Q.QG_ERR_UNSUPPORTED           # m = 1: VALU calls
    # (Long rows are accepted: x too long to stage in LDS is read from memory.)
    assert f(W, X, Y, 2, 16, 96, 96, 16, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, X, Y, 2, 16, K, K - 2, 16, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, X, Y, 2, 16, K, K, 15, None) == Q.QG_ERR_INVALID_ARG
    assert f(W + 16, X, Y, 2, 16, K, K, 16, None) == Q.QG_ERR_ALIGNMENT
    assert f(W, X, Y, 2, 16, K, K + 1, 16, None) == Q.QG_ERR_ALIGNMENT
    assert f(W, X, Y, 0, 16, K, K, 16, None) == Q.QG_OK
    fid = {"q8g64": Q.FMT_Q8G64_MMA, "q8g128": Q.FMT_Q8G128_MMA, "q8pc": Q.FMT_Q8PC_MMA}[fmt]
    assert Q.variant_name(fid, 16, 151936, 2560) == "%s_mma_m16" % fmt


def test_q8g64_mma_pack_layout():
    # The 8-bit matrix-core packing against the documented formula: block
    # (tile t, step j) at (t J + j) KiB, lane l = 16 qs + rho holding the
    # codes of row 16 t + rho at k = 64 j + 16 qs .. + 15; then the fp16
    # scales at [tile][group][row].
    N = 40
    for K in (192, 1280):
        q = ((np.arange(N)[:, None] * 5 + np.arange(K)[None, :] * 3) % 251 - 125).astype(np.int8)
        sc = (np.arange(N * K // 64, dtype=np.uint16).reshape(N, K // 64) + 0x3C00).astype(np.uint16)
        buf = Q.qpack_q8g64_mma(q, sc)
        # float16 arrays are taken as their bits; other float arrays are refused.
        assert np.array_equal(Q.qpack_q8g64_mma(q, sc.view(np.float16)), buf)
        with pytest.raises(Q.QGError):
            Q.qpack_q8g64_mma(q, sc.view(np.float16).astype(np.float32))
        tiles, J = (N + 15) // 16, K // 64
        for (t, j, qs, rho) in [(0, 0, 0, 0), (1, J - 1, 3, 7), (2, J // 2, 1, 7), (1, 1, 2, 15)]:
            n = 16 * t + rho
            off = (t * J + j) * 1024 + (16 * qs + rho) * 16
            assert np.array_equal(buf[off:off + 16].view(np.int8), q[n, 64 * j + 16 * qs:64 * j + 16 * qs + 16])
            moff = tiles * J * 1024 + (t * J + j) * 32 + rho * 2
            assert int(buf[moff:moff + 2].view(np.uint16)[0]) == int(sc[n, j])


def test_q4g32_mma_pack_layout_and_roundtrip():
    # Layout of the Q4G32 matrix-core packing, checked against the
    # documented formula: in block (tile t, step j), lane l = 16 qs + rho,
    # dword g holds the codes of row 16 t + rho at k = 128 j + 32 g + 8 qs + e
    # in canonical byte order (e at nibble position e: byte e // 2, low
    # nibble for even e); the block sits at (t J + j) KiB; then the meta
    # dwords scale | min << 16 at [tile][step][row][group].
    N = 37
    for K in (384, 1024):
        n_idx = np.arange(N)[:, None]
        k_idx = np.arange(K)[None, :]
        c = (k_idx * 7 + n_idx * 3) % 16
        codes = synth.pack_nibbles(c)
        s = (np.arange(N * K // 32, dtype=np.uint16).reshape(N, K // 32) + 0x3C00).astype(np.uint16)
        mn = (np.arange(N * K // 32, dtype=np.uint16).reshape(N, K // 32) + 0x8000).astype(np.uint16)
        buf = Q.qpack_q4g32_mma(codes, s, mn)
        tiles, J = (N + 15) // 16, K // 128
        assert buf.nbytes == Q.qpack_mma_size("q4g32", N, K) == -(-(tiles * J * 1024 + tiles * J * 256) // 256) * 256

        def block(t, j):
            return (t * J + j) * 1024

        pos = tuple(range(8))
        for (t, j, qs, rho, g) in [(0, 0, 0, 0, 0), (1, 2, 3, 5, 1), (2, 1, 2, 4, 3), (0, 2, 1, 15, 2),
                                   (1, J - 1, 0, 7, 0), (2, J - 1, 3, 3, 2)]:
            n = 16 * t + rho
            word = int(buf[block(t, j) + (16 * qs + rho) * 16 + 4 * g:][:4].view(np.uint32)[0])
            for e in range(8):
                assert (word >> (4 * pos[e])) & 15 == c[n, 128 * j + 32 * g + 8 * qs + e]
            meta = buf[tiles * J * 1024 + ((t * J + j) * 16 + rho) * 16 + 4 * g:][:4].view(np.uint16)
            assert meta[0] == s[n, 4 * j + g] and meta[1] == mn[n, 4 * j + g]
        # Padding rows of the last tile are all zero.
        pad = np.stack([buf[block(2, j):block(2, j) + 1024] for j in range(J)]).reshape(J, 64, 16)
        assert not pad[:, [16 * q + r for q in range(4) for r in range(5, 16)]].any()
        c2, s2, m2 = Q.qunpack_mma("q4g32", buf, N, K)
        assert np.array_equal(c2, codes) and np.array_equal(s2, s) and np.array_equal(m2, mn)
    assert Q.qpack_mma_size("q4g32", N, 320) == 0          # K not a multiple of 128
    f = Q.lib().qgemv_q4g32_mma
    assert f(W, X, Y, 2, 16, 320, 320, 16, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, X, Y, 17, 16, 256, 256, 16, None) == Q.QG_ERR_UNSUPPORTED
    assert f(W, X, Y, 1, 16, 256, 256, 16, None) == Q.QG_ERR_UNSUPPORTED
    assert f(W + 16, X, Y, 2, 16, 256, 256, 16, None) == Q.QG_ERR_ALIGNMENT
    assert f(W, X, Y, 0, 16, 256, 256, 16, None) == Q.QG_OK
    assert Q.variant_name(Q.FMT_Q4G32_MMA, 4, 9216, 2560) == "q4g32_mma_m4"


def test_launch_override_validation():
    # Values outside the documented ranges are rejected; valid ones and the
    # reset to defaults are accepted (no kernel is launched here).
    for args in [(-1, -1, 0), (0, 2, 0), (0, -2, 0), (0, -1, 3), (1 << 25, -1, 0)]:
        with pytest.raises(Q.QGError):
            Q.set_launch_override(*args)
    try:
        Q.set_launch_override(7, 1, 4)
        Q.set_launch_override(1 << 24, 0, 2)
    finally:
        Q.set_launch_override()


def test_read_stream_validation():
    # Argument checks run before anything touches a device.
    f = Q.lib().qg_read_stream
    assert f(None, 16, 64, 0, None) == Q.QG_ERR_INVALID_ARG
    assert f(256, 16, None, 0, None) == Q.QG_ERR_INVALID_ARG
    assert f(256, 0, 64, 0, None) == Q.QG_ERR_INVALID_ARG
    assert f(256, 24, 64, 0, None) == Q.QG_ERR_INVALID_ARG
    assert f(256, 16, 64, 33, None) == Q.QG_ERR_INVALID_ARG
    assert f(256, 16, 64, -1, None) == Q.QG_ERR_INVALID_ARG
    assert f(264, 16, 64, 0, None) == Q.QG_ERR_ALIGNMENT
    assert f(256, 16, 66, 0, None) == Q.QG_ERR_ALIGNMENT


def test_binding_checks_tensors_before_calling_the_library():
    # The torch-facing wrappers reject a wrong element type, a tensor too
    # short for the shape and a tensor that is not on a GPU, with
    # QG_ERR_INVALID_ARG, before any pointer reaches the C ABI (no GPU
    # needed: the checks run on the host and nothing is launched).
    torch = pytest.importorskip("torch")
    N, K, m = 64, 128, 2
    w = torch.zeros(Q.qpack_q8g64_size(N, K), dtype=torch.uint8)
    x = torch.zeros((m, K), dtype=torch.bfloat16)
    y = torch.zeros((m, N), dtype=torch.float32)

    def rejects(fn, *a, **kw):
        with pytest.raises(Q.QGError) as e:
            fn(*a, **kw)
        assert e.value.status == Q.QG_ERR_INVALID_ARG
        return str(e.value)

    assert "dtype" in rejects(Q.qgemv_q8g64, w, x.float(), y, N, K)
    assert "dtype" in rejects(Q.qgemv_q8g64, w, x, y.double(), N, K)
    assert "dtype" in rejects(Q.qgemv_q8g64, w.to(torch.int32), x, y, N, K)
    assert "elements" in rejects(Q.qgemv_q8g64, w[:-1], x, y, N, K)
    assert "elements" in rejects(Q.qgemv_q8g64, w, x[:, :K - 2], y, N, K, m=m, ldx=K)
    assert "elements" in rejects(Q.qgemv_q8g64, w, x, y[:1], N, K, m=m, ldy=N)
    assert "GPU" in rejects(Q.qgemv_q8g64, w, x, y, N, K)
    # routed experts: int64 ids (torch's default integer type) are refused
    Ne, Ke, E = 32, 64, 3
    stride = Q.expert_stride(Ne, Ke)
    we = torch.zeros(E * stride, dtype=torch.uint8)
    ids = torch.zeros(2, dtype=torch.int64)
    xe = torch.zeros((2, Ke), dtype=torch.int16)
    ye = torch.zeros((2, Ne), dtype=torch.float32)
    assert "dtype" in rejects(Q.qgemv_grouped_q4g32, we, stride, E, ids, xe, Ke, ye, Ne, Ne, Ke)
    ids32 = ids.to(torch.int32)
    assert "elements" in rejects(Q.qgemv_grouped_q4g32, we[:-256], stride, E, ids32, xe, Ke, ye, Ne, Ne, Ke)
    assert "elements" in rejects(Q.qgemv_grouped_q4g32, we, stride, E, ids32, xe[:1], Ke, ye, Ne, Ne, Ke)
    assert "GPU" in rejects(Q.qgemv_grouped_q4g32, we, stride, E, ids32, xe, Ke, ye, Ne, Ne, Ke)
    # argmax: the logits must cover m rows of N at stride ldx
    lg = torch.zeros((2, 100), dtype=torch.float32)
    idx = torch.zeros(2, dtype=torch.int32)
    ws = torch.zeros(Q.argmax_workspace_size(2), dtype=torch.uint8)
    assert "elements" in rejects(Q.argmax_f32, lg[:1], idx, ws, N=100, m=2, ldx=100)
    assert "dtype" in rejects(Q.argmax_f32, lg, idx.long(), ws, N=100, m=2)
    assert "GPU" in rejects(Q.argmax_f32, lg, idx, ws, N=100, m=2)
