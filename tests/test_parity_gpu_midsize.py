"""GPU parity on mid-size dense matrices with ragged N, every lane-group
width and many steps per tile: shapes between the launch-bound small
matrices and the stream-bound LM head, where few tiles per wave leave the
launch uneven.  (A work-group split of such matrices, with tiles cut
across waves and folded through LDS, was built and measured slower on
MI355X; these cases stay as mid-size coverage.)  Acceptance as in the
other parity tests.
"""
import os

import numpy as np
import pytest

import oracle
from weight_only_block_amd import qgemv as Q
from weight_only_block_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3
CANARY_BITS = 0x7FC0DEAD
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))

# (format, N, K): G, tiles, steps per tile in the comment.
MID_SHAPES = [
    ("q8g64", 3001, 2560),    # G=32, 751 tiles, J=5
    ("q8g64", 5000, 1536),    # G=32, 1250 tiles, J=3
    ("q4g32", 2049, 9216),    # G=32, 513 tiles, J=9
    ("q4g32", 9216, 2560),    # G=16, 1152 tiles, J=5
    ("q4g32", 700, 4096),     # G=64, 350 tiles, J=2
    ("q8pc", 1500, 4352),     # G=16, 188 tiles, J=17
    ("q8pc", 5120, 1280),     # G=16, 640 tiles, J=5
    ("q8g128", 3000, 4096),   # G=64, 1500 tiles, J=4
]

FMT = {
    "q8g64": (synth.q8g64_weights, Q.qpack_q8g64, Q.qgemv_q8g64, oracle.q8g64),
    "q8g128": (synth.q8g128_weights, Q.qpack_q8g128, Q.qgemv_q8g128, oracle.q8g128),
    "q8pc": (synth.q8pc_weights, Q.qpack_q8pc, Q.qgemv_q8pc, oracle.q8pc),
    "q4g32": (synth.q4g32_weights, Q.qpack_q4g32, Q.qgemv_q4g32, oracle.q4g32),
}


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    Q.lib()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to("cuda")


def canary(shape):
    return torch.full(shape, CANARY_BITS, dtype=torch.int32, device="cuda").view(torch.float32)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def run(fmt, weights, x, N, K, ldx=None, ldy=None, packed=None):
    _, pack, gemv, _ = FMT[fmt]
    m = x.shape[0]
    ldx = K if ldx is None else ldx
    ldy = N if ldy is None else ldy
    xb = np.zeros((m, ldx), np.uint16)
    xb[:, :K] = x[:, :K]
    y = canary((m, ldy))
    w = packed if packed is not None else dev(pack(*weights))
    gemv(w, dev(xb), y, N, K, m=m, ldx=ldx, ldy=ldy)
    return host(y)


@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("fmt,N,K", MID_SHAPES)
def test_mid_size_shapes_match_the_oracle(fmt, N, K, m):
    gen, _, _, ref = FMT[fmt]
    rng = synth.rng_for(80, N, K, m)
    weights = gen(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run(fmt, weights, x, N, K, ldx=K + 2, ldy=N + 3)
    assert np.all(y[:, N:].view(np.uint32) == CANARY_BITS), "wrote past N"
    y_ref, a_ref = ref(*weights, x, threads=THREADS)
    ok = oracle.within_tolerance(y[:, :N], y_ref, a_ref, TOL)
    assert ok.all(), "%s N=%d K=%d m=%d: %d bad" % (fmt, N, K, m, (~ok).sum())


@pytest.mark.parametrize("fmt,N,K", [s for s in MID_SHAPES if s[0] in ("q8pc", "q4g32")])
def test_mid_size_rows_do_not_depend_on_m(fmt, N, K):
    # The launch and the order of the sums depend on the matrix only, so the
    # rows of an m = 4 call equal four m = 1 calls bit for bit (batch
    # invariance).
    gen, pack, _, _ = FMT[fmt]
    rng = synth.rng_for(81, N, K)
    weights = gen(rng, N, K)
    w = dev(pack(*weights))
    x = synth.activations(rng, 4, K)
    y4 = run(fmt, weights, x, N, K, packed=w)
    for i in range(4):
        assert np.array_equal(y4[i], run(fmt, weights, x[i:i + 1], N, K, packed=w)[0])


def test_mid_size_repeat_calls_are_bitwise_identical():
    N, K = 1500, 4352
    rng = synth.rng_for(82, 0)
    weights = synth.q8pc_weights(rng, N, K)
    w = dev(Q.qpack_q8pc(*weights))
    x = synth.activations(rng, 2, K)
    outs = [run("q8pc", weights, x, N, K, packed=w) for _ in range(4)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("N,K", [(2049, 9216), (9216, 2560)])
def test_mid_size_exact_inputs_bit_exact(N, K):
    rng = synth.rng_for(83, N, K)
    codes, _, _ = synth.q4g32_weights(rng, N, K)
    e = rng.integers(-6, -2, size=(N, K // 32))
    s = synth.to_fp16_bits(2.0 ** e)
    mn = synth.to_fp16_bits(-(2.0 ** e) * rng.integers(0, 9, size=(N, K // 32)))
    x = synth.to_bf16_bits(rng.integers(-4, 5, size=(3, K)).astype(np.float32))
    y = run("q4g32", (codes, s, mn), x, N, K)
    y_ref, _ = oracle.q4g32(codes, s, mn, x, threads=THREADS)
    assert np.array_equal(y.astype(np.float64), y_ref)
