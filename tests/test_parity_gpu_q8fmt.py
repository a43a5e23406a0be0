"""GPU parity for the two further 8-bit formats, through the C ABI:
Q8G128 (one fp16 scale per 128 K) and Q8PC (one fp32 scale per output row).

Same acceptance as the Q8G64/Q4G32 parity tests: per output element
|y_gpu - y_ref| <= 2e-3 * sum_k |w x| against the fp64 oracle, bit-exact on
exact-arithmetic inputs, a NaN canary in every output buffer and untouched
canaries past N in strided rows.
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

FORMATS = {
    "q8g128": (Q.qpack_q8g128, Q.qgemv_q8g128, oracle.q8g128, synth.q8g128_weights, 128),
    "q8pc": (Q.qpack_q8pc, Q.qgemv_q8pc, oracle.q8pc, synth.q8pc_weights, 16),
}


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    Q.lib()


def dev(a: np.ndarray) -> "torch.Tensor":
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to("cuda")


def canary(shape) -> "torch.Tensor":
    return torch.full(shape, CANARY_BITS, dtype=torch.int32, device="cuda").view(torch.float32)


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_parity(y_gpu, y_ref, a_ref, what=""):
    y_gpu = np.asarray(y_gpu, np.float64)
    ok = oracle.within_tolerance(y_gpu, y_ref, a_ref, TOL)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        details = [(tuple(b), y_gpu[tuple(b)], y_ref[tuple(b)], a_ref[tuple(b)]) for b in bad]
        raise AssertionError("%s: %d of %d outputs out of tolerance, e.g. %s"
                             % (what, (~ok).sum(), ok.size, details))


def run(fmt, q, s, x, ldx=None, ldy=None):
    pack, gemv = FORMATS[fmt][:2]
    N, K = q.shape
    m = x.shape[0]
    ldx = K if ldx is None else ldx
    ldy = N if ldy is None else ldy
    xb = np.zeros((m, ldx), np.uint16)
    xb[:, :K] = x[:, :K]
    y = canary((m, ldy))
    gemv(dev(pack(q, s)), dev(xb), y, N, K, m=m, ldx=ldx, ldy=ldy)
    return host(y)


def reference(fmt, q, s, x):
    return FORMATS[fmt][2](q, s, x, threads=THREADS)


def weights(fmt, rng, N, K):
    return FORMATS[fmt][3](rng, N, K)


# ----------------------------------------------------------- workload configs

def test_lm_head_q8g128_full_size():
    # The LM-head shape in its own per-operator format (one scale per 128),
    # in the launch configuration the benchmark times; every row checked.
    _, _, N, K = synth.LM_HEAD
    rng = synth.rng_for(30, 0)
    q, s = synth.q8g128_weights(rng, N, K)
    x = synth.activations(rng, 1, K)
    y = run("q8g128", q, s, x)
    y_ref, a_ref = reference("q8g128", q, s, x)
    assert_parity(y, y_ref, a_ref, "lm_head q8g128")


@pytest.mark.parametrize("m", [1, 4])
@pytest.mark.parametrize("j,label,N,K", [(j, c[0], c[2], c[3])
                                         for j, c in enumerate(synth.W8A16_QWEN3_14B_TP4)])
def test_w8a16_qwen3_14b_tp4(j, label, N, K, m):
    rng = synth.rng_for(31, j, m)
    q, s = synth.q8pc_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run("q8pc", q, s, x)
    y_ref, a_ref = reference("q8pc", q, s, x)
    assert_parity(y, y_ref, a_ref, "w8a16 %s m=%d" % (label, m))


# ------------------------------------------------------------ shape sweep

@pytest.mark.parametrize("N", [1, 7, 129, 1000])
@pytest.mark.parametrize("K", [128, 384, 2560])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_q8g128_ragged_shapes_and_strides(N, K, m):
    rng = synth.rng_for(32, N, K, m)
    q, s = synth.q8g128_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run("q8g128", q, s, x, ldx=K + 6, ldy=N + 5)
    assert np.all(y[:, N:].view(np.uint32) == CANARY_BITS), "wrote past N"
    y_ref, a_ref = reference("q8g128", q, s, x)
    assert_parity(y[:, :N], y_ref, a_ref, "q8g128 N=%d K=%d m=%d" % (N, K, m))


@pytest.mark.parametrize("N", [1, 7, 129, 1000])
@pytest.mark.parametrize("K", [16, 48, 1280, 4352])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_q8pc_ragged_shapes_and_strides(N, K, m):
    rng = synth.rng_for(33, N, K, m)
    q, s = synth.q8pc_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run("q8pc", q, s, x, ldx=K + 2, ldy=N + 3)
    assert np.all(y[:, N:].view(np.uint32) == CANARY_BITS), "wrote past N"
    y_ref, a_ref = reference("q8pc", q, s, x)
    assert_parity(y[:, :N], y_ref, a_ref, "q8pc N=%d K=%d m=%d" % (N, K, m))


# ------------------------------------------------------- exact arithmetic

def _exact_x(rng, m, K):
    return synth.to_bf16_bits(rng.integers(-4, 5, size=(m, K)).astype(np.float32))


@pytest.mark.parametrize("N,K,m", [(1024, 1024, 1), (2048, 2560, 4), (151936, 2560, 1)])
def test_q8g128_exact_inputs_bit_exact(N, K, m):
    rng = synth.rng_for(34, N, K)
    q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    s = synth.to_fp16_bits(2.0 ** rng.integers(-6, -2, size=(N, K // 128)))
    x = _exact_x(rng, m, K)
    y_ref, _ = reference("q8g128", q, s, x)
    assert np.array_equal(run("q8g128", q, s, x).astype(np.float64), y_ref)


@pytest.mark.parametrize("N,K,m", [(1792, 5120, 1), (5120, 1280, 4), (8704, 5120, 2), (5120, 4352, 3)])
def test_q8pc_exact_inputs_bit_exact(N, K, m):
    rng = synth.rng_for(35, N, K)
    q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    # fp32 row scales far outside fp16's range: only an fp32 scale path is exact.
    s = (2.0 ** rng.integers(-40, -30, size=N)).astype(np.float32).view(np.uint32)
    x = _exact_x(rng, m, K)
    y_ref, _ = reference("q8pc", q, s, x)
    assert np.array_equal(run("q8pc", q, s, x).astype(np.float64), y_ref)


# -------------------------------------------------------- degenerate cases

@pytest.mark.parametrize("fmt", ["q8g128", "q8pc"])
def test_zero_scales_and_zero_codes_give_exact_zero(fmt):
    rng = synth.rng_for(36, 0)
    q, s = weights(fmt, rng, 300, 2560)
    x = synth.activations(rng, 2, 2560)
    assert np.all(run(fmt, q, np.zeros_like(s), x) == 0.0)
    assert np.all(run(fmt, np.zeros_like(q), s, x) == 0.0)
    assert np.all(run(fmt, q, s, np.zeros((1, 2560), np.uint16)) == 0.0)


def test_q8pc_extreme_codes_and_row_scales():
    # int8 -128 and 127 against large, tiny and subnormal fp32 row scales.
    N, K = 16, 256
    q = np.where(np.arange(K)[None, :] % 2 == 0, -128, 127).astype(np.int8).repeat(N, 0)
    s = np.full(N, 1.0e30, np.float32)
    s[1::4] = 1.0e-30
    s[2::4] = 1.0e-40                                  # fp32 subnormal
    s[3::4] = 65504.0
    x = synth.activations(synth.rng_for(36, 1), 1, K)
    y = run("q8pc", q, s.view(np.uint32), x)
    y_ref, a_ref = reference("q8pc", q, s.view(np.uint32), x)
    assert_parity(y, y_ref, a_ref, "extreme q8pc")


def test_q8g128_extreme_codes_and_scales():
    N, K = 16, 512
    q = np.where(np.arange(K)[None, :] % 2 == 0, -128, 127).astype(np.int8).repeat(N, 0)
    s = np.full((N, K // 128), 0x7BFF, np.uint16)      # 65504
    s[1::2] = 0x0001                                    # 2^-24 (subnormal)
    x = synth.activations(synth.rng_for(36, 2), 1, K)
    y = run("q8g128", q, s, x)
    y_ref, a_ref = reference("q8g128", q, s, x)
    assert_parity(y, y_ref, a_ref, "extreme q8g128")


# ------------------------------------------------- structural identities

@pytest.mark.parametrize("fmt,K", [("q8g128", 2560), ("q8pc", 4352)])
def test_m4_rows_equal_m1_calls_bitwise(fmt, K):
    rng = synth.rng_for(37, K)
    q, s = weights(fmt, rng, 777, K)
    x = synth.activations(rng, 4, K)
    y4 = run(fmt, q, s, x)
    for i in range(4):
        assert np.array_equal(y4[i], run(fmt, q, s, x[i:i + 1])[0])


def test_q8pc_equals_q8g128_with_row_constant_scales_within_rounding():
    # A per-row fp32 scale that is an fp16 value is the same weight matrix as
    # Q8G128 with that scale in every group.
    rng = synth.rng_for(38, 0)
    N, K = 640, 2560
    q = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    s16 = synth.to_fp16_bits(rng.uniform(1e-3, 2e-2, size=N))
    s32 = s16.view(np.float16).astype(np.float32).view(np.uint32)
    x = synth.activations(rng, 2, K)
    y_pc = run("q8pc", q, s32, x)
    y_g = run("q8g128", q, np.repeat(s16[:, None], K // 128, axis=1), x)
    _, a_ref = reference("q8pc", q, s32, x)
    assert np.all(np.abs(y_pc.astype(np.float64) - y_g) <= 2 * TOL * a_ref)


def test_route_counters_name_the_launched_variant():
    rng = synth.rng_for(39, 0)
    Q.route_counts_reset()
    q, s = synth.q8pc_weights(rng, 64, 1280)
    run("q8pc", q, s, synth.activations(rng, 2, 1280))
    q2, s2 = synth.q8g128_weights(rng, 64, 2560)
    run("q8g128", q2, s2, synth.activations(rng, 1, 2560))
    assert Q.route_count(Q.variant_name(4, 2, 64, 1280)) == 1
    assert Q.route_count(Q.variant_name(3, 1, 64, 2560)) == 1
    assert Q.route_count(Q.variant_name(0, 1, 64, 2560)) == 0


def test_graph_replays_match_eager_calls():
    rng = synth.rng_for(40, 0)
    q, s = synth.q8pc_weights(rng, 1792, 5120)
    w = dev(Q.qpack_q8pc(q, s))
    x = dev(synth.activations(rng, 2, 5120))
    y = canary((2, 1792))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call = Q.bound_q8pc(w, x, y, 1792, 5120, m=2)
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    for r in range(3):
        x.copy_(dev(synth.activations(synth.rng_for(40, 100 + r), 2, 5120)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(y).copy()
        ye = canary((2, 1792))
        Q.qgemv_q8pc(w, x, ye, 1792, 5120, m=2)
        assert np.array_equal(got, host(ye)), "replay %d" % r
