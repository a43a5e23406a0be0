"""GPU parity for the Q4G32 matrix-core decode kernel (m = 2..16), through
the C ABI: qgemv_q4g32_mma on weights packed by qpack_q4g32_mma.  Same
acceptance as the other GEMV parity tests (|y - y_ref| <= 2e-3 sum|w x| per
output, bit-exact on exact inputs, NaN canary, untouched elements past N).
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


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    Q.lib()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def run(W, x, ldx=None, ldy=None, packed=None):
    codes = W[0]
    N, K = codes.shape[0], 2 * codes.shape[1]
    m = x.shape[0]
    ldx = K if ldx is None else ldx
    ldy = N if ldy is None else ldy
    xb = np.zeros((m, ldx), np.uint16)
    xb[:, :K] = x[:, :K]
    y = torch.full((m, ldy), CANARY_BITS, dtype=torch.int32, device="cuda").view(torch.float32)
    w = packed if packed is not None else dev(Q.qpack_q4g32_mma(*W))
    Q.qgemv_q4g32_mma(w, dev(xb), y, N, K, m=m, ldx=ldx, ldy=ldy)
    return host(y)


def check(W, x, y, what):
    y_ref, a_ref = oracle.q4g32(*W, x, threads=THREADS)
    ok = oracle.within_tolerance(y, y_ref, a_ref, TOL)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        raise AssertionError("%s: %d of %d bad, e.g. %s" % (
            what, (~ok).sum(), ok.size, [(tuple(b), y[tuple(b)], y_ref[tuple(b)]) for b in bad]))


# ----------------------------------------------------------- workload configs

@pytest.mark.parametrize("m", [4, 8, 16])
@pytest.mark.parametrize("N,K", [(9216, 2560), (2560, 9216)])
def test_q4_k2560_family_batched(N, K, m):
    # The Q4G32 K=2560 family (gate/up 2560 -> 9216, down 9216 -> 2560); at
    # m = 16 the down projection's x does not fit in LDS and is read from
    # memory.
    rng = synth.rng_for(110, N, K, m)
    W = synth.q4g32_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    check(W, x, run(W, x), "N=%d K=%d m=%d" % (N, K, m))


# ------------------------------------------------------------ shape sweep

@pytest.mark.parametrize("m", [2, 3, 5, 16])
@pytest.mark.parametrize("N", [1, 15, 17, 1000])
@pytest.mark.parametrize("K", [128, 384, 2560])
def test_ragged_shapes_and_strides(K, N, m):
    rng = synth.rng_for(111, N, K, m)
    W = synth.q4g32_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run(W, x, ldx=K + 4, ldy=N + 3)
    assert np.all(y[:, N:].view(np.uint32) == CANARY_BITS), "wrote past N"
    check(W, x, y[:, :N], "N=%d K=%d m=%d" % (N, K, m))


# How a tile's K is shared: by no wave (many tiles), by four waves (4..63
# steps of 128, or whenever the sixteen-way split's sums do not fit beside
# x), by sixteen (64 or more steps); x read from memory where it does not
# fit in LDS.
@pytest.mark.parametrize("N,K,m,pad", [
    (70000, 256, 3, 0),       # many tiles: whole tiles per wave
    (1000, 512, 9, 2),        # four steps: four waves, one step each
    (300, 8192, 6, 0),        # 64 steps: sixteen waves
    (33, 8320, 4, 8),         # 65 steps: uneven sixteen-way shares
    (500, 4864, 16, 0),       # x fills the LDS: four waves, x from memory
    (70, 16384, 16, 2),       # 512 KiB of x: x from memory, 4-byte loads
])
def test_k_split_choices(N, K, m, pad):
    rng = synth.rng_for(112, N, K, m)
    W = synth.q4g32_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run(W, x, ldx=K + pad, ldy=N + 1)
    assert np.all(y[:, N:].view(np.uint32) == CANARY_BITS), "wrote past N"
    check(W, x, y[:, :N], "N=%d K=%d m=%d" % (N, K, m))


def test_every_m_from_2_to_16():
    N, K = 3000, 1024
    rng = synth.rng_for(113, 0)
    W = synth.q4g32_weights(rng, N, K)
    w = dev(Q.qpack_q4g32_mma(*W))
    x = synth.activations(rng, 16, K)
    y_ref, a_ref = oracle.q4g32(*W, x, threads=THREADS)
    for m in range(2, 17):
        y = run(W, x[:m], packed=w)
        assert oracle.within_tolerance(y, y_ref[:m], a_ref[:m], TOL).all(), "m=%d" % m


# ------------------------------------------------------- exact arithmetic

@pytest.mark.parametrize("N,K,m", [(9216, 2560, 16), (1000, 8192, 5), (70, 384, 12)])
def test_exact_inputs_bit_exact(N, K, m):
    # Power-of-two scales, mins that are multiples of the scale and integer
    # x make every partial sum exact in fp32: any summation order gives the
    # oracle's value.
    rng = synth.rng_for(114, N, K)
    codes, _, _ = synth.q4g32_weights(rng, N, K)
    e = rng.integers(-6, -2, size=(N, K // 32))
    s = synth.to_fp16_bits(2.0 ** e)
    mn = synth.to_fp16_bits(-(2.0 ** e) * rng.integers(0, 9, size=(N, K // 32)))
    x = synth.to_bf16_bits(rng.integers(-4, 5, size=(m, K)).astype(np.float32))
    y = run((codes, s, mn), x)
    y_ref, _ = oracle.q4g32(codes, s, mn, x, threads=THREADS)
    assert np.array_equal(y.astype(np.float64), y_ref)


# -------------------------------------------------------- degenerate cases

def test_zero_scales_mins_and_activations_give_exact_zero():
    rng = synth.rng_for(115, 0)
    codes, s, mn = synth.q4g32_weights(rng, 300, 2560)
    x = synth.activations(rng, 7, 2560)
    z = np.zeros_like(s)
    assert np.all(run((codes, z, z), x) == 0.0)
    assert np.all(run((codes, s, mn), np.zeros_like(x)) == 0.0)


def test_zero_scales_leave_min_times_group_sums():
    # With every scale 0, y = sum over groups of min * (sum of the group's x):
    # the oracle's closed form, within the tolerance.
    rng = synth.rng_for(116, 0)
    codes, s, mn = synth.q4g32_weights(rng, 200, 1024)
    x = synth.activations(rng, 3, 1024)
    W = (codes, np.zeros_like(s), mn)
    check(W, x, run(W, x), "zero scales")


# ------------------------------------------------- structural identities

def test_rows_do_not_depend_on_the_batch():
    N, K = 2000, 2560
    rng = synth.rng_for(117, 0)
    W = synth.q4g32_weights(rng, N, K)
    w = dev(Q.qpack_q4g32_mma(*W))
    x = synth.activations(rng, 16, K)
    y16 = run(W, x, packed=w)
    for i in (0, 7, 14):
        assert np.array_equal(y16[i:i + 2], run(W, x[i:i + 2], packed=w))


def test_matches_the_plain_gemv_within_rounding():
    N, K, m = 4000, 2560, 4
    rng = synth.rng_for(118, 0)
    W = synth.q4g32_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    y_mma = run(W, x)
    y = torch.full((m, N), CANARY_BITS, dtype=torch.int32, device="cuda").view(torch.float32)
    Q.qgemv_q4g32(dev(Q.qpack_q4g32(*W)), dev(x), y, N, K, m=m)
    _, a_ref = oracle.q4g32(*W, x, threads=THREADS)
    assert np.all(np.abs(y_mma.astype(np.float64) - host(y)) <= 2 * TOL * a_ref)


def test_route_counter_names_the_variant():
    Q.route_counts_reset()
    rng = synth.rng_for(119, 0)
    W = synth.q4g32_weights(rng, 64, 1280)
    run(W, synth.activations(rng, 11, 1280))
    assert Q.route_count("q4g32_mma_m11") == 1
    assert Q.variant_name(Q.FMT_Q4G32_MMA, 11, 64, 1280) == "q4g32_mma_m11"


def test_graph_replays_match_eager_calls():
    N, K, m = 9216, 2560, 8
    rng = synth.rng_for(121, 0)
    W = synth.q4g32_weights(rng, N, K)
    w = dev(Q.qpack_q4g32_mma(*W))
    x = dev(synth.activations(rng, m, K))
    y = torch.full((m, N), CANARY_BITS, dtype=torch.int32, device="cuda").view(torch.float32)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call = Q.bound_mma("q4g32", w, x, y, N, K, m=m)
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    for r in range(3):
        x.copy_(dev(synth.activations(synth.rng_for(121, 100 + r), m, K)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(y).copy()
        ye = torch.full((m, N), CANARY_BITS, dtype=torch.int32, device="cuda").view(torch.float32)
        Q.qgemv_q4g32_mma(w, x, ye, N, K, m=m)
        assert np.array_equal(got, host(ye)), "replay %d" % r
