"""GPU parity for the matrix-core decode kernel (m = 2..16), through the
C ABI: qgemv_q8g64_mma, qgemv_q8g128_mma, qgemv_q8pc_mma on weights packed
in the matrix-core layout.  Same acceptance as the other GEMV parity tests
(|y - y_ref| <= 2e-3 sum|w x| per output, bit-exact on exact inputs, NaN
canary, untouched elements past N).
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

FMT = {
    "q8g64": (synth.q8g64_weights, Q.qpack_q8g64_mma, Q.qgemv_q8g64_mma, oracle.q8g64, 64),
    "q8g128": (synth.q8g128_weights, Q.qpack_q8g128_mma, Q.qgemv_q8g128_mma, oracle.q8g128, 128),
    "q8pc": (synth.q8pc_weights, Q.qpack_q8pc_mma, Q.qgemv_q8pc_mma, oracle.q8pc, 64),
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


def run(fmt, q, s, x, ldx=None, ldy=None, packed=None):
    _, pack, gemv, _, _ = FMT[fmt]
    N, K = q.shape
    m = x.shape[0]
    ldx = K if ldx is None else ldx
    ldy = N if ldy is None else ldy
    xb = np.zeros((m, ldx), np.uint16)
    xb[:, :K] = x[:, :K]
    y = canary((m, ldy))
    w = packed if packed is not None else dev(pack(q, s))
    gemv(w, dev(xb), y, N, K, m=m, ldx=ldx, ldy=ldy)
    return host(y)


def check(fmt, q, s, x, y, what):
    ref = FMT[fmt][3]
    y_ref, a_ref = ref(q, s, x, threads=THREADS)
    ok = oracle.within_tolerance(y, y_ref, a_ref, TOL)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        raise AssertionError("%s: %d of %d bad, e.g. %s" % (
            what, (~ok).sum(), ok.size, [(tuple(b), y[tuple(b)], y_ref[tuple(b)]) for b in bad]))


# ----------------------------------------------------------- workload configs

@pytest.mark.parametrize("m", [8, 16])
@pytest.mark.parametrize("fmt", ["q8g64", "q8g128"])
def test_lm_head_batched_full_size(fmt, m):
    _, _, N, K = synth.LM_HEAD
    gen = FMT[fmt][0]
    rng = synth.rng_for(100, m)
    q, s = gen(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run(fmt, q, s, x)
    check(fmt, q, s, x, y, "lm_head %s m=%d" % (fmt, m))


# m = 2 to 4, 8 and 16 take the shape policy's launch choices on some of
# these shapes (even rounds; a four-way K split with x read from memory).
@pytest.mark.parametrize("m", [2, 3, 4, 8, 15, 16])
@pytest.mark.parametrize("j,label,N,K", [(j, c[0], c[2], c[3])
                                         for j, c in enumerate(synth.W8A16_QWEN3_14B_TP4)])
def test_w8a16_qwen3_14b_tp4_batched(j, label, N, K, m):
    rng = synth.rng_for(101, j, m)
    q, s = synth.q8pc_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run("q8pc", q, s, x)
    check("q8pc", q, s, x, y, "w8a16 %s m=%d" % (label, m))


# ------------------------------------------------------------ shape sweep

@pytest.mark.parametrize("m", [2, 3, 5, 16])
@pytest.mark.parametrize("N", [1, 15, 17, 1000])
@pytest.mark.parametrize("K", [128, 384, 2560])
@pytest.mark.parametrize("fmt", ["q8g64", "q8g128", "q8pc"])
def test_ragged_shapes_and_strides(fmt, K, N, m):
    gen = FMT[fmt][0]
    rng = synth.rng_for(102, N, K, m)
    q, s = gen(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run(fmt, q, s, x, ldx=K + 4, ldy=N + 3)
    assert np.all(y[:, N:].view(np.uint32) == CANARY_BITS), "wrote past N"
    check(fmt, q, s, x, y[:, :N], "%s N=%d K=%d m=%d" % (fmt, N, K, m))


# Rows of x that are not a whole number of 128-wide groups (K = 64 mod
# 128) are swizzled in LDS in groups of 8 chunks instead of 16.
@pytest.mark.parametrize("m", [2, 9, 16])
@pytest.mark.parametrize("N,K", [(1000, 320), (70000, 192), (40, 1344)])
@pytest.mark.parametrize("fmt", ["q8g64", "q8pc"])
def test_rows_of_an_odd_number_of_steps(fmt, N, K, m):
    gen = FMT[fmt][0]
    rng = synth.rng_for(112, N, K, m)
    q, s = gen(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run(fmt, q, s, x)
    check(fmt, q, s, x, y, "%s N=%d K=%d m=%d" % (fmt, N, K, m))


# Whole tiles per wave (many rows) with activation rows that are 4-byte but
# not 16-byte aligned: x is staged into LDS in 4-byte pieces.
@pytest.mark.parametrize("m", [2, 7, 16])
@pytest.mark.parametrize("fmt", ["q8g64", "q8g128", "q8pc"])
def test_whole_tiles_with_unaligned_rows(fmt, m):
    N, K = 70000, 256
    gen = FMT[fmt][0]
    rng = synth.rng_for(113, m)
    q, s = gen(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run(fmt, q, s, x, ldx=K + 2)
    check(fmt, q, s, x, y, "%s N=%d K=%d m=%d ldx=K+2" % (fmt, N, K, m))


# The launch picks how a tile's K is shared: by no wave (many tiles), by
# the four waves of a work-group (4..63 scale groups per row), or by
# sixteen (64 or more groups, when the staged x leaves room in LDS); where
# no split's partial sums fit beside the staged x, four waves share the
# tile and read x from memory.  These shapes reach each choice, with
# uneven shares, ragged tiles and both x load widths.
@pytest.mark.parametrize("fmt,N,K,m,pad", [
    ("q8g64", 1000, 4096, 3, 0),       # 64 groups: sixteen waves, four groups each
    ("q8g64", 17, 4160, 12, 2),        # 65 groups: uneven sixteen-way shares
    ("q8pc", 333, 6400, 9, 0),         # 100 steps over sixteen waves
    ("q8g128", 500, 8192, 5, 0),       # 64 groups of two steps
    ("q8g128", 64, 4096, 16, 0),       # 32 groups: four waves
    ("q8g64", 1000, 4864, 16, 0),      # x fills the LDS: x from memory
    ("q8pc", 700, 4864, 16, 2),        # the same with 4-byte x loads
    ("q8g128", 130, 4864, 16, 8),      # 38 groups, x from memory, 16-byte loads
    ("q8g64", 40, 16384, 16, 0),       # 512 KiB of x: x from memory
])
def test_k_split_choices(fmt, N, K, m, pad):
    gen = FMT[fmt][0]
    rng = synth.rng_for(109, N, K, m)
    q, s = gen(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run(fmt, q, s, x, ldx=K + pad, ldy=N + 1)
    assert np.all(y[:, N:].view(np.uint32) == CANARY_BITS), "wrote past N"
    check(fmt, q, s, x, y[:, :N], "%s N=%d K=%d m=%d" % (fmt, N, K, m))


def test_x_from_memory_without_a_split():
    # Many tiles (no K split) and rows too long to stage: every wave reads
    # x with its items.  Rows are checked against the oracle on slices (the
    # oracle on the whole matrix would take minutes).
    N, K, m = 65600, 5120, 16
    rng = synth.rng_for(122, 0)
    q, s = synth.q8g64_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run("q8g64", q, s, x)
    for lo, hi in ((0, 1500), (31000, 32000), (N - 1500, N)):
        check("q8g64", q[lo:hi], s[lo:hi], x, y[:, lo:hi], "rows %d..%d" % (lo, hi))


def test_every_m_from_2_to_16():
    N, K = 3000, 1024
    rng = synth.rng_for(103, 0)
    q, s = synth.q8g64_weights(rng, N, K)
    w = dev(Q.qpack_q8g64_mma(q, s))
    x = synth.activations(rng, 16, K)
    y_ref, a_ref = oracle.q8g64(q, s, x, threads=THREADS)
    for m in range(2, 17):
        y = run("q8g64", q, s, x[:m], packed=w)
        assert oracle.within_tolerance(y, y_ref[:m], a_ref[:m], TOL).all(), "m=%d" % m


# ------------------------------------------------------- exact arithmetic

@pytest.mark.parametrize("fmt,N,K,m", [("q8g64", 4096, 2560, 16), ("q8g128", 1000, 4096, 9),
                                       ("q8pc", 5120, 1280, 12)])
def test_exact_inputs_bit_exact(fmt, N, K, m):
    rng = synth.rng_for(104, N, K)
    q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    if fmt == "q8pc":
        s = (2.0 ** rng.integers(-40, -30, size=N)).astype(np.float32).view(np.uint32)
    else:
        s = synth.to_fp16_bits(2.0 ** rng.integers(-6, -2, size=(N, K // FMT[fmt][4])))
    x = synth.to_bf16_bits(rng.integers(-4, 5, size=(m, K)).astype(np.float32))
    y = run(fmt, q, s, x)
    y_ref, _ = FMT[fmt][3](q, s, x, threads=THREADS)
    assert np.array_equal(y.astype(np.float64), y_ref)


# -------------------------------------------------------- degenerate cases

@pytest.mark.parametrize("fmt", ["q8g64", "q8g128", "q8pc"])
def test_zero_codes_scales_and_activations_give_exact_zero(fmt):
    gen = FMT[fmt][0]
    rng = synth.rng_for(105, 0)
    q, s = gen(rng, 300, 2560)
    x = synth.activations(rng, 7, 2560)
    assert np.all(run(fmt, np.zeros_like(q), s, x) == 0.0)
    assert np.all(run(fmt, q, np.zeros_like(s), x) == 0.0)
    assert np.all(run(fmt, q, s, np.zeros_like(x)) == 0.0)


# ------------------------------------------------- structural identities

def test_rows_do_not_depend_on_the_batch():
    # Each output row of the matrix product is computed on its own, so the
    # rows of an m = 16 call equal those of m = 2 calls bit for bit.
    N, K = 2000, 2560
    rng = synth.rng_for(106, 0)
    q, s = synth.q8g64_weights(rng, N, K)
    w = dev(Q.qpack_q8g64_mma(q, s))
    x = synth.activations(rng, 16, K)
    y16 = run("q8g64", q, s, x, packed=w)
    for i in (0, 5, 14):
        y2 = run("q8g64", q, s, x[i:i + 2], packed=w)
        assert np.array_equal(y16[i:i + 2], y2)


def test_matches_the_plain_gemv_within_rounding():
    N, K, m = 4000, 2560, 4
    rng = synth.rng_for(107, 0)
    q, s = synth.q8g64_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    y_mma = run("q8g64", q, s, x)
    y = canary((m, N))
    Q.qgemv_q8g64(dev(Q.qpack_q8g64(q, s)), dev(x), y, N, K, m=m)
    _, a_ref = oracle.q8g64(q, s, x, threads=THREADS)
    assert np.all(np.abs(y_mma.astype(np.float64) - host(y)) <= 2 * TOL * a_ref)


def test_route_counter_names_the_variant():
    Q.route_counts_reset()
    rng = synth.rng_for(108, 0)
    q, s = synth.q8pc_weights(rng, 64, 1280)
    run("q8pc", q, s, synth.activations(rng, 11, 1280))
    assert Q.route_count("q8pc_mma_m11") == 1
    assert Q.variant_name(Q.FMT_Q8PC_MMA, 11, 64, 1280) == "q8pc_mma_m11"


@pytest.mark.parametrize("fmt,N,K,m", [("q8pc", 1792, 5120, 8),      # sixteen-wave K split
                                       ("q8g64", 70000, 512, 12),     # whole tiles per wave
                                       ("q8pc", 300, 4864, 16)])      # x read from memory
def test_graph_replays_match_eager_calls(fmt, N, K, m):
    # Captured once, replayed with new activations in place: every replay
    # equals an eager call bit for bit (the K split's LDS fold and the
    # staging are per launch, nothing is recorded that replays differently).
    gen, pack, gemv, _, _ = FMT[fmt]
    rng = synth.rng_for(120, N, K)
    q, s = gen(rng, N, K)
    w = dev(pack(q, s))
    x = dev(synth.activations(rng, m, K))
    y = canary((m, N))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call = Q.bound_mma(fmt, w, x, y, N, K, m=m)
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    for r in range(3):
        x.copy_(dev(synth.activations(synth.rng_for(120, 100 + r), m, K)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(y).copy()
        ye = canary((m, N))
        gemv(w, x, ye, N, K, m=m)
        assert np.array_equal(got, host(ye)), "replay %d" % r


# ------------------------------------------------ per-call variant forcing

@pytest.mark.parametrize("spec", ["ksplit=1", "ksplit=4", "ksplit=16", "ksplit=4,xg=1", "ksplit=4,xg=0",
                                  "mmawaves=64", "policy=0"])
def test_forced_matrix_core_variants_meet_the_bar(spec, monkeypatch):
    # QG_FORCE_VARIANT is read at every call, so one process can force each
    # K split and x path in turn; every one must meet the oracle's bar.
    N, K, m = 1792, 5120, 6
    rng = synth.rng_for(109, 0)
    q, s = synth.q8pc_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    w = dev(Q.qpack_q8pc_mma(q, s))
    monkeypatch.setenv("QG_FORCE_VARIANT", spec)
    y = run("q8pc", q, s, x, packed=w)
    monkeypatch.delenv("QG_FORCE_VARIANT")
    check("q8pc", q, s, x, y, "forced %s" % spec)


def test_work_group_policy_keeps_the_bits():
    # The shape policy only changes how many work-groups share the tiles
    # (even rounds at this shape); each tile is computed the same way.
    N, K, m = 8704, 5120, 4
    rng = synth.rng_for(110, 0)
    q, s = synth.q8pc_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    w = dev(Q.qpack_q8pc_mma(q, s))
    y_policy = run("q8pc", q, s, x, packed=w)
    os.environ["QG_FORCE_VARIANT"] = "policy=0"
    try:
        y_default = run("q8pc", q, s, x, packed=w)
    finally:
        del os.environ["QG_FORCE_VARIANT"]
    assert np.array_equal(y_policy.view(np.uint32), y_default.view(np.uint32))
