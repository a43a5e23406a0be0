"""GPU parity: the HIP path against the fp64 CPU oracle, through the C ABI.

Acceptance per output element (i, n):  |y_gpu - y_ref| <= 2e-3 * sum_k |w x|
(fp64, y_gpu finite).  Exact-arithmetic inputs (integer x in [-4, 4],
power-of-two scales, mins that are multiples of the scale) make every fp32
partial sum exact, so there the GPU must equal the oracle bit for bit.
Every output buffer starts filled with a NaN canary so an unwritten element
fails, and elements outside [0, N) of a strided row must keep the canary.
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
    # A GPU run that finds no device must fail, not skip.
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    Q.lib()


def dev(a: np.ndarray) -> "torch.Tensor":
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
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


def run_q8(q, s, x, m=None, ldx=None, ldy=None, N=None):
    N_, K = q.shape
    packed = dev(Q.qpack_q8g64(q, s))
    m = x.shape[0] if m is None else m
    ldx = K if ldx is None else ldx
    ldy = N_ if ldy is None else ldy
    xb = np.zeros((m, ldx), np.uint16)
    xb[:, :K] = x[:, :K]
    xd = dev(xb)
    y = canary((m, ldy))
    Q.qgemv_q8g64(packed, xd, y, N_, K, m=m, ldx=ldx, ldy=ldy)
    return host(y)


def run_q4(codes, s, mn, x, m=None, ldx=None, ldy=None):
    N_, half_k = codes.shape
    K = 2 * half_k
    packed = dev(Q.qpack_q4g32(codes, s, mn))
    m = x.shape[0] if m is None else m
    ldx = K if ldx is None else ldx
    ldy = N_ if ldy is None else ldy
    xb = np.zeros((m, ldx), np.uint16)
    xb[:, :K] = x[:, :K]
    y = canary((m, ldy))
    Q.qgemv_q4g32(packed, dev(xb), y, N_, K, m=m, ldx=ldx, ldy=ldy)
    return host(y)


def check_canary_tail(y, N):
    tail = y[:, N:].view(np.uint32)
    assert np.all(tail == CANARY_BITS), "wrote past N"


# ----------------------------------------------------------- workload configs

def test_q8_small_1024x1024():
    rng = synth.rng_for(0, 0)
    q, s = synth.q8g64_weights(rng, 1024, 1024)
    x = synth.activations(rng, 1, 1024)
    y = run_q8(q, s, x)
    y_ref, a_ref = oracle.q8g64(q, s, x, threads=THREADS)
    assert_parity(y, y_ref, a_ref, "q8 1024x1024")


@pytest.mark.parametrize("j,label,N,K", [(j,) + tuple(c[:1]) + tuple(c[2:])
                                         for j, c in enumerate(synth.QWEN3_06B_LAYER)])
def test_qwen3_06b_layer(j, label, N, K):
    rng = synth.rng_for(1, j)
    q, s = synth.q8g64_weights(rng, N, K)
    x = synth.activations(rng, 1, K)
    y = run_q8(q, s, x)
    y_ref, a_ref = oracle.q8g64(q, s, x, threads=THREADS)
    assert_parity(y, y_ref, a_ref, "qwen3-0.6b " + label)


@pytest.mark.parametrize("m", [1, 4])
@pytest.mark.parametrize("j,label,N,K", [(j,) + tuple(c[:1]) + tuple(c[2:])
                                         for j, c in enumerate(synth.Q4_K2560)])
def test_q4_k2560(j, label, N, K, m):
    rng = synth.rng_for(2, j)
    codes, s, mn = synth.q4g32_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    y = run_q4(codes, s, mn, x)
    y_ref, a_ref = oracle.q4g32(codes, s, mn, x, threads=THREADS)
    assert_parity(y, y_ref, a_ref, "q4 %s m=%d" % (label, m))


def test_lm_head_full_size():
    # Full lm_head shape in the launch configuration the benchmark times;
    # the oracle covers every row.
    _, _, N, K = synth.LM_HEAD
    rng = synth.rng_for(3, 0)
    q, s = synth.q8g64_weights(rng, N, K)
    x = synth.activations(rng, 1, K)
    y = run_q8(q, s, x)
    y_ref, a_ref = oracle.q8g64(q, s, x, threads=THREADS)
    assert_parity(y, y_ref, a_ref, "lm_head")


def _moe_experts(proj, n_experts, used, seed_base):
    """Canonical experts: real seeded data for the ids in ``used``; every other
    expert holds one shared seeded decoy, so reading a wrong expert shows."""
    N, K = synth.MOE[proj]
    decoy = synth.q4g32_weights(synth.rng_for(seed_base, 999), N, K)
    return [synth.q4g32_weights(synth.rng_for(seed_base, e), N, K) if e in used else decoy
            for e in range(n_experts)], N, K


def _upload_experts(experts, N, K):
    stride = Q.expert_stride(N, K)
    buf = torch.empty(len(experts) * stride, dtype=torch.uint8, device="cuda")
    packed_cache = {}
    for e, ex in enumerate(experts):
        key = id(ex)
        if key not in packed_cache:
            packed_cache[key] = torch.from_numpy(Q.qpack_q4g32(*ex)).to("cuda")
        buf[e * stride:(e + 1) * stride].copy_(packed_cache[key])
    return buf, stride


@pytest.mark.parametrize("proj", ["gate", "up", "down"])
def test_moe_grouped_full_size(proj):
    n_experts, n_slots = synth.MOE["n_experts"], synth.MOE["n_slots"]
    ids = synth.expert_ids(synth.rng_for(4, 1000, 0), n_experts, n_slots)
    experts, N, K = _moe_experts(proj, n_experts, set(ids.tolist()), 40 + ["gate", "up", "down"].index(proj))
    buf, stride = _upload_experts(experts, N, K)
    rng = synth.rng_for(4, 2000)
    if proj == "down":
        xs = synth.activations(rng, n_slots, K)      # one activation per slot
        x_stride = K
    else:
        x1 = synth.activations(rng, 1, K)            # gate/up share the token's x
        xs = np.repeat(x1, n_slots, axis=0)
        x_stride = 0
    y = canary((n_slots, N))
    Q.qgemv_grouped_q4g32(buf, stride, n_experts, dev(ids), dev(xs if x_stride else xs[:1]),
                          x_stride, y, N, N, K)
    y_gpu = host(y)
    y_ref, a_ref = oracle.grouped_q4g32(experts, ids, xs, threads=THREADS)
    assert_parity(y_gpu, y_ref, a_ref, "moe " + proj)


def test_moe_merged_gate_up_full_size():
    # The routed-expert step the benchmark times beside the LM head: each
    # expert's gate and up rows stacked into one 3072 x 4096 matrix, 128
    # experts, 8 routed; the first 1536 outputs of a slot are gate, the rest up.
    n_experts, n_slots = synth.MOE["n_experts"], synth.MOE["n_slots"]
    ids = synth.expert_ids(synth.rng_for(4, 1000, 1), n_experts, n_slots)
    used = set(ids.tolist())
    gate, N, K = _moe_experts("gate", n_experts, used, 43)
    up, _, _ = _moe_experts("up", n_experts, used, 44)
    merged, cache = [], {}
    for g, u in zip(gate, up):
        key = (id(g), id(u))
        if key not in cache:
            cache[key] = tuple(np.concatenate([a, b]) for a, b in zip(g, u))
        merged.append(cache[key])
    buf, stride = _upload_experts(merged, 2 * N, K)
    x1 = synth.activations(synth.rng_for(4, 2001), 1, K)
    y = canary((n_slots, 2 * N))
    Q.qgemv_grouped_q4g32(buf, stride, n_experts, dev(ids), dev(x1), 0, y, 2 * N, 2 * N, K)
    y_gpu = host(y)
    xs = np.repeat(x1, n_slots, axis=0)
    g_ref, g_a = oracle.grouped_q4g32(gate, ids, xs, threads=THREADS)
    u_ref, u_a = oracle.grouped_q4g32(up, ids, xs, threads=THREADS)
    assert_parity(y_gpu[:, :N], g_ref, g_a, "merged gate half")
    assert_parity(y_gpu[:, N:], u_ref, u_a, "merged up half")


# ------------------------------------------------------------ shape sweep

@pytest.mark.parametrize("N", [1, 7, 129, 1000])
@pytest.mark.parametrize("K", [64, 192, 2560])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_q8_ragged_shapes_and_strides(N, K, m):
    rng = synth.rng_for(10, N, K, m)
    q, s = synth.q8g64_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    ldx, ldy = K + 34, N + 5
    y = run_q8(q, s, x, ldx=ldx, ldy=ldy)
    check_canary_tail(y, N)
    y_ref, a_ref = oracle.q8g64(q, s, x, threads=THREADS)
    assert_parity(y[:, :N], y_ref, a_ref, "q8 N=%d K=%d m=%d" % (N, K, m))


@pytest.mark.parametrize("N", [1, 7, 129, 1000])
@pytest.mark.parametrize("K", [32, 96, 1536])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_q4_ragged_shapes_and_strides(N, K, m):
    rng = synth.rng_for(11, N, K, m)
    codes, s, mn = synth.q4g32_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    ldx, ldy = K + 2, N + 3
    y = run_q4(codes, s, mn, x, ldx=ldx, ldy=ldy)
    check_canary_tail(y, N)
    y_ref, a_ref = oracle.q4g32(codes, s, mn, x, threads=THREADS)
    assert_parity(y[:, :N], y_ref, a_ref, "q4 N=%d K=%d m=%d" % (N, K, m))


# ------------------------------------------------------- exact arithmetic

def _exact_x(rng, m, K):
    return synth.to_bf16_bits(rng.integers(-4, 5, size=(m, K)).astype(np.float32))


@pytest.mark.parametrize("N,K,m", [(1024, 1024, 1), (2048, 1024, 4), (1024, 3072, 2), (151936, 2560, 1)])
def test_q8_exact_inputs_bit_exact(N, K, m):
    rng = synth.rng_for(12, N, K)
    q = rng.integers(-128, 128, size=(N, K), dtype=np.int8)      # includes -128
    s = synth.to_fp16_bits(2.0 ** rng.integers(-6, -2, size=(N, K // 64)))
    x = _exact_x(rng, m, K)
    y = run_q8(q, s, x)
    y_ref, _ = oracle.q8g64(q, s, x, threads=THREADS)
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("N,K,m", [(9216, 2560, 4), (2560, 9216, 1), (1536, 4096, 1), (4096, 1536, 3)])
def test_q4_exact_inputs_bit_exact(N, K, m):
    rng = synth.rng_for(13, N, K)
    codes, _, _ = synth.q4g32_weights(rng, N, K)
    e = rng.integers(-6, -2, size=(N, K // 32))
    s = synth.to_fp16_bits(2.0 ** e)
    mn = synth.to_fp16_bits(-(2.0 ** e) * rng.integers(0, 9, size=(N, K // 32)))
    x = _exact_x(rng, m, K)
    y = run_q4(codes, s, mn, x)
    y_ref, _ = oracle.q4g32(codes, s, mn, x, threads=THREADS)
    assert np.array_equal(y.astype(np.float64), y_ref)


# -------------------------------------------------------- degenerate cases

def test_zero_scales_and_zero_codes_give_exact_zero():
    rng = synth.rng_for(14, 0)
    q, s = synth.q8g64_weights(rng, 300, 2560)
    x = synth.activations(rng, 2, 2560)
    assert np.all(run_q8(q, np.zeros_like(s), x) == 0.0)
    assert np.all(run_q8(np.zeros_like(q), s, x) == 0.0)
    codes, s4, mn4 = synth.q4g32_weights(rng, 300, 1536)
    x4 = synth.activations(rng, 3, 1536)
    assert np.all(run_q4(codes, np.zeros_like(s4), np.zeros_like(mn4), x4) == 0.0)
    assert np.all(run_q4(np.zeros_like(codes), s4, np.zeros_like(mn4), x4) == 0.0)


def test_zero_activation_gives_exact_zero():
    rng = synth.rng_for(14, 1)
    q, s = synth.q8g64_weights(rng, 64, 1024)
    x = np.zeros((1, 1024), np.uint16)
    assert np.all(run_q8(q, s, x) == 0.0)


def test_extreme_codes_and_scales():
    # int8 -128 and 127, the largest fp16 scale, subnormal fp16 scales.
    N, K = 16, 256
    q = np.where(np.arange(K)[None, :] % 2 == 0, -128, 127).astype(np.int8).repeat(N, 0)
    s = np.full((N, K // 64), 0x7BFF, np.uint16)        # 65504
    s[1::2] = 0x0001                                      # 2^-24 (subnormal)
    x = synth.activations(synth.rng_for(14, 2), 1, K)
    y = run_q8(q, s, x)
    y_ref, a_ref = oracle.q8g64(q, s, x)
    assert_parity(y, y_ref, a_ref, "extreme q8")


# ------------------------------------------------- structural identities

def test_m4_rows_equal_m1_calls_bitwise():
    rng = synth.rng_for(15, 0)
    q, s = synth.q8g64_weights(rng, 777, 2560)
    x = synth.activations(rng, 4, 2560)
    y4 = run_q8(q, s, x)
    for i in range(4):
        assert np.array_equal(y4[i], run_q8(q, s, x[i:i + 1])[0])
    codes, s4, mn4 = synth.q4g32_weights(rng, 777, 2560)
    y4 = run_q4(codes, s4, mn4, x)
    for i in range(4):
        assert np.array_equal(y4[i], run_q4(codes, s4, mn4, x[i:i + 1])[0])


def test_repeat_calls_are_bitwise_identical():
    rng = synth.rng_for(15, 1)
    codes, s, mn = synth.q4g32_weights(rng, 9216, 2560)
    packed = dev(Q.qpack_q4g32(codes, s, mn))
    x = dev(synth.activations(rng, 1, 2560))
    outs = []
    for _ in range(3):
        y = canary((1, 9216))
        Q.qgemv_q4g32(packed, x, y, 9216, 2560)
        outs.append(host(y))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_grouped_slots_equal_single_calls_and_bad_ids_give_nan():
    n_experts, N, K = 12, 300, 1536
    experts = [synth.q4g32_weights(synth.rng_for(16, e), N, K) for e in range(n_experts)]
    buf, stride = _upload_experts(experts, N, K)
    ids = np.array([3, 11, 0, 3, -1, 12, 7], np.int32)    # repeats and two bad ids
    xs = synth.activations(synth.rng_for(16, 100), len(ids), K)
    y = canary((len(ids), N + 4))
    Q.qgemv_grouped_q4g32(buf, stride, n_experts, dev(ids), dev(xs), K, y, N + 4, N, K)
    y = host(y)
    for j, e in enumerate(ids):
        if 0 <= e < n_experts:
            packed = dev(Q.qpack_q4g32(*experts[e]))
            yj = canary((1, N))
            Q.qgemv_q4g32(packed, dev(xs[j:j + 1]), yj, N, K)
            assert np.array_equal(y[j, :N], host(yj)[0])
        else:
            assert np.all(np.isnan(y[j, :N]))
        assert np.all(y[j, N:].view(np.uint32) == CANARY_BITS)


def test_route_counters_name_the_launched_variant():
    rng = synth.rng_for(17, 0)
    q, s = synth.q8g64_weights(rng, 64, 2560)
    Q.route_counts_reset()
    run_q8(q, s, synth.activations(rng, 3, 2560))
    assert Q.route_count(Q.variant_name(0, 3, 64, 2560)) == 1
    assert Q.route_count(Q.variant_name(0, 1, 64, 2560)) == 0


def test_graph_replays_match_eager_calls():
    # Decode loops replay captured launches.  Capture one dense and one
    # grouped call, replay several times with eager work (new activations)
    # between replays, and compare every replay with the eager result.
    rng = synth.rng_for(18, 0)
    q, s = synth.q8g64_weights(rng, 1000, 2560)
    w = dev(Q.qpack_q8g64(q, s))
    experts = [synth.q4g32_weights(synth.rng_for(18, e), 256, 1536) for e in range(6)]
    buf, stride = _upload_experts(experts, 256, 1536)
    ids = dev(np.array([5, 2, 0], np.int32))
    x = dev(synth.activations(rng, 1, 2560))
    xg = dev(synth.activations(rng, 3, 1536))
    y = canary((1, 1000))
    yg = canary((3, 256))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dense = Q.bound_q8g64(w, x, y, 1000, 2560)
        grouped = Q.bound_grouped_q4g32(buf, stride, 6, ids, xg, 1536, yg, 256, 256, 1536)
        dense()
        grouped()                                   # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dense()
        grouped()
    for r in range(4):
        x.copy_(dev(synth.activations(synth.rng_for(18, 100 + r), 1, 2560)))
        xg.copy_(dev(synth.activations(synth.rng_for(18, 200 + r), 3, 1536)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got, got_g = host(y).copy(), host(yg).copy()
        ye, yge = canary((1, 1000)), canary((3, 256))
        Q.qgemv_q8g64(w, x, ye, 1000, 2560)
        Q.qgemv_grouped_q4g32(buf, stride, 6, ids, xg, 1536, yge, 256, 256, 1536)
        assert np.array_equal(got, host(ye)), "replay %d dense" % r
        assert np.array_equal(got_g, host(yge)), "replay %d grouped" % r


@pytest.mark.parametrize("fmt,parts,K", [
    ("q8g64", (2048, 1024, 1024), 1024),     # q, k, v of the 0.6B layer
    ("q8g64", (3072, 3072), 1024),           # gate, up
    ("q4g32", (9216, 9216), 2560),
    ("q8g128", (701, 1299), 2048),           # a part ending inside a tile
    ("q8pc", (8704, 8704), 5120)])
@pytest.mark.parametrize("m", [1, 2])
def test_stacked_rows_equal_separate_calls_bitwise(fmt, parts, K, m):
    # A matrix made of several matrices' rows stacked in order (the stacked
    # projections of a layer) gives each part's outputs bit for bit, because
    # every output row is computed the same way in any matrix, whatever
    # launch shape the stacked and the separate calls take (at m = 1 the
    # stacked gate+up matrices hold x in registers, their parts stage it).
    gen = {"q8g64": synth.q8g64_weights, "q4g32": synth.q4g32_weights,
           "q8g128": synth.q8g128_weights, "q8pc": synth.q8pc_weights}[fmt]
    pack = getattr(Q, "qpack_" + fmt)
    call = getattr(Q, "qgemv_" + fmt)
    mats = [gen(synth.rng_for(20, j, K), N, K) for j, N in enumerate(parts)]
    stacked = tuple(np.concatenate(arrs) for arrs in zip(*mats))
    x = dev(synth.activations(synth.rng_for(20, 99, K), m, K))
    Ns = sum(parts)
    ys = canary((m, Ns))
    call(dev(pack(*stacked)), x, ys, Ns, K)
    ys = host(ys)
    off = 0
    for j, (w, N) in enumerate(zip(mats, parts)):
        y = canary((m, N))
        call(dev(pack(*w)), x, y, N, K)
        assert np.array_equal(host(y).view(np.uint32), ys[:, off:off + N].view(np.uint32)), "part %d" % j
        off += N


def test_merged_gate_up_equals_separate_calls_bitwise():
    # Stacking each expert's gate and up rows into one [2N][K] matrix is a row
    # concatenation; every output row is computed the same way, so the merged
    # grouped call must equal the two separate calls bit for bit.
    n_experts, N, K = 5, 384, 4096
    gate = [synth.q4g32_weights(synth.rng_for(19, 0, e), N, K) for e in range(n_experts)]
    up = [synth.q4g32_weights(synth.rng_for(19, 1, e), N, K) for e in range(n_experts)]
    merged = [tuple(np.concatenate([a, b]) for a, b in zip(g, u)) for g, u in zip(gate, up)]
    bg, sg = _upload_experts(gate, N, K)
    bu, su = _upload_experts(up, N, K)
    bm, sm = _upload_experts(merged, 2 * N, K)
    ids = dev(np.array([4, 1, 3], np.int32))
    x = dev(synth.activations(synth.rng_for(19, 9), 1, K))
    yg, yu, ym = canary((3, N)), canary((3, N)), canary((3, 2 * N))
    Q.qgemv_grouped_q4g32(bg, sg, n_experts, ids, x, 0, yg, N, N, K)
    Q.qgemv_grouped_q4g32(bu, su, n_experts, ids, x, 0, yu, N, N, K)
    Q.qgemv_grouped_q4g32(bm, sm, n_experts, ids, x, 0, ym, 2 * N, 2 * N, K)
    ym = host(ym)
    assert np.array_equal(ym[:, :N], host(yg)) and np.array_equal(ym[:, N:], host(yu))
