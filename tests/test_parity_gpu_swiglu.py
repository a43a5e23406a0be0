"""GPU parity for the routed-expert gate+up call with the SwiGLU epilogue
(qgemv_grouped_q4g32_swiglu), through the C ABI.

Acceptance per output (slot j, n): the bf16 result is within
oracle.swiglu_tolerance of the fp64 oracle's silu(g) * u, a bound derived
from the GEMV bar (|g' - g| <= 2e-3 sum|w x|, same for u), the slope of
silu and bf16 rounding.  Outputs start as a canary so unwritten elements
fail, and elements past N of each slot must keep it.
"""
import os

import numpy as np
import pytest

import oracle
from weight_only_block_amd import qgemv as Q
from weight_only_block_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
CANARY16 = 0x7FAB          # a NaN pattern the kernel never writes
NAN16 = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    Q.lib()


def dev(a: np.ndarray) -> "torch.Tensor":
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def act_canary(rows, cols):
    return torch.full((rows, cols), CANARY16, dtype=torch.int16, device="cuda")


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def upload_pairs(gates, ups, N, K):
    """One gate/up pair buffer per expert at the minimum stride."""
    stride = Q.gate_up_expert_stride(N, K)
    buf = torch.empty(len(gates) * stride, dtype=torch.uint8, device="cuda")
    cache = {}
    for e, (g, u) in enumerate(zip(gates, ups)):
        key = (id(g), id(u))
        if key not in cache:
            cache[key] = torch.from_numpy(Q.qpack_q4g32_gate_up(g, u)).to("cuda")
        buf[e * stride:(e + 1) * stride].copy_(cache[key])
    return buf, stride


def run_swiglu(buf, stride, n_experts, ids, xs, x_stride, N, K, act_stride=None):
    act_stride = N if act_stride is None else act_stride
    act = act_canary(len(ids), act_stride)
    Q.qgemv_grouped_q4g32_swiglu(buf, stride, n_experts, dev(np.asarray(ids, np.int32)), dev(xs),
                                 x_stride, act, act_stride, N, K)
    return host(act).view(np.uint16)


def assert_swiglu_parity(act_bits, gates, ups, ids, xs_full, N, what):
    act = bf16_to_f64(act_bits[:, :N])
    ref, g, u, a_g, a_u = oracle.grouped_q4g32_swiglu(gates, ups, ids, xs_full, threads=THREADS)
    tol = oracle.swiglu_tolerance(ref, g, u, a_g, a_u)
    ok = np.isfinite(act) & (np.abs(act - ref) <= tol)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        raise AssertionError("%s: %d of %d outside tolerance, e.g. %s" % (
            what, (~ok).sum(), ok.size,
            [(tuple(b), act[tuple(b)], ref[tuple(b)], tol[tuple(b)]) for b in bad]))


# ----------------------------------------------------------- workload config

def test_moe_gate_up_swiglu_full_size():
    # 128 experts of gate/up 4096 -> 1536, 8 routed per token, shared x.
    n_experts, n_slots = synth.MOE["n_experts"], synth.MOE["n_slots"]
    N, K = synth.MOE["gate"]
    ids = synth.expert_ids(synth.rng_for(60, 0), n_experts, n_slots)
    used = set(ids.tolist())
    decoy_g = synth.q4g32_weights(synth.rng_for(60, 998), N, K)
    decoy_u = synth.q4g32_weights(synth.rng_for(60, 999), N, K)
    gates = [synth.q4g32_weights(synth.rng_for(61, e), N, K) if e in used else decoy_g
             for e in range(n_experts)]
    ups = [synth.q4g32_weights(synth.rng_for(62, e), N, K) if e in used else decoy_u
           for e in range(n_experts)]
    buf, stride = upload_pairs(gates, ups, N, K)
    x1 = synth.activations(synth.rng_for(60, 1), 1, K)
    act = run_swiglu(buf, stride, n_experts, ids, x1, 0, N, K)
    assert_swiglu_parity(act, gates, ups, ids, np.repeat(x1, n_slots, axis=0), N, "moe gate/up")


# ------------------------------------------------------------- shape sweep

@pytest.mark.parametrize("N", [1, 7, 100, 1000])
@pytest.mark.parametrize("K", [32, 96, 1536, 4096])
@pytest.mark.parametrize("shared_x", [True, False])
def test_ragged_shapes_and_strides(N, K, shared_x):
    n_experts = 5
    gates = [synth.q4g32_weights(synth.rng_for(63, N, K, e), N, K) for e in range(n_experts)]
    ups = [synth.q4g32_weights(synth.rng_for(64, N, K, e), N, K) for e in range(n_experts)]
    buf, stride = upload_pairs(gates, ups, N, K)
    ids = [4, 0, 2]
    rng = synth.rng_for(65, N, K)
    if shared_x:
        x1 = synth.activations(rng, 1, K)
        xs, x_stride, xs_full = x1, 0, np.repeat(x1, len(ids), axis=0)
    else:
        xs_full = synth.activations(rng, len(ids), K)
        xb = np.zeros((len(ids), K + 6), np.uint16)
        xb[:, :K] = xs_full
        xs, x_stride = xb, K + 6
    act = run_swiglu(buf, stride, n_experts, ids, xs, x_stride, N, K, act_stride=N + 3)
    assert np.all(act[:, N:] == CANARY16), "wrote past N"
    assert_swiglu_parity(act, gates, ups, ids, xs_full, N, "N=%d K=%d" % (N, K))


# ------------------------------------------------------- exact arithmetic

@pytest.mark.parametrize("N,K", [(1536, 4096), (300, 1536), (64, 32)])
def test_exact_gemv_sums_leave_only_the_epilogue_rounding(N, K):
    # Power-of-two scales, mins that are multiples of the scale and integer x
    # make g and u exact in fp32 on both sides; what remains is fp32 silu and
    # the bf16 rounding.
    rng = synth.rng_for(66, N, K)

    def exact(seed):
        r = synth.rng_for(67, seed, N, K)
        codes, _, _ = synth.q4g32_weights(r, N, K)
        e = r.integers(-6, -2, size=(N, K // 32))
        s = synth.to_fp16_bits(2.0 ** e)
        mn = synth.to_fp16_bits(-(2.0 ** e) * r.integers(0, 9, size=(N, K // 32)))
        return codes, s, mn

    gates, ups = [exact(0), exact(1)], [exact(2), exact(3)]
    buf, stride = upload_pairs(gates, ups, N, K)
    ids = [1, 0]
    xs = synth.to_bf16_bits(rng.integers(-4, 5, size=(2, K)).astype(np.float32))
    act = bf16_to_f64(run_swiglu(buf, stride, 2, ids, xs, K, N, K))
    ref = oracle.grouped_q4g32_swiglu(gates, ups, ids, xs, threads=THREADS)[0]
    # bf16 rounding (8 significant bits) plus the fp32 evaluation of silu;
    # below the smallest normal bf16 an output may also come out as zero.
    assert np.all(np.abs(act - ref) <= (2.0 ** -8 + 2.0 ** -19) * np.abs(ref) + 2.0 ** -126)


def test_epilogue_applies_to_the_plain_gemv_sums():
    # The same pair buffer through the plain grouped call (as a 2*N-row
    # matrix in the pair order) gives the fp32 gate and up sums; the fused
    # call must equal bf16(silu(g) * u) of exactly those sums, up to one
    # bf16 ulp for the fp32 evaluation of silu.
    n_experts, N, K = 4, 1000, 1536
    gates = [synth.q4g32_weights(synth.rng_for(68, 0, e), N, K) for e in range(n_experts)]
    ups = [synth.q4g32_weights(synth.rng_for(68, 1, e), N, K) for e in range(n_experts)]
    buf, stride = upload_pairs(gates, ups, N, K)
    ids = [3, 1, 2, 3]
    xs = synth.activations(synth.rng_for(68, 9), len(ids), K)
    act = run_swiglu(buf, stride, n_experts, ids, xs, K, N, K)
    G = int(Q.variant_name(Q.FMT_GROUPED_Q4G32_SWIGLU, 1, N, K).split("_g")[-1].split("_")[0])
    rps = 64 // G
    Nv = 2 * (-(-N // rps)) * rps
    y = torch.empty((len(ids), Nv), dtype=torch.float32, device="cuda")
    Q.qgemv_grouped_q4g32(buf, stride, n_experts, dev(np.asarray(ids, np.int32)), dev(xs), K,
                          y, Nv, Nv, K)
    y = host(y).astype(np.float64)
    n = np.arange(N)
    v_gate = (n // rps) * 2 * rps + n % rps
    g, u = y[:, v_gate], y[:, v_gate + rps]
    want = oracle.swiglu(g, u)
    got = bf16_to_f64(act)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 2.0 ** -126))) - 7)
    assert np.all(np.abs(got - want) <= ulp + 2.0 ** -126 * (np.abs(want) < 2.0 ** -126))


# -------------------------------------------------------- degenerate cases

def test_bad_ids_give_nan_and_good_slots_are_unaffected():
    n_experts, N, K = 6, 200, 1536
    gates = [synth.q4g32_weights(synth.rng_for(69, 0, e), N, K) for e in range(n_experts)]
    ups = [synth.q4g32_weights(synth.rng_for(69, 1, e), N, K) for e in range(n_experts)]
    buf, stride = upload_pairs(gates, ups, N, K)
    ids = np.array([2, -1, 5, 6, 0], np.int32)
    xs = synth.activations(synth.rng_for(69, 2), len(ids), K)
    act = run_swiglu(buf, stride, n_experts, ids, xs, K, N, K, act_stride=N + 2)
    for j, e in enumerate(ids):
        if 0 <= e < n_experts:
            assert_swiglu_parity(act[j:j + 1], gates, ups, [e], xs[j:j + 1], N, "slot %d" % j)
        else:
            assert np.all(act[j, :N] == NAN16)
        assert np.all(act[j, N:] == CANARY16)


def test_zero_gate_gives_exact_zero():
    N, K = 256, 1536
    g = synth.q4g32_weights(synth.rng_for(70, 0), N, K)
    u = synth.q4g32_weights(synth.rng_for(70, 1), N, K)
    zero = (g[0], np.zeros_like(g[1]), np.zeros_like(g[2]))
    buf, stride = upload_pairs([zero], [u], N, K)
    act = run_swiglu(buf, stride, 1, [0, 0], synth.activations(synth.rng_for(70, 2), 2, K), K, N, K)
    assert np.all(bf16_to_f64(act) == 0.0)


# ------------------------------------------------- structural identities

def upload_downs(downs, N, K):
    ds = Q.expert_stride(N, K)
    dbuf = torch.zeros(len(downs) * ds, dtype=torch.uint8, device="cuda")
    for e, d in enumerate(downs):
        p = torch.from_numpy(Q.qpack_q4g32(*d))
        dbuf[e * ds:e * ds + p.numel()].copy_(p)
    return dbuf, ds


def run_chain(buf, stride, dbuf, ds, n_experts, ids, xs, x_stride, Ng, Kg):
    """gate/up + SwiGLU, then the down projection reading that activation."""
    n = len(ids)
    ids_d = dev(np.asarray(ids, np.int32))
    act = act_canary(n, Ng)
    y = torch.full((n, Kg), 0x7FC0DEAD, dtype=torch.int32, device="cuda").view(torch.float32)
    Q.qgemv_grouped_q4g32_swiglu(buf, stride, n_experts, ids_d, dev(xs), x_stride, act, Ng, Ng, Kg)
    Q.qgemv_grouped_q4g32(dbuf, ds, n_experts, ids_d, act, Ng, y, Kg, Kg, Ng)
    return host(act).view(np.uint16), host(y)


def test_down_projection_consumes_the_activation():
    # The fused call's output is the down projection's input: the chain
    # gate/up+SwiGLU -> down (grouped, per-slot x = act) against the
    # oracle's MLP, y = Down bf16(silu(Gate x) Up x), within the bound
    # oracle.expert_mlp_tolerance derives from the GEMV bar of both calls.
    n_experts, n_slots = 8, 4
    Ng, Kg = 512, 1024
    gates = [synth.q4g32_weights(synth.rng_for(71, 0, e), Ng, Kg) for e in range(n_experts)]
    ups = [synth.q4g32_weights(synth.rng_for(71, 1, e), Ng, Kg) for e in range(n_experts)]
    downs = [synth.q4g32_weights(synth.rng_for(71, 2, e), Kg, Ng) for e in range(n_experts)]
    buf, stride = upload_pairs(gates, ups, Ng, Kg)
    dbuf, ds = upload_downs(downs, Kg, Ng)
    ids = [6, 1, 3, 0]
    x = synth.activations(synth.rng_for(71, 3), 1, Kg)
    act, y = run_chain(buf, stride, dbuf, ds, n_experts, ids, x, 0, Ng, Kg)
    ref = oracle.expert_mlp(gates, ups, downs, ids, np.repeat(x, n_slots, axis=0), threads=THREADS)
    tol_act, tol_y = oracle.expert_mlp_tolerance(ref, downs, ids, threads=THREADS)
    assert np.all(np.abs(bf16_to_f64(act) - ref.act) <= tol_act)
    assert np.all(np.isfinite(y)) and np.all(np.abs(y.astype(np.float64) - ref.y) <= tol_y)


def exact_mlp_experts(seed, n_experts, hidden, inter):
    """Experts on which every sum of the chain is exact in fp32 for a
    one-hot x of value 1: gate weights 16 c + 256 (g in [256, 496], so
    silu(g) = g in fp32 and fp64), up weights c - 8, act = g u with at most
    8 significant bits (16 (16 + c) (c' - 8)), down weights c / 16 - 1/2,
    so y is an integer below 2^22."""
    def mk(kind, e, N, K, scale, minv):
        codes, _, _ = synth.q4g32_weights(synth.rng_for(92, seed, kind, e), N, K)
        return (codes, synth.to_fp16_bits(np.full((N, K // 32), scale)),
                synth.to_fp16_bits(np.full((N, K // 32), minv)))
    return ([mk(0, e, inter, hidden, 16.0, 256.0) for e in range(n_experts)],
            [mk(1, e, inter, hidden, 1.0, -8.0) for e in range(n_experts)],
            [mk(2, e, hidden, inter, 1.0 / 16, -0.5) for e in range(n_experts)])


def test_chain_bit_exact_on_exact_inputs():
    # Routed-expert shape (gate/up 4096 -> 1536, down 1536 -> 4096), per-slot
    # one-hot x: act and y must equal the oracle's bit for bit.
    Ng, Kg = synth.MOE["gate"]
    gates, ups, downs = exact_mlp_experts(0, 5, Kg, Ng)
    buf, stride = upload_pairs(gates, ups, Ng, Kg)
    dbuf, ds = upload_downs(downs, Kg, Ng)
    ids = [3, 0, 4, 4, 1, 2, 0, 3]
    xs = np.zeros((len(ids), Kg + 2), np.uint16)
    xs[np.arange(len(ids)), synth.rng_for(93, 0).integers(0, Kg, len(ids))] = 0x3F80   # 1.0
    act, y = run_chain(buf, stride, dbuf, ds, 5, ids, xs, Kg + 2, Ng, Kg)
    ref = oracle.expert_mlp(gates, ups, downs, ids, xs[:, :Kg], threads=THREADS)
    assert np.array_equal(bf16_to_f64(ref.act_bits), ref.act), "inputs not exact"
    assert np.array_equal(act, ref.act_bits)
    assert np.array_equal(y.astype(np.float64), ref.y)


def test_graph_replays_match_eager_calls():
    n_experts, N, K = 6, 384, 4096
    gates = [synth.q4g32_weights(synth.rng_for(72, 0, e), N, K) for e in range(n_experts)]
    ups = [synth.q4g32_weights(synth.rng_for(72, 1, e), N, K) for e in range(n_experts)]
    buf, stride = upload_pairs(gates, ups, N, K)
    ids = dev(np.array([5, 2, 0], np.int32))
    x = dev(synth.activations(synth.rng_for(72, 2), 1, K))
    act = act_canary(3, N)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call = Q.bound_grouped_q4g32_swiglu(buf, stride, n_experts, ids, x, 0, act, N, N, K)
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    for r in range(3):
        x.copy_(dev(synth.activations(synth.rng_for(72, 100 + r), 1, K)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(act).copy()
        eager = act_canary(3, N)
        Q.qgemv_grouped_q4g32_swiglu(buf, stride, n_experts, ids, x, 0, eager, N, N, K)
        assert np.array_equal(got, host(eager)), "replay %d" % r


def test_route_counter_names_the_swiglu_variant():
    N, K = 128, 1536
    g = synth.q4g32_weights(synth.rng_for(73, 0), N, K)
    u = synth.q4g32_weights(synth.rng_for(73, 1), N, K)
    buf, stride = upload_pairs([g], [u], N, K)
    Q.route_counts_reset()
    run_swiglu(buf, stride, 1, [0], synth.activations(synth.rng_for(73, 2), 1, K), 0, N, K)
    name = Q.variant_name(Q.FMT_GROUPED_Q4G32_SWIGLU, 1, N, K)
    assert name.startswith("q4g32_grouped_swiglu_m1_")
    assert Q.route_count(name) == 1
