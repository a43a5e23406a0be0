"""GPU: the VALU kernels give the same bits under every launch geometry.

qg_set_launch_override changes how tiles map to waves (total wave count,
contiguous runs or a grid-stride sweep, ring depth 2 or 4, or x held in
registers with a ring of one tile), and QG_FORCE_VARIANT does the same per
call.  Each tile is
computed the same way under any mapping, so every output must equal the
default launch's bit for bit; the default itself is checked against the
oracle.  Few waves give each wave hundreds of tiles, which drives the
routed-expert SwiGLU epilogue through many full batches and a partial one,
and the grid-stride sweep gives the batch tiles that are not adjacent.
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
CANARY16 = 0x7FAB

# (target_waves, contig, ring_depth); the first entry is the default.
# ring_depth 1 holds x in registers (where the layout allows it).
GEOMETRIES = [(0, -1, 0), (1, 1, 2), (1, 0, 4), (3, 0, 4), (7, 1, 4), (64, 0, 2), (4096, 1, 2),
              (4096, 0, 4), (0, -1, 1), (1, 1, 1), (7, 0, 1), (4096, 1, 1)]
# The same choices through QG_FORCE_VARIANT, which the library reads at every
# call (the override above must be at its default for it to apply).
FORCED = ["ring=xr", "waves=5,contig=0,ring=xr", "wpcu=2,contig=1,ring=4", "waves=3,ring=2", "policy=0"]


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    Q.lib()


@pytest.fixture(autouse=True)
def _restore_default_geometry():
    Q.set_launch_override()
    yield
    Q.set_launch_override()


def dev(a: np.ndarray) -> "torch.Tensor":
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def over_geometries(run):
    """run() -> numpy array of output bits; returns the default's result
    after checking that every other geometry reproduces it exactly."""
    results = []
    for geo in GEOMETRIES:
        Q.set_launch_override(*geo)
        results.append((geo, run()))
    Q.set_launch_override()
    for spec in FORCED:
        os.environ["QG_FORCE_VARIANT"] = spec
        try:
            results.append((spec, run()))
        finally:
            del os.environ["QG_FORCE_VARIANT"]
    base = results[0][1]
    for geo, r in results[1:]:
        diff = np.argwhere(r != base)
        assert diff.size == 0, "geometry %s differs from the default at %d outputs, e.g. %s" % (
            geo, len(diff), [tuple(d) for d in diff[:4]])
    return base


@pytest.mark.parametrize("N,K", [(1000, 4096), (777, 2048), (1000, 1536), (130, 96), (65, 32)])
def test_swiglu_batches_under_every_geometry(N, K):
    # G = 64, 32, 16, 1, 1: gate/up sums transposed onto lane bit 5, bit 4,
    # or kept in two registers; batches of 32, 16, 16 and 1 tiles.
    n_experts = 4
    gates = [synth.q4g32_weights(synth.rng_for(90, N, K, e), N, K) for e in range(n_experts)]
    ups = [synth.q4g32_weights(synth.rng_for(91, N, K, e), N, K) for e in range(n_experts)]
    stride = Q.gate_up_expert_stride(N, K)
    buf = torch.empty(n_experts * stride, dtype=torch.uint8, device="cuda")
    for e in range(n_experts):
        buf[e * stride:(e + 1) * stride].copy_(torch.from_numpy(Q.qpack_q4g32_gate_up(gates[e], ups[e])))
    ids = np.array([3, 0, 2], np.int32)
    xs = synth.activations(synth.rng_for(92, N, K), len(ids), K)
    ids_d, xs_d = dev(ids), dev(xs)

    def run():
        act = torch.full((len(ids), N + 5), CANARY16, dtype=torch.int16, device="cuda")
        Q.qgemv_grouped_q4g32_swiglu(buf, stride, n_experts, ids_d, xs_d, K, act, N + 5, N, K)
        return host(act).view(np.uint16)

    act = over_geometries(run)
    assert np.all(act[:, N:] == CANARY16), "wrote past N"
    ref, g, u, a_g, a_u = oracle.grouped_q4g32_swiglu(gates, ups, ids, xs, threads=THREADS)
    got = (act[:, :N].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    tol = oracle.swiglu_tolerance(ref, g, u, a_g, a_u)
    ok = np.isfinite(got) & (np.abs(got - ref) <= tol)
    assert ok.all(), "%d of %d outside tolerance" % ((~ok).sum(), ok.size)


@pytest.mark.parametrize("N,K", [(1000, 1536), (513, 4096)])
def test_grouped_under_every_geometry(N, K):
    n_experts = 5
    experts = [synth.q4g32_weights(synth.rng_for(93, N, K, e), N, K) for e in range(n_experts)]
    stride = Q.expert_stride(N, K)
    buf = torch.cat([torch.from_numpy(Q.qpack_q4g32(*e)) for e in experts]).to("cuda")
    ids = np.array([4, 1, 1, 0], np.int32)
    xs = synth.activations(synth.rng_for(94, N, K), len(ids), K)
    ids_d, xs_d = dev(ids), dev(xs)

    def run():
        y = torch.full((len(ids), N + 3), float("nan"), dtype=torch.float32, device="cuda")
        Q.qgemv_grouped_q4g32(buf, stride, n_experts, ids_d, xs_d, K, y, N + 3, N, K)
        return host(y).view(np.uint32)

    y = over_geometries(run).view(np.float32)
    assert np.all(np.isnan(y[:, N:])), "wrote past N"
    y_ref, a_ref = oracle.grouped_q4g32(experts, ids, xs, threads=THREADS)
    assert oracle.within_tolerance(y[:, :N], y_ref, a_ref, 2e-3).all()


@pytest.mark.parametrize("fmt,m,N,K", [("q8g64", 1, 3001, 2560), ("q8g64", 4, 1000, 1024),
                                       ("q4g32", 2, 1000, 2560), ("q8g128", 3, 700, 1024),
                                       ("q8pc", 1, 2049, 640)])
def test_dense_under_every_geometry(fmt, m, N, K):
    rng = synth.rng_for(95, m, N, K)
    if fmt == "q4g32":
        wts = synth.q4g32_weights(rng, N, K)
    elif fmt == "q8g128":
        wts = synth.q8g128_weights(rng, N, K)
    elif fmt == "q8pc":
        wts = synth.q8pc_weights(rng, N, K)
    else:
        wts = synth.q8g64_weights(rng, N, K)
    w = dev(getattr(Q, "qpack_" + fmt)(*wts))
    x = dev(synth.activations(rng, m, K))

    def run():
        y = torch.full((m, N), float("nan"), dtype=torch.float32, device="cuda")
        getattr(Q, "qgemv_" + fmt)(w, x, y, N, K)
        return host(y).view(np.uint32)

    y = over_geometries(run).view(np.float32)
    y_ref, a_ref = getattr(oracle, fmt)(*wts, host(x).view(np.uint16), threads=THREADS)
    assert oracle.within_tolerance(y, y_ref, a_ref, 2e-3).all()


def test_fused_argmax_under_every_geometry():
    m, N, K = 2, 5000, 1024
    rng = synth.rng_for(96, N, K)
    q, s = synth.q8g64_weights(rng, N, K)
    w = dev(Q.qpack_q8g64(q, s))
    x = dev(synth.activations(rng, m, K))
    ws = torch.zeros(Q.argmax_workspace_size(m), dtype=torch.uint8, device="cuda")

    def run():
        logits = torch.empty((m, N), dtype=torch.float32, device="cuda")
        idx = torch.full((m,), -1, dtype=torch.int32, device="cuda")
        Q.qgemv_q8g64_argmax(w, x, logits, idx, ws, N, K, m=m)
        return np.concatenate([host(logits).view(np.uint32).ravel(), host(idx).view(np.uint32)])

    out = over_geometries(run)
    logits = out[:m * N].view(np.float32).reshape(m, N)
    idx = out[m * N:].view(np.int32)
    for i in range(m):
        row = logits[i].astype(np.float64)
        assert idx[i] == int(np.flatnonzero(row == row.max())[0])
