"""GPU: the largest activations and slot counts the VALU kernels accept.

The staged activation rows (bf16 plus one fp32 sum per unit, for m rows) must
fit in the 159 KiB of dynamic LDS a work-group may use.  For each format and
row count the test finds the largest K the library accepts (its own check,
through qg_variant_name), confirms that one more scale group is rejected
with QG_ERR_UNSUPPORTED, and checks the call at that K against the oracle.
These launches stage x over many rounds and use more than the default
64 KiB of dynamic LDS.  The grouped calls are also run at their 64-slot limit.
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
FMT_ID = {"q8g64": Q.FMT_Q8G64, "q4g32": Q.FMT_Q4G32, "q8g128": Q.FMT_Q8G128, "q8pc": Q.FMT_Q8PC}
STEP = {"q8g64": 64, "q4g32": 32, "q8g128": 128, "q8pc": 16}


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    Q.lib()


def dev(a: np.ndarray) -> "torch.Tensor":
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def accepted(fmt, m, N, K):
    try:
        Q.variant_name(FMT_ID[fmt], m, N, K)
        return True
    except Q.QGError as e:
        assert e.status == Q.QG_ERR_UNSUPPORTED, e
        return False


def largest_k(fmt, m, N):
    step = STEP[fmt]
    K = (1 << 17) // step * step
    while not accepted(fmt, m, N, K):
        K -= step
    return K


@pytest.mark.parametrize("fmt,m,N", [("q8g64", 1, 300), ("q8g64", 4, 129), ("q4g32", 1, 257),
                                     ("q4g32", 4, 64), ("q8g128", 3, 100), ("q8pc", 2, 77)])
def test_largest_staged_activation(fmt, m, N):
    K = largest_k(fmt, m, N)
    assert K > 16384 // m, "staging limit lower than expected: K=%d" % K
    assert not accepted(fmt, m, N, K + STEP[fmt])
    rng = synth.rng_for(102, m, N, K)
    gen = {"q8g64": synth.q8g64_weights, "q4g32": synth.q4g32_weights,
           "q8g128": synth.q8g128_weights, "q8pc": synth.q8pc_weights}[fmt]
    wts = gen(rng, N, K)
    x = synth.activations(rng, m, K)
    y = torch.full((m, N), float("nan"), dtype=torch.float32, device="cuda")
    getattr(Q, "qgemv_" + fmt)(dev(getattr(Q, "qpack_" + fmt)(*wts)), dev(x), y, N, K)
    torch.cuda.synchronize()
    y_ref, a_ref = getattr(oracle, fmt)(*wts, x, threads=THREADS)
    ok = oracle.within_tolerance(y.cpu().numpy(), y_ref, a_ref, 2e-3)
    assert ok.all(), "%s m=%d N=%d K=%d: %d outputs out of tolerance" % (fmt, m, N, K, (~ok).sum())


def test_grouped_calls_at_the_slot_limit():
    # 64 slots (the most a grouped call takes), expert ids repeating, one x
    # per slot; the plain grouped call and the SwiGLU call against the oracle.
    n_experts, n_slots, N, K = 9, 64, 200, 512
    ids = synth.rng_for(103, 0).integers(0, n_experts, n_slots).astype(np.int32)
    xs = synth.activations(synth.rng_for(103, 1), n_slots, K)
    experts = [synth.q4g32_weights(synth.rng_for(103, 2, e), N, K) for e in range(n_experts)]
    stride = Q.expert_stride(N, K)
    buf = torch.cat([torch.from_numpy(Q.qpack_q4g32(*e)) for e in experts]).to("cuda")
    y = torch.full((n_slots, N), float("nan"), dtype=torch.float32, device="cuda")
    Q.qgemv_grouped_q4g32(buf, stride, n_experts, dev(ids), dev(xs), K, y, N, N, K)
    torch.cuda.synchronize()
    y_ref, a_ref = oracle.grouped_q4g32(experts, ids, xs, threads=THREADS)
    assert oracle.within_tolerance(y.cpu().numpy(), y_ref, a_ref, 2e-3).all()

    ups = [synth.q4g32_weights(synth.rng_for(103, 3, e), N, K) for e in range(n_experts)]
    gstride = Q.gate_up_expert_stride(N, K)
    gbuf = torch.cat([torch.from_numpy(Q.qpack_q4g32_gate_up(g, u)) for g, u in zip(experts, ups)]).to("cuda")
    act = torch.full((n_slots, N), 0x7FAB, dtype=torch.int16, device="cuda")
    Q.qgemv_grouped_q4g32_swiglu(gbuf, gstride, n_experts, dev(ids), dev(xs), K, act, N, N, K)
    torch.cuda.synchronize()
    ref, g, u, a_g, a_u = oracle.grouped_q4g32_swiglu(experts, ups, ids, xs, threads=THREADS)
    got = (act.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    tol = oracle.swiglu_tolerance(ref, g, u, a_g, a_u)
    assert (np.isfinite(got) & (np.abs(got - ref) <= tol)).all()
