"""The allocation-free LM head with the fused greedy choice
(qgemv_q8g64_argmax_noalloc) against the workspace entry point
(qgemv_q8g64_argmax), through the C ABI.

Two calls in a row on the library's own scratch, the second on a smaller
input (fewer rows, fewer vocabulary rows): each call's indices must equal
the workspace call's exactly, and its logits must be the same bits (both
run the same kernel).  The decision is an integer taken on identical fp32
logits, so exact equality is the bar; the logits themselves are also held
to the oracle's tolerance.
"""
import numpy as np
import pytest

import oracle
from weight_only_block_amd import qgemv as Q
from weight_only_block_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    Q.lib()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def _case(seed, m, N, K):
    rng = synth.rng_for(90, seed)
    q, s = synth.q8g64_weights(rng, N, K)
    x = synth.activations(rng, m, K)
    return q, s, x, dev(Q.qpack_q8g64(q, s)), dev(x)


def _with_workspace(w, xd, m, N, K):
    logits = torch.full((m, N), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(Q.argmax_workspace_size(m), dtype=torch.uint8, device="cuda")
    Q.qgemv_q8g64_argmax(w, xd, logits, idx, ws, N, K)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), idx.cpu().numpy()


def _noalloc(w, xd, m, N, K, with_logits=True):
    logits = torch.full((m, N), float("nan"), dtype=torch.float32, device="cuda") if with_logits else None
    idx = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    Q.qgemv_q8g64_argmax_noalloc(w, xd, logits, idx, N, K)
    torch.cuda.synchronize()
    return (logits.cpu().numpy() if with_logits else None), idx.cpu().numpy()


def test_noalloc_matches_workspace_call_twice_second_smaller():
    cases = [(0, 4, synth.LM_HEAD[2], synth.LM_HEAD[3]), (1, 2, 5003, 2560)]
    for seed, m, N, K in cases:
        q, s, x, w, xd = _case(seed, m, N, K)
        ref_logits, ref_idx = _with_workspace(w, xd, m, N, K)
        got_logits, got_idx = _noalloc(w, xd, m, N, K)
        assert np.array_equal(got_idx, ref_idx), (seed, got_idx, ref_idx)
        assert np.array_equal(got_logits.view(np.uint32), ref_logits.view(np.uint32))
        assert np.array_equal(got_idx, oracle.argmax_f32(got_logits))
        y_ref, a_ref = oracle.q8g64(q, s, x, threads=16)
        assert oracle.within_tolerance(got_logits.astype(np.float64), y_ref, a_ref, 2e-3).all()


def test_noalloc_without_logits_and_repeated():
    # No logits written; repeated calls keep choosing the same indices (the
    # scratch is left zeroed by every call).
    seed, m, N, K = 2, 3, 40000, 2560
    _, _, _, w, xd = _case(seed, m, N, K)
    _, ref_idx = _with_workspace(w, xd, m, N, K)
    for _ in range(3):
        _, got_idx = _noalloc(w, xd, m, N, K, with_logits=False)
        assert np.array_equal(got_idx, ref_idx)


def test_noalloc_rejects_before_launch():
    # m beyond the scratch's 4 rows, and the call's own argument checks.
    f = Q.lib().qgemv_q8g64_argmax_noalloc
    W, X, Y, I = 1 << 20, 1 << 21, 1 << 22, 1 << 23
    assert f(W, X, Y, I, 5, 64, 64, 64, 64, None) == Q.QG_ERR_UNSUPPORTED
    assert f(W, X, Y, None, 1, 64, 64, 64, 64, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, X, Y, I, 1, 64, 96, 96, 64, None) == Q.QG_ERR_INVALID_ARG
    assert f(W, X, Y, I, 0, 64, 64, 64, 64, None) == Q.QG_OK
