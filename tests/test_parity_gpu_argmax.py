"""GPU parity for the greedy argmax over fp32 logits (qg_argmax_f32),
through the C ABI.  The decision is an integer taken on the same fp32
values on both sides, so the GPU index must equal the oracle's exactly.
"""
import numpy as np
import pytest

import oracle
from weight_only_block_amd import qgemv as Q
from weight_only_block_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

VOCAB = synth.LM_HEAD[2]          # 151936


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    Q.lib()


def workspace(m):
    return torch.zeros(Q.argmax_workspace_size(m), dtype=torch.uint8, device="cuda")


def gpu_argmax(x: np.ndarray, ldx=None, ws=None):
    m, N = x.shape
    ldx = N if ldx is None else ldx
    xb = np.zeros((m, ldx), np.float32)
    xb[:, :N] = x
    xd = torch.from_numpy(xb).to("cuda")
    out = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    ws = workspace(m) if ws is None else ws
    Q.argmax_f32(xd, out, ws, N=N, m=m, ldx=ldx)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.int64), ws


def logits(rng, m, N):
    return (rng.standard_normal((m, N)) * 3).astype(np.float32)


@pytest.mark.parametrize("m", [1, 2, 4, 7])
def test_full_vocabulary_rows(m):
    rng = np.random.default_rng(m)
    x = logits(rng, m, VOCAB)
    got, ws = gpu_argmax(x, ldx=VOCAB + 5)
    assert np.array_equal(got, oracle.argmax_f32(x))
    assert not ws.any().item(), "workspace not left zeroed"


@pytest.mark.parametrize("N", [1, 2, 7, 255, 2047, 2048, 2049, 4096, 10001])
def test_ragged_lengths(N):
    rng = np.random.default_rng(N)
    x = logits(rng, 3, N)
    got, _ = gpu_argmax(x)
    assert np.array_equal(got, oracle.argmax_f32(x))


def test_ties_across_work_groups_take_the_lowest_index():
    x = np.zeros((5, VOCAB), np.float32)
    x[0, [100, 70000, 151935]] = 9.0            # tie in three different work-groups
    x[1, [151935, 5]] = np.inf
    x[2, :] = -np.inf                           # all -inf: index 0
    x[3, :] = 1.5                               # all equal: index 0
    x[4, 3] = -0.0                              # -0 ties +0 (row max 0): index 0
    got, _ = gpu_argmax(x)
    assert got.tolist() == [100, 5, 0, 0, 0]
    assert np.array_equal(got, oracle.argmax_f32(x))


def test_nan_counts_as_largest_and_first_nan_wins():
    rng = np.random.default_rng(3)
    x = logits(rng, 3, VOCAB)
    x[0, [90000, 20]] = np.nan
    x[1, VOCAB - 1] = np.nan
    x[2, 0] = np.float32("-nan")
    got, _ = gpu_argmax(x)
    assert got.tolist() == [20, VOCAB - 1, 0]
    assert np.array_equal(got, oracle.argmax_f32(x))


def test_coarse_values_with_many_ties():
    rng = np.random.default_rng(4)
    x = rng.integers(-5, 6, size=(4, 50000)).astype(np.float32)
    got, _ = gpu_argmax(x)
    assert np.array_equal(got, oracle.argmax_f32(x))


def test_workspace_is_reusable_across_calls():
    rng = np.random.default_rng(5)
    ws = workspace(4)
    for r in range(5):
        x = logits(rng, 4, VOCAB)
        got, ws = gpu_argmax(x, ws=ws)
        assert np.array_equal(got, oracle.argmax_f32(x)), "call %d" % r
    assert not ws.any().item()


def test_graph_replays_match_eager_calls():
    rng = np.random.default_rng(6)
    m = 2
    x = torch.from_numpy(logits(rng, m, VOCAB)).to("cuda")
    out = torch.zeros(m, dtype=torch.int32, device="cuda")
    ws = workspace(m)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call = Q.bound_argmax_f32(x, out, ws, VOCAB, m=m)
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    for r in range(4):
        new = logits(np.random.default_rng(100 + r), m, VOCAB)
        x.copy_(torch.from_numpy(new).to("cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), oracle.argmax_f32(new)), "replay %d" % r


def test_lm_head_then_argmax_picks_a_valid_token():
    # The GEMV's fp32 logits feed the argmax; the GPU index must equal the
    # oracle's argmax of those same logits, and the chosen token must be a
    # maximum of the fp64 logits to within the GEMV tolerance.
    _, _, N, K = synth.LM_HEAD
    rng = synth.rng_for(90, 0)
    q, s = synth.q8g64_weights(rng, N, K)
    x = synth.activations(rng, 2, K)
    w = torch.from_numpy(Q.qpack_q8g64(q, s)).to("cuda")
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    y = torch.empty((2, N), dtype=torch.float32, device="cuda")
    idx = torch.zeros(2, dtype=torch.int32, device="cuda")
    Q.qgemv_q8g64(w, xd, y, N, K)
    Q.argmax_f32(y, idx, workspace(2))
    torch.cuda.synchronize()
    y_gpu = y.cpu().numpy()
    got = idx.cpu().numpy().astype(np.int64)
    assert np.array_equal(got, oracle.argmax_f32(y_gpu))
    y_ref, a_ref = oracle.q8g64(q, s, x, threads=16)
    for i in range(2):
        best = y_ref[i].max()
        assert y_ref[i, got[i]] >= best - 2e-3 * (a_ref[i, got[i]] + a_ref[i, y_ref[i].argmax()])
