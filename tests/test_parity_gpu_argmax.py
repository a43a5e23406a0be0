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


# ------------------------------------------------ LM head with fused argmax

FUSED = {"q8g64": (synth.q8g64_weights, Q.qpack_q8g64, Q.qgemv_q8g64, Q.qgemv_q8g64_argmax,
                   oracle.q8g64, Q.FMT_Q8G64_ARGMAX),
         "q8g128": (synth.q8g128_weights, Q.qpack_q8g128, Q.qgemv_q8g128, Q.qgemv_q8g128_argmax,
                    oracle.q8g128, Q.FMT_Q8G128_ARGMAX)}


@pytest.mark.parametrize("fmt", ["q8g64", "q8g128"])
@pytest.mark.parametrize("m", [1, 4])
def test_fused_lm_head_argmax_full_size(fmt, m):
    # Same launch configuration as the plain GEMV: the fused call's logits
    # must equal the plain call's bit for bit, its index must equal the
    # argmax of those logits, and the logits must meet the GEMV bar.
    gen, pack, plain, fused, ref, _ = FUSED[fmt]
    _, _, N, K = synth.LM_HEAD
    rng = synth.rng_for(91, m)
    q, s = gen(rng, N, K)
    x = synth.activations(rng, m, K)
    w = torch.from_numpy(pack(q, s)).to("cuda")
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    y_plain = torch.empty((m, N), dtype=torch.float32, device="cuda")
    y_fused = torch.full((m, N), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    ws = workspace(m)
    plain(w, xd, y_plain, N, K)
    fused(w, xd, y_fused, idx, ws, N, K)
    torch.cuda.synchronize()
    yp, yf = y_plain.cpu().numpy(), y_fused.cpu().numpy()
    assert np.array_equal(yp.view(np.uint32), yf.view(np.uint32))
    assert np.array_equal(idx.cpu().numpy().astype(np.int64), oracle.argmax_f32(yf))
    y_ref, a_ref = ref(q, s, x, threads=16)
    assert oracle.within_tolerance(yf, y_ref, a_ref).all()
    assert not ws.any().item()


@pytest.mark.parametrize("N,K", [(1, 64), (7, 128), (1000, 2560), (5003, 1024), (40000, 256)])
def test_fused_argmax_ragged_shapes_without_logits(N, K):
    # With logits=None nothing but the index is written.
    gen, pack, plain, fused, _, _ = FUSED["q8g64"]
    rng = synth.rng_for(92, N, K)
    q, s = gen(rng, N, K)
    x = synth.activations(rng, 3, K)
    w = torch.from_numpy(pack(q, s)).to("cuda")
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    y = torch.empty((3, N), dtype=torch.float32, device="cuda")
    plain(w, xd, y, N, K)
    idx = torch.full((3,), -7, dtype=torch.int32, device="cuda")
    ws = workspace(3)
    for _ in range(3):                       # the workspace is reused
        fused(w, xd, None, idx, ws, N, K, m=3)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy().astype(np.int64), oracle.argmax_f32(y.cpu().numpy()))
    assert not ws.any().item()


def test_fused_argmax_ties_take_the_lowest_index():
    # Four identical weight rows (codes of the sign of x, the largest scale)
    # give four identical logits far above the rest: the first of them wins.
    N, K = 3000, 512
    rng = synth.rng_for(93, 0)
    q, s = synth.q8g64_weights(rng, N, K)
    x = synth.activations(rng, 1, K)
    sign = np.where(x[0] & 0x8000, -1, 1)
    for r in (17, 1500, 2000, 2999):
        q[r] = (100 * sign).astype(np.int8)
        s[r] = synth.to_fp16_bits(np.full(K // 64, 0.05))
    w = torch.from_numpy(Q.qpack_q8g64(q, s)).to("cuda")
    xd = torch.from_numpy(x.view(np.int16)).to("cuda")
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    Q.qgemv_q8g64_argmax(w, xd, y, idx, workspace(1), N, K)
    torch.cuda.synchronize()
    yv = y.cpu().numpy()[0]
    assert yv[17] == yv[1500] == yv[2000] == yv[2999] == yv.max()
    assert idx.item() == 17


def test_fused_argmax_graph_replays():
    _, _, N, K = synth.LM_HEAD
    rng = synth.rng_for(94, 0)
    q, s = synth.q8g64_weights(rng, 20000, K)
    w = torch.from_numpy(Q.qpack_q8g64(q, s)).to("cuda")
    xd = torch.from_numpy(synth.activations(rng, 1, K).view(np.int16)).to("cuda")
    y = torch.empty((1, 20000), dtype=torch.float32, device="cuda")
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = workspace(1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call = Q.bound_q8g64_argmax(w, xd, y, idx, ws, 20000, K)
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    for r in range(4):
        xd.copy_(torch.from_numpy(synth.activations(synth.rng_for(94, 10 + r), 1, K).view(np.int16)).to("cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy().astype(np.int64), oracle.argmax_f32(y.cpu().numpy()))


def test_fused_route_counter_and_variant_name():
    Q.route_counts_reset()
    N, K = 640, 1024
    rng = synth.rng_for(95, 0)
    q, s = synth.q8g128_weights(rng, N, K)
    w = torch.from_numpy(Q.qpack_q8g128(q, s)).to("cuda")
    xd = torch.from_numpy(synth.activations(rng, 2, K).view(np.int16)).to("cuda")
    idx = torch.zeros(2, dtype=torch.int32, device="cuda")
    Q.qgemv_q8g128_argmax(w, xd, None, idx, workspace(2), N, K)
    torch.cuda.synchronize()
    name = Q.variant_name(Q.FMT_Q8G128_ARGMAX, 2, N, K)
    assert name.startswith("q8g128_argmax_m2_")
    assert Q.route_count(name) == 1
