"""GPU: seeded random shapes for every dense entry point against the oracle.

Each case draws a format, a row count, N, K and row strides from a fixed
seed: the plain kernels at m = 1..4 and the matrix-core kernels at m = 2..16,
K any whole number of scale groups (matrix cores: of 64-wide steps, 128 for
Q8G128 and Q4G32).  Outputs must meet the oracle's bar, and the canary past
N in each output row must survive.
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
CANARY_BITS = 0x7FA01234
GEN = {"q8g64": synth.q8g64_weights, "q4g32": synth.q4g32_weights,
       "q8g128": synth.q8g128_weights, "q8pc": synth.q8pc_weights}
GROUP = {"q8g64": 64, "q4g32": 32, "q8g128": 128, "q8pc": 16}
MMA_STEP = {"q8g64": 64, "q4g32": 128, "q8g128": 128, "q8pc": 64}


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    Q.lib()


def draw_case(i):
    rng = synth.rng_for(104, i)
    mma = bool(i % 3 == 2)
    fmt = ["q8g64", "q4g32", "q8g128", "q8pc"][int(rng.integers(0, 4))]
    m = int(rng.integers(2, 17)) if mma else int(rng.integers(1, 5))
    N = int(rng.choice([1, 2, 3, 15, 16, 17, 63, 100, 255, 256, 257, 1000, 2049, 3001]))
    step = MMA_STEP[fmt] if mma else GROUP[fmt]
    K = step * int(rng.integers(1, max(2, 6144 // step)))
    ldx = K + 2 * int(rng.integers(0, 3))      # even: rows of x stay 4-byte aligned
    ldy = N + int(rng.integers(0, 5))
    return mma, fmt, m, N, K, ldx, ldy


CASES = [draw_case(i) for i in range(48)]


@pytest.mark.parametrize("case", CASES, ids=["%s%s-m%d-N%d-K%d" % (c[1], "_mma" if c[0] else "", c[2], c[3], c[4])
                                            for c in CASES])
def test_random_shape_against_oracle(case):
    mma, fmt, m, N, K, ldx, ldy = case
    rng = synth.rng_for(105, m, N, K, int(mma))
    wts = GEN[fmt](rng, N, K)
    x = synth.activations(rng, m, K)
    xb = np.zeros((m, ldx), np.uint16)
    xb[:, :K] = x
    suffix = "_mma" if mma else ""
    w = torch.from_numpy(getattr(Q, "qpack_" + fmt + suffix)(*wts)).to("cuda")
    xd = torch.from_numpy(xb.view(np.int16)).to("cuda")
    y = torch.full((m, ldy), CANARY_BITS, dtype=torch.int32, device="cuda").view(torch.float32)
    getattr(Q, "qgemv_" + fmt + suffix)(w, xd, y, N, K, m=m, ldx=ldx, ldy=ldy)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.all(yh[:, N:].view(np.uint32) == CANARY_BITS), "wrote past N"
    y_ref, a_ref = getattr(oracle, fmt)(*wts, x, threads=THREADS)
    ok = oracle.within_tolerance(yh[:, :N], y_ref, a_ref, 2e-3)
    assert ok.all(), "%d of %d outputs out of tolerance" % ((~ok).sum(), ok.size)
