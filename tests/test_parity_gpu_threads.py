"""GPU: calls from several host threads, each on its own stream, give the
same bits as the same calls made from one thread.

The launch path keeps only per-device lookups and counters as shared state;
this drives it from four threads at once (default-priority streams created
by torch) with different shapes and formats per thread.
"""
import threading

import numpy as np
import pytest

from weight_only_block_amd import qgemv as Q
from weight_only_block_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    Q.lib()


def dev(a: np.ndarray) -> "torch.Tensor":
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


CASES = [("q8g64", 1, 3001, 2560), ("q4g32", 2, 1000, 4096), ("q8g128", 1, 2048, 1024),
         ("q8pc", 3, 777, 1280)]


def make_case(t, fmt, m, N, K):
    rng = synth.rng_for(101, t)
    wts = {"q8g64": synth.q8g64_weights, "q4g32": synth.q4g32_weights,
           "q8g128": synth.q8g128_weights, "q8pc": synth.q8pc_weights}[fmt](rng, N, K)
    return dev(getattr(Q, "qpack_" + fmt)(*wts)), dev(synth.activations(rng, m, K))


def test_concurrent_threads_match_single_thread():
    cases = [make_case(t, *c) for t, c in enumerate(CASES)]
    ref = []
    for (fmt, m, N, K), (w, x) in zip(CASES, cases):
        y = torch.empty((m, N), dtype=torch.float32, device="cuda")
        getattr(Q, "qgemv_" + fmt)(w, x, y, N, K)
        torch.cuda.synchronize()
        ref.append(y.cpu().numpy().view(np.uint32).copy())

    iters = 40
    errors = []

    def worker(t):
        try:
            fmt, m, N, K = CASES[t]
            w, x = cases[t]
            stream = torch.cuda.Stream()
            ys = [torch.empty((m, N), dtype=torch.float32, device="cuda") for _ in range(iters)]
            with torch.cuda.stream(stream):
                for i in range(iters):
                    getattr(Q, "qgemv_" + fmt)(w, x, ys[i], N, K, stream=stream)
            stream.synchronize()
            for i in range(iters):
                got = ys[i].cpu().numpy().view(np.uint32)
                if not np.array_equal(got, ref[t]):
                    errors.append("thread %d call %d differs" % (t, i))
                    return
        except Exception as e:  # reported below, in the main thread
            errors.append("thread %d: %r" % (t, e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(len(CASES))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
