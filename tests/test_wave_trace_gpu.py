"""GPU: the per-wave timeline (qg_set_wave_trace) records every wave of every
traced launch once, with ordered times, drops what does not fit, and leaves
the results unchanged.

The timeline is a diagnostic: its records are checked for completeness and
order here, and the outputs of traced launches must equal untraced ones bit
for bit (the oracle checks of the untraced kernels live in the parity
tests).
"""
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
    yield
    Q.set_wave_trace(None)


def dev(a: np.ndarray) -> "torch.Tensor":
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def _inputs():
    rng = synth.rng_for(4242, 0)
    N, K = 4096, 1024
    q, s = synth.q8g64_weights(rng, N, K)
    w = dev(Q.qpack_q8g64(q, s))
    x = dev(synth.activations(rng, 1, K))
    Ng, Kg, n_exp, n_slots = 512, 1024, 6, 3
    stride = Q.expert_stride(Ng, Kg)
    buf = torch.empty(n_exp * stride, dtype=torch.uint8, device="cuda")
    for e in range(n_exp):
        c, sc, mn = synth.q4g32_weights(synth.rng_for(4242, 1, e), Ng, Kg)
        buf[e * stride:(e + 1) * stride].copy_(dev(Q.qpack_q4g32(c, sc, mn)))
    ids = dev(np.array([4, 1, 5], dtype=np.int32))
    xg = dev(synth.activations(rng, n_slots, Kg))
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    yg = torch.empty((n_slots, Ng), dtype=torch.float32, device="cuda")

    def run():
        Q.qgemv_q8g64(w, x, y, N, K)
        Q.qgemv_grouped_q4g32(buf, stride, n_exp, ids, xg, Kg, yg, Ng, Ng, Kg)

    return run, y, yg, n_slots


def test_trace_records_every_wave_once_and_changes_no_result():
    run, y, yg, n_slots = _inputs()
    run()
    torch.cuda.synchronize()
    ref = (y.clone(), yg.clone())
    cap = 1 << 14
    rec = torch.zeros(cap * 8, dtype=torch.int64, device="cuda")
    Q.set_wave_trace(rec)
    run()
    records, launches, dropped = Q.wave_trace_state()
    Q.set_wave_trace(None)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), ref[0].view(torch.int32))
    assert torch.equal(yg.view(torch.int32), ref[1].view(torch.int32))
    assert launches == 2 and dropped == 0 and 0 < records <= cap
    r = rec[:records * 8].view(-1, 8).cpu().numpy().astype(np.int64)
    assert not rec[records * 8:].any().item()
    for li, slots in ((0, 1), (1, n_slots)):
        w = r[r[:, 7] == li]
        assert len(w) % slots == 0 and len(w) > 0
        per_slot = len(w) // slots
        pairs = sorted(zip(w[:, 5].tolist(), w[:, 6].tolist()))
        assert pairs == [(s, g) for s in range(slots) for g in range(per_slot)]
        t0, t1, t2 = w[:, 0], w[:, 1], w[:, 2]
        assert (t0 > 0).all() and (t2 >= t0).all()
        got = t1 > 0
        assert got.any()
        assert ((t1[got] >= t0[got]) & (t1[got] <= t2[got])).all()
        # One launch's waves run within a few milliseconds of each other.
        assert t2.max() - t0.min() < 100 * 5000
        assert (w[:, 4] < 8).all()
    # The second launch starts after the first has ended (same stream).
    a, b = r[r[:, 7] == 0], r[r[:, 7] == 1]
    assert b[:, 0].min() >= a[:, 2].max()


def test_trace_drops_launches_that_do_not_fit():
    run, y, yg, _ = _inputs()
    rec = torch.zeros(8, dtype=torch.int64, device="cuda")   # one record: fits neither launch
    Q.set_wave_trace(rec)
    run()
    records, launches, dropped = Q.wave_trace_state()
    Q.set_wave_trace(None)
    torch.cuda.synchronize()
    assert (records, launches, dropped) == (0, 0, 2)
    assert not rec.any().item()


def test_trace_rejects_bad_buffers():
    rec = torch.zeros(8, dtype=torch.int64, device="cuda")
    with pytest.raises(Q.QGError):
        Q.set_wave_trace(rec[1:])   # 56 bytes: not one whole record
    assert Q.lib().qg_set_wave_trace(rec.data_ptr() + 4, 1) == Q.QG_ERR_INVALID_ARG
    assert Q.lib().qg_set_wave_trace(rec.data_ptr(), 0) == Q.QG_ERR_INVALID_ARG
    assert Q.wave_trace_state() == (0, 0, 0)
