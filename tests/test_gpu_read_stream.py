"""GPU: the plain read stream (qg_read_stream, the bandwidth reference the
bench compares the GEMV kernels with) reads every 16-byte unit.

A lane XOR-folds the 32-bit words of the units it reads and stores the fold
to the sink when it equals 0x9E3779B9.  In an all-zero buffer with one unit
(0x9E3779B9, 0, 0, 0) planted, only the lane that reads that unit can store,
so the sink changes exactly when the planted unit was read.
"""
import numpy as np
import pytest

from weight_only_block_amd import qgemv as Q

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PATTERN = 0x9E3779B9
UNSET = 0x1234567


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    Q.lib()


def run(units, planted, waves_per_cu):
    words = np.zeros(units * 4, np.uint32)
    if planted is not None:
        words[4 * planted] = PATTERN
    buf = torch.from_numpy(words.view(np.int32)).to("cuda")
    sink = torch.full((1,), UNSET, dtype=torch.int32, device="cuda")
    Q.read_stream(buf, sink, waves_per_cu=waves_per_cu)
    torch.cuda.synchronize()
    return int(sink.cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("units", [1, 63, 511, 512, 513, 4096 * 8 + 3, 1 << 20])
@pytest.mark.parametrize("waves_per_cu", [0, 1, 32])
def test_every_unit_is_read(units, waves_per_cu):
    for planted in sorted({0, units // 2, units - 1}):
        assert run(units, planted, waves_per_cu) == PATTERN, "unit %d of %d not read" % (planted, units)
    assert run(units, None, waves_per_cu) == UNSET


def test_two_planted_units_in_one_lane_cancel():
    # A wave reads 512-unit chunks, lane l taking units l, l + 64, ...: two
    # patterns planted 64 units apart in one chunk fold to zero in one lane.
    units = 1 << 16
    words = np.zeros(units * 4, np.uint32)
    words[4 * 512 * 3 + 4 * 5] = PATTERN
    words[4 * 512 * 3 + 4 * 69] = PATTERN
    buf = torch.from_numpy(words.view(np.int32)).to("cuda")
    sink = torch.full((1,), UNSET, dtype=torch.int32, device="cuda")
    Q.read_stream(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == UNSET
