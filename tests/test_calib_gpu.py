"""GPU test of the pure-read streaming kernel behind the bench's read-ceiling measurement
(gemv_read_stream): it reads every vector of every row it is given, in the lane layout of
the GEMV's weight stream, and nothing else."""
import pytest
import torch

import bandwidth_bound_decode_amd as bbd

pytestmark = pytest.mark.gpu

FOLD = 0x9E3779B9          # the one fold value the kernel stores


@pytest.mark.parametrize("unroll,waves", [(1, 0), (2, 3), (4, 8), (8, 32)])
def test_every_vector_is_read(unroll, waves):
    """Only lane 2 of the last row gets a nonzero word, placed in its last vector: the fold
    reaches the stored value only if that vector was loaded and folded into that lane."""
    rows, row_bytes = 33, 1024 * unroll * 3
    buf = torch.zeros(rows * row_bytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    words_per_row = row_bytes // 4
    steps = row_bytes // 1024
    lane, last = 2, steps - 1
    # vector v = lane + 64 * step holds bytes [16 v, 16 v + 16) of the row
    word = (rows - 1) * words_per_row + (lane + 64 * last) * 4 + 3
    signed = FOLD - (1 << 32)
    buf[word] = signed
    bbd.read_stream(buf, rows, row_bytes, unroll, waves, sink)
    torch.cuda.synchronize()
    assert sink.item() == signed
    # the same word one row short of the launch: never read, nothing stored
    sink.zero_()
    bbd.read_stream(buf, rows - 1, row_bytes, unroll, waves, sink)
    torch.cuda.synchronize()
    assert sink.item() == 0
    # two lanes' words cancel only if a lane folded both: they sit in different lanes
    buf.zero_()
    buf[word] = signed
    buf[word - 4 * 64] = signed          # the same lane, one step earlier: folds to 0
    bbd.read_stream(buf, rows, row_bytes, unroll, waves, sink)
    torch.cuda.synchronize()
    assert sink.item() == 0
