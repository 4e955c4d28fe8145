"""The measurement aids (contiguous read stream, scattered row gather): the
word each leaves in its sink is the XOR of exactly the bytes it was asked to
read, checked against numpy on the host."""

import numpy as np
import pytest
import torch

from long_context_sparse_approx_amd import ssa

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def xor_words(a: np.ndarray) -> int:
    w = np.ascontiguousarray(a).view(np.uint32).ravel()
    return int(np.bitwise_xor.reduce(w)) if w.size else 0


def sink_value(sink):
    return xor_words(sink.cpu().numpy())


def new_sink():
    return torch.zeros(ssa.MEASURE_SINK_WORDS, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 1 << 20, (64 << 20) + 48])
def test_stream_folds_exactly_the_bytes_read(nbytes):
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(-2**31, 2**31 - 1, ((nbytes + 4096) // 4,), generator=g, dtype=torch.int32)
    sink = new_sink()
    print(f"stream {nbytes} bytes", flush=True)
    ssa.measure_stream(src.to(DEV), nbytes, sink)
    assert sink_value(sink) == xor_words(src.numpy()[: nbytes // 4])


@pytest.mark.parametrize("row_bytes", [16, 256, 1024])
@pytest.mark.parametrize("n", [1, 37, 5000, 300000])
def test_gather_folds_exactly_the_rows_read(row_bytes, n):
    g = torch.Generator().manual_seed(row_bytes * 1000003 + n)
    num_rows = 4099
    src = torch.randint(-2**31, 2**31 - 1, (num_rows * row_bytes // 4,), generator=g,
                        dtype=torch.int32)
    # ids out of range are clamped to the first and last row
    rows = torch.randint(-50, num_rows + 50, (n,), generator=g, dtype=torch.int32)
    sink = new_sink()
    print(f"gather {n} rows of {row_bytes} bytes", flush=True)
    ssa.measure_gather(src.to(DEV), row_bytes, rows.to(DEV), sink)
    table = src.numpy().reshape(num_rows, row_bytes // 4)
    picked = table[np.clip(rows.numpy(), 0, num_rows - 1)]
    assert sink_value(sink) == xor_words(picked)


def test_bad_sizes_are_rejected_before_launch():
    src = torch.zeros(1024, dtype=torch.int32, device=DEV)
    sink = new_sink()
    rows = torch.zeros(4, dtype=torch.int32, device=DEV)
    with pytest.raises(ssa.SsaError):
        ssa.measure_stream(src, 24, sink)
    with pytest.raises(ssa.SsaError):
        ssa.measure_gather(src, 48, rows, sink)
    # nothing to read (n = 0 with a valid id array)
    rc = ssa.lib().ssa_measure_gather(src.data_ptr(), 256, 16, rows.data_ptr(), 0,
                                      sink.data_ptr(), None)
    assert rc == ssa.SSA_OK
    assert sink_value(sink) == 0
