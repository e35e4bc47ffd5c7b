"""The measured-ceiling kernels (needs an MI355X): the streaming read must read every
word of the buffer (its XOR is checked on the host), and the MFMA kernel's accumulators
must hold the exact count of products it claims to have issued."""
import numpy as np
import pytest
import torch

import block_ar_canvas_amd as dg
from gpu_util import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 64 << 20])
def test_stream_read_reads_every_word(dg_ctx, nbytes):
    words = np.random.default_rng(nbytes).integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(DEV)
    sink = torch.zeros(dg.PEAK_STREAM_BLOCKS, dtype=torch.int32, device=DEV)
    dg_ctx.peak_stream_read(buf, sink)
    dg_ctx.sync()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


def test_mfma_peak_counts_every_product(dg_ctx):
    sink = torch.zeros(dg.PEAK_MFMA_BLOCKS * 4, dtype=torch.float32, device=DEV)
    flop = dg_ctx.peak_mfma(64, sink)
    dg_ctx.sync()
    assert flop == dg.PEAK_MFMA_BLOCKS * 4 * 64 * 4 * 32768
    assert torch.all(sink == 1024.0 * 64)


def test_peak_calls_reject_bad_arguments(dg_ctx):
    sink = torch.zeros(dg.PEAK_STREAM_BLOCKS, dtype=torch.int32, device=DEV)
    with pytest.raises(dg.DGError):
        dg_ctx.peak_stream_read(torch.zeros(17, dtype=torch.uint8, device=DEV), sink)
    fs = torch.zeros(dg.PEAK_MFMA_BLOCKS * 4, dtype=torch.float32, device=DEV)
    for bad in (0, 16385):
        with pytest.raises(dg.DGError):
            dg_ctx.peak_mfma(bad, fs)
