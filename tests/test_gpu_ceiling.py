"""tg_mfma_ceiling on gfx950: every MFMA of the measurement loop runs and
accumulates (all-ones operands give each thread an exactly known sum), zero
operands give zeros, and buffers that do not fit their allocation are
rejected before launch."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import tiled_dense_gemm_08_amd as tg  # noqa: E402

ONE_F16 = 0x3C00


def log(msg):
    sys.stderr.write("[gpu] %s\n" % msg)
    sys.stderr.flush()


def operands(bits):
    n = tg.TG_CEILING_OPERAND_BYTES // 2
    return torch.full((n,), np.int16(np.uint16(bits).view(np.int16)), dtype=torch.int16,
                      device="cuda:0")


@pytest.mark.parametrize("mfma", [32, 16])
@pytest.mark.parametrize("iters", [2, 4, 10])
def test_all_ones_count_every_product(mfma, iters):
    # Each wave holds a 128 x 128 accumulator tile, 256 values per lane, and
    # every k-step adds 32 products of ones to each: a thread's accumulators
    # sum to 256 * 32 * iters, exact in fp32.
    log("mfma_ceiling ones mfma=%d iters=%d" % (mfma, iters))
    wg = 300
    ops = operands(ONE_F16)
    sink = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    st = tg.tg_mfma_ceiling(mfma, ops.data_ptr(), sink.data_ptr(), iters, wg,
                            torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_SUCCESS
    torch.cuda.synchronize()
    got = sink.cpu().numpy()
    assert np.all(got == 256.0 * 32 * iters)


@pytest.mark.parametrize("mfma", [32, 16])
def test_zero_operands_give_zero(mfma):
    log("mfma_ceiling zeros mfma=%d" % mfma)
    ops = operands(0)
    sink = torch.full((64 * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    assert tg.tg_mfma_ceiling(mfma, ops.data_ptr(), sink.data_ptr(), 2, 64,
                              torch.cuda.current_stream().cuda_stream) == tg.TG_SUCCESS
    torch.cuda.synchronize()
    assert np.all(sink.cpu().numpy() == 0.0)


def test_buffers_must_fit_their_allocation():
    log("mfma_ceiling short buffers")
    s = torch.cuda.current_stream().cuda_stream
    # with no cached free blocks, a 64 MiB request is a segment of its own,
    # so nothing follows its last KiB inside the allocation
    torch.cuda.empty_cache()
    big = torch.empty(64 << 20, dtype=torch.uint8, device="cuda:0")
    tail_ops = big[big.numel() - 1024:]
    sink = torch.zeros(4 * 256, dtype=torch.float32, device="cuda:0")
    assert tg.tg_mfma_ceiling(32, tail_ops.data_ptr(), sink.data_ptr(), 2, 4, s) == \
        tg.TG_ERROR_INVALID_VALUE
    host = np.zeros(tg.TG_CEILING_OPERAND_BYTES, np.uint8)
    assert tg.tg_mfma_ceiling(32, host.ctypes.data, sink.data_ptr(), 2, 4, s) == \
        tg.TG_ERROR_NOT_DEVICE_MEMORY
    torch.cuda.synchronize()
