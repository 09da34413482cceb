"""tg_mfma_ceiling on gfx950: every MFMA of the measurement loop runs and
accumulates (all-ones operands give each thread an exactly known sum, for
the fp16 and the int8 shapes), zero operands give zeros, and buffers that do
not fit their allocation are rejected before launch."""
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
    # Each wave holds a 128 x 64 accumulator tile, 128 values per lane, and
    # every k-step adds 32 products of ones to each: a thread's accumulators
    # sum to 128 * 32 * iters, exact in fp32.
    log("mfma_ceiling ones mfma=%d iters=%d" % (mfma, iters))
    wg = 300
    ops = operands(ONE_F16)
    sink = torch.full((wg * 512,), float("nan"), dtype=torch.float32, device="cuda:0")
    st = tg.tg_mfma_ceiling(mfma, ops.data_ptr(), sink.data_ptr(), iters, wg,
                            torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_SUCCESS
    torch.cuda.synchronize()
    got = sink.cpu().numpy()
    assert np.all(got == 128.0 * 32 * iters)


@pytest.mark.parametrize("iters", [2, 6])
def test_int8_all_ones_count_every_product(iters):
    # int8 ones (every byte 1): each k-step of 64 adds 64 products to each of
    # a lane's 128 int32 accumulators
    log("mfma_ceiling int8 ones iters=%d" % iters)
    wg = 300
    ops = operands(0x0101)
    sink = torch.full((wg * 512,), float("nan"), dtype=torch.float32, device="cuda:0")
    st = tg.tg_mfma_ceiling(64, ops.data_ptr(), sink.data_ptr(), iters, wg,
                            torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_SUCCESS
    torch.cuda.synchronize()
    assert np.all(sink.cpu().numpy() == 128.0 * 64 * iters)


@pytest.mark.parametrize("mfma", [32, 16, 64])
def test_zero_operands_give_zero(mfma):
    log("mfma_ceiling zeros mfma=%d" % mfma)
    ops = operands(0)
    sink = torch.full((64 * 512,), float("nan"), dtype=torch.float32, device="cuda:0")
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
    sink = torch.zeros(4 * 512, dtype=torch.float32, device="cuda:0")
    assert tg.tg_mfma_ceiling(32, tail_ops.data_ptr(), sink.data_ptr(), 2, 4, s) == \
        tg.TG_ERROR_INVALID_VALUE
    # a sink of 256 floats per workgroup is half of what the call writes
    short_sink = big[big.numel() - 4 * 256 * 4:]
    ops = operands(0)
    assert tg.tg_mfma_ceiling(16, ops.data_ptr(), short_sink.data_ptr(), 2, 4, s) == \
        tg.TG_ERROR_INVALID_VALUE
    host = np.zeros(tg.TG_CEILING_OPERAND_BYTES, np.uint8)
    assert tg.tg_mfma_ceiling(32, host.ctypes.data, sink.data_ptr(), 2, 4, s) == \
        tg.TG_ERROR_NOT_DEVICE_MEMORY
    torch.cuda.synchronize()
