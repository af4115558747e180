"""GPU: the measured-ceiling kernels do the work they claim (the MFMA loop's
closed-form sum, the copy byte for byte, the read's XOR of every word), so
the figures bench.py reports from them are real."""
import numpy as np
import pytest

from w8a8_post_quantization_channel_amd import capi, ceiling

pytestmark = pytest.mark.gpu


def _operands(kind):
    if kind == "ones":
        return np.ones(ceiling.CEILING_OPERAND_BYTES, np.int8)
    rng = np.random.default_rng(7)
    if kind == "random":
        return rng.integers(-128, 128, ceiling.CEILING_OPERAND_BYTES).astype(np.int8)
    # small codes, like most of a quantized tensor's
    return np.clip(np.rint(rng.normal(0, 20, ceiling.CEILING_OPERAND_BYTES)), -127, 127).astype(np.int8)


@pytest.mark.parametrize("kind", ["ones", "random", "small"])
def test_mfma_loop_sum(kind):
    import torch
    host = _operands(kind)
    operands = torch.from_numpy(host).cuda()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    limit = (1 << 31) // max(1, max(abs(d) for d in ceiling.ceiling_chain_dots(host)))
    for iters, per_cu in ((1, 1), (37, 2), (1000, 1), (min(20000, limit - 1), 2)):
        sink.zero_()
        ops = ceiling.sq_ceiling_mfma(iters, per_cu, operands, sink)
        torch.cuda.synchronize()
        waves = ops // (8 * iters * 2 * 32 * 32 * 32)
        assert waves == per_cu * torch.cuda.get_device_properties(0).multi_processor_count * 4
        assert int(sink[0].item()) % (1 << 32) == ceiling.ceiling_expected_sink(host, iters, waves)


SIZES = [16, 4096 + 48, 3 * (1 << 20) + 16 * 7, 64 << 20, (64 << 20) + 32768 * 3 + 16 * 5]


@pytest.mark.parametrize("nbytes", SIZES)
def test_copy(nbytes):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.full((nbytes + 64,), 7, dtype=torch.uint8, device="cuda")
    ceiling.sq_ceiling_copy(src, dst[:nbytes])
    torch.cuda.synchronize()
    assert torch.equal(src, dst[:nbytes])
    assert bool((dst[nbytes:] == 7).all())  # nothing written past the end


@pytest.mark.parametrize("nbytes", SIZES)
def test_read(nbytes):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes + 1)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    expect = int(np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32)))
    sink = torch.full((4,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    ceiling.sq_ceiling_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink[0].item()) % (1 << 32) == expect ^ 0x5A5A5A5A


@pytest.mark.parametrize("nbytes", SIZES)
def test_narrow(nbytes):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes + 2)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.full((nbytes // 2 + 64,), 7, dtype=torch.uint8, device="cuda")
    ceiling.sq_ceiling_narrow(src, dst[:nbytes // 2])
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes // 2], src.view(-1, 16)[:, :8].reshape(-1))
    assert bool((dst[nbytes // 2:] == 7).all())
