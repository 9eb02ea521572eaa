"""GPU checks of the measurement probes bench.py reports the box's peaks with: the copy
probe moves every byte, the MFMA probe's sums are the exact products of its operands."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_probe_copy_moves_every_byte(gdn_lib):
    g = torch.Generator(device="cuda").manual_seed(5)
    for n in (16, 4096 + 16, (1 << 22) + 48):      # one element, a partial pass, several passes
        src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=g)
        dst = torch.zeros_like(src)
        gdn_lib.probe_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(src, dst), n


def test_probe_mfma_sums(gdn_lib):
    blocks, iters = 3, 7
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flop = gdn_lib.probe_mfma(out, blocks, iters)
    torch.cuda.synchronize()
    assert flop == blocks * 4 * 4 * iters * 32768
    # B is b = 2^-10 everywhere; lane l supplies row l % 32 of A with its eight k slots,
    # whose even slots are a1 = 2^-10 (1 + 2^-7) for odd lanes and a0 = 2^-10 otherwise,
    # odd slots a0.  So D[i][j] = b (8 a(i) + 8 a0) per MFMA, a(i) = a1 for odd rows i;
    # a thread's 16 accumulator rows are half even, half odd: its sum over 4 chains of
    # iters MFMAs is 4 iters b (192 a0 + 64 a1).  Every partial sum is exact in fp32.
    a0, a1, b = 2.0 ** -10, 2.0 ** -10 * (1 + 2.0 ** -7), 2.0 ** -10
    expect = 4 * iters * b * (192 * a0 + 64 * a1)
    assert torch.equal(out.double(), torch.full_like(out, expect, dtype=torch.float64))


def test_probe_copy_in_place(gdn_lib):
    g = torch.Generator(device="cuda").manual_seed(6)
    x = torch.randint(0, 256, ((1 << 20) + 32,), dtype=torch.uint8, device="cuda", generator=g)
    ref = x.clone()
    gdn_lib.probe_copy(x, x)
    torch.cuda.synchronize()
    assert torch.equal(x, ref)
