"""The measurement kernels behind bench.py --peaks read and multiply what
they claim to: the streaming read's per-block checksums XOR to the XOR of
every 32-bit word of the bytes read, and the matrix-rate kernel's sums are
the closed-form products of its constant operands."""
import numpy as np
import pytest
import torch

from test_gpu_parity import dev  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (1 << 20, 7), ((3 << 20) + 48, 1024),
                                           (64 << 20, 8192)])
def test_stream_read_checksum(dev, nbytes, blocks):
    from routed_expert_mxfp4_amd import moe
    g = torch.Generator().manual_seed(nbytes)
    n = (nbytes + 3) // 4 + 5
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), dtype=torch.int32, generator=g)
    src = host.to(dev)
    out = torch.full((blocks,), -1, dtype=torch.int32, device=dev)
    moe.diag_stream_read(src, nbytes, out, blocks)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host[: nbytes // 4].numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == want


def test_stream_read_refuses_unaligned(dev):
    from routed_expert_mxfp4_amd import moe
    src = torch.zeros(64, dtype=torch.int32, device=dev)
    out = torch.zeros(4, dtype=torch.int32, device=dev)
    with pytest.raises(RuntimeError):
        moe.diag_stream_read(src, 24, out, 4)          # not a multiple of 16


# The kernels' operands are v = 0x22222222 ^ (lane & 7) (the 16x16 kinds: ^
# (chain << 8)) for A and v ^ 1 for B, in every register, so every product is
# fixed; the FP4 x FP4 kinds are checked in closed form (E2M1 magnitudes 0,
# 0.5, 1, 1.5, 2, 3, 4, 6, bit 3 the sign), the others for finiteness.
def _fp4(code):
    mag = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0][code & 7]
    return -mag if code & 8 else mag


def _fp4_row(v):
    # the 32 FP4 elements a lane holds in its first four registers (16 bytes)
    words = [v] * 4
    return [_fp4((w >> (4 * i)) & 15) for w in words for i in range(8)]


def _product(M, K, xor):
    """C = A B^T of the operands every lane builds from v = 0x22222222 ^
    (lane & 7) ^ xor (A) and v ^ 1 (B): lane l holds row l % M, K block
    l // M."""
    A = np.zeros((M, K))
    B = np.zeros((M, K))
    for lane in range(64):
        v = 0x22222222 ^ (lane & 7) ^ xor
        r, g = lane % M, lane // M
        A[r, 32 * g:32 * g + 32] = _fp4_row(v)
        B[r, 32 * g:32 * g + 32] = _fp4_row(v ^ 1)
    return A @ B.T


@pytest.mark.parametrize("kind", ["fp4xfp4", "fp4xfp4_32x32x64"])
def test_mfma_rate_fp4_closed_form(dev, kind):
    from routed_expert_mxfp4_amd import moe
    blocks, iters = 2, 8
    out = torch.zeros(4 * blocks, dtype=torch.float32, device=dev)
    moe.diag_mfma_rate(kind, blocks, iters, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if kind == "fp4xfp4":
        # sixteen chains of iters / 4 products; chain j's operands are built
        # from v ^ (j << 8) and the sum takes its entry j % 4, which lane 0
        # holds as C[j % 4][0]
        want = sum(iters // 4 * _product(16, 128, j << 8)[j % 4, 0] for j in range(16))
    else:
        # four chains of iters products on the same operands; register r of
        # lane 0 holds row 8 (r / 4) + r % 4, column 0, and the sum takes
        # registers 0, 5, 10, 15 of chains 0..3
        C = _product(32, 64, 0)
        want = iters * sum(C[8 * (r // 4) + r % 4, 0] for r in (0, 5, 10, 15))
    np.testing.assert_allclose(got, want, rtol=1e-6)


@pytest.mark.parametrize("kind", ["fp6xfp4", "fp8xfp4", "fp8xfp8", "bf16", "fp6xfp4_32x32x64"])
def test_mfma_rate_other_kinds_finite(dev, kind):
    from routed_expert_mxfp4_amd import moe
    out = torch.full((8,), float("nan"), dtype=torch.float32, device=dev)
    flops = moe.diag_mfma_rate(kind, 2, 8, out)
    torch.cuda.synchronize()
    assert flops > 0 and torch.isfinite(out).all()


def test_mfma_rate_refuses_iterations_not_multiple_of_four(dev):
    from routed_expert_mxfp4_amd import moe
    out = torch.zeros(8, dtype=torch.float32, device=dev)
    with pytest.raises(RuntimeError):
        moe.diag_mfma_rate("fp6xfp4", 2, 6, out)
