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


# E2M1 0x2 = 1.0, 0x3 = 1.5; E2M3 0x22 pattern: fields of 6 bits; E4M3 0x22 =
# 2^-3 * 1.25.  The kernels' operands are v = 0x22222222 ^ (lane & 7) and v ^ 1
# in every register, so every product is fixed; here only the FP4 x FP4 kinds
# are checked in closed form, the others for finiteness and sign.
def _fp4(code):
    mag = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0][code & 7]
    return -mag if code & 8 else mag


def _fp4_row(v):
    # the 32 FP4 elements a lane holds in its first four registers (16 bytes)
    words = [v] * 4
    return [_fp4((w >> (4 * i)) & 15) for w in words for i in range(8)]


@pytest.mark.parametrize("kind", ["fp4xfp4", "fp4xfp4_32x32x64"])
def test_mfma_rate_fp4_closed_form(dev, kind):
    from routed_expert_mxfp4_amd import moe
    blocks, iters = 2, 3
    out = torch.zeros(4 * blocks, dtype=torch.float32, device=dev)
    moe.diag_mfma_rate(kind, blocks, iters, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # lane 0 of each wave writes its accumulator entries; every lane's A and
    # B rows are the same within a K block group because lanes 0..7 differ
    # only in the low 3 bits of each word, so compute C = A B^T explicitly
    if kind == "fp4xfp4":
        M = N = 16
        K = 128
        groups = 4
    else:
        M = N = 32
        K = 64
        groups = 2
    A = np.zeros((M, K))
    B = np.zeros((N, K))
    for lane in range(64):
        v = 0x22222222 ^ (lane & 7)
        r, g = lane % M, lane // M
        A[r, 32 * g:32 * g + 32] = _fp4_row(v)
        B[r, 32 * g:32 * g + 32] = _fp4_row(v ^ 1)
    C = A @ B.T
    if kind == "fp4xfp4":
        # lane 0 holds C[0][0] .. C[3][0]; the sum takes c0[0] + c1[1] + c2[2] + c3[3]
        want = iters * (C[0, 0] + C[1, 0] + C[2, 0] + C[3, 0])
    else:
        # 32x32: register r of lane 0 holds row 8 (r / 4) + r % 4, column 0
        rows = [8 * (r // 4) + r % 4 for r in (0, 5, 10, 15)]
        want = iters * sum(C[m, 0] for m in rows)
    np.testing.assert_allclose(got, want, rtol=1e-6)


@pytest.mark.parametrize("kind", ["fp6xfp4", "fp8xfp4", "fp8xfp8", "bf16", "fp6xfp4_32x32x64"])
def test_mfma_rate_other_kinds_finite(dev, kind):
    from routed_expert_mxfp4_amd import moe
    out = torch.full((8,), float("nan"), dtype=torch.float32, device=dev)
    flops = moe.diag_mfma_rate(kind, 2, 5, out)
    torch.cuda.synchronize()
    assert flops > 0 and torch.isfinite(out).all()
