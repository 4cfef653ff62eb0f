"""GPU checks of the calibration probes: the copy copies, and the matrix-core loop
computes what its operands define (so the ceiling it measures is real work)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from state_space_sequence_amd.inputs import round_bf16

pytestmark = pytest.mark.gpu


def test_probe_copy_copies():
    from state_space_sequence_amd import m3
    g = torch.Generator(device="cpu").manual_seed(5)
    n = (3 << 20) + 48  # not a multiple of the grid's stride
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros_like(src)
    m3.probe_copy(src, dst)
    m3.probe_copy(src[:16 * 1000], dst[:16 * 1000], blocks=3)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_probe_mfma_checksum_and_clock():
    from state_space_sequence_amd import m3
    blocks, iters, seed = 6, 40, 1.5
    out, clk = m3.probe_mfma_bf16(blocks, iters, seed)
    torch.cuda.synchronize()
    # the operands as the kernel forms them, lane l: A[l%16][8(l/16)+j], B[8(l/16)+j][l%16]
    l = np.arange(64)[:, None]
    j = np.arange(8)[None, :]
    a = round_bf16((seed * (((l + 3 * j) % 17) - 8) / 1024.0).astype(np.float32)).astype(np.float64)
    b = round_bf16(((((5 * l + j) % 13) - 6) / 1024.0).astype(np.float32)).astype(np.float64)
    A = np.zeros((16, 32))
    B = np.zeros((32, 16))
    for lane in range(64):
        for jj in range(8):
            A[lane % 16, 8 * (lane // 16) + jj] = a[lane, jj]
            B[8 * (lane // 16) + jj, lane % 16] = b[lane, jj]
    per_chain = iters * float((A @ B).sum())
    want = 4 * 2 * per_chain  # 4 waves x 2 chains per workgroup
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= 1e-4 * abs(want) + 1e-6), (got, want)
    c = clk.cpu().numpy().reshape(blocks, 2)
    assert (c > 0).all()
