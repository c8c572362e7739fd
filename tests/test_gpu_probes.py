"""GPU checks of the measurement aids in fa_probe.hip (the matrix-core, atomic and issue
probes that the hardware facts of the design rest on): each computes a value known in closed
form, or the same value along two code paths, so a probe that issued the wrong operands or
lost work would be caught, not only timed.

- fa_mfma_probe: lane t holds A[m][k] = (m mod 8) / 8 + (k mod 8) and B[k][n] = (k mod 8) / 2 - 1
  (m = t mod 32, k = 8 (t / 32 mod 2) + i), so C[m][n] = 2 sum_j ((m mod 8) / 8 + j)(j / 2 - 1)
  = 1.5 (m mod 8) + 84 for every n; after `iters` products on each of four chains, a lane's
  sum of its 16 accumulator registers (rows 8 (i / 4) + 4 h + i mod 4, h = t / 32 mod 2) is
  4 iters (96 h + 1380).  All values are small multiples of 1/2, so the float32 result is
  exact.
- fa_atomic_probe: blocks * iters * 4096 adds of 1/1024 into a zeroed accumulator sum to
  blocks * iters * 4, exactly, and touch columns 0..127 of each row only.
- fa_issue_probe kind 3: the same LDS operands and products with the accumulators in VGPRs
  (params 0-2) or AGPRs through assembly products (params 10-12) give bitwise equal results
  (this caught missing wait states between the vector writes of the register operands and
  the first assembly product); kind 6 (operands from global memory) launches and completes.
"""

import pytest
import torch

from exact_io_aware_fa2_amd import fa

pytestmark = pytest.mark.gpu


def test_mfma_probe_exact_sums():
    blocks, iters = 8, 100
    out = torch.full((blocks * 256,), float("nan"), device="cuda", dtype=torch.float32)
    assert fa.fa_mfma_probe(out, blocks, iters) == fa.FA_OK, fa.fa_last_error()
    torch.cuda.synchronize()
    t = torch.arange(blocks * 256, device="cuda")
    h = (t % 64) // 32
    want = (4 * iters * (96 * h + 1380)).to(torch.float32)
    assert torch.equal(out, want), (out[:4], want[:4])


def test_atomic_probe_adds_every_value():
    row_blocks, stride, blocks, iters = 16, 160, 64, 5
    acc = torch.zeros((row_blocks * 32, stride), device="cuda", dtype=torch.float32)
    assert fa.fa_atomic_probe(acc, row_blocks, stride, blocks, iters) == fa.FA_OK
    torch.cuda.synchronize()
    assert acc.double().sum().item() == blocks * iters * 4096 / 1024
    assert torch.count_nonzero(acc[:, 128:]).item() == 0
    # every touched value is a whole number of adds of 1/1024
    assert torch.equal(acc * 1024, torch.round(acc * 1024))


@pytest.mark.parametrize("nr", [0, 1, 2])
def test_issue_probe_agpr_accumulators_match_vgpr(nr):
    blocks, wps, iters = 16, 2, 40
    a = torch.zeros(blocks * 256 * wps, device="cuda", dtype=torch.float32)
    b = torch.zeros_like(a)
    assert fa.fa_issue_probe(a, 3, nr, wps, blocks, iters) == fa.FA_OK, fa.fa_last_error()
    assert fa.fa_issue_probe(b, 3, 10 + nr, wps, blocks, iters) == fa.FA_OK, fa.fa_last_error()
    torch.cuda.synchronize()
    assert torch.isfinite(a).all() and (a != 0).any()
    assert torch.equal(a, b)


@pytest.mark.parametrize("kind,param", [(0, 4), (1, 2), (2, 1), (3, 20), (3, 22), (6, 1), (6, 2),
                                        (6, 3)])
def test_issue_probe_kinds_complete(kind, param):
    blocks, wps, iters = 32, 1, 40
    out = torch.zeros(blocks * 256 * wps, device="cuda", dtype=torch.float32)
    assert fa.fa_issue_probe(out, kind, param, wps, blocks, iters) == fa.FA_OK, fa.fa_last_error()
    torch.cuda.synchronize()
    if kind != 6:  # kind 6 reads its operands from `out` while other workgroups write it
        assert torch.isfinite(out).all()
