"""GPU check of the bound the 8-bit forward's tolerances rest on: the 32x32x64 E4M3 product
of the matrix core (v_mfma_f32_32x32x64_f8f6f4, run one product at a time by
fa_fp8_product_probe) against exact sums.

Every E4M3 value is an integer multiple of 2^-9 (the smallest subnormal), so each product of
two codes is an integer multiple of 2^-18 below 2^36 and a 64-term sum is exact in int64.
The tolerance derivation (tests/_parity.py) takes the error of one such sum to be below
2^-9 * 2^E, E the largest exponent sum e(a_k) + e(b_k) over the 64 pairs (a subnormal code
counted at exponent -6), and doubles it; this test holds the hardware to the undoubled
bound on operand sets built to stress it: uniform codes, log-uniform magnitudes, one
dominant product per output, and cancelling pairs (largest error seen: 1.05 * 2^-10 * 2^E).  (Measured against the largest actual
product instead, a set whose largest exponent sum involves a subnormal operand exceeds any
bound of that form: the hardware aligns at the exponent, not at the value.)
"""

import numpy as np
import pytest
import torch

from exact_io_aware_fa2_amd import fa
from oracle.fp8 import e4m3_decode

pytestmark = pytest.mark.gpu

BOUND = 2.0 ** -9  # times 2^E
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _code(sign, exp_field, mant):
    return ((sign << 7) | (exp_field << 3) | mant).astype(np.uint8)


def _sets(kind, n, rng):
    """n operand sets of one kind: (a, bt), each [n, 32, 64] uint8 E4M3 codes."""
    shape = (n, 32, 64)
    if kind == "uniform":
        return rng.choice(FINITE, size=shape), rng.choice(FINITE, size=shape)
    if kind == "loguniform":
        def draw():
            e = rng.integers(0, 16, size=shape)
            m = rng.integers(0, 8, size=shape)
            m = np.where(e == 15, np.minimum(m, 6), m)  # 0x7F / 0xFF are NaN
            return _code(rng.integers(0, 2, size=shape), e, m)
        return draw(), draw()
    if kind == "dominant":
        # per set: small codes everywhere, one large pair per (row, column) at k0 = row
        a = _code(rng.integers(0, 2, size=shape), rng.integers(0, 4, size=shape),
                  rng.integers(0, 8, size=shape))
        bt = _code(rng.integers(0, 2, size=shape), rng.integers(0, 4, size=shape),
                   rng.integers(0, 8, size=shape))
        big = _code(rng.integers(0, 2, size=(n, 32)), rng.integers(12, 15, size=(n, 32)),
                    rng.integers(0, 8, size=(n, 32)))
        rows = np.arange(32)
        a[:, rows, rows] = big
        bt[:, rows, rows] = big[:, ::-1]
        return a, bt
    if kind == "cancel":
        # products in pairs of equal magnitude and opposite sign, plus a few small terms
        a, bt = _sets("loguniform", n, rng)
        a[:, :, 1:48:2] = a[:, :, 0:48:2] ^ np.uint8(0x80)
        bt[:, :, 1:48:2] = bt[:, :, 0:48:2]
        small = _code(rng.integers(0, 2, size=(n, 32, 16)), rng.integers(0, 3, size=(n, 32, 16)),
                      rng.integers(0, 8, size=(n, 32, 16)))
        a[:, :, 48:] = small
        return a, bt
    raise ValueError(kind)


def _exp(codes):
    """Unbiased exponent of each code, subnormals (exponent field 0) at -6."""
    return np.maximum((codes.astype(np.int64) >> 3) & 0xF, 1) - 7


def _exact(a, bt):
    """Exact A B as float64 from int64 sums of products in units of 2^-18; the largest
    |product|; 2^E with E the largest exponent sum over the pairs with a nonzero product."""
    ia = np.rint(e4m3_decode(a) * 512.0).astype(np.int64)   # value * 2^9, exact
    ib = np.rint(e4m3_decode(bt) * 512.0).astype(np.int64)
    s = np.einsum("smk,snk->smn", ia, ib)                     # integers < 2^42
    prods = ia[:, :, None, :] * ib[:, None, :, :]
    prod_max = np.abs(prods).max(axis=3)
    esum = _exp(a)[:, :, None, :] + _exp(bt)[:, None, :, :]
    emax = np.where(prods != 0, esum, -64).max(axis=3)
    return (s.astype(np.float64) * 2.0 ** -18, prod_max.astype(np.float64) * 2.0 ** -18,
            np.exp2(emax.astype(np.float64)))


@pytest.mark.parametrize("kind", ["uniform", "loguniform", "dominant", "cancel"])
def test_fp8_product_error_within_truncation_bound(kind):
    rng = np.random.default_rng({"uniform": 11, "loguniform": 12, "dominant": 13, "cancel": 14}[kind])
    n = 256
    a, bt = _sets(kind, n, rng)
    assert not np.isnan(e4m3_decode(a)).any() and not np.isnan(e4m3_decode(bt)).any()
    da = torch.from_numpy(a).cuda()
    db = torch.from_numpy(bt).cuda()
    dc = torch.empty((n, 32, 32), dtype=torch.float32, device="cuda")
    print(f"fp8 products, {kind}: {n} sets", flush=True)
    assert fa.fa_fp8_product_probe(da, db, dc, n) == fa.FA_OK, fa.fa_last_error()
    torch.cuda.synchronize()
    got = dc.cpu().numpy().astype(np.float64)
    exact, pmax, align = _exact(a, bt)
    err = np.abs(got - exact)
    zero = pmax == 0
    assert (err[zero] == 0).all()
    ratio = err[~zero] / align[~zero]
    print(f"fp8 products, {kind}: max |error| / 2^E = {ratio.max() * 2**24:.0f} * 2^-24 "
          f"(bound {BOUND * 2**24:.0f} * 2^-24); max |error| / max |product| = "
          f"{(err[~zero] / pmax[~zero]).max() * 2**24:.0f} * 2^-24; exact results "
          f"{np.mean(err == 0) * 100:.1f} %", flush=True)
    assert ratio.max() <= BOUND
