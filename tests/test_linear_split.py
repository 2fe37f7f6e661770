"""The FP8 expansion the prefill indexer uses for the linear part of its score (CPU).

With ReLU(x) = (x + |x|) / 2 the score's linear part is k . u, u = sum_j w'_j/2 q_j (DeepSeek-V3.2-Exp
overview, indexer formula, restated), and the kernel feeds u to the FP8 matrix cores as six e4m3
terms u = sum_i 2^(E-7-4i) c_i, E = max(exponent of max|u|, -100), each term rounding (to nearest,
ties to even) the fp32 residual of the ones before.  This restates that split with the oracle's
e4m3 rounding and checks the three facts the kernel's comments rely on: every scaled residual
stays below 256 (no term reaches the e4m3 saturation at 448), each fp32 residual is exact, and
what six terms leave is at most 2^(E-24) <= 2^-24 max|u| per component.  The kernel's own
results are compared with the oracle by the GPU parity tests."""
import numpy as np
import pytest

import oracle

TERMS = 6


def split_u(u32):
    m = float(np.max(np.abs(u32)))
    e = (int(np.float32(m).view(np.uint32)) >> 23 & 0xFF) - 127
    E = max(e, -100)
    res = u32.astype(np.float32).copy()
    codes = []
    for i in range(TERMS):
        up = np.float32(np.ldexp(1.0, 7 + 4 * i - E))
        dn = np.float32(np.ldexp(1.0, E - 7 - 4 * i))
        y = res * up  # exact: a power of two, no overflow below 256
        assert np.all(np.abs(y.astype(np.float64)) < 256.0), f"term {i} leaves the e4m3 range"
        c = oracle.encode_e4m3(y)
        back = oracle.decode_e4m3(c).astype(np.float32)
        new = (res.astype(np.float64) - back.astype(np.float64) * float(dn))
        res32 = np.float32(res) - back * dn
        assert np.array_equal(res32.astype(np.float64), new), f"term {i}: fp32 residual not exact"
        res = res32.astype(np.float32)
        codes.append(c)
    return E, res, codes


def vectors():
    rng = np.random.default_rng(21)
    out = []
    for scale in (1e-30, 1e-6, 1.0, 3e4, 1e30):
        out.append((rng.standard_normal(128) * scale).astype(np.float32))
        out.append((rng.standard_cauchy(128) * scale).astype(np.float32))
    one = np.zeros(128, np.float32)
    one[17] = 3.0e3
    one[5] = 1.0e-4
    out += [np.zeros(128, np.float32), one, np.full(128, -7.25, np.float32),
            (np.arange(128) - 64).astype(np.float32) * np.float32(1e-3),
            (rng.standard_normal(128) * 1e-33).astype(np.float32)]  # max|u| below 2^-100
    return out


@pytest.mark.parametrize("which", range(15))
def test_six_term_split_bound(which):
    u = vectors()[which]
    E, res, codes = split_u(u)
    bound = np.ldexp(1.0, E - 4 * TERMS)
    assert np.all(np.abs(res.astype(np.float64)) <= bound)
    if np.max(np.abs(u)) > 0:
        assert bound <= np.ldexp(np.max(np.abs(u.astype(np.float64))), -4 * TERMS) or E == -100
    # the terms reproduce u to within the bound
    total = sum(oracle.decode_e4m3(c).astype(np.float64) * np.ldexp(1.0, E - 7 - 4 * i) for i, c in enumerate(codes))
    assert np.all(np.abs(total - u.astype(np.float64)) <= bound)
