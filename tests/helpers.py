"""Shared test helpers: host copies of generated inputs and the parity checks."""
from __future__ import annotations

import numpy as np
import torch


def host(t):
    """Exact bytes of a tensor as numpy (bf16 -> uint16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def host_inputs(inp: dict) -> dict:
    out = {}
    for k, v in inp.items():
        out[k] = host(v) if torch.is_tensor(v) else v
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_attention(got_bits: np.ndarray, ref: np.ndarray, max_abs=2e-2, rel=1e-2, what=""):
    """Attention parity: max |g - o| <= 2e-2 and ||g - o||_2 / ||o||_2 <= 1e-2."""
    g = bf16_to_f64(got_bits)
    err = np.abs(g - ref)
    m = float(err.max()) if err.size else 0.0
    den = float(np.linalg.norm(ref))
    r = float(np.linalg.norm(g - ref) / den) if den > 0 else float(np.linalg.norm(g - ref))
    assert m <= max_abs and r <= rel, f"{what}: max abs {m:.3e} (<= {max_abs}), rel {r:.3e} (<= {rel})"
    return m, r


# Accumulation error of gfx950's FP8 MFMA relative to A (the summed product magnitudes), on
# codes quantised like the workload: the bound tests/test_gpu_fp8_accumulation.py asserts from
# its measurement through the indexer, and the term the score check allows (twice that).
EPS_MEASURED_BOUND = 2.0 ** -15.5
EPS_ACC = 2.0 * EPS_MEASURED_BOUND


def check_scores(got: np.ndarray, ref: np.ndarray, mag: np.ndarray, mag_abs: np.ndarray,
                 tol=1e-3, eps_acc=EPS_ACC, what=""):
    """Indexer parity: |g - o| <= tol * M + eps_acc * A, where
    M = s_k sum_j |w'_j| ReLU(D_j)           (the oracle's score with |w| in place of w) and
    A = s_k sum_j |w'_j| sum_d |q_jd k_d|    (the score with |w| and sign-free codes).
    The second term bounds the accumulation error of the gfx950 FP8 MFMA, which does not sum
    the (exact) products in full fp32; its size is measured through the indexer on workload
    codes by tests/test_gpu_fp8_accumulation.py, and eps_acc is twice the bound that test
    asserts.  It only matters where the head dot products D_j cancel to nearly nothing, which
    a bound relative to M alone cannot cover."""
    bound = tol * mag + eps_acc * mag_abs + 1e-30
    diff = np.abs(got.astype(np.float64) - ref)
    bad = diff > bound
    if bad.any():
        i = int(np.argmax(diff - bound))
        raise AssertionError(f"{what}: {int(bad.sum())} scores out of tolerance; worst at {i}: "
                             f"gpu {got[i]!r} oracle {ref[i]!r} M {mag[i]!r} A {mag_abs[i]!r}")


def check_sets(gpu_idx: np.ndarray, orc_idx: np.ndarray, orc_scores: np.ndarray, k: int, tol=1e-3):
    """End-to-end selected sets: positions may differ only where the oracle score is within
    tol * max(|theta|, rms) of the oracle's k-th score theta."""
    a = set(int(x) for x in gpu_idx if x >= 0)
    b = set(int(x) for x in orc_idx if x >= 0)
    if a == b:
        return 0
    n = len(orc_scores)
    theta = np.sort(orc_scores)[::-1][min(k, n) - 1]
    rms = float(np.sqrt(np.mean(orc_scores ** 2)))
    band = tol * max(abs(theta), rms)
    for s in a ^ b:
        assert abs(orc_scores[s] - theta) <= band, (
            f"position {s} differs with score {orc_scores[s]} vs threshold {theta} (band {band})")
    return len(a ^ b)
