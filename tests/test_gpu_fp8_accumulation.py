"""Evidence for the accumulation term of the indexer tolerance.

The indexer parity bound is |g - o| <= 1e-3 * M + eps_acc * A per (t, s), where
M = s_k sum_j |w'_j| ReLU(D_j) and A = s_k sum_j |w'_j| sum_d |q_jd k_d| (tests/helpers.py).
The second term exists because gfx950's FP8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) does not
add the exact products of a 128-long dot product in full fp32: its error scales with the summed
product magnitudes, so where the head dot products D_j cancel, no bound relative to M alone
holds.  This file measures that error through the product path itself.

With one-hot head weights (row t keeps head j = t % 64 with weight 1) and unit scales, the
score of (t, s) is exactly ReLU(D_j) with D_j the dot product of two FP8 code rows: the oracle
computes it without rounding (every product is a multiple of 2^-18 and the sum stays far inside
double's range).  The kernel's deviation from it, divided by A_j = sum_d |q_jd k_d|, is then the
matrix cores' accumulation error (plus the fp32 epilogue's and the FP8 expansion of the linear
part's, both orders of magnitude smaller), on codes quantised like the workload (per-row
amax/448 scales of N(0,1) vectors).  Measured on MI355X over 605,550 pairs (seed 7): exact
for most pairs, 2^-17.05 at the 99.9th percentile, 2^-15.87 at most.  The test asserts it stays
below EPS_MEASURED_BOUND = 2^-15.5 on two seeds and prints its distribution;
helpers.check_scores uses EPS_ACC = 2 * EPS_MEASURED_BOUND.

It also runs the standard workload (Gaussian head weights, real scales) and reports how many
scores need the accumulation term at all, i.e. fall outside 1e-3 * M alone.
"""
import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
import sparse_attention_long_lightning_amd as dsa
from helpers import EPS_ACC, EPS_MEASURED_BOUND, check_scores, host, host_inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def scores_of(inp, dims, dev):
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=dev)
    stride = (batch.max_len_k + 3) // 4 * 4
    sc = torch.full((batch.n_q, stride), float("nan"), dtype=torch.float32, device=dev)
    dsa.indexer_scores(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], sc, stride)
    torch.cuda.synchronize()
    return host(sc)


def oracle_rows(h, L, absolute=False):
    q8, k8, w = h["q8"], h["k8"], h["w"]
    if absolute:
        q8, k8, w = q8 & np.uint8(0x7F), k8 & np.uint8(0x7F), np.abs(w)
    return oracle.indexer_rows(q8, h["q_scale"], w, k8, h["k_scale"], np.arange(L), np.arange(L))


@pytest.mark.parametrize("seed", [7, 8])
def test_fp8_mfma_accumulation_error_one_head(cuda, seed):
    dims, L, H = dsa_inputs.PROD, 1100, 64
    say(f"FP8 MFMA accumulation error: prod L={L} seed {seed}, one head per row, unit scales")
    inp = dsa_inputs.prefill_inputs(L, dims, seed=seed, device=cuda, needles=False)
    w = torch.zeros(L, H, device=cuda)
    w[torch.arange(L, device=cuda), torch.arange(L, device=cuda) % H] = 1.0
    inp["w"] = w.contiguous()
    inp["q_scale"] = torch.ones(L, H, device=cuda)
    inp["k_scale"] = torch.ones(L, device=cuda)
    got = scores_of(inp, dims, cuda)
    h = host_inputs({k: v for k, v in inp.items() if k not in ("q", "kv")})
    exact = oracle_rows(h, L)            # ReLU(D_j), exact
    A = oracle_rows(h, L, absolute=True)  # sum_d |q_jd k_d|, exact
    rel = np.concatenate([np.abs(got[t, : t + 1].astype(np.float64) - exact[t]) / A[t] for t in range(L)])
    neg = np.concatenate([exact[t] == 0 for t in range(L)])
    lg = lambda x: np.log2(max(x, 1e-300))  # noqa: E731
    q = np.quantile(rel, [0.5, 0.9, 0.99, 0.999, 1.0])
    say(f"{rel.size} pairs: |err|/A exact on {np.mean(rel == 0):.1%}; p90 2^{lg(q[1]):.2f}, p99 2^{lg(q[2]):.2f}, "
        f"p99.9 2^{lg(q[3]):.2f}, max 2^{lg(q[4]):.2f} (D < 0 on {neg.mean():.1%}); "
        f"asserted bound 2^{lg(EPS_MEASURED_BOUND):.2f}")
    assert q[4] <= EPS_MEASURED_BOUND


def test_scores_needing_the_accumulation_term(cuda):
    dims, L = dsa_inputs.PROD, 1100
    say(f"standard workload prod L={L}: share of scores outside 1e-3 M alone")
    inp = dsa_inputs.prefill_inputs(L, dims, seed=1, device=cuda, needles=False)
    got = scores_of(inp, dims, cuda)
    h = host_inputs({k: v for k, v in inp.items() if k not in ("q", "kv")})
    ref = oracle.indexer_rows(h["q8"], h["q_scale"], h["w"], h["k8"], h["k_scale"], np.arange(L), np.arange(L))
    M = oracle.indexer_rows(h["q8"], h["q_scale"], np.abs(h["w"]), h["k8"], h["k_scale"], np.arange(L), np.arange(L))
    A = oracle_rows(h, L, absolute=True)
    need = total = 0
    ratio = []
    for t in range(L):
        g = got[t, : t + 1].astype(np.float64)
        d = np.abs(g - ref[t])
        need += int(np.sum(d > 1e-3 * M[t]))
        total += t + 1
        ratio.append(A[t] / np.maximum(M[t], 1e-300))
        check_scores(got[t, : t + 1], ref[t], M[t], A[t], what=f"row {t}")
    r = np.concatenate(ratio)
    r = r[np.isfinite(r)]
    say(f"{need} of {total} scores ({need / total:.2e}) lie outside 1e-3 M alone; A/M median {np.median(r):.1f}, "
        f"p95 {np.quantile(r, 0.95):.1f}; bound used 1e-3 M + 2^{np.log2(EPS_ACC):.2f} A")
