"""Targeted test of the sparse MQA's lazy running maximum against the oracle.

The kernel keeps a running maximum of the base-2 logits per head and rescales its output
accumulators (hand-written AGPR code with fixed hazard waits) only when a block of 32 slots
brings a maximum more than 64 above it.  Here every head's logits follow a chosen pattern so
that the rescale branch is taken, skipped at the gap, taken in the first and in the last block,
after empty blocks and from very negative starts; the output and lse must still match the
oracle's softmax (DeepSeek-V3.2 explained, section 二.1: attention of the query over the
selected latent rows).

Construction (production and tiny shapes): the latent rows' value dims are N(0,1); rope dim
DV + k holds pattern k's logit for the row, and head h's query is 1 (or -1 for the upper half
of the heads, which reverses every pattern) at dim DV + h % 8 and 0 elsewhere, so its logit is
exactly sm_scale * (+-) pattern value.  sm_scale is chosen so that one unit of a pattern is
1/8 of a base-2 unit."""
import math

import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
import sparse_attention_long_lightning_amd as dsa
from helpers import check_attention, host

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def patterns(n_slots, rng):
    """Base-2 logits y[k, j] of 8 patterns over slot j (blocks of 32 slots)."""
    b = np.arange(n_slots) // 32
    nb = int(b.max()) + 1
    u = rng.uniform
    y = np.zeros((8, n_slots))
    y[0] = np.where(b < 8, 65.0 * b, 65.0 * 7 - 100.0) + u(-2, 0, n_slots)         # +65 each block
    y[1] = np.where(b < 6, 64.0 * b, 320.0) + np.where(b % 2 == 0, -0.05, 0.05) * (b < 6)  # ~64 steps
    y[2] = np.where(b == nb - 1, 90.0, 0.0) + u(-5, 5, n_slots) * (b != nb - 1)     # jump in the last block
    y[3] = -10.0 * b + u(-3, 0, n_slots)                                            # decreasing
    y[4] = rng.normal(0, 120, n_slots)                                              # many rescales
    y[5] = np.where(b == 0, -100.0, np.where(b == 1, -140.0, u(0, 1, n_slots)))     # very negative start
    y[6] = 3.0                                                                      # constant
    y[7] = np.where(b >= 1, 65.0, 0.0) + u(-0.5, 0, n_slots)                        # one jump at block 1
    return y


def build(dims, n_rows, seed):
    rng = np.random.default_rng(seed)
    H, DQK, DV, k = dims.n_heads, dims.qk_dim, dims.v_dim, dims.topk
    S = k
    kv = rng.normal(size=(S, DQK))
    y = patterns(S, rng)
    kv[:, DV:DV + 8] = 8.0 * y.T  # one unit of y per 8 units of the rope entry
    q = np.zeros((n_rows, H, DQK))
    heads = np.arange(H)
    q[:, heads, DV + heads % 8] = np.where(heads < H // 2, 1.0, -1.0)
    idx = np.empty((n_rows, k), np.int32)
    for r in range(n_rows):
        kind = r % 8
        row = np.arange(k, dtype=np.int32)
        if kind == 1:
            row = row[::-1].copy()                       # big blocks first
        elif kind == 2:
            row[rng.random(k) < 0.4] = -1                # scattered empty slots
        elif kind == 3:
            row[:32] = -1                                # first block empty
        elif kind == 4:
            row[:-32] = -1                               # only the last block
        elif kind == 5:
            row[:] = -1
            row[k // 2] = k // 2                         # a single slot
        elif kind == 6:
            row = rng.permutation(row).astype(np.int32)
        elif kind == 7:
            row[:] = -1                                  # no slot: out = 0, lse = -inf
        idx[r] = row
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)  # noqa: E731
    return bf(q).contiguous(), bf(kv).contiguous(), idx


@pytest.mark.parametrize("shape,n_rows", [("prod", 128), ("prod", 8), ("tiny", 128), ("tiny", 8)])
def test_lazy_rescale_against_oracle(cuda, shape, n_rows):
    base = dsa_inputs.PROD if shape == "prod" else dsa_inputs.TINY
    sm = 0.125 / math.log2(math.e)  # one pattern unit = 1/8 base-2 unit
    dims = dsa_inputs.Dims(base.n_idx_heads, base.idx_dim, 2048 if shape == "prod" else 256, base.n_heads,
                           base.qk_dim, base.v_dim, sm)
    say(f"lazy rescale: {shape} rows {n_rows} (split path: {n_rows < 128}), k={dims.topk}")
    q, kv, idx = build(dims, n_rows, seed=31 + n_rows)
    S = kv.shape[0]
    # one sequence per row, all sharing the same latent rows (a row's slots name positions 0..S-1)
    batch = dsa.Batch(list(range(n_rows + 1)), [S * i for i in range(n_rows + 1)], device=cuda)
    kv_all = kv.repeat(n_rows, 1).to(cuda)
    out = torch.empty(n_rows, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=cuda)
    lse = torch.empty(n_rows, dims.n_heads, dtype=torch.float32, device=cuda)
    ws = torch.empty(max(dsa.workspace_size(dims, batch), 16), dtype=torch.uint8, device=cuda)
    dsa.sparse_mqa(dims, batch, q.to(cuda), kv_all, torch.from_numpy(idx).to(cuda), out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_mqa(host(q), host(kv), idx, dims.v_dim, dims.sm_scale)
    got_o, got_l = host(out), host(lse)
    for r in range(n_rows):
        check_attention(got_o[r:r + 1], ro[r:r + 1], what=f"{shape} row {r} (kind {r % 8})")
        fin = np.isfinite(rl[r])
        assert np.array_equal(np.isfinite(got_l[r]), fin), f"row {r}: lse finiteness"
        np.testing.assert_allclose(got_l[r][fin], rl[r][fin], rtol=0, atol=2e-3, err_msg=f"row {r}")
    assert np.all(got_o[7::8] == 0)  # rows without slots
