"""Index-row checks on the GPU (the selected positions are the attention's gather addresses:
lightning-indexer walk-through, step 4).

- dsa_check_indices flags nothing on the index rows dsa_forward writes (prefill and decode),
  and flags each kind of bad entry in hand-made rows: out of range (below -1, at len_k, huge),
  past the query's position, not in the top-k's ascending-then-pad form, pages outside a pool
  of known size.
- The gathers treat such entries as empty slots: dsa_sparse_mqa and dsa_indexer_kl give
  bit-identical results on a row with bad entries and on the same row with those entries
  replaced by -1 (the kernels' own range test makes them load row 0 in place and mask it, so
  every load stays inside the caches).
- DSA_DEBUG_CHECKS=1 makes the gathering calls report the flags through dsa_debug_flags; with
  the variable unset nothing is reported."""
import os

import numpy as np
import pytest
import torch

import dsa_inputs
import sparse_attention_long_lightning_amd as dsa
from helpers import host

pytestmark = pytest.mark.gpu

OOR, NC, NS, BP = dsa.IDX_OUT_OF_RANGE, dsa.IDX_NOT_CAUSAL, dsa.IDX_NOT_SORTED, dsa.IDX_BAD_PAGE


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def flags_of(dims, batch, idx, dev):
    f = torch.full((idx.shape[0],), 0xFFFFFFFF, dtype=torch.int64, device=dev).to(torch.int32)
    dsa.check_indices(dims, batch, idx, f)
    torch.cuda.synchronize()
    return host(f).view(np.uint32)


def run_forward(inp, dims, dev):
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=dev)
    T = batch.n_q
    out = torch.empty(T, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=dev)
    idx = torch.empty(T, dims.topk, dtype=torch.int32, device=dev)
    ws = torch.empty(dsa.workspace_size(dims, batch), dtype=torch.uint8, device=dev)
    dsa.forward(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], inp["q"], inp["kv"],
                out, None, idx, ws)
    torch.cuda.synchronize()
    return batch, idx


def test_forward_index_rows_pass_the_check(cuda):
    dims = dsa_inputs.PROD
    say("dsa_check_indices on dsa_forward's rows: prefill L=3000 and decode B=6")
    inp = dsa_inputs.prefill_inputs(3000, dims, seed=2, device=cuda)
    batch, idx = run_forward(inp, dims, cuda)
    assert not flags_of(dims, batch, idx, cuda).any()
    inp = dsa_inputs.decode_inputs(dims=dims, seed=4, device=cuda, lens=[1500, 2048, 2049, 7000, 12345, 20000])
    batch, idx = run_forward(inp, dims, cuda)
    assert not flags_of(dims, batch, idx, cuda).any()


def bad_rows(k):
    """Five query rows of one sequence of 100 keys (positions 95..99) and the flags they carry."""
    rows = np.full((5, k), -1, np.int32)
    rows[0, :4] = [0, 5, 50, 95]                 # what the top-k could write: no flag
    rows[1, :4] = [3, -3, 100, 1 << 30]          # below -1, at len_k, huge
    rows[2, :3] = [10, 20, 99]                   # 99 is past position 97
    rows[3, :3] = [5, 3, -1]
    rows[3, 5] = 7                               # descending, then a valid entry after a -1
    rows[4, :3] = [1, 2, 3]
    rows[4, k - 1] = 4                           # a valid entry after the pads
    want = [0, OOR, NC, NS, NS]
    return rows, want


def test_check_flags_hand_made_rows(cuda):
    k = 16
    dims = dsa_inputs.Dims(64, 128, k, 128, 576, 512, 0.0721)
    say("dsa_check_indices on hand-made rows (out of range, not causal, not sorted)")
    rows, want = bad_rows(k)
    batch = dsa.Batch([0, 5], [0, 100], device=cuda)
    got = flags_of(dims, batch, torch.from_numpy(rows).to(cuda), cuda)
    assert got.tolist() == want


def cleaned(rows, lim, row_ok=None):
    r = rows.copy()
    bad = (r < -1) | (r > lim)
    if row_ok is not None:
        bad |= (r >= 0) & ~row_ok(np.clip(r, 0, lim))
    r[bad] = -1
    return r


def test_gathers_skip_out_of_range_slots(cuda):
    k, L = 16, 100
    dims = dsa_inputs.Dims(64, 128, k, 128, 576, 512, 0.0721)
    say("sparse MQA and KL target: a row with bad entries == the row with them emptied")
    rows, _ = bad_rows(k)
    g = torch.Generator().manual_seed(3)
    q = torch.randn(5, 128, 576, generator=g).to(torch.bfloat16).to(cuda)
    kv = torch.randn(L, 576, generator=g).to(torch.bfloat16).to(cuda)
    scores = torch.randn(5, L, generator=g).to(cuda)
    batch = dsa.Batch([0, 5], [0, L], device=cuda)
    ws = torch.empty(dsa.workspace_size(dims, batch), dtype=torch.uint8, device=cuda)
    res = []
    for r in (rows, cleaned(rows, L - 1)):
        idx = torch.from_numpy(r).to(cuda)
        out = torch.empty(5, 128, 512, dtype=torch.bfloat16, device=cuda)
        lse = torch.empty(5, 128, dtype=torch.float32, device=cuda)
        dsa.sparse_mqa(dims, batch, q, kv, idx, out, lse, ws)
        kl = torch.empty(5, device=cuda)
        rev = torch.empty(5, device=cuda)
        dsa.indexer_kl(dims, batch, q, kv, lse, idx, scores, L, kl, rev)
        torch.cuda.synchronize()
        res.append([host(t).copy() for t in (out, lse, kl, rev)])
    for a, b, name in zip(res[0], res[1], ("out", "lse", "kl", "kl_rev")):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name


def test_bad_pages_are_flagged_and_skipped(cuda):
    k, L = 16, 100
    dims = dsa_inputs.Dims(64, 128, k, 128, 576, 512, 0.0721)
    say("paged pool of 4 pages: an entry whose page id is 9 is flagged and skipped")
    table = np.array([[2, 9]], np.int32)         # positions 64..99 live on page 9, outside the pool
    pool_rows = 4 * 64
    rows = np.full((2, k), -1, np.int32)
    rows[0, :3] = [1, 30, 63]
    rows[1, :4] = [1, 30, 63, 70]
    batch = dsa.Batch([0, 2], [0, L], device=cuda, page_table=table, pool_rows=pool_rows)
    assert flags_of(dims, batch, torch.from_numpy(rows).to(cuda), cuda).tolist() == [0, BP]
    g = torch.Generator().manual_seed(5)
    q = torch.randn(2, 128, 576, generator=g).to(torch.bfloat16).to(cuda)
    kv = torch.randn(pool_rows, 576, generator=g).to(torch.bfloat16).to(cuda)
    ws = torch.empty(dsa.workspace_size(dims, batch), dtype=torch.uint8, device=cuda)
    res = []
    for r in (rows, np.where(rows >= 64, -1, rows).astype(np.int32)):
        out = torch.empty(2, 128, 512, dtype=torch.bfloat16, device=cuda)
        lse = torch.empty(2, 128, dtype=torch.float32, device=cuda)
        dsa.sparse_mqa(dims, batch, q, kv, torch.from_numpy(r).to(cuda), out, lse, ws)
        torch.cuda.synchronize()
        res.append((host(out).copy(), host(lse).copy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


def test_debug_checks_report_through_the_flag_word(cuda):
    k, L = 16, 100
    dims = dsa_inputs.Dims(64, 128, k, 128, 576, 512, 0.0721)
    say("DSA_DEBUG_CHECKS=1: the gathering calls report bad rows; unset: nothing")
    rows, want = bad_rows(k)
    g = torch.Generator().manual_seed(6)
    q = torch.randn(5, 128, 576, generator=g).to(torch.bfloat16).to(cuda)
    kv = torch.randn(L, 576, generator=g).to(torch.bfloat16).to(cuda)
    batch = dsa.Batch([0, 5], [0, L], device=cuda)
    ws = torch.empty(dsa.workspace_size(dims, batch), dtype=torch.uint8, device=cuda)
    out = torch.empty(5, 128, 512, dtype=torch.bfloat16, device=cuda)
    idx = torch.from_numpy(rows).to(cuda)
    dsa.debug_flags(clear=True)
    old = os.environ.pop("DSA_DEBUG_CHECKS", None)
    try:
        dsa.sparse_mqa(dims, batch, q, kv, idx, out, None, ws)
        assert dsa.debug_flags() == 0
        os.environ["DSA_DEBUG_CHECKS"] = "1"
        dsa.sparse_mqa(dims, batch, q, kv, idx, out, None, ws)
        assert dsa.debug_flags(clear=True) == OOR | NC | NS
        assert dsa.debug_flags() == 0  # cleared
        good = torch.from_numpy(bad_rows(k)[0][:1].repeat(5, 0)).to(cuda)
        dsa.sparse_mqa(dims, batch, q, kv, good, out, None, ws)
        assert dsa.debug_flags() == 0
        # the forward checks its own rows before the attention: nothing to report
        inp = dsa_inputs.decode_inputs(dims=dsa_inputs.PROD, seed=4, device=cuda, lens=[3000, 9000])
        run_forward(inp, dsa_inputs.PROD, cuda)
        inp = dsa_inputs.prefill_inputs(2500, dsa_inputs.PROD, seed=3, device=cuda)
        run_forward(inp, dsa_inputs.PROD, cuda)
        assert dsa.debug_flags() == 0
    finally:
        os.environ.pop("DSA_DEBUG_CHECKS", None)
        if old is not None:
            os.environ["DSA_DEBUG_CHECKS"] = old
