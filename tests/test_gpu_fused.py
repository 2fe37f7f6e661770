"""GPU parity of the fused indexer -> top-k path of dsa_forward, through the C ABI.

In a prefill pass the indexer counts each row's scores as it stores them and the top-k starts
from those counts (one read of the row instead of two).  The selection is unique, so the
index rows that dsa_forward returns must equal, bit for bit, dsa_topk run on the scores of
dsa_indexer_scores for the same inputs (the unfused path, itself bit-exact against the
oracle).  Cases: random rows with planted needles (the list path), negative head weights
(fewer than k non-negative scores: the fallback), identical keys (one score per row: ties
everywhere, list overflow for long rows, partial tie selection for short ones) and a handful
of distinct keys (many ties at the threshold)."""
import numpy as np
import pytest
import torch

import dsa_inputs
import sparse_attention_long_lightning_amd as dsa

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def unfused_idx(dims, inp, dev):
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=dev)
    T, L = batch.n_q, batch.max_len_k
    stride = (L + 3) // 4 * 4
    scores = torch.empty(T, stride, dtype=torch.float32, device=dev)
    dsa.indexer_scores(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], scores,
                       stride)
    idx = torch.empty(T, dims.topk, dtype=torch.int32, device=dev)
    dsa.topk(dims, batch, scores, stride, idx)
    torch.cuda.synchronize()
    return idx


def fused_idx(dims, inp, dev, ws_bytes=None):
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=dev)
    T = batch.n_q
    out = torch.empty(T, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=dev)
    idx = torch.empty(T, dims.topk, dtype=torch.int32, device=dev)
    n = dsa.workspace_size(dims, batch) if ws_bytes is None else ws_bytes
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    dsa.forward(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], inp["q"], inp["kv"],
                out, None, idx, ws)
    torch.cuda.synchronize()
    return idx


def compare(dims, inp, dev, what, ws_bytes=None):
    a = fused_idx(dims, inp, dev, ws_bytes)
    b = unfused_idx(dims, inp, dev)
    bad = torch.nonzero((a != b).any(dim=1)).flatten().tolist()
    assert not bad, f"{what}: {len(bad)} index rows differ, first row {bad[0]}"


@pytest.mark.parametrize("case", ["random", "negative_w", "identical_keys", "few_keys"])
def test_fused_topk_equals_unfused(cuda, case):
    dims = dsa_inputs.PROD
    L = 20000 if case != "identical_keys" else 12000
    say(f"fused indexer->top-k vs unfused, L={L}, {case}")
    inp = dsa_inputs.prefill_inputs(L, dims, seed=6, device=cuda, needles=case == "random")
    if case == "negative_w":
        inp["w"] = -inp["w"].abs()
    elif case == "identical_keys":
        inp["k8"] = inp["k8"][:1].expand(L, -1).contiguous()
        inp["k_scale"] = inp["k_scale"][:1].expand(L).contiguous()
    elif case == "few_keys":
        sel = torch.arange(L, device=cuda) % 5
        inp["k8"] = inp["k8"][sel].contiguous()
        inp["k_scale"] = inp["k_scale"][sel].contiguous()
    compare(dims, inp, cuda, case)


def test_fused_topk_small_passes_and_tiny_shape(cuda):
    say("fused top-k: minimal workspace (8-row passes) at L=3000, and the tiny shape")
    dims = dsa_inputs.PROD
    inp = dsa_inputs.prefill_inputs(3000, dims, seed=7, device=cuda)
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=cuda)
    compare(dims, inp, cuda, "minimal workspace", ws_bytes=dsa.workspace_min(dims, batch))
    tiny = dsa_inputs.TINY
    inp = dsa_inputs.prefill_inputs(700, tiny, seed=8, device=cuda, needles=False)
    compare(tiny, inp, cuda, "tiny")


def score_keys(s):
    """The order-preserving 32-bit keys of float32 scores (NaN lowest, -0 = +0)."""
    u = s.view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    u = np.where(u == 0x80000000, 0, u)
    k = np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000)
    return np.where(nan, 0, k).astype(np.uint64)


def test_counted_stages_match_the_plain_ones(cuda):
    dims = dsa_inputs.PROD
    lq, lk = [3000, 900], [5000, 900]
    say(f"indexer_scores_counted / topk_counted vs plain stages, lq {lq} lk {lk}")
    parts = [dsa_inputs.prefill_inputs(n, dims, seed=9 + i, device=cuda, needles=False) for i, n in enumerate(lk)]
    inp = {}
    for key in ("k8", "k_scale", "kv"):
        inp[key] = torch.cat([p[key] for p in parts])
    for key in ("q8", "q_scale", "w", "q"):
        inp[key] = torch.cat([p[key][n - m:] for p, n, m in zip(parts, lk, lq)])
    cu_q = [0, lq[0], lq[0] + lq[1]]
    cu_k = [0, lk[0], lk[0] + lk[1]]
    batch = dsa.Batch(cu_q, cu_k, device=cuda)
    T, stride = cu_q[-1], (max(lk) + 3) // 4 * 4
    s1 = torch.zeros(T, stride, device=cuda)
    s2 = torch.zeros(T, stride, device=cuda)
    counts = torch.full((T, dsa.COUNT_BINS), 7, dtype=torch.int32, device=cuda)
    dsa.indexer_scores(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], s1, stride)
    dsa.indexer_scores_counted(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], s2,
                               stride, counts)
    i1 = torch.empty(T, dims.topk, dtype=torch.int32, device=cuda)
    i2 = torch.empty(T, dims.topk, dtype=torch.int32, device=cuda)
    dsa.topk(dims, batch, s1, stride, i1)
    dsa.topk_counted(dims, batch, s2, stride, counts, i2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(i1, i2)
    # the counts are the histogram of the stored scores >= +0 by key bits 30..21
    hs, hc = s2.cpu().numpy(), counts.cpu().numpy()
    for b in range(2):
        for r in (0, lq[b] // 2, lq[b] - 1):
            t = cu_q[b] + r
            p = lk[b] - lq[b] + r
            k = score_keys(hs[t, :p + 1])
            k = k[(k >> 31) == 1]
            ref = np.bincount(((k >> 21) & 1023).astype(np.int64), minlength=1024)
            assert np.array_equal(hc[t], ref), f"seq {b} row {r}"


def decode_unfused_idx(dims, inp, dev):
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=dev)
    T, L = batch.n_q, batch.max_len_k
    stride = (L + 3) // 4 * 4
    scores = torch.empty(T, stride, dtype=torch.float32, device=dev)
    dsa.indexer_scores(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], scores, stride)
    idx = torch.empty(T, dims.topk, dtype=torch.int32, device=dev)
    dsa.topk(dims, batch, scores, stride, idx)
    torch.cuda.synchronize()
    return idx


def test_decode_forward_topk_equals_two_stage(cuda):
    # decode batches select with segment workgroups and a merge (no counts): the index rows of
    # dsa_forward must equal dsa_indexer_scores + dsa_topk on one workgroup per row
    dims = dsa_inputs.PROD
    lens = [100, 2048, 2049, 16384, 16385, 40000, 91529, 131072, 70000, 30000]
    say(f"decode forward index rows vs indexer_scores + topk, lens {lens}")
    inp = dsa_inputs.decode_inputs(dims=dims, seed=11, device=cuda, lens=lens)
    # row 8: negative head weights (few non-negative scores); row 9: one key repeated (ties)
    inp["w"][8] = -inp["w"][8].abs()
    k0 = inp["cu_k"][9]
    inp["k8"][k0:k0 + lens[9]] = inp["k8"][k0]
    inp["k_scale"][k0:k0 + lens[9]] = inp["k_scale"][k0]
    a = fused_idx(dims, inp, cuda)
    b = decode_unfused_idx(dims, inp, cuda)
    bad = torch.nonzero((a != b).any(dim=1)).flatten().tolist()
    assert not bad, f"decode rows differ: {bad}"
    a2 = fused_idx(dims, inp, cuda)
    assert torch.equal(a, a2)


def test_decode_forward_topk_many_rows(cuda):
    # 160 decode rows (more than the segmented dsa_topk handles) of mixed lengths, some below k,
    # some at segment boundaries; every fifth row has only five distinct keys (a crowded
    # threshold bin)
    dims = dsa_inputs.PROD
    rng = np.random.default_rng(12)
    lens = [int(x) for x in rng.integers(1, 40000, 160)]
    lens[:4] = [2048, 2049, 16384, 32769]
    say(f"decode forward index rows vs indexer_scores + topk, {len(lens)} rows")
    inp = dsa_inputs.decode_inputs(dims=dims, seed=13, device=cuda, lens=lens, needles=False)
    for b in range(4, len(lens), 5):
        k0 = inp["cu_k"][b]
        sel = torch.arange(lens[b], device=cuda) % 5 + k0
        inp["k8"][k0:k0 + lens[b]] = inp["k8"][sel]
        inp["k_scale"][k0:k0 + lens[b]] = inp["k_scale"][sel]
    a = fused_idx(dims, inp, cuda)
    b_ = decode_unfused_idx(dims, inp, cuda)
    bad = torch.nonzero((a != b_).any(dim=1)).flatten().tolist()
    assert not bad, f"decode rows differ: {bad[:10]}"
