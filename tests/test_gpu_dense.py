"""GPU parity of the dense short-sequence path and of k other than 2048, through the C ABI.

dsa_dense_mqa against the oracle's textbook causal attention (max abs 2e-2, relative L2 1e-2,
lse 2e-3, as for the sparse attention); the dense path against the sparse kernel on full
index rows (the same sums in the same order: equal values); dsa_forward on sequences no
longer than k against dense attention; end-to-end forward at k = 512 and k = 8192."""
import math

import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
import sparse_attention_long_lightning_amd as dsa
from helpers import check_attention, host, host_inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def rand_case(dims, lq, lk, seed, dev):
    g = torch.Generator().manual_seed(seed)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    T, S = int(cu_q[-1]), int(cu_k[-1])
    q = torch.randn(T, dims.n_heads, dims.qk_dim, generator=g).to(torch.bfloat16).to(dev)
    kv = torch.randn(S, dims.qk_dim, generator=g).to(torch.bfloat16).to(dev)
    return cu_q, cu_k, q, kv


def run_dense(dims, cu_q, cu_k, q, kv, dev):
    batch = dsa.Batch(cu_q, cu_k, device=dev)
    T = batch.n_q
    out = torch.empty(T, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(T, dims.n_heads, dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, dsa.workspace_size(dims, batch)), dtype=torch.uint8, device=dev)
    dsa.dense_mqa(dims, batch, q, kv, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def check_dense(dims, cu_q, cu_k, q, kv, out, lse, what, rows_per_seq=None):
    hq, hkv, ho, hl = host(q), host(kv), host(out), lse.cpu().numpy()
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        rows = np.arange(q1 - q0)
        if rows_per_seq is not None and len(rows) > rows_per_seq:
            rows = np.unique(np.r_[rows[:rows_per_seq // 2], rows[-(rows_per_seq // 2):]])
        if len(rows) == 0:
            continue
        pos = ((k1 - k0) - (q1 - q0) + rows).astype(np.int32)
        ro, rl = oracle.dense_causal(hq[q0 + rows], hkv[k0:k1], pos, dims.v_dim, dims.sm_scale)
        check_attention(ho[q0 + rows], ro, what=f"{what} seq {b}")
        np.testing.assert_allclose(hl[q0 + rows], rl, rtol=0, atol=2e-3)


@pytest.mark.parametrize("shape", ["tiny", "prod"])
def test_dense_mqa_prefill_sequences(cuda, shape):
    dims = dsa_inputs.TINY if shape == "tiny" else dsa_inputs.PROD
    lq, lk = ([200, 1, 77], [200, 40, 77]) if shape == "tiny" else ([700, 130], [700, 1300])
    say(f"dense MQA {shape} lq {lq} lk {lk}")
    cu_q, cu_k, q, kv = rand_case(dims, lq, lk, 1, cuda)
    out, lse = run_dense(dims, cu_q, cu_k, q, kv, cuda)
    check_dense(dims, cu_q, cu_k, q, kv, out, lse, f"dense {shape}", rows_per_seq=64)


def test_dense_mqa_decode_split(cuda):
    dims = dsa_inputs.PROD
    lk = [1, 31, 33, 1000, 4097, 9000]
    say(f"dense MQA decode rows (split over workgroups) lens {lk}")
    cu_q, cu_k, q, kv = rand_case(dims, [1] * len(lk), lk, 2, cuda)
    out, lse = run_dense(dims, cu_q, cu_k, q, kv, cuda)
    check_dense(dims, cu_q, cu_k, q, kv, out, lse, "dense decode")


def test_dense_equals_sparse_on_full_index_rows(cuda):
    dims = dsa_inputs.PROD
    L = 600
    say(f"dense MQA == sparse MQA with index rows 0..p (L={L})")
    cu_q, cu_k, q, kv = rand_case(dims, [L], [L], 3, cuda)
    idx = np.full((L, dims.topk), -1, np.int32)
    for t in range(L):
        idx[t, :t + 1] = np.arange(t + 1)
    batch = dsa.Batch(cu_q, cu_k, device=cuda)
    o_s = torch.empty(L, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=cuda)
    l_s = torch.empty(L, dims.n_heads, dtype=torch.float32, device=cuda)
    dsa.sparse_mqa(dims, batch, q, kv, torch.from_numpy(idx).to(cuda), o_s, l_s)
    o_d, l_d = run_dense(dims, cu_q, cu_k, q, kv, cuda)
    assert torch.equal(o_s.float(), o_d.float()) and torch.equal(l_s, l_d)


def run_forward(inp, dims, dev, with_idx=True):
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=dev)
    T = batch.n_q
    out = torch.empty(T, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(T, dims.n_heads, dtype=torch.float32, device=dev)
    idx = torch.empty(T, dims.topk, dtype=torch.int32, device=dev) if with_idx else None
    ws = torch.empty(dsa.workspace_size(dims, batch), dtype=torch.uint8, device=dev)
    dsa.forward(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], inp["q"],
                inp["kv"], out, lse, idx, ws)
    torch.cuda.synchronize()
    return out, lse, idx


def test_forward_short_sequence_is_dense_attention(cuda):
    dims = dsa_inputs.PROD
    L = 1500
    say(f"forward prod L={L} <= k: dense causal attention, with and without index rows")
    inp = dsa_inputs.prefill_inputs(L, dims, seed=4, device=cuda, needles=False)
    o1, l1, idx = run_forward(inp, dims, cuda)
    o2, l2, _ = run_forward(inp, dims, cuda, with_idx=False)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    gi = idx.cpu().numpy()
    for t in (0, 1, 777, L - 1):
        assert np.array_equal(gi[t], np.r_[np.arange(t + 1), np.full(dims.topk - t - 1, -1)])
    h = host_inputs(inp)
    rows = np.r_[0:8, 700:708, L - 8:L]
    ro, rl = oracle.dense_causal(h["q"][rows], h["kv"], rows.astype(np.int32), dims.v_dim, dims.sm_scale)
    check_attention(host(o1)[rows], ro, what="short forward")
    np.testing.assert_allclose(l1.cpu().numpy()[rows], rl, rtol=0, atol=2e-3)


@pytest.mark.parametrize("k", [512, 8192])
def test_forward_other_k(cuda, k):
    from test_gpu_parity import compare_forward_rows
    L = 12000
    dims = dsa_inputs.Dims(64, 128, k, 128, 576, 512, 1.0 / math.sqrt(192.0), w_std=0.125)
    say(f"forward prod L={L} k={k} sampled rows")
    inp = dsa_inputs.prefill_inputs(L, dims, seed=5, device=cuda)
    out, lse, idx = run_forward(inp, dims, cuda)
    h = host_inputs(inp)
    rows = sorted(set([0, k - 2, k - 1, k, k + 1, L - 1] + [int(x) for x in np.linspace(k, L - 1, 6)]))
    rows = [r for r in rows if 0 <= r < L]
    compare_forward_rows(inp, h, out, lse, idx, rows, dims, f"k={k} forward")
