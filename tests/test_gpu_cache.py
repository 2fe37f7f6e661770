"""GPU parity of the decode cache producer and of paged caches, through the C ABI.

dsa_cache_append against the oracle's RoPE + e4m3 quantisation: codes and scales bit-exact
(both sides round every product, sum and quotient to float32 and encode round-to-nearest-even),
cache rows written exactly where the packed or paged layout puts them and nowhere else.
Paged caches against packed ones: the same kernels read the same values through another row
map, so indexer scores, selected indices, attention outputs and LSE are bit-identical."""
import math

import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
import sparse_attention_long_lightning_amd as dsa
from helpers import host

pytestmark = pytest.mark.gpu

PAGE = dsa.PAGE_SIZE


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def rope_tables(n_pos, rope_dim, base=10000.0):
    """cos / sin [n_pos, rope_dim / 2] of the usual rotary angles pos * base^(-2i / rope_dim)."""
    i = np.arange(rope_dim // 2, dtype=np.float64)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * base ** (-2.0 * i / rope_dim)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def page_layout(lens, rng, spare=5, base_page=0):
    """A shuffled page pool for sequences of the given lengths: page table [B, pps] (slots past
    a sequence's end point at page 0, never read) and the pool row of each packed row.  With
    base_page > 0 the sequences' pages are ids base_page and above of a larger pool."""
    need = [(n + PAGE - 1) // PAGE for n in lens]
    pps = max(max(need), 1)
    n_pages = sum(need) + spare
    perm = rng.permutation(n_pages) + base_page
    table = np.zeros((len(lens), pps), np.int32)
    rows = []
    at = 0
    for b, n in enumerate(lens):
        table[b, :need[b]] = perm[at:at + need[b]]
        at += need[b]
        p = np.arange(n)
        rows.append(table[b, p // PAGE].astype(np.int64) * PAGE + p % PAGE)
    return table, np.concatenate(rows) if rows else np.zeros(0, np.int64), (base_page + n_pages) * PAGE


def append_case(dims, lens, lq, seed, dev):
    """Sequences of lengths lens whose last lq[b] positions are the new tokens."""
    g = torch.Generator().manual_seed(seed)
    T = sum(lq)
    H, d = dims.n_idx_heads, dims.idx_dim
    q_idx = torch.randn(T, H, d, generator=g) * 3.0
    k_idx = torch.randn(T, d, generator=g) * 0.7
    q_idx[0, 1] = 0.0                       # an all-zero row: scale 1, codes 0
    k_idx[T - 1, :] = 0.0
    q_idx[T - 1, 0, :] = 1e-3 * torch.randn(d, generator=g)
    q_idx[T - 1, 0, 5] = 2.0e3              # one dominant value: the rest near e4m3's subnormals
    kv_new = torch.randn(T, dims.qk_dim, generator=g).to(torch.bfloat16)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(n - m, n) for n, m in zip(lens, lq)]).astype(np.int64)
    return dict(q_idx=q_idx.to(dev), k_idx=k_idx.to(dev), kv_new=kv_new.to(dev), cu_q=cu_q, cu_k=cu_k,
                pos=pos, T=T)


def run_append(dims, c, cos, sin, n_rows, dev, page_table=None, row_of=None):
    batch = dsa.Batch(c["cu_q"], c["cu_k"], device=dev, page_table=page_table)
    T, H, d = c["T"], dims.n_idx_heads, dims.idx_dim
    q8 = torch.full((T, H, d), 0xEE, dtype=torch.uint8, device=dev)
    qs = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)
    k8 = torch.full((n_rows, d), 0xAA, dtype=torch.uint8, device=dev)
    ks = torch.full((n_rows,), -7.0, dtype=torch.float32, device=dev)
    kv = torch.full((n_rows, dims.qk_dim), -3.0, dtype=torch.bfloat16, device=dev)
    dsa.cache_append(dims, batch, c["q_idx"], c["k_idx"], c["kv_new"], torch.from_numpy(cos).to(dev),
                     torch.from_numpy(sin).to(dev), q8, qs, k8, ks, kv)
    torch.cuda.synchronize()
    return host(q8), host(qs), host(k8), host(ks), host(kv)


def check_append(dims, c, cos, sin, got, crow, n_rows, what):
    q8, qs, k8, ks, kv = got
    oq8, oqs, ok8, oks = oracle.cache_append(c["q_idx"].cpu().numpy(), c["k_idx"].cpu().numpy(), c["pos"],
                                             cos, sin, dims.idx_dim // 2)
    assert np.array_equal(qs.view(np.uint32), oqs.view(np.uint32)), f"{what}: query scales"
    bad = np.argwhere(q8 != oq8)
    assert len(bad) == 0, f"{what}: {len(bad)} query codes differ, first {bad[0]}: {q8[tuple(bad[0])]:#x} vs {oq8[tuple(bad[0])]:#x}"
    assert np.array_equal(k8[crow], ok8), f"{what}: key codes"
    assert np.array_equal(ks[crow].view(np.uint32), oks.view(np.uint32)), f"{what}: key scales"
    assert np.array_equal(kv[crow], host(c["kv_new"])), f"{what}: latent rows"
    rest = np.setdiff1d(np.arange(n_rows), crow)
    assert (k8[rest] == 0xAA).all() and (ks[rest] == -7.0).all(), f"{what}: rows outside the new tokens written"
    assert (kv[rest] == host(torch.tensor(-3.0, dtype=torch.bfloat16))).all(), f"{what}: latent rows outside"


@pytest.mark.parametrize("shape", ["tiny", "prod"])
def test_cache_append_packed(cuda, shape):
    dims = dsa_inputs.TINY if shape == "tiny" else dsa_inputs.PROD
    lens, lq = [1, 70, 3000, 129], [1, 1, 5, 16]
    say(f"cache_append packed {shape} lens {lens} new {lq}")
    c = append_case(dims, lens, lq, seed=1, dev=cuda)
    cos, sin = rope_tables(max(lens), dims.idx_dim // 2)
    crow = np.concatenate([np.arange(k1 - m, k1) for k1, m in zip(c["cu_k"][1:], lq)])
    got = run_append(dims, c, cos, sin, int(c["cu_k"][-1]), cuda)
    check_append(dims, c, cos, sin, got, crow, int(c["cu_k"][-1]), f"packed {shape}")


def test_cache_append_paged(cuda):
    dims = dsa_inputs.PROD
    lens, lq = [64, 65, 2000, 127, 1], [1, 1, 3, 2, 1]
    say(f"cache_append paged prod lens {lens} new {lq}")
    rng = np.random.default_rng(3)
    table, row_of, n_rows = page_layout(lens, rng)
    c = append_case(dims, lens, lq, seed=2, dev=cuda)
    cos, sin = rope_tables(max(lens), dims.idx_dim // 2)
    crow = np.concatenate([row_of[k1 - m:k1] for k1, m in zip(c["cu_k"][1:], lq)])
    got = run_append(dims, c, cos, sin, n_rows, cuda, page_table=table)
    check_append(dims, c, cos, sin, got, crow, n_rows, "paged prod")


def test_cache_append_without_latent(cuda):
    dims = dsa_inputs.TINY
    lens, lq = [10, 20], [1, 1]
    say("cache_append without the latent copy")
    c = append_case(dims, lens, lq, seed=4, dev=cuda)
    cos, sin = rope_tables(max(lens), dims.idx_dim // 2)
    batch = dsa.Batch(c["cu_q"], c["cu_k"], device=cuda)
    n = int(c["cu_k"][-1])
    q8 = torch.empty(c["T"], dims.n_idx_heads, dims.idx_dim, dtype=torch.uint8, device=cuda)
    qs = torch.empty(c["T"], dims.n_idx_heads, dtype=torch.float32, device=cuda)
    k8 = torch.zeros(n, dims.idx_dim, dtype=torch.uint8, device=cuda)
    ks = torch.zeros(n, dtype=torch.float32, device=cuda)
    dsa.cache_append(dims, batch, c["q_idx"], c["k_idx"], None, torch.from_numpy(cos).to(cuda),
                     torch.from_numpy(sin).to(cuda), q8, qs, k8, ks, None)
    torch.cuda.synchronize()
    _, _, ok8, oks = oracle.cache_append(c["q_idx"].cpu().numpy(), c["k_idx"].cpu().numpy(), c["pos"],
                                         cos, sin, dims.idx_dim // 2)
    crow = c["cu_k"][1:] - 1
    assert np.array_equal(host(k8)[crow], ok8) and np.array_equal(host(ks)[crow], oks)


# ------------------------------------------------------------------ paged caches -----------

def to_pool(t, row_of, n_rows, fill=0):
    pool = torch.full((n_rows,) + tuple(t.shape[1:]), fill, dtype=t.dtype, device=t.device)
    pool[torch.from_numpy(row_of).to(t.device)] = t
    return pool


def paged_inputs(inp, seed, base_page=0):
    rng = np.random.default_rng(seed)
    table, row_of, n_rows = page_layout(inp["lens"], rng, base_page=base_page)
    p = dict(inp)
    p["k8"] = to_pool(inp["k8"], row_of, n_rows, 0x3C)
    p["k_scale"] = to_pool(inp["k_scale"], row_of, n_rows, 1.0)
    p["kv"] = to_pool(inp["kv"], row_of, n_rows, 0.5)
    return p, table


def forward(dims, inp, dev, page_table=None):
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=dev, page_table=page_table)
    T = batch.n_q
    out = torch.empty(T, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(T, dims.n_heads, dtype=torch.float32, device=dev)
    idx = torch.empty(T, dims.topk, dtype=torch.int32, device=dev)
    ws = torch.empty(dsa.workspace_size(dims, batch), dtype=torch.uint8, device=dev)
    dsa.forward(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], inp["q"],
                inp["kv"], out, lse, idx, ws)
    stride = (batch.max_len_k + 3) // 4 * 4
    sc = torch.zeros(T, stride, dtype=torch.float32, device=dev)
    dsa.indexer_scores(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], sc, stride)
    torch.cuda.synchronize()
    return out, lse, idx, sc


# Pages from id 60,000 on: pool rows above 3.84M, i.e. latent rows more than 4 GiB into the pool
# (1,152 bytes each), which the gathers reach through 64-bit addresses.
HIGH_PAGE = 60000


@pytest.mark.parametrize("shape,base_page", [("tiny", 0), ("prod", 0), ("prod", HIGH_PAGE)])
def test_paged_decode_forward_equals_packed(cuda, shape, base_page):
    dims = dsa_inputs.TINY if shape == "tiny" else dsa_inputs.PROD
    lens = [1, 63, 64, 65, 2048, 2049, 9000, 20001] if shape == "prod" else [1, 31, 64, 65, 300, 1000]
    say(f"paged decode forward {shape} lens {lens}, pages from id {base_page}")
    inp = dsa_inputs.decode_inputs(dims=dims, seed=5, device=cuda, lens=lens)
    ref = forward(dims, inp, cuda)
    pinp, table = paged_inputs(inp, seed=6, base_page=base_page)
    got = forward(dims, pinp, cuda, page_table=table)
    for name, a, b in zip(("out", "lse", "idx", "scores"), ref, got):
        if name == "scores":
            a = torch.cat([a[i, :n] for i, n in enumerate(lens)])
            b = torch.cat([b[i, :n] for i, n in enumerate(lens)])
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), f"{shape} paged {name}"


@pytest.mark.parametrize("base_page", [0, HIGH_PAGE])
def test_paged_sparse_mqa_prefill_rows_equal_packed(cuda, base_page):
    dims = dsa_inputs.PROD
    lens, lq = [3000, 700, 130], [40, 7, 130]
    say(f"paged sparse MQA, several rows per sequence, lens {lens} rows {lq}, pages from id {base_page}")
    g = torch.Generator().manual_seed(7)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, S = int(cu_q[-1]), int(cu_k[-1])
    q = torch.randn(T, dims.n_heads, dims.qk_dim, generator=g).to(torch.bfloat16).to(cuda)
    kv = torch.randn(S, dims.qk_dim, generator=g).to(torch.bfloat16).to(cuda)
    idx = torch.full((T, dims.topk), -1, dtype=torch.int32)
    t = 0
    for n, m in zip(lens, lq):
        for i in range(m):
            p = n - m + i
            sel = torch.randperm(p + 1, generator=g)[:min(dims.topk, p + 1)]
            idx[t, :len(sel)] = sel.to(torch.int32)
            t += 1
    idx = idx.to(cuda)
    rng = np.random.default_rng(8)
    table, row_of, n_rows = page_layout(lens, rng, base_page=base_page)
    kvp = to_pool(kv, row_of, n_rows, 0.25)
    res = []
    for pt, cache in ((None, kv), (table, kvp)):
        batch = dsa.Batch(cu_q, cu_k, device=cuda, page_table=pt)
        out = torch.empty(T, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=cuda)
        lse = torch.empty(T, dims.n_heads, dtype=torch.float32, device=cuda)
        dsa.sparse_mqa(dims, batch, q, cache, idx, out, lse)
        torch.cuda.synchronize()
        res.append((out, lse))
    assert torch.equal(res[0][0].view(torch.uint8), res[1][0].view(torch.uint8))
    assert torch.equal(res[0][1], res[1][1])
