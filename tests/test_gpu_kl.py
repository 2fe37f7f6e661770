"""GPU parity of the indexer KL target (forward only), through the C ABI.

dsa_indexer_kl against the oracle's definition on the same inputs (bf16 query and latent rows,
the attention LSE computed by the oracle, seeded indexer scores).  Tolerance
|g - o| <= 2e-4 + 1e-3 |o|: the kernel's logits carry the fp32 accumulation error of the bf16
MFMA (relative ~1e-6 per logit at these magnitudes) and its exponentials and logarithms are
fp32 (~1e-6 relative); KL(P||Q) = A/Z - ln Z - B/Z + LSE(I) loses about one more digit to the
cancellation between B/Z and LSE(I) for scores of magnitude ~10, which leaves 2e-4 ample."""
import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
import sparse_attention_long_lightning_amd as dsa
from helpers import host

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def check_kl(got, ref, what):
    got = np.asarray(got, np.float64)
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf), f"{what}: infinite entries differ"
    err = np.abs(got[~inf] - ref[~inf])
    bound = 2e-4 + 1e-3 * np.abs(ref[~inf])
    bad = np.flatnonzero(err > bound)
    assert len(bad) == 0, f"{what}: {len(bad)} rows out of tolerance, first {bad[0]}: {got[~inf][bad[0]]} vs {ref[~inf][bad[0]]}"


def case(dims, lq, lk, seed, dev, sparse, empty_frac=0.1, score_scale=3.0):
    """One sequence of lk keys whose last lq positions are query rows."""
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    q = torch.randn(lq, dims.n_heads, dims.qk_dim, generator=g).to(torch.bfloat16)
    kv = torch.randn(lk, dims.qk_dim, generator=g).to(torch.bfloat16)
    stride = (lk + 3) // 4 * 4
    scores = (torch.randn(lq, stride, generator=g) * score_scale).float()
    pos = np.arange(lk - lq, lk)
    hq, hkv = host(q), host(kv)
    if sparse:
        k = dims.topk
        idx = np.full((lq, k), -1, np.int32)
        for i, p in enumerate(pos):
            n = min(k, p + 1)
            sel = rng.permutation(p + 1)[:n]
            keep = rng.random(n) >= empty_frac
            slots = rng.permutation(k)[:n]
            idx[i, slots[keep]] = sel[keep]
        _, lse = oracle.sparse_mqa(hq, hkv, idx, dims.v_dim, dims.sm_scale)
        slots_of = [idx[i] for i in range(lq)]
    else:
        idx = None
        _, lse = oracle.dense_causal(hq, hkv, pos.astype(np.int32), dims.v_dim, dims.sm_scale)
        slots_of = [np.arange(p + 1) for p in pos]
    lse = lse.astype(np.float32)
    kl, rev = oracle.indexer_kl(hq, hkv, lse, slots_of, list(scores.numpy()), dims.sm_scale)
    batch = dsa.Batch([0, lq], [0, lk], device=dev)
    return dict(q=q.to(dev), kv=kv.to(dev), lse=torch.from_numpy(lse).to(dev), scores=scores.to(dev),
                idx=None if idx is None else torch.from_numpy(idx).to(dev), stride=stride, batch=batch,
                kl=kl, rev=rev, lq=lq, lk=lk)


def run(dims, c, dev, batch=None, kv=None):
    kl = torch.full((c["lq"],), float("nan"), device=dev)
    rev = torch.full((c["lq"],), float("nan"), device=dev)
    dsa.indexer_kl(dims, batch or c["batch"], c["q"], c["kv"] if kv is None else kv, c["lse"], c["idx"],
                   c["scores"], c["stride"], kl, rev)
    torch.cuda.synchronize()
    return kl.cpu().numpy(), rev.cpu().numpy()


@pytest.mark.parametrize("sparse", [True, False])
def test_indexer_kl_tiny_every_row(cuda, sparse):
    dims = dsa_inputs.TINY
    say(f"indexer KL tiny L=200, {'selected slots' if sparse else 'every earlier position'}")
    c = case(dims, 200, 200, 1, cuda, sparse)
    kl, rev = run(dims, c, cuda)
    check_kl(kl, c["kl"], "tiny KL(P||Q)")
    check_kl(rev, c["rev"], "tiny KL(Q||P)")


@pytest.mark.parametrize("sparse", [True, False])
def test_indexer_kl_prod(cuda, sparse):
    dims = dsa_inputs.PROD
    lq, lk = (48, 3000) if sparse else (24, 1100)
    say(f"indexer KL prod {lq} rows of a {lk}-token sequence, {'top-k slots' if sparse else 'dense'}")
    c = case(dims, lq, lk, 2, cuda, sparse)
    kl, rev = run(dims, c, cuda)
    check_kl(kl, c["kl"], "prod KL(P||Q)")
    check_kl(rev, c["rev"], "prod KL(Q||P)")


@pytest.mark.parametrize("base_page", [0, 60000])
def test_indexer_kl_paged_equals_packed(cuda, base_page):
    # base_page 60,000: pool rows above 3.84M, latent rows more than 4 GiB into the pool
    dims = dsa_inputs.PROD
    say(f"indexer KL with a paged latent cache == packed, pages from id {base_page}")
    c = case(dims, 16, 700, 3, cuda, True)
    ref = run(dims, c, cuda)
    rng = np.random.default_rng(4)
    n_pages = (700 + 63) // 64 + 3
    perm = rng.permutation(n_pages) + base_page
    table = perm[: (700 + 63) // 64].astype(np.int32)[None, :]
    p = np.arange(700)
    rows = table[0, p // 64].astype(np.int64) * 64 + p % 64
    pool = torch.zeros((base_page + n_pages) * 64, dims.qk_dim, dtype=torch.bfloat16, device=cuda)
    pool[torch.from_numpy(rows).to(cuda)] = c["kv"]
    batch = dsa.Batch([0, 16], [0, 700], device=cuda, page_table=table)
    got = run(dims, c, cuda, batch=batch, kv=pool)
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])
