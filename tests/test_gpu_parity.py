"""GPU parity of every stage and of the whole path against the CPU oracle, through the C ABI.

Tolerances: indexer |g - o| <= 1e-3 * M + eps_acc * A (M = the score with |w| in place of w,
A = the same with sign-free codes, eps_acc = twice the FP8 MFMA accumulation error that
tests/test_gpu_fp8_accumulation.py measures and asserts); top-k on the
same fp32 arrays bit-exact; end-to-end sets identical except positions within 1e-3 of the
oracle's k-th score; attention max abs 2e-2 and relative L2 1e-2 against the oracle run on
the GPU's own index rows."""
import math

import numpy as np
import pytest
import torch

import dsa_inputs
import oracle
import sparse_attention_long_lightning_amd as dsa
from helpers import check_attention, check_scores, check_sets, host, host_inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def stride_for(n):
    return (n + 3) // 4 * 4


def run_indexer(inp, dims, dev, rows=None):
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=dev)
    T = batch.n_q
    stride = stride_for(batch.max_len_k)
    scores = torch.full((T, stride), float("nan"), dtype=torch.float32, device=dev)
    dsa.indexer_scores(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"],
                       scores, stride)
    torch.cuda.synchronize()
    return scores


def oracle_scores(h, rows, seq=0, mode="score"):
    """The oracle's scores; mode "absw" uses |w| (magnitude M), mode "abs" uses |w| and the
    codes with their sign bits cleared (magnitude A of the summed products)."""
    cu_q, cu_k = h["cu_q"], h["cu_k"]
    q0, q1, k0, k1 = cu_q[seq], cu_q[seq + 1], cu_k[seq], cu_k[seq + 1]
    rows = np.asarray(rows)
    pos = (k1 - k0) - (q1 - q0) + rows
    w = np.abs(h["w"]) if mode != "score" else h["w"]
    q8, k8 = h["q8"], h["k8"]
    if mode == "abs":
        q8, k8 = q8 & np.uint8(0x7F), k8 & np.uint8(0x7F)
    return oracle.indexer_rows(q8[q0 + rows], h["q_scale"][q0 + rows], w[q0 + rows],
                               k8[k0:k1], h["k_scale"][k0:k1], np.arange(len(rows)), pos)


def compare_indexer_rows(scores, h, rows, what, seq=0):
    ref = oracle_scores(h, rows, seq)
    mag = oracle_scores(h, rows, seq, mode="absw")
    mag_abs = oracle_scores(h, rows, seq, mode="abs")
    base = h["cu_q"][seq]
    for i, r in enumerate(rows):
        n = len(ref[i])
        got = scores[base + r, :n]
        assert np.isfinite(got).all(), f"{what}: row {r} has unwritten entries"
        check_scores(got, ref[i], mag[i], mag_abs[i], what=f"{what} row {r}")


# ------------------------------------------------------------------ indexer ---------------

def test_indexer_tiny_all_rows(cuda):
    say("indexer tiny L=256 all rows")
    dims = dsa_inputs.TINY
    inp = dsa_inputs.prefill_inputs(256, dims, seed=0, device=cuda, needles=False)
    scores = host(run_indexer(inp, dims, cuda))
    compare_indexer_rows(scores, host_inputs(inp), np.arange(256), "tiny")


def test_indexer_prod_ragged_all_rows(cuda):
    say("indexer prod L=1100 all rows (ragged tiles)")
    dims = dsa_inputs.PROD
    inp = dsa_inputs.prefill_inputs(1100, dims, seed=1, device=cuda, needles=False)
    scores = host(run_indexer(inp, dims, cuda))
    compare_indexer_rows(scores, host_inputs(inp), np.arange(1100), "prod-1100")


@pytest.mark.parametrize("dims_name,L", [("prod", 700), ("tiny", 300)])
def test_indexer_head_weight_extremes(cuda, dims_name, L):
    # The prefill kernel computes the linear half of w * ReLU(x) = w/2 * (x + |x|) as one dot
    # product with u = sum_j w'_j/2 q_j, expanded in FP8 terms scaled by the exponent of
    # max|u|.  Rows cycle through weights of tiny and huge magnitude, all zero (u = 0), a single
    # head, magnitudes spread over twelve decades with alternating signs, and all negative.
    dims = dsa_inputs.PROD if dims_name == "prod" else dsa_inputs.TINY
    say(f"indexer {dims_name} L={L}, extreme head weights")
    inp = dsa_inputs.prefill_inputs(L, dims, seed=4, device=cuda, needles=False)
    H = dims.n_idx_heads
    w = inp["w"].clone()
    kind = torch.arange(L, device=cuda) % 6
    j = torch.arange(H, device=cuda)
    spread = torch.where(j % 2 == 0, 1.0, -1.0) * torch.pow(10.0, (j % 12 - 6).float())
    one = torch.zeros(H, device=cuda)
    one[H // 3] = 1.7
    w[kind == 0] *= 1e-33
    w[kind == 1] *= 1e25
    w[kind == 2] = 0.0
    w[kind == 3] = one
    w[kind == 4] = spread
    w[kind == 5] = -w[kind == 5].abs()
    inp["w"] = w.contiguous()
    scores = host(run_indexer(inp, dims, cuda))
    compare_indexer_rows(scores, host_inputs(inp), np.arange(L), f"{dims_name} weight extremes")
    assert np.all(scores[2::6][np.isfinite(scores[2::6])] == 0.0)


def test_indexer_prod_16k_sampled_rows(cuda):
    say("indexer prod L=16384 sampled rows")
    dims = dsa_inputs.PROD
    inp = dsa_inputs.prefill_inputs(16384, dims, seed=0, device=cuda)
    scores = run_indexer(inp, dims, cuda)
    rows = np.array([0, 7, 8, 511, 512, 2047, 2048, 5000, 8191, 12345, 16376, 16383])
    h = host_inputs({k: v for k, v in inp.items() if k not in ("q", "kv")})
    compare_indexer_rows(host(scores), h, rows, "prod-16k")


def test_indexer_decode_batch(cuda):
    say("indexer decode B=5 lens 3000..9000")
    dims = dsa_inputs.PROD
    lens = [3000, 4097, 5555, 8191, 9000]
    inp = dsa_inputs.decode_inputs(dims=dims, seed=3, device=cuda, lens=lens)
    scores = host(run_indexer(inp, dims, cuda))
    h = host_inputs({k: v for k, v in inp.items() if k not in ("q", "kv")})
    for b in range(len(lens)):
        compare_indexer_rows(scores, h, np.array([0]), f"decode seq {b}", seq=b)


# ------------------------------------------------------------------ top-k -----------------

def adversarial_rows(k, rng):
    """Score rows of chosen lengths and contents (each row is its own one-query sequence)."""
    rows = []
    rows.append(rng.normal(size=k - 1))                     # shorter than k
    rows.append(rng.normal(size=k))                         # exactly k
    rows.append(rng.normal(size=k + 1))                     # k + 1
    rows.append(np.array([3.5]))                            # length 1
    rows.append(np.full(5000, 0.25))                        # constant row
    rows.append(np.full(20000, -1.5))                       # constant row beyond the LDS list
    x = rng.normal(size=9000)
    x[rng.permutation(9000)[:4000]] = np.sort(x)[-1500]     # huge tie group at the threshold
    rows.append(x)
    x = rng.integers(-3, 4, 7000).astype(np.float64)        # few distinct values
    rows.append(x)
    x = rng.normal(size=6000)
    x[::3] = 0.0
    x[1::7] = -0.0
    x[5::11] = -np.inf
    x[2::13] = np.nan
    x[4::17] = np.inf
    rows.append(x)
    rows.append(np.arange(10000, dtype=np.float64))         # ascending
    rows.append(-np.arange(10000, dtype=np.float64))        # descending
    bits = rng.integers(0, 2 ** 32, 12000, dtype=np.uint64).astype(np.uint32)
    rows.append(bits.view(np.float32).astype(np.float64))   # random fp32 bit patterns (incl. NaN)
    rows.append(rng.normal(size=131072) * 1e-3)             # longest prefill row
    rows.append(np.abs(rng.normal(size=50000)) + 10.0)      # one exponent range
    rows.append(np.full(70000, 2.0))                        # ties across five 16K segments
    x = rng.normal(size=50000)
    x[rng.permutation(50000)[:6000]] = np.sort(x)[-1000]    # threshold ties in every segment
    rows.append(x)
    rows.append(rng.normal(size=16384))                     # one full segment
    rows.append(rng.normal(size=16385))                     # a segment plus one element
    x = rng.normal(size=40000)
    x[16384 - 3000:16384 + 3000] = 7.0                      # a tie block across a boundary
    rows.append(x)
    return [r.astype(np.float32) for r in rows]


def topk_ws(dims, batch, split, cuda):
    """Workspace for the segmented path (split=True) or None (one workgroup per row)."""
    if not split:
        return None
    n = dsa.topk_workspace_size(dims, batch)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device=cuda)


@pytest.mark.parametrize("k,split", [(2048, False), (2048, True), (32, False), (32, True), (1, False),
                                     (1, True), (4096, False), (8192, False)])
def test_topk_bit_exact_on_identical_arrays(cuda, k, split):
    say(f"topk adversarial rows k={k} split={split}")
    rng = np.random.default_rng(7 + k)
    rows = adversarial_rows(max(k, 4), rng)
    lens = [len(r) for r in rows]
    stride = stride_for(max(lens))
    buf = np.full((len(rows), stride), np.nan, np.float32)
    for i, r in enumerate(rows):
        buf[i, : len(r)] = r
    cu_q = list(range(len(rows) + 1))
    cu_k = [0] + list(np.cumsum(lens))
    dims = dsa.Dims(64, 128, k, 128, 576, 512, 0.07)
    batch = dsa.Batch(cu_q, cu_k, device=cuda)
    scores = torch.from_numpy(buf).to(cuda)
    idx = torch.empty(len(rows), k, dtype=torch.int32, device=cuda)
    dsa.topk(dims, batch, scores, stride, idx, ws=topk_ws(dims, batch, split, cuda))
    torch.cuda.synchronize()
    ref = oracle.topk_rows(rows, k)
    got = idx.cpu().numpy()
    for i in range(len(rows)):
        assert np.array_equal(got[i], ref[i]), f"row {i} (len {lens[i]}) differs"


def test_topk_prefill_rows_with_shortcut(cuda):
    say("topk prefill rows of one sequence (rows < k take every position)")
    L, k = 3000, 2048
    rng = np.random.default_rng(11)
    buf = rng.normal(size=(L, stride_for(L))).astype(np.float32)
    dims = dsa.Dims(64, 128, k, 128, 576, 512, 0.07)
    batch = dsa.Batch([0, L], [0, L], device=cuda)
    idx = torch.empty(L, k, dtype=torch.int32, device=cuda)
    dsa.topk(dims, batch, torch.from_numpy(buf).to(cuda), buf.shape[1], idx)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    rows = [0, 1, 2046, 2047, 2048, 2500, 2999]
    ref = oracle.topk_rows([buf[r, : r + 1] for r in rows], k)
    for i, r in enumerate(rows):
        assert np.array_equal(got[r], ref[i]), f"row {r}"


@pytest.mark.parametrize("split", [False, True])
def test_topk_few_prefill_rows(cuda, split):
    say(f"topk 120 rows of two sequences (one of them all below k) split={split}")
    k = 2048
    rng = np.random.default_rng(12)
    lq, lk = [60, 60], [60, 30000]
    stride = stride_for(max(lk))
    buf = rng.normal(size=(sum(lq), stride)).astype(np.float32)
    dims = dsa.Dims(64, 128, k, 128, 576, 512, 0.07)
    batch = dsa.Batch([0, 60, 120], [0, 60, 30060], device=cuda)
    idx = torch.empty(sum(lq), k, dtype=torch.int32, device=cuda)
    dsa.topk(dims, batch, torch.from_numpy(buf).to(cuda), stride, idx, ws=topk_ws(dims, batch, split, cuda))
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    rows = [buf[i, : i + 1] for i in range(60)] + [buf[60 + i, : lk[1] - lq[1] + i + 1] for i in range(60)]
    ref = oracle.topk_rows(rows, k)
    for i in range(120):
        assert np.array_equal(got[i], ref[i]), f"row {i}"


# ------------------------------------------------------------------ sparse MQA ------------

def random_idx(T, k, S, rng, empty_frac=0.1):
    idx = np.stack([rng.permutation(S)[:k] for _ in range(T)]).astype(np.int32)
    idx[rng.random(idx.shape) < empty_frac] = -1
    idx[0, :] = -1  # a row with no valid slot
    idx[1, 1:] = -1  # a row with one valid slot
    return idx


@pytest.mark.parametrize("shape,T,S", [("tiny", 40, 300), ("prod", 24, 5000), ("prod", 300, 3000)])
def test_sparse_mqa_against_oracle(cuda, shape, T, S):
    say(f"sparse MQA {shape} T={T} S={S}")
    dims = dsa_inputs.TINY if shape == "tiny" else dsa_inputs.PROD
    rng = np.random.default_rng(5)
    g = torch.Generator(device=cuda).manual_seed(5)
    q = torch.randn(T, dims.n_heads, dims.qk_dim, generator=g, device=cuda).to(torch.bfloat16)
    kv = torch.randn(S, dims.qk_dim, generator=g, device=cuda).to(torch.bfloat16)
    idx = random_idx(T, dims.topk, S, rng)
    batch = dsa.Batch([0, T], [0, S], device=cuda)
    out = torch.empty(T, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=cuda)
    lse = torch.empty(T, dims.n_heads, dtype=torch.float32, device=cuda)
    ws = torch.empty(max(16, dsa.workspace_size(dims, batch)), dtype=torch.uint8, device=cuda)
    dsa.sparse_mqa(dims, batch, q, kv, torch.from_numpy(idx).to(cuda), out, lse, ws)
    torch.cuda.synchronize()
    check_rows = np.arange(T) if T <= 40 else np.r_[0:8, T - 8:T]
    ref_o, ref_l = oracle.sparse_mqa(host(q)[check_rows], host(kv), idx[check_rows], dims.v_dim, dims.sm_scale)
    check_attention(host(out)[check_rows], ref_o, what=f"mqa {shape}")
    got_l = lse.cpu().numpy()[check_rows]
    assert np.all(np.isneginf(got_l[0])) and np.all(np.isneginf(ref_l[0]))
    fin = np.isfinite(ref_l)
    np.testing.assert_allclose(got_l[fin], ref_l[fin], rtol=0, atol=2e-3)


def test_sparse_mqa_split_path_decode_shape(cuda):
    say("sparse MQA decode shape (split over slots) B=32")
    dims = dsa_inputs.PROD
    B, S = 32, 4000
    rng = np.random.default_rng(9)
    g = torch.Generator(device=cuda).manual_seed(9)
    q = torch.randn(B, dims.n_heads, dims.qk_dim, generator=g, device=cuda).to(torch.bfloat16)
    kv = torch.randn(B * S, dims.qk_dim, generator=g, device=cuda).to(torch.bfloat16)
    idx = random_idx(B, dims.topk, S, rng, empty_frac=0.0)
    batch = dsa.Batch(list(range(B + 1)), [b * S for b in range(B + 1)], device=cuda)
    out = torch.empty(B, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=cuda)
    lse = torch.empty(B, dims.n_heads, dtype=torch.float32, device=cuda)
    ws = torch.empty(dsa.workspace_size(dims, batch), dtype=torch.uint8, device=cuda)
    dsa.sparse_mqa(dims, batch, q, kv, torch.from_numpy(idx).to(cuda), out, lse, ws)
    torch.cuda.synchronize()
    rows = [0, 1, 2, 17, 31]
    for b in rows:
        ro, rl = oracle.sparse_mqa(host(q)[b:b + 1], host(kv)[b * S:(b + 1) * S], idx[b:b + 1],
                                   dims.v_dim, dims.sm_scale)
        check_attention(host(out)[b:b + 1], ro, what=f"decode seq {b}")
        if np.isfinite(rl).all():
            np.testing.assert_allclose(lse.cpu().numpy()[b], rl[0], atol=2e-3)


# ------------------------------------------------------------------ whole path ------------

def run_forward(inp, dims, dev, ws_bytes=None):
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=dev)
    T = batch.n_q
    out = torch.empty(T, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(T, dims.n_heads, dtype=torch.float32, device=dev)
    idx = torch.empty(T, dims.topk, dtype=torch.int32, device=dev)
    n = dsa.workspace_size(dims, batch) if ws_bytes is None else ws_bytes
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    dsa.forward(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"],
                inp["q"], inp["kv"], out, lse, idx, ws)
    torch.cuda.synchronize()
    return out, lse, idx


def compare_forward_rows(inp, h, out, lse, idx, rows, dims, what, seq=0, needles=None):
    orc = oracle.forward_rows(h, rows, seq=seq)
    gi = idx.cpu().numpy()[h["cu_q"][seq] + np.asarray(rows)]
    ndiff = 0
    for i in range(len(rows)):
        ndiff += check_sets(gi[i], orc["idx"][i], orc["scores"][i], dims.topk)
    k0, k1 = h["cu_k"][seq], h["cu_k"][seq + 1]
    qr = h["cu_q"][seq] + np.asarray(rows)
    ro, rl = oracle.sparse_mqa(h["q"][qr], h["kv"][k0:k1], gi, dims.v_dim, dims.sm_scale)
    check_attention(host(out)[qr], ro, what=what)
    np.testing.assert_allclose(lse.cpu().numpy()[qr], rl, rtol=0, atol=2e-3)
    return orc, ndiff


def test_forward_tiny_end_to_end(cuda):
    say("forward tiny L=256 k=32")
    dims = dsa_inputs.TINY
    inp = dsa_inputs.prefill_inputs(256, dims, seed=0, device=cuda, needles=False)
    out, lse, idx = run_forward(inp, dims, cuda)
    h = host_inputs(inp)
    compare_forward_rows(inp, h, out, lse, idx, np.arange(256), dims, "tiny forward")


def test_forward_tiny_dense_when_k_is_L(cuda):
    say("forward tiny L=256 k=256 equals dense causal attention")
    dims = dsa_inputs.Dims(4, 32, 256, 8, 80, 64, 1 / math.sqrt(80))
    inp = dsa_inputs.prefill_inputs(256, dims, seed=0, device=cuda, needles=False)
    out, lse, idx = run_forward(inp, dims, cuda)
    h = host_inputs(inp)
    gi = idx.cpu().numpy()
    for t in range(256):
        assert np.array_equal(gi[t], np.r_[np.arange(t + 1), np.full(255 - t, -1)])
    ro, rl = oracle.dense_causal(h["q"], h["kv"], np.arange(256, dtype=np.int32), dims.v_dim, dims.sm_scale)
    check_attention(host(out), ro, what="dense")


def test_forward_prod_16k_sampled(cuda):
    say("forward prod L=16384 sampled rows + needle recall")
    dims = dsa_inputs.PROD
    inp = dsa_inputs.prefill_inputs(16384, dims, seed=0, device=cuda)
    out, lse, idx = run_forward(inp, dims, cuda)
    h = host_inputs(inp)
    needles = inp["needles"]
    rng = np.random.default_rng(0)
    nrows = sorted(set([t for t, s in needles[::97]]))[:10]
    rows = sorted(set([0, 1, 2047, 2048, 2049, 16383] + list(rng.integers(2048, 16384, 6)) + nrows))
    orc, ndiff = compare_forward_rows(inp, h, out, lse, idx, rows, dims, "prod-16k forward")
    gi = idx.cpu().numpy()
    planted = [(t, s) for t, s in needles if t in set(rows)]
    rec_g = np.mean([s in set(gi[t]) for t, s in planted])
    rec_o = np.mean([s in set(orc["idx"][rows.index(t)]) for t, s in planted])
    say(f"needle recall gpu {rec_g:.3f} oracle {rec_o:.3f} over {len(planted)}; set diffs {ndiff}")
    assert rec_g == rec_o


def test_forward_small_workspace_is_identical(cuda):
    say("forward prod L=3000 default vs minimal and a third of the default workspace (bit-identical)")
    dims = dsa_inputs.PROD
    inp = dsa_inputs.prefill_inputs(3000, dims, seed=2, device=cuda)
    o1, l1, i1 = run_forward(inp, dims, cuda)
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=cuda)
    o2, l2, i2 = run_forward(inp, dims, cuda, ws_bytes=dsa.workspace_min(dims, batch))
    assert torch.equal(i1, i2) and torch.equal(o1, o2) and torch.equal(l1, l2)
    # a third of the default: three passes of different row counts at different score strides
    o4, l4, i4 = run_forward(inp, dims, cuda, ws_bytes=dsa.workspace_size(dims, batch) // 3)
    assert torch.equal(i1, i4) and torch.equal(o1, o4) and torch.equal(l1, l4)
    o3, l3, i3 = run_forward(inp, dims, cuda)  # determinism
    assert torch.equal(i1, i3) and torch.equal(o1, o3) and torch.equal(l1, l3)


def test_forward_decode_small(cuda):
    say("forward decode B=6 lens 1500..20000")
    dims = dsa_inputs.PROD
    lens = [1500, 2048, 2049, 7000, 12345, 20000]
    inp = dsa_inputs.decode_inputs(dims=dims, seed=4, device=cuda, lens=lens)
    out, lse, idx = run_forward(inp, dims, cuda)
    h = host_inputs(inp)
    for b in range(len(lens)):
        compare_forward_rows(inp, h, out, lse, idx, [0], dims, f"decode seq {b}", seq=b)


def test_forward_decode_32_full_size_all_sequences(cuda):
    say("forward decode B=32 lens U[32768,131072], every sequence + needle recall")
    from concurrent.futures import ThreadPoolExecutor

    dims = dsa_inputs.PROD
    inp = dsa_inputs.decode_inputs(32, dims=dims, seed=0, device=cuda)
    out, lse, idx = run_forward(inp, dims, cuda)
    h = host_inputs(inp)
    # one oracle row per sequence: the sequences run side by side (the oracle call releases
    # the interpreter while it computes)
    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(lambda b: compare_forward_rows(inp, h, out, lse, idx, [0], dims, f"decode32 seq {b}",
                                                         seq=b), range(32)))
    gi = idx.cpu().numpy()
    rec_g = np.mean([s in set(gi[b]) for b, s in inp["needles"]])
    rec_o = np.mean([s in set(res[b][0]["idx"][0]) for b, s in inp["needles"]])
    say(f"decode32: set differences {sum(r[1] for r in res)}, needle recall gpu {rec_g:.4f} oracle {rec_o:.4f} "
        f"over {len(inp['needles'])} needles")
    assert rec_g == rec_o


def test_forward_ragged_prefill_batch(cuda):
    # three sequences in one call: a full prefill, a short one below k, and a chunk of 2500 new
    # rows continuing a 9000-token cache (len_q < len_k); small workspace so passes split rows
    dims = dsa_inputs.PROD
    lq, lk = [3000, 700, 2500], [3000, 700, 9000]
    say(f"forward prod ragged prefill batch lq {lq} lk {lk}")
    parts = [dsa_inputs.prefill_inputs(n, dims, seed=20 + i, device=cuda) for i, n in enumerate(lk)]
    inp = {"dims": dims}
    for key in ("k8", "k_scale", "kv"):
        inp[key] = torch.cat([p[key] for p in parts])
    for key in ("q8", "q_scale", "w", "q"):
        inp[key] = torch.cat([p[key][n - m:] for p, n, m in zip(parts, lk, lq)])
    inp["cu_q"] = [0] + list(np.cumsum(lq))
    inp["cu_k"] = [0] + list(np.cumsum(lk))
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=cuda)
    out, lse, idx = run_forward(inp, dims, cuda, ws_bytes=dsa.workspace_min(dims, batch) + (64 << 20))
    h = host_inputs(inp)
    for seq, rows in ((0, [0, 2047, 2048, 2999]), (1, [0, 350, 699]), (2, [0, 1, 1250, 2499])):
        compare_forward_rows(inp, h, out, lse, idx, rows, dims, f"ragged seq {seq}", seq=seq)
