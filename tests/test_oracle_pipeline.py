"""Pins of the oracle's whole pipeline (indexer -> top-k -> sparse MQA, ``oracle.forward_rows``)
and of the cache producer's composition (``oracle.cache_append``), against facts fixed outside
the composition:

- DSA equals dense causal attention whenever k covers every earlier position ("DeepSeek-V3.2
  explained", section 二.1: DSA is attention over TopK(Indexer); DSA deep dive, section 4: the
  short-sequence masked-MHA mode stands in for DSA), checked against the separately written
  textbook two-pass attention ``oracle.dense_causal``;
- the query position p = len_k - len_q + i of a batch row, the key rows of its own sequence,
  and the causal extent 0..p, on prefill, continuation and decode batches;
- a hand-worked four-token example of the whole path (tests/golden/forward_worked_example.json);
- the cache producer at angle 0 and at a quarter turn against torch's float8 cast (a library
  routine) of the same rows.
"""
import dataclasses
import json
import math
import os

import numpy as np
import torch

import dsa_inputs
import oracle
from helpers import host_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_prefill(L, topk, seed=0):
    dims = dataclasses.replace(dsa_inputs.TINY, topk=topk)
    inp = dsa_inputs.prefill_inputs(L, dims, seed=seed, device="cpu", needles=False)
    return dims, host_inputs(inp)


def brute_top(scores, k):
    """Positions of the k best scores by an O(n^2) rank count (ties -> lower position)."""
    n = len(scores)
    sel = [s for s in range(n)
           if sum(1 for u in range(n) if scores[u] > scores[s] or (u < s and scores[u] == scores[s])) < k]
    return sel + [-1] * (k - len(sel))


def test_forward_equals_dense_causal_when_k_is_L():
    L = 256
    dims, h = tiny_prefill(L, topk=L)
    rows = np.arange(L)
    orc = oracle.forward_rows(h, rows)
    assert np.array_equal(orc["pos"], rows)
    for t in rows:
        assert len(orc["scores"][t]) == t + 1  # causal extent: keys 0..t, the own position included
        assert orc["idx"][t].tolist() == list(range(t + 1)) + [-1] * (L - t - 1)
    ref_o, ref_l = oracle.dense_causal(h["q"], h["kv"], rows.astype(np.int32), dims.v_dim, dims.sm_scale)
    assert np.max(np.abs(orc["out"] - ref_o)) < 1e-13
    assert np.max(np.abs(orc["lse"] - ref_l)) < 1e-13


def test_forward_at_k32_dense_below_k_and_top_k_above():
    L = 256
    dims, h = tiny_prefill(L, topk=32)
    rows = np.array([0, 1, 30, 31, 32, 33, 100, 255])
    orc = oracle.forward_rows(h, rows)
    pos = rows.astype(np.int32)
    ref_o, ref_l = oracle.dense_causal(h["q"][rows], h["kv"], pos, dims.v_dim, dims.sm_scale)
    for i, t in enumerate(rows):
        # every score is the pair function of (query row t, key s) on the sequence's own rows
        for s in (0, t // 2, t):
            assert orc["scores"][i][s] == oracle.index_score(h["q8"][t], h["q_scale"][t], h["w"][t],
                                                             h["k8"][s], h["k_scale"][s])
        if t + 1 <= 32:  # k covers every earlier position: exactly dense attention
            assert orc["idx"][i].tolist() == list(range(t + 1)) + [-1] * (31 - t)
            assert np.max(np.abs(orc["out"][i] - ref_o[i])) < 1e-13
            assert np.max(np.abs(orc["lse"][i] - ref_l[i])) < 1e-13
        else:
            assert orc["idx"][i].tolist() == brute_top(orc["scores"][i].tolist(), 32)
            # sparse attention only ever sees part of the dense softmax mass
            assert np.all(orc["lse"][i] < ref_l[i] + 1e-12)


def test_forward_continuation_rows_sit_at_len_k_minus_len_q():
    # the last 3 queries of a 40-token sequence as a batch of their own (len_q = 3, len_k = 40)
    # give exactly what the full prefill gives for rows 37..39
    L, n = 40, 3
    dims, h = tiny_prefill(L, topk=8)
    full = oracle.forward_rows(h, [L - 3, L - 2, L - 1])
    part = dict(h)
    for key in ("q8", "q_scale", "w", "q"):
        part[key] = h[key][L - n:]
    part["cu_q"], part["cu_k"] = [0, n], [0, L]
    cont = oracle.forward_rows(part, [0, 1, 2])
    assert cont["pos"].tolist() == [37, 38, 39]
    assert np.array_equal(cont["idx"], full["idx"])
    assert all(np.array_equal(a, b) for a, b in zip(cont["scores"], full["scores"]))
    assert np.array_equal(cont["out"], full["out"]) and np.array_equal(cont["lse"], full["lse"])


def test_decode_batch_scores_positions_0_to_n_minus_1_of_its_own_sequence():
    lens = [5, 40, 77]
    dims = dataclasses.replace(dsa_inputs.TINY, topk=32)
    h = host_inputs(dsa_inputs.decode_inputs(3, dims, seed=3, device="cpu", lens=lens, needles=False))
    assert h["cu_q"] == [0, 1, 2, 3]
    for b, n in enumerate(lens):
        orc = oracle.forward_rows(h, [0], seq=b)
        k0 = h["cu_k"][b]
        assert orc["pos"].tolist() == [n - 1]
        sc = orc["scores"][0]
        assert len(sc) == n
        for s in (0, n // 3, n - 1):
            assert sc[s] == oracle.index_score(h["q8"][b], h["q_scale"][b], h["w"][b], h["k8"][k0 + s],
                                               h["k_scale"][k0 + s])
        kv_b = h["kv"][k0:k0 + n]
        ref_o, ref_l = oracle.dense_causal(h["q"][b:b + 1], kv_b, np.array([n - 1], np.int32), dims.v_dim,
                                           dims.sm_scale)
        if n <= 32:
            assert orc["idx"][0].tolist() == list(range(n)) + [-1] * (32 - n)
            assert np.max(np.abs(orc["out"] - ref_o)) < 1e-13
        else:
            assert orc["idx"][0].tolist() == brute_top(sc.tolist(), 32)
            o2, l2 = oracle.sparse_mqa(h["q"][b:b + 1], kv_b, orc["idx"], dims.v_dim, dims.sm_scale)
            assert np.array_equal(orc["out"], o2) and np.array_equal(orc["lse"], l2)


def _e4m3(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_golden_forward_example():
    ex = json.load(open(os.path.join(GOLDEN, "forward_worked_example.json")))
    dims = dsa_inputs.Dims(**ex["dims"])
    L = len(ex["k_idx"])
    inp = dict(q8=_e4m3(ex["q_idx"]), q_scale=np.ones((L, 1), np.float32), w=np.ones((L, 1), np.float32),
               k8=_e4m3(ex["k_idx"]), k_scale=np.array(ex["k_scale"], np.float32), q=_bf16(ex["q_main"]),
               kv=_bf16(ex["latent"]), cu_q=[0, L], cu_k=[0, L], dims=dims)
    orc = oracle.forward_rows(inp, np.arange(L))
    assert orc["idx"].tolist() == ex["expected_idx"]
    assert [s.tolist() for s in orc["scores"]] == ex["expected_scores"]
    env = {"e": math.e, "ln": math.log}
    for t in range(L):
        assert abs(orc["out"][t, 0, 0] - eval(ex["expected_out"][t], env)) < 1e-15
        assert abs(orc["lse"][t, 0] - eval(ex["expected_lse"][t], env)) < 1e-15


def _usual_tables(n_pos, rope_dim):
    ang = np.arange(n_pos)[:, None] * 10000.0 ** (-2.0 * np.arange(rope_dim // 2) / rope_dim)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def test_cache_append_against_torch_cast_at_angle_0_and_quarter_turn():
    rng = np.random.default_rng(11)
    H, d, R = 64, 128, 64
    q = (rng.normal(size=(4, H, d)) * rng.uniform(0.01, 50, size=(4, 1, 1))).astype(np.float32)
    k = (rng.normal(size=(4, d)) * 3).astype(np.float32)
    cos_t, sin_t = _usual_tables(8, R)
    cos_t[5], sin_t[5] = 0.0, 1.0  # position 5: a quarter turn, (x0, x1) -> (-x1, x0) exactly
    pos = np.array([0, 5, 0, 5])
    q8, qs, k8, ks = oracle.cache_append(q, k, pos, cos_t, sin_t, R)
    for i, p in enumerate(pos):
        qr, kr = q[i].copy(), k[i].copy()
        if p == 5:
            for x in (qr, kr):
                x0, x1 = x[..., 0:R:2].copy(), x[..., 1:R:2].copy()
                x[..., 0:R:2], x[..., 1:R:2] = -x1, x0
        c, s = dsa_inputs.quantize_e4m3_rows(torch.from_numpy(qr))
        assert np.array_equal(q8[i], c.numpy()) and np.array_equal(qs[i], s.numpy())
        c, s = dsa_inputs.quantize_e4m3_rows(torch.from_numpy(kr[None]))
        assert np.array_equal(k8[i], c.numpy()[0]) and ks[i] == s.numpy()[0]


def test_cache_append_is_rope_then_row_quantiser_at_every_position():
    rng = np.random.default_rng(12)
    H, d, R = 4, 32, 16
    q = rng.normal(size=(6, H, d)).astype(np.float32)
    k = rng.normal(size=(6, d)).astype(np.float32)
    cos_t, sin_t = _usual_tables(300, R)
    pos = np.array([0, 1, 2, 63, 64, 299])
    q8, qs, k8, ks = oracle.cache_append(q, k, pos, cos_t, sin_t, R)
    for i, p in enumerate(pos):
        a, sa = oracle.quantize_row_e4m3(oracle.rope_f32(q[i], p, cos_t, sin_t, R))
        b, sb = oracle.quantize_row_e4m3(oracle.rope_f32(k[i], p, cos_t, sin_t, R))
        assert np.array_equal(q8[i], a) and np.array_equal(qs[i], sa)
        assert np.array_equal(k8[i], b) and ks[i] == sb
    # positions differ in their rotation: the same vector at two positions gives two code rows
    q8b, _, _, _ = oracle.cache_append(np.repeat(q[:1], 2, 0), np.repeat(k[:1], 2, 0), np.array([1, 200]),
                                       cos_t, sin_t, R)
    assert not np.array_equal(q8b[0], q8b[1])
    assert np.array_equal(q8b[0][:, R:], q8b[0][:, R:])  # dims past the rope part: same values
