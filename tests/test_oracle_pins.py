"""Pins of the CPU oracle against facts fixed outside the oracle itself: library codecs,
closed forms of the indexer score, brute-force ranks for the selection, textbook attention
(torch's scaled_dot_product_attention) and hand-worked fixtures under tests/golden/.

Each test is chosen so that a plausible slip in the oracle (a dropped head or dim, a scale
applied per token instead of per head, w inside the ReLU, a wrong tie rule, an off-by-one
causal bound, a transposed operand) fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest
import torch

import dsa_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def e4m3_code(x: float) -> int:
    """Code of an exactly representable e4m3 value (via torch's cast, a library routine)."""
    t = torch.tensor([x], dtype=torch.float32).to(torch.float8_e4m3fn)
    assert float(t.float()) == x, x
    return int(t.view(torch.uint8))


def finite_codes(n, rng=RNG):
    c = rng.integers(0, 256, n).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # replace the NaN patterns by 1.0
    return c


# ---------------------------------------------------------------- codecs ------------------

def test_e4m3_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(mine[~nan], ref[~nan])


def test_e4m3_spot_values():
    assert oracle.decode_e4m3([0x7E])[0] == 448.0
    assert oracle.decode_e4m3([0xFE])[0] == -448.0
    assert oracle.decode_e4m3([0x08])[0] == 2.0 ** -6  # smallest normal
    assert oracle.decode_e4m3([0x01])[0] == 2.0 ** -9  # smallest subnormal
    assert oracle.decode_e4m3([0x07])[0] == 7 * 2.0 ** -9
    assert oracle.decode_e4m3([0x38])[0] == 1.0
    assert oracle.decode_e4m3([0x80])[0] == 0.0 and math.copysign(1, oracle.decode_e4m3([0x80])[0]) < 0


def test_e4m3_fixed_point_is_value_times_512():
    for b in range(256):
        if (b & 0x7F) == 0x7F:
            continue
        assert oracle.e4m3_fixed(b) == oracle.decode_e4m3([b])[0] * 512


def test_bf16_matches_torch():
    bits = RNG.integers(0, 1 << 16, 4096).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # drop inf/nan exponents
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    assert np.array_equal(oracle.decode_bf16(bits), ref)


# ---------------------------------------------------------------- indexer -----------------

def test_dot_is_exact_fixed_vs_double_vs_matmul():
    for d in (32, 128):
        for _ in range(50):
            a, b = finite_codes(d), finite_codes(d)
            dd = oracle.dot_e4m3(a, b)
            assert dd * 2.0 ** 18 == oracle.dot_e4m3_fixed(a, b)
            lut = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
            assert dd == float(lut[a] @ lut[b])  # every partial sum is exact in double


def test_index_score_one_hot_closed_form():
    H, d = 4, 32
    # head j has a single non-zero code at dim j, the key has non-zeros at dims 0 and 2
    q = np.zeros((H, d), np.uint8)
    vals_q = [2.0, -3.0, 0.5, 6.0]
    for j in range(H):
        q[j, j] = e4m3_code(vals_q[j])
    k = np.zeros(d, np.uint8)
    k[0] = e4m3_code(1.5)
    k[2] = e4m3_code(-4.0)
    k[3] = e4m3_code(0.25)
    qs = np.array([0.5, 2.0, 4.0, 0.125], np.float32)
    w = np.array([1.0, -2.0, 0.75, 3.0], np.float32)
    ks = 0.0625
    D = [2.0 * 1.5, 0.0, 0.5 * -4.0, 6.0 * 0.25]
    expect = sum(w[j] * max(0.0, qs[j] * ks * D[j]) for j in range(H))
    # head 0: 1*(0.5*0.0625*3) ; head 1: D = 0 ; head 2: D < 0 ; head 3: 3*(0.125*0.0625*1.5)
    assert expect == 0.09375 + 0.03515625
    assert oracle.index_score(q, qs, w, k, ks) == expect


def test_index_score_constant_vectors():
    H, d = 64, 128
    a, b = 0.75, -1.25
    q = np.full((H, d), e4m3_code(a), np.uint8)
    k = np.full(d, e4m3_code(b), np.uint8)
    qs = RNG.uniform(0.1, 2, H).astype(np.float32)
    w = RNG.normal(size=H).astype(np.float32)
    ks = np.float32(0.3)
    # D = d * a * b < 0 for every head -> I = 0 ; flip the key sign -> every head positive
    assert oracle.index_score(q, qs, w, k, ks) == 0.0
    k2 = np.full(d, e4m3_code(-b), np.uint8)
    expect = sum(float(w[j]) * (float(qs[j]) * float(ks) * d * a * -b) for j in range(H))
    assert oracle.index_score(q, qs, w, k2, ks) == pytest.approx(expect, rel=1e-14)


def test_index_score_weight_outside_relu_and_homogeneity():
    H, d = 4, 32
    q = finite_codes(H * d).reshape(H, d)
    k = finite_codes(d)
    qs = RNG.uniform(0.01, 1, H).astype(np.float32)
    w = RNG.normal(size=H).astype(np.float32)
    ks = 0.5
    base = oracle.index_score(q, qs, w, k, ks)
    assert oracle.index_score(q, qs, (4 * w).astype(np.float32), k, ks) == 4 * base
    assert oracle.index_score(q, qs, -w, k, ks) == -base
    # a negative weight on a positive head must contribute (w outside the ReLU)
    q1 = np.zeros((1, d), np.uint8)
    q1[0, 0] = e4m3_code(1.0)
    k1 = np.zeros(d, np.uint8)
    k1[0] = e4m3_code(2.0)
    assert oracle.index_score(q1, np.array([1.0], np.float32), np.array([-3.0], np.float32), k1, 1.0) == -6.0


def test_indexer_rows_match_pair_function_and_causal_extent():
    T, H, d = 12, 4, 32
    q8 = finite_codes(T * H * d).reshape(T, H, d)
    k8 = finite_codes(T * d).reshape(T, d)
    qs = RNG.uniform(0.01, 1, (T, H)).astype(np.float32)
    w = RNG.normal(size=(T, H)).astype(np.float32)
    ks = RNG.uniform(0.01, 1, T).astype(np.float32)
    rows = np.arange(T)
    pos = np.arange(T)
    res = oracle.indexer_rows(q8, qs, w, k8, ks, rows, pos)
    for t in range(T):
        assert len(res[t]) == t + 1  # keys 0..t, the query's own position included
        for s in range(t + 1):
            assert res[t][s] == oracle.index_score(q8[t], qs[t], w[t], k8[s], ks[s])


def test_golden_indexer_example():
    ex = json.load(open(os.path.join(GOLDEN, "indexer_worked_example.json")))
    q = np.array([[e4m3_code(x) for x in row] for row in ex["q"]], np.uint8)
    k = np.array([e4m3_code(x) for x in ex["k"]], np.uint8)
    got = oracle.index_score(q, np.array(ex["q_scale"], np.float32), np.array(ex["w"], np.float32),
                             k, ex["k_scale"])
    assert got == ex["expected"]


# ---------------------------------------------------------------- top-k -------------------

def brute_topk(x, k):
    """s is selected iff #{u: x_u > x_s} + #{u < s: x_u == x_s} < k (NaN ranked lowest)."""
    n = len(x)
    key = [(-math.inf if math.isnan(v) else v, math.isnan(v)) for v in x]
    sel = []
    for s in range(n):
        above = 0
        for u in range(n):
            gu = (not key[u][1] and (key[s][1] or key[u][0] > key[s][0]))
            eq = (key[u][1] and key[s][1]) or (not key[u][1] and not key[s][1] and key[u][0] == key[s][0])
            if gu or (u < s and eq):
                above += 1
        if above < k:
            sel.append(s)
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("n,k", [(1, 4), (3, 4), (4, 4), (5, 4), (40, 7), (64, 32), (200, 32)])
def test_topk_matches_brute_force_rank(n, k):
    for trial in range(5):
        x = RNG.integers(-5, 6, n).astype(np.float64)  # many duplicates
        if trial == 1:
            x = np.zeros(n)
        if trial == 2:
            x = np.arange(n, dtype=np.float64)
        if trial == 3:
            x = -np.arange(n, dtype=np.float64)
        got = oracle.topk_rows([x], k)[0]
        assert got.tolist() == brute_topk(x.tolist(), k)


def test_topk_special_values():
    x = np.array([0.0, -0.0, np.nan, -np.inf, 1.0, np.inf, -0.0, np.nan, -1.0], np.float32)
    got = oracle.topk_rows([x], 9)[0].tolist()
    assert got == list(range(9))  # everything selected, ascending positions
    got = oracle.topk_rows([x], 5)[0].tolist()
    # ranking: inf(5), 1(4), 0(0), -0(1), -0(6) | -1, -inf, nan, nan
    assert got == [0, 1, 4, 5, 6]
    got = oracle.topk_rows([x], 8)[0].tolist()  # -inf in, first NaN (lower position) in
    assert got == [0, 1, 2, 3, 4, 5, 6, 8]
    assert brute_topk(x.astype(np.float64).tolist(), 8) == got


def test_topk_invariants_random_rows():
    for n in (100, 2049, 5000):
        x = RNG.normal(size=n).astype(np.float32)
        x[RNG.integers(0, n, n // 10)] = 0.5  # a tie group
        k = 2048
        sel = oracle.topk_rows([x], k)[0]
        valid = sel[sel >= 0]
        assert len(valid) == min(k, n)
        assert np.all(np.diff(valid) > 0)
        mask = np.zeros(n, bool)
        mask[valid] = True
        if (~mask).any():
            assert x[mask].min() >= x[~mask].max()
            thr = x[mask].min()
            if (x[~mask] == thr).any():  # ties at the threshold: selected ones have lower positions
                assert np.flatnonzero(mask & (x == thr)).max() < np.flatnonzero(~mask & (x == thr)).min()


def test_topk_short_rows_are_all_positions():
    got = oracle.topk_rows([np.ones(5)], 8)[0].tolist()
    assert got == [0, 1, 2, 3, 4, -1, -1, -1]


def test_golden_topk_example():
    ex = json.load(open(os.path.join(GOLDEN, "topk_worked_example.json")))
    x = np.array(ex["scores"], np.float32)
    assert oracle.topk_rows([x], ex["k"])[0].tolist() == ex["expected"]


# ---------------------------------------------------------------- attention ---------------

def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rand_bf16(shape):
    return bf16_bits(RNG.normal(size=shape))


def test_dense_causal_matches_torch_sdpa():
    T, H, Dqk, Dv = 24, 8, 80, 64
    sm = 1 / math.sqrt(Dqk)
    q = rand_bf16((T, H, Dqk))
    kv = rand_bf16((T, Dqk))
    pos = np.arange(T, dtype=np.int32)
    out, lse = oracle.dense_causal(q, kv, pos, Dv, sm)
    qd = torch.from_numpy(oracle.decode_bf16(q)).permute(1, 0, 2)  # [H, T, D]
    kd = torch.from_numpy(oracle.decode_bf16(kv))
    K = kd.unsqueeze(0).expand(H, T, Dqk)
    V = kd[:, :Dv].unsqueeze(0).expand(H, T, Dv)
    ref = torch.nn.functional.scaled_dot_product_attention(qd, K, V, is_causal=True, scale=sm)
    logits = (qd @ K.transpose(1, 2)) * sm
    logits = logits.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), -math.inf)
    ref_lse = torch.logsumexp(logits, dim=-1).permute(1, 0)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def all_positions_idx(T, k, pos0=0):
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        n = min(k, pos0 + t + 1)
        idx[t, :n] = np.arange(n)
    return idx


def test_sparse_equals_dense_when_k_covers_every_position():
    T, H, Dqk, Dv, k = 40, 8, 80, 64, 64
    sm = 1 / math.sqrt(Dqk)
    q, kv = rand_bf16((T, H, Dqk)), rand_bf16((T, Dqk))
    o1, l1 = oracle.sparse_mqa(q, kv, all_positions_idx(T, k), Dv, sm)
    o2, l2 = oracle.dense_causal(q, kv, np.arange(T, dtype=np.int32), Dv, sm)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


def test_single_key_returns_its_value():
    H, Dqk, Dv = 8, 80, 64
    q, kv = rand_bf16((1, H, Dqk)), rand_bf16((5, Dqk))
    idx = np.array([[-1, 3, -1, -1]], np.int32)
    out, lse = oracle.sparse_mqa(q, kv, idx, Dv, 0.1)
    v = oracle.decode_bf16(kv[3, :Dv])
    for h in range(H):
        assert np.array_equal(out[0, h], v)
        z = 0.1 * float(oracle.decode_bf16(q[0, h]) @ oracle.decode_bf16(kv[3]))
        assert lse[0, h] == pytest.approx(z, rel=1e-15)


def test_zero_query_gives_mean_of_selected_values():
    H, Dqk, Dv = 8, 80, 64
    q = np.zeros((1, H, Dqk), np.uint16)
    kv = rand_bf16((10, Dqk))
    sel = [0, 2, 3, 7, 9]
    idx = np.array([sel + [-1] * 3], np.int32)
    out, lse = oracle.sparse_mqa(q, kv, idx, Dv, 0.3)
    mean = oracle.decode_bf16(kv[sel, :Dv]).mean(axis=0)
    np.testing.assert_allclose(out[0], np.broadcast_to(mean, (H, Dv)), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse[0], math.log(5), rtol=1e-15)


def test_slot_order_and_empty_slots_do_not_matter():
    T, H, Dqk, Dv = 6, 8, 80, 64
    q, kv = rand_bf16((T, H, Dqk)), rand_bf16((50, Dqk))
    idx = np.stack([RNG.permutation(50)[:20] for _ in range(T)]).astype(np.int32)
    idx = np.concatenate([idx, np.full((T, 12), -1, np.int32)], axis=1)
    o1, l1 = oracle.sparse_mqa(q, kv, idx, Dv, 0.11)
    perm = np.stack([RNG.permutation(32) for _ in range(T)])
    o2, l2 = oracle.sparse_mqa(q, kv, np.take_along_axis(idx, perm, 1), Dv, 0.11)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_needle_dominates():
    H, Dqk, Dv = 8, 80, 64
    qf = RNG.normal(size=(1, H, Dqk))
    kvf = RNG.normal(size=(30, Dqk)) * 0.01
    kvf[17] = qf[0, 5] * 3  # logit of head 5 on row 17: >= 40 above the rest
    q, kv = bf16_bits(qf), bf16_bits(kvf)
    idx = np.arange(30, dtype=np.int32)[None]
    out, _ = oracle.sparse_mqa(q, kv, idx, Dv, 1.0)
    z = oracle.decode_bf16(q[0, 5]) @ oracle.decode_bf16(kv).T
    assert np.sort(z)[-1] - np.sort(z)[-2] > 40
    np.testing.assert_allclose(out[0, 5], oracle.decode_bf16(kv[17, :Dv]), atol=1e-12)


def test_golden_attention_example():
    ex = json.load(open(os.path.join(GOLDEN, "attention_worked_example.json")))
    q = bf16_bits(np.array(ex["q"], np.float32)[None, None])
    kv = bf16_bits(np.array(ex["kv"], np.float32))
    out, lse = oracle.sparse_mqa(q, kv, np.array([ex["idx"]], np.int32), ex["v_dim"], ex["sm_scale"])
    np.testing.assert_allclose(out[0, 0], ex["expected_out"], rtol=1e-14)
    assert lse[0, 0] == pytest.approx(ex["expected_lse"], rel=1e-14)


# ---------------------------------------------------------------- input contract ----------

def test_quantiser_round_trip():
    import dsa_inputs

    x = torch.randn(64, 128) * 3
    codes, scale = dsa_inputs.quantize_e4m3_rows(x)
    dec = torch.from_numpy(oracle.decode_e4m3(codes.numpy())) * scale.double()[:, None]
    assert torch.all(scale == x.abs().amax(1) / 448)
    # the largest element of each row maps to +-448 exactly
    assert np.all(np.abs(oracle.decode_e4m3(codes.numpy())).max(1) == 448.0)
    # round to nearest: error at most half a code step (relative 2^-4 for normal codes)
    err = (dec - x.double()).abs()
    assert torch.all(err <= x.double().abs() * 2.0 ** -4 + scale.double()[:, None] * 2.0 ** -10)


# ---- cache producer: e4m3 encoder, RoPE, row quantiser ------------------------------------

def test_encode_e4m3_round_trips_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    back = oracle.encode_e4m3(oracle.decode_e4m3(codes).astype(np.float32))
    assert np.array_equal(back, codes)  # including -0 -> 0x80


def test_encode_e4m3_ties_go_to_the_even_code_and_saturate():
    codes = np.arange(0, 0x7E, dtype=np.uint8)  # non-negative finite codes, ascending values
    vals = oracle.decode_e4m3(codes)
    mid = (vals[:-1] + vals[1:]) / 2  # exact in float32 for this format
    got = oracle.encode_e4m3(mid.astype(np.float32))
    want = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert np.array_equal(got, want)
    above = oracle.encode_e4m3((mid * (1 + 1e-4)).astype(np.float32))
    assert np.array_equal(above, codes[1:])
    below = oracle.encode_e4m3((mid * (1 - 1e-4)).astype(np.float32))
    assert np.array_equal(below, codes[:-1])
    assert list(oracle.encode_e4m3(np.array([448, 449, 1e30, -1e30], np.float32))) == [0x7E, 0x7E, 0x7E, 0xFE]
    assert oracle.encode_e4m3(np.array([np.nan], np.float32))[0] == 0x7F


def test_encode_e4m3_matches_torch_cast():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(size=4000) * s for s in (1e-3, 1.0, 60.0)]).astype(np.float32)
    x = np.clip(x, -448, 448)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_e4m3(x), want)


def test_rope_closed_forms():
    rng = np.random.default_rng(6)
    x = rng.normal(size=(3, 128)).astype(np.float32)
    P = 4
    cos_tab = np.ones((P, 32), np.float32)
    sin_tab = np.zeros((P, 32), np.float32)
    cos_tab[1], sin_tab[1] = 0.0, 1.0        # a quarter turn: (x0, x1) -> (-x1, x0) exactly
    ang = rng.uniform(-np.pi, np.pi, 32)
    cos_tab[2], sin_tab[2] = np.cos(ang), np.sin(ang)
    assert np.array_equal(oracle.rope_f32(x, 0, cos_tab, sin_tab, 64), x)
    q = oracle.rope_f32(x, 1, cos_tab, sin_tab, 64)
    assert np.array_equal(q[:, 0:64:2], -x[:, 1:64:2]) and np.array_equal(q[:, 1:64:2], x[:, 0:64:2])
    assert np.array_equal(q[:, 64:], x[:, 64:])  # dims past the rope part are untouched
    r = oracle.rope_f32(x, 2, cos_tab, sin_tab, 64).astype(np.float64)
    c, s = cos_tab[2].astype(np.float64), sin_tab[2].astype(np.float64)
    x0, x1 = x[:, 0:64:2].astype(np.float64), x[:, 1:64:2].astype(np.float64)
    assert np.allclose(r[:, 0:64:2], x0 * c - x1 * s, rtol=0, atol=1e-6)
    assert np.allclose(r[:, 1:64:2], x0 * s + x1 * c, rtol=0, atol=1e-6)


def test_quantize_row_e4m3_properties():
    rng = np.random.default_rng(8)
    x = (rng.normal(size=(50, 128)) * rng.uniform(0.01, 100, size=(50, 1))).astype(np.float32)
    x[3] = 0.0
    codes, scale = oracle.quantize_row_e4m3(x)
    assert scale[3] == 1.0 and not codes[3].any()
    dec = oracle.decode_e4m3(codes) * scale[:, None].astype(np.float64)
    amax = np.abs(x).max(axis=1)
    for i in range(50):
        if i == 3:
            continue
        j = np.argmax(np.abs(x[i]))
        assert codes[i, j] in (0x7E, 0xFE)  # the largest entry takes the largest code
        # round to nearest: half a step of 3 mantissa bits, or half the subnormal step
        err = np.abs(dec[i] - x[i])
        assert np.all(err <= np.maximum(np.abs(x[i]) / 16, 2.0 ** -10 * scale[i]) * (1 + 1e-6))
    # the input recipe's quantiser (torch's cast) makes the same codes and scales
    c2, s2 = dsa_inputs.quantize_e4m3_rows(torch.from_numpy(x))
    assert np.array_equal(codes, c2.numpy()) and np.array_equal(scale, s2.numpy())


# ---- indexer KL target ----------------------------------------------------------------

def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_indexer_kl_uniform_target_closed_form():
    # a zero query gives every slot the same logit, so P is uniform over the n slots and
    # KL(U || Q) = -ln n - mean(log Q), KL(Q || U) = sum Q log Q + ln n
    rng = np.random.default_rng(21)
    H, D, n = 3, 8, 7
    q = _bf16_bits(np.zeros((1, H, D)))
    kv = _bf16_bits(rng.normal(size=(n, D)))
    lse = np.full((1, H), np.log(n))
    I = rng.normal(size=n) * 2.0
    kl, rev = oracle.indexer_kl(q, kv, lse, [np.arange(n)], [I], 0.5)
    logQ = I - np.log(np.exp(I).sum())
    assert np.isclose(kl[0], -np.log(n) - logQ.mean(), rtol=0, atol=1e-12)
    assert np.isclose(rev[0], np.sum(np.exp(logQ) * logQ) + np.log(n), rtol=0, atol=1e-12)


def test_indexer_kl_two_slots_worked_example():
    # one head, two slots with logits 0 and ln 3 (q = [1, 0], rows [0, *] and [ln 3, *],
    # sm_scale 1): P = (1/4, 3/4); indexer scores (0, 0): Q = (1/2, 1/2)
    # KL(P || Q) = 1/4 ln(1/2) + 3/4 ln(3/2) ; KL(Q || P) = 1/2 ln 2 + 1/2 ln(2/3)
    ln3 = float(np.log(np.float32(3.0)))
    q = _bf16_bits([[[1.0, 0.0]]])
    kvf = np.array([[0.0, 5.0], [ln3, -2.0]], np.float32)
    kv = _bf16_bits(kvf)
    z1 = float(oracle.decode_bf16(kv)[1, 0])  # the bf16 value of ln 3
    lse = np.array([[np.log(1.0 + np.exp(z1))]])
    kl, rev = oracle.indexer_kl(q, kv, lse, [np.array([0, 1])], [np.zeros(2)], 1.0)
    p1 = np.exp(z1) / (1 + np.exp(z1))
    p0 = 1 - p1
    assert np.isclose(kl[0], p0 * np.log(2 * p0) + p1 * np.log(2 * p1), rtol=0, atol=1e-12)
    assert np.isclose(rev[0], 0.5 * np.log(0.5 / p0) + 0.5 * np.log(0.5 / p1), rtol=0, atol=1e-12)
    assert abs(p1 - 0.75) < 2e-3  # bf16 rounding of ln 3 only


def test_indexer_kl_matches_scipy_and_properties():
    from scipy.special import rel_entr, softmax
    rng = np.random.default_rng(22)
    H, D, S = 4, 16, 40
    qf = rng.normal(size=(3, H, D))
    kvf = rng.normal(size=(S, D))
    q, kv = _bf16_bits(qf), _bf16_bits(kvf)
    qd, kvd = oracle.decode_bf16(q), oracle.decode_bf16(kv)
    slots = [np.arange(S), np.r_[rng.permutation(S)[:10], -1, -1], np.array([-1, 5, -1])]
    scores = [rng.normal(size=S) * 3 for _ in range(3)]
    # lse of each head over the row's own slots (as the attention reports it)
    lse = np.zeros((3, H))
    for t in range(3):
        p = slots[t][slots[t] >= 0]
        z = 0.3 * kvd[p] @ qd[t].T
        lse[t] = np.log(np.exp(z).sum(axis=0))
    kl, rev = oracle.indexer_kl(q, kv, lse, slots, scores, 0.3)
    for t in range(3):
        p = slots[t][slots[t] >= 0]
        P = softmax(0.3 * kvd[p] @ qd[t].T, axis=0).mean(axis=1)  # per-head softmax, head mean
        Q = softmax(scores[t][p])
        assert np.isclose(kl[t], rel_entr(P, Q).sum(), rtol=1e-12, atol=1e-12)
        assert np.isclose(rev[t], rel_entr(Q, P).sum(), rtol=1e-12, atol=1e-12)
        assert kl[t] >= 0 and rev[t] >= 0
    assert kl[2] == 0 and rev[2] == 0  # one slot: P = Q = 1
    # Q equal to P: both divergences vanish
    p = slots[0]
    P = softmax(0.3 * kvd[p] @ qd[0].T, axis=0).mean(axis=1)
    kl0, rev0 = oracle.indexer_kl(q[:1], kv, lse[:1], [p], [np.log(P) + 7.0], 0.3)
    assert abs(kl0[0]) < 1e-12 and abs(rev0[0]) < 1e-12
    # a row without slots
    kl1, rev1 = oracle.indexer_kl(q[:1], kv, lse[:1], [np.array([-1, -1])], [scores[0]], 0.3)
    assert kl1[0] == 0 and rev1[0] == 0
