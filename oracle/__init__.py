"""Python face of the DSA oracle (``oracle.c``): plain CPU reference for the hot path.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.  It shares nothing with the HIP library.

Functions take numpy arrays holding the exact bytes the GPU consumes (uint8 FP8 codes,
uint16 bf16 bits, float32 scales and weights) and return float64 results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` next to its source with gcc + OpenMP."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                        "-Wall", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P, I, I64, D, F = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double,
                           ctypes.c_float)
        L.orc_e4m3.restype = D
        L.orc_e4m3.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_fixed.restype = I64
        L.orc_e4m3_fixed.argtypes = [ctypes.c_uint8]
        L.orc_bf16.restype = D
        L.orc_bf16.argtypes = [ctypes.c_uint16]
        L.orc_decode_e4m3.argtypes = [I64, P, P]
        L.orc_decode_bf16.argtypes = [I64, P, P]
        L.orc_dot_e4m3.restype = D
        L.orc_dot_e4m3.argtypes = [I, P, P]
        L.orc_dot_e4m3_fixed.restype = I64
        L.orc_dot_e4m3_fixed.argtypes = [I, P, P]
        L.orc_index_score.restype = D
        L.orc_index_score.argtypes = [I, I, P, P, P, P, F]
        L.orc_indexer_rows.argtypes = [I, I, P, P, P, P, P, I, P, P, P, I64]
        L.orc_topk_rows_f64.argtypes = [I, P, P, I64, I, P]
        L.orc_topk_rows_f32.argtypes = [I, P, P, I64, I, P]
        L.orc_sparse_mqa.argtypes = [I, I, I, D, I, P, P, I, P, P, P]
        L.orc_dense_causal.argtypes = [I, I, I, D, I, P, P, P, P, P]
        L.orc_encode_e4m3_n.argtypes = [I64, P, P]
        L.orc_rope_f32.argtypes = [I, I, P, I64, P, P, I64, I, P]
        L.orc_quantize_rows_e4m3.argtypes = [I, I, P, P, P]
        L.orc_cache_append.argtypes = [I, I, I, P, P, P, P, P, I64, I, P, P, P, P]
        L.orc_indexer_kl.argtypes = [I, I, D, I, P, P, P, I, P, P, I64, P, P]
        L.orc_num_threads.restype = I
        L.orc_set_num_threads.argtypes = [I]
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops from now on."""
    lib().orc_set_num_threads(int(n))


# ---- codecs ---------------------------------------------------------------------------

def decode_e4m3(codes) -> np.ndarray:
    a, p = _c(codes, np.uint8)
    out = np.empty(a.shape, np.float64)
    lib().orc_decode_e4m3(a.size, p, out.ctypes.data_as(ctypes.c_void_p))
    return out


def decode_bf16(bits) -> np.ndarray:
    a, p = _c(bits, np.uint16)
    out = np.empty(a.shape, np.float64)
    lib().orc_decode_bf16(a.size, p, out.ctypes.data_as(ctypes.c_void_p))
    return out


def e4m3_fixed(code: int) -> int:
    return int(lib().orc_e4m3_fixed(code))


# ---- indexer --------------------------------------------------------------------------

def dot_e4m3(a, b) -> float:
    a, pa = _c(a, np.uint8)
    b, pb = _c(b, np.uint8)
    return float(lib().orc_dot_e4m3(a.size, pa, pb))


def dot_e4m3_fixed(a, b) -> int:
    a, pa = _c(a, np.uint8)
    b, pb = _c(b, np.uint8)
    return int(lib().orc_dot_e4m3_fixed(a.size, pa, pb))


def index_score(q8_row, qs_row, w_row, k8_row, ks) -> float:
    """Score of one (query row, key row) pair; q8_row [H, d], k8_row [d]."""
    q, pq = _c(q8_row, np.uint8)
    H, d = q.shape
    qs, ps = _c(qs_row, np.float32)
    wq, pw = _c(w_row, np.float32)
    k, pk = _c(k8_row, np.uint8)
    return float(lib().orc_index_score(H, d, pq, ps, pw, pk, float(ks)))


def indexer_rows(q8, q_scale, w, k8, k_scale, rows, pos) -> list:
    """Scores of query ``rows`` (absolute positions ``pos``) against keys 0..pos.

    q8 [T, H, d] uint8, q_scale/w [T, H] float32, k8 [S, d] uint8, k_scale [S] float32.
    Returns a list of float64 arrays, row i of length pos[i] + 1."""
    q8, pq = _c(q8, np.uint8)
    T, H, d = q8.shape
    qs, pqs = _c(q_scale, np.float32)
    wv, pw = _c(w, np.float32)
    k8, pk = _c(k8, np.uint8)
    ks, pks = _c(k_scale, np.float32)
    rows_a, pr = _c(rows, np.int32)
    pos_a, pp = _c(pos, np.int32)
    n = len(rows_a)
    if n == 0:
        return []
    stride = int(pos_a.max()) + 1
    out = np.zeros((n, stride), np.float64)
    lib().orc_indexer_rows(H, d, pq, pqs, pw, pk, pks, n, pr, pp,
                           out.ctypes.data_as(ctypes.c_void_p), stride)
    return [out[i, : int(pos_a[i]) + 1] for i in range(n)]


# ---- top-k ----------------------------------------------------------------------------

def topk_rows(rows, k: int) -> np.ndarray:
    """Top-k positions (ascending, -1 padded) of each score row.  Rows are float32 or
    float64 arrays; float32 rows are widened exactly."""
    n = len(rows)
    if n == 0:
        return np.zeros((0, k), np.int32)
    f32 = all(np.asarray(r).dtype == np.float32 for r in rows)
    lens = np.array([len(r) for r in rows], np.int64)
    stride = max(1, int(lens.max()))
    buf = np.zeros((n, stride), np.float32 if f32 else np.float64)
    for i, r in enumerate(rows):
        buf[i, : len(r)] = r
    out = np.empty((n, k), np.int32)
    fn = lib().orc_topk_rows_f32 if f32 else lib().orc_topk_rows_f64
    fn(n, lens.ctypes.data_as(ctypes.c_void_p), buf.ctypes.data_as(ctypes.c_void_p), stride, k,
       out.ctypes.data_as(ctypes.c_void_p))
    return out


# ---- attention ------------------------------------------------------------------------

def sparse_mqa(q_bits, kv_bits, idx, v_dim: int, sm_scale: float):
    """q_bits [T, H, Dqk] uint16 (bf16), kv_bits [S, Dqk] uint16, idx [T, k] int32 positions
    (-1 = empty).  Returns (out [T, H, v_dim] float64, lse [T, H] float64)."""
    q, pq = _c(q_bits, np.uint16)
    T, H, Dqk = q.shape
    kv, pkv = _c(kv_bits, np.uint16)
    ix, pix = _c(idx, np.int32)
    k = ix.shape[1] if ix.ndim == 2 else 0
    assert ix.shape[0] == T and (ix.size == 0 or int(ix.max()) < kv.shape[0]), "one index row per query row"
    out = np.zeros((T, H, v_dim), np.float64)
    lse = np.zeros((T, H), np.float64)
    if T == 0:
        return out, lse
    lib().orc_sparse_mqa(H, Dqk, v_dim, float(sm_scale), T, pq, pkv, k, pix,
                         out.ctypes.data_as(ctypes.c_void_p), lse.ctypes.data_as(ctypes.c_void_p))
    return out, lse


def dense_causal(q_bits, kv_bits, pos, v_dim: int, sm_scale: float):
    """Textbook causal attention over keys 0..pos[t] (MQA: one latent row per key)."""
    q, pq = _c(q_bits, np.uint16)
    T, H, Dqk = q.shape
    kv, pkv = _c(kv_bits, np.uint16)
    p, pp = _c(pos, np.int32)
    assert p.shape == (T,) and (T == 0 or int(p.max()) < kv.shape[0]), "one position per query row, within kv"
    out = np.zeros((T, H, v_dim), np.float64)
    lse = np.zeros((T, H), np.float64)
    lib().orc_dense_causal(H, Dqk, v_dim, float(sm_scale), T, pp, pq, pkv,
                           out.ctypes.data_as(ctypes.c_void_p), lse.ctypes.data_as(ctypes.c_void_p))
    return out, lse


# ---- the whole path -------------------------------------------------------------------

def forward_rows(inp: dict, rows, seq: int = 0):
    """Oracle DSA forward for selected query rows of sequence ``seq`` of a batch produced by
    the input generator (numpy views of the exact bytes).  Returns a dict with the double
    scores of each row, the selected index rows, the attention output and lse."""
    cu_q, cu_k = inp["cu_q"], inp["cu_k"]
    dims = inp["dims"]
    q0, q1 = cu_q[seq], cu_q[seq + 1]
    k0, k1 = cu_k[seq], cu_k[seq + 1]
    rows = np.asarray(rows, np.int64)
    pos = (k1 - k0) - (q1 - q0) + rows
    qr = q0 + rows
    q8 = np.asarray(inp["q8"])[qr]
    qs = np.asarray(inp["q_scale"])[qr]
    w = np.asarray(inp["w"])[qr]
    scores = indexer_rows(q8, qs, w, np.asarray(inp["k8"])[k0:k1], np.asarray(inp["k_scale"])[k0:k1],
                          np.arange(len(rows)), pos)
    idx = topk_rows(scores, dims.topk)
    out, lse = sparse_mqa(np.asarray(inp["q"])[qr], np.asarray(inp["kv"])[k0:k1], idx,
                          dims.v_dim, dims.sm_scale)
    return dict(scores=scores, idx=idx, out=out, lse=lse, pos=pos)


# ---- cache producer: RoPE, FP8 quantisation, cache append ---------------------------------
# (DeepSeek-V3.2-Exp lightning-indexer walk-through, step 2: rotary position encoding of the
# first 64 dims of the indexer query and key, then FP8 quantisation of both with the key
# codes and their scale kept in the cache.)  oracle.c evaluates the rotation and the
# quantiser in float32 with every product, sum and quotient rounded separately, the precision
# in which the GPU path decides each FP8 code, so both sides make the same rounding decisions.

def encode_e4m3(x) -> np.ndarray:
    """Nearest e4m3fn code of each float32 value, ties to the even code, saturating at +-448;
    the sign bit follows the input (-0 -> 0x80), NaN -> 0x7f."""
    a, p = _c(x, np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().orc_encode_e4m3_n(a.size, p, out.ctypes.data_as(ctypes.c_void_p))
    return out


def _tables(cos_tab, sin_tab):
    c, pc = _c(cos_tab, np.float32)
    s, ps = _c(sin_tab, np.float32)
    assert c.shape == s.shape and c.ndim == 2
    return c, pc, s, ps, c.shape[1]


def rope_f32(x, pos, cos_tab, sin_tab, rope_dim: int):
    """Rotary encoding of the first rope_dim dims of x[..., d] (float32) at position pos:
    pairs (2i, 2i+1) rotate by the table's angle for (pos, i),
        r0 = x0*c - x1*s,  r1 = x0*s + x1*c,
    each product and sum rounded to float32; the other dims pass unchanged."""
    a, pa = _c(x, np.float32)
    c, pc, s, ps, stride = _tables(cos_tab, sin_tab)
    assert rope_dim // 2 <= stride and 0 <= int(pos) < c.shape[0]
    d = a.shape[-1]
    out = np.empty(a.shape, np.float32)
    lib().orc_rope_f32(a.size // d, d, pa, int(pos), pc, ps, stride, rope_dim,
                       out.ctypes.data_as(ctypes.c_void_p))
    return out


def quantize_row_e4m3(x):
    """One scale per row of x[..., d] (float32): amax/448 (1 for an all-zero row), codes of
    x / scale clamped to +-448, all in float32."""
    a, pa = _c(x, np.float32)
    d = a.shape[-1]
    codes = np.empty(a.shape, np.uint8)
    scale = np.empty(a.shape[:-1], np.float32)
    lib().orc_quantize_rows_e4m3(a.size // d, d, pa, codes.ctypes.data_as(ctypes.c_void_p),
                                 scale.ctypes.data_as(ctypes.c_void_p))
    return codes, scale


def cache_append(q_idx, k_idx, pos, cos_tab, sin_tab, rope_dim: int):
    """New tokens' indexer entries: q_idx [n, H, d] and k_idx [n, d] float32 at positions
    pos[n] -> (q8 [n, H, d], q_scale [n, H], k8 [n, d], k_scale [n])."""
    q, pq = _c(q_idx, np.float32)
    k, pk = _c(k_idx, np.float32)
    ps_, ppos = _c(pos, np.int64)
    n, H, d = q.shape
    assert k.shape == (n, d) and ps_.shape == (n,)
    c, pc, s, pss, stride = _tables(cos_tab, sin_tab)
    assert rope_dim // 2 <= stride and (n == 0 or (ps_.min() >= 0 and ps_.max() < c.shape[0]))
    q8 = np.empty((n, H, d), np.uint8)
    qs = np.empty((n, H), np.float32)
    k8 = np.empty((n, d), np.uint8)
    ks = np.empty(n, np.float32)
    if n:
        vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
        lib().orc_cache_append(n, H, d, pq, pk, ppos, pc, pss, stride, rope_dim, vp(q8), vp(qs), vp(k8), vp(ks))
    return q8, qs, k8, ks


def indexer_kl(q_bits, kv_bits, lse, slots, scores, sm_scale: float):
    """Indexer training target and its KL divergences, forward only (DeepSeek-V3.2-Exp
    overview, "训练"; 解析 §二; deep dive §3): for query row t over its slot positions S_t
    (every s <= p in the dense warm-up, the selected set in the sparse stage),
        P_t[s] = sum_h exp(z[t,h,s] - lse[t,h]),   z = sm_scale * q[t,h,:] . kv[s,:]
    (the main attention probabilities summed over heads), L1-normalised over S_t, and
        Q_t = softmax over S_t of the indexer scores I[t,s];
    returns (KL(P_t || Q_t), KL(Q_t || P_t)) per row, 0 for a row without slots.
      q_bits [T, H, Dqk] uint16 (bf16), kv_bits [S, Dqk] uint16 (the rows of the row's
      sequence), lse [T, H] float (natural log), slots: T arrays of positions (-1 = empty),
      scores: T arrays with I[t, s] at index s."""
    q, pq = _c(q_bits, np.uint16)
    T, H, Dqk = q.shape
    kv, pkv = _c(kv_bits, np.uint16)
    ls, pls = _c(lse, np.float64)
    k = max([len(s) for s in slots] + [1])
    sl = np.full((T, k), -1, np.int32)
    for t in range(T):
        sl[t, : len(slots[t])] = slots[t]
    width = max([len(s) for s in scores] + [1])
    sc = np.zeros((T, width), np.float64)
    for t in range(T):
        sc[t, : len(scores[t])] = scores[t]
    assert sl.max() < min(kv.shape[0], width), "slot outside the key rows or the score row"
    kl = np.zeros(T)
    rev = np.zeros(T)
    if T:
        lib().orc_indexer_kl(H, Dqk, float(sm_scale), T, pq, pkv, pls, k, sl.ctypes.data_as(ctypes.c_void_p),
                             sc.ctypes.data_as(ctypes.c_void_p), width, kl.ctypes.data_as(ctypes.c_void_p),
                             rev.ctypes.data_as(ctypes.c_void_p))
    return kl, rev
