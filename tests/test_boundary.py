"""The C-ABI boundary on the host: the library loads, exports every function declared in
include/dsa.h, and rejects invalid arguments with the documented status before enqueueing
anything (these calls never touch device memory, so they run without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_attention_long_lightning_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 1 << 20  # 16-byte aligned address; never dereferenced on the error paths below


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"dsa_indexer_scores", "dsa_topk", "dsa_sparse_mqa", "dsa_forward",
            "dsa_workspace_size", "dsa_status_string"} <= set(names)
    lib = dsa.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = dsa.lib()
    for s, name in dsa.STATUS.items():
        assert lib.dsa_status_string(s).decode().startswith(name)


def cpu_batch(cu_q, cu_k):
    return dsa.Batch(cu_q, cu_k, device="cpu")


def call_forward(dims, batch, ptr=FAKE, ws_bytes=1 << 40, **over):
    args = dict(q8=ptr, q_scale=ptr, w=ptr, k8=ptr, k_scale=ptr, q=ptr, kv=ptr, out=ptr, lse=None,
                idx=None, ws=ptr)
    args.update(over)
    return dsa.lib().dsa_forward(ctypes.byref(dims), ctypes.byref(batch.c), args["q8"],
                                 args["q_scale"], args["w"], args["k8"], args["k_scale"], args["q"],
                                 args["kv"], args["out"], args["lse"], args["idx"], args["ws"],
                                 ws_bytes, None)


def dims_with(**kw):
    d = dsa.Dims(64, 128, 2048, 128, 576, 512, 0.0721)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(topk=0), INVALID), (dict(topk=8193), INVALID), (dict(topk=-5), INVALID),
    (dict(sm_scale=0.0), INVALID), (dict(sm_scale=float("nan")), INVALID),
    (dict(sm_scale=float("inf")), INVALID), (dict(n_idx_heads=32), UNSUPPORTED),
    (dict(idx_dim=64), UNSUPPORTED), (dict(n_heads=64), UNSUPPORTED), (dict(qk_dim=512), UNSUPPORTED),
    (dict(v_dim=576), UNSUPPORTED)])
def test_invalid_dims(kw, status):
    b = cpu_batch([0, 4096], [0, 4096])
    assert call_forward(dims_with(**kw), b) == status
    out = ctypes.c_size_t(0)
    assert dsa.lib().dsa_workspace_size(ctypes.byref(dims_with(**kw)), ctypes.byref(b.c),
                                        ctypes.byref(out)) == status


@pytest.mark.parametrize("cu_q,cu_k", [
    ([1, 4], [0, 4]),          # not zero-based
    ([0, 4], [1, 4]),
    ([0, 8], [0, 4]),          # more queries than keys
    ([0, 4, 2], [0, 4, 8]),    # decreasing offsets
    ([0, 2, 4], [0, 8, 6])])
def test_invalid_batches(cu_q, cu_k):
    assert call_forward(dims_with(), cpu_batch(cu_q, cu_k)) == INVALID


def test_null_and_misaligned_pointers():
    d, b = dims_with(), cpu_batch([0, 64], [0, 64])
    for name in ("q8", "q_scale", "w", "k8", "k_scale", "q", "kv", "out"):
        assert call_forward(d, b, **{name: None}) == INVALID, name
        assert call_forward(d, b, **{name: FAKE + 4}) == INVALID, name
    assert call_forward(d, b, lse=FAKE + 8) == INVALID
    assert call_forward(d, b, idx=FAKE + 2) == INVALID
    assert call_forward(d, b, ws=None) == WORKSPACE
    lib = dsa.lib()
    assert lib.dsa_topk(ctypes.byref(d), ctypes.byref(b.c), FAKE, 64, None, None, 0, None) == INVALID
    assert lib.dsa_topk(ctypes.byref(d), ctypes.byref(b.c), FAKE, 60, FAKE, None, 0, None) == INVALID  # stride < len
    assert lib.dsa_topk(ctypes.byref(d), ctypes.byref(b.c), FAKE, 66, FAKE, None, 0, None) == INVALID  # not x4
    assert lib.dsa_topk(ctypes.byref(d), ctypes.byref(b.c), FAKE, 64, FAKE, FAKE + 4, 1 << 20,
                        None) == WORKSPACE  # misaligned workspace
    assert lib.dsa_indexer_scores(ctypes.byref(d), ctypes.byref(b.c), FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE + 4, 64, None) == INVALID
    assert lib.dsa_sparse_mqa(ctypes.byref(d), ctypes.byref(b.c), FAKE, FAKE, None, FAKE, None, None,
                              0, None) == INVALID


def test_workspace_too_small_is_rejected():
    d, b = dims_with(), cpu_batch([0, 4096], [0, 4096])
    lo = dsa.workspace_min(d, b)
    hi = dsa.workspace_size(d, b)
    assert 0 < lo <= hi
    assert call_forward(d, b, ws_bytes=lo - 1) == WORKSPACE
    # decode batches need the split partials of the attention as well
    db = cpu_batch(list(range(33)), [i * 40000 for i in range(33)])
    assert call_forward(d, db, ws_bytes=dsa.workspace_size(d, db) - 1) == WORKSPACE
    assert dsa.lib().dsa_sparse_mqa(ctypes.byref(d), ctypes.byref(db.c), FAKE, FAKE, FAKE, FAKE, None,
                                    FAKE, 16, None) == WORKSPACE


def test_workspace_policy_is_bounded_by_chunking():
    d = dims_with()
    b128 = cpu_batch([0, 131072], [0, 131072])
    ws = dsa.workspace_size(d, b128)
    # one pass of 8192 query rows of fp32 scores (+ their index rows), never the full L x L
    assert ws < 131072 * 131072 * 4 / 8
    assert ws >= 8192 * 131072 * 4


def test_empty_batch_is_a_no_op():
    d = dims_with()
    b = cpu_batch([0, 0], [0, 100])
    assert call_forward(d, b, ptr=None, ws_bytes=0) == OK


def test_topk_workspace_covers_the_segment_candidates():
    d = dims_with()
    # 32 one-query sequences, the longest 91,529 keys: six 16K-score segments per row, each
    # keeping k (key, position) candidates of 8 bytes
    db = cpu_batch(list(range(33)), [0] + [91529 * (i + 1) for i in range(32)])
    assert dsa.topk_workspace_size(d, db) == 32 * 6 * 2048 * 8
    # rows longer than eight segments, or batches of 128 rows and more, are selected by one
    # workgroup per row: no workspace
    assert dsa.topk_workspace_size(d, cpu_batch([0, 1], [0, 8 * 16384 + 1])) == 0
    assert dsa.topk_workspace_size(d, cpu_batch([0, 128], [0, 5000])) == 0


def call_append(dims, batch, ptr=FAKE, n_pos=1 << 20, **over):
    args = dict(q_idx=ptr, k_idx=ptr, kv_new=ptr, cos=ptr, sin=ptr, q8=ptr, q_scale=ptr, k8=ptr,
                k_scale=ptr, kv=ptr)
    args.update(over)
    return dsa.lib().dsa_cache_append(ctypes.byref(dims), ctypes.byref(batch.c), args["q_idx"],
                                      args["k_idx"], args["kv_new"], args["cos"], args["sin"], n_pos,
                                      args["q8"], args["q_scale"], args["k8"], args["k_scale"],
                                      args["kv"], None)


def test_cache_append_rejects_bad_arguments():
    d, b = dims_with(), cpu_batch([0, 1, 2], [0, 100, 300])
    for name in ("q_idx", "k_idx", "cos", "sin", "q8", "q_scale", "k8", "k_scale"):
        assert call_append(d, b, **{name: None}) == INVALID, name
        assert call_append(d, b, **{name: FAKE + 4}) == INVALID, name
    assert call_append(d, b, kv_new=None) == INVALID       # latent row without a latent cache
    assert call_append(d, b, kv=None) == INVALID
    assert call_append(d, b, kv=FAKE + 2) == INVALID
    assert call_append(d, b, n_pos=199) == INVALID          # no table row for position 199
    assert call_append(dims_with(idx_dim=64), b) == UNSUPPORTED
    assert call_append(d, cpu_batch([0, 0], [0, 5]), ptr=None) == OK  # nothing to append


def test_paged_batches_are_validated():
    d = dims_with()
    pt = np.zeros((2, 4), np.int32)
    dec = dsa.Batch([0, 1, 2], [0, 256, 356], device="cpu", page_table=pt)
    assert dec.c.pages_per_seq == 4
    short = dsa.Batch([0, 1, 2], [0, 257, 300], device="cpu", page_table=pt)  # 257 keys > 4 pages
    assert call_forward(d, short) == INVALID
    assert call_append(d, short) == INVALID
    bad = dsa.Batch([0, 1, 2], [0, 256, 356], device="cpu", page_table=pt)
    bad.c.pages_per_seq = 0
    assert call_forward(d, bad) == INVALID
    # prefill (a sequence with several query rows) reads packed caches only
    pre = dsa.Batch([0, 2, 3], [0, 256, 356], device="cpu", page_table=pt)
    assert call_forward(d, pre) == UNSUPPORTED
    assert dsa.lib().dsa_indexer_scores(ctypes.byref(d), ctypes.byref(pre.c), FAKE, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, 256, None) == UNSUPPORTED
    with pytest.raises(ValueError):
        dsa.Batch([0, 1, 2], [0, 5, 6], device="cpu", page_table=np.zeros((3, 1), np.int32))


def test_workspace_size_covers_the_attention_split_of_small_batches():
    d = dims_with()
    # 24 query rows of one sequence: dsa_sparse_mqa splits each row over several workgroups
    b = cpu_batch([0, 24], [0, 5000])
    need = dsa.workspace_size(d, b)
    assert dsa.lib().dsa_sparse_mqa(ctypes.byref(d), ctypes.byref(b.c), FAKE, FAKE, FAKE, FAKE, None,
                                    FAKE, need - 16, None) == WORKSPACE


def test_indexer_kl_rejects_bad_arguments():
    d, b = dims_with(), cpu_batch([0, 4], [0, 100])
    lib = dsa.lib()

    def call(q=FAKE, kv=FAKE, lse=FAKE, idx=FAKE, scores=FAKE, stride=100, kl=FAKE, rev=None):
        return lib.dsa_indexer_kl(ctypes.byref(d), ctypes.byref(b.c), q, kv, lse, idx, scores, stride, kl,
                                  rev, None)
    for name in ("q", "kv", "lse", "scores", "kl"):
        assert call(**{name: None}) == INVALID, name
        assert call(**{name: FAKE + 4}) == INVALID, name
    assert call(idx=FAKE + 4) == INVALID
    assert call(rev=FAKE + 8) == INVALID
    assert call(stride=96) == INVALID    # shorter than the longest row
    assert call(stride=102) == INVALID   # not a multiple of 4
    assert lib.dsa_indexer_kl(ctypes.byref(dims_with(n_heads=64)), ctypes.byref(b.c), FAKE, FAKE, FAKE, None,
                              FAKE, 100, FAKE, None, None) == UNSUPPORTED
    e = cpu_batch([0, 0], [0, 7])
    assert lib.dsa_indexer_kl(ctypes.byref(d), ctypes.byref(e.c), None, None, None, None, None, 8, None, None,
                              None) == OK  # no rows


def test_counted_stages_reject_bad_arguments():
    d, b = dims_with(), cpu_batch([0, 64], [0, 64])
    lib = dsa.lib()
    args = [FAKE] * 6
    assert lib.dsa_indexer_scores_counted(ctypes.byref(d), ctypes.byref(b.c), *args, 64, None, None) == INVALID
    assert lib.dsa_indexer_scores_counted(ctypes.byref(d), ctypes.byref(b.c), *args, 64, FAKE + 4, None) == INVALID
    dec = cpu_batch([0, 1, 2], [0, 100, 300])  # decode batches are scored by the decode kernel: no counts
    assert lib.dsa_indexer_scores_counted(ctypes.byref(d), ctypes.byref(dec.c), *args, 200, FAKE, None) == UNSUPPORTED
    assert lib.dsa_topk_counted(ctypes.byref(d), ctypes.byref(b.c), FAKE, 64, None, FAKE, None) == INVALID
    assert lib.dsa_topk_counted(ctypes.byref(d), ctypes.byref(b.c), FAKE, 64, FAKE, None, None) == INVALID
    assert lib.dsa_topk_counted(ctypes.byref(d), ctypes.byref(b.c), FAKE, 60, FAKE, FAKE, None) == INVALID


def test_index_check_and_debug_flags_reject_bad_arguments():
    d, b = dims_with(), cpu_batch([0, 4], [0, 100])
    lib = dsa.lib()
    assert lib.dsa_check_indices(ctypes.byref(d), ctypes.byref(b.c), None, FAKE, None) == INVALID
    assert lib.dsa_check_indices(ctypes.byref(d), ctypes.byref(b.c), FAKE, None, None) == INVALID
    assert lib.dsa_check_indices(ctypes.byref(d), ctypes.byref(b.c), FAKE + 4, FAKE, None) == INVALID
    assert lib.dsa_check_indices(ctypes.byref(dims_with(qk_dim=512)), ctypes.byref(b.c), FAKE, FAKE, None) == UNSUPPORTED
    assert lib.dsa_check_indices(ctypes.byref(d), ctypes.byref(cpu_batch([0, 0], [0, 9]).c), None, None, None) == OK
    assert lib.dsa_debug_flags(None, 0) == INVALID


def test_sequences_past_the_32_bit_row_offsets_are_unsupported():
    # latent rows are addressed by 32-bit byte offsets from a sequence's first row
    d = dims_with()
    longest = (1 << 32) // 1152 - 1
    assert call_forward(d, cpu_batch([0, 1], [0, longest])) != UNSUPPORTED
    assert call_forward(d, cpu_batch([0, 1], [0, longest + 1])) == UNSUPPORTED


def test_negative_pool_size_is_invalid():
    d = dims_with()
    b = dsa.Batch([0, 1], [0, 100], device="cpu", page_table=np.zeros((1, 2), np.int32), pool_rows=128)
    assert b.c.pool_rows == 128
    b.c.pool_rows = -1
    assert call_forward(d, b) == INVALID
