"""dsa_forward_noalloc (the forward with the library's fixed per-device scratch array as its
workspace) against dsa_forward with a caller workspace, through the C ABI: bit-identical index
rows, outputs and lse on calls in a row whose sizes shrink (a prefill, a decode batch, a
smaller decode batch), so that every call runs over what the previous one left in the array."""
import ctypes

import pytest
import torch

import dsa_inputs
import sparse_attention_long_lightning_amd as dsa

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def both(inp, dims, dev):
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=dev)
    T = batch.n_q
    res = []
    for noalloc in (False, True):
        out = torch.full((T, dims.n_heads, dims.v_dim), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((T, dims.n_heads), float("nan"), dtype=torch.float32, device=dev)
        idx = torch.full((T, dims.topk), -7, dtype=torch.int32, device=dev)
        args = (dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], inp["q"], inp["kv"],
                out, lse, idx)
        if noalloc:
            dsa.forward_noalloc(*args)
        else:
            ws = torch.empty(dsa.workspace_size(dims, batch), dtype=torch.uint8, device=dev)
            dsa.forward(*args, ws)
        torch.cuda.synchronize()
        res.append((out, lse, idx))
    (o1, l1, i1), (o2, l2, i2) = res
    assert torch.equal(i1, i2) and torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_forward_noalloc_equals_forward_on_shrinking_calls(cuda):
    dims = dsa_inputs.PROD
    say("noalloc: prefill L=3000 (passes sized to the scratch array)")
    both(dsa_inputs.prefill_inputs(3000, dims, seed=2, device=cuda), dims, cuda)
    lens = [1500, 2048, 2049, 7000, 12345, 20000]
    say(f"noalloc: decode B=6 lens {lens}")
    both(dsa_inputs.decode_inputs(dims=dims, seed=4, device=cuda, lens=lens), dims, cuda)
    lens = [100, 3000, 9000]
    say(f"noalloc: decode B=3 lens {lens} (smaller, after the larger call)")
    both(dsa_inputs.decode_inputs(dims=dims, seed=5, device=cuda, lens=lens), dims, cuda)
    say("noalloc: tiny prefill L=256")
    both(dsa_inputs.prefill_inputs(256, dsa_inputs.TINY, seed=0, device=cuda, needles=False), dsa_inputs.TINY,
         cuda)


def test_forward_noalloc_rejects_a_batch_beyond_the_array(cuda):
    dims = dsa.PROD_DIMS
    lens = [131072] * 64
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    batch = dsa.Batch(list(range(65)), cu, device=cuda)
    need = dsa.workspace_min(dims, batch)
    assert need > dsa.NOALLOC_SCRATCH_BYTES
    fake = 1 << 20  # never dereferenced: the call returns before enqueueing anything
    st = dsa.lib().dsa_forward_noalloc(ctypes.byref(dims), ctypes.byref(batch.c), *([fake] * 8), None, None,
                                       None)
    assert st == 3  # DSA_ERR_WORKSPACE
