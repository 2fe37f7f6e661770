"""Seeded synthetic inputs for the DSA hot path (lightning indexer -> top-k -> sparse MQA).

This module is shared by the tests, the benchmark and the oracle harness.  It holds only
random draws, the input encoding that the method's caches use (FP8 e4m3 codes with a
per-row scale for the indexer query/key, bf16 for the main query and the latent cache) and
the placement of planted "needle" keys.  It holds none of the scoring, selection or
attention arithmetic.

Encoding of the indexer inputs (DeepSeek-V3.2-Exp lightning-indexer walk-through, step 2
"RoPE and FP8 quantisation"): the query and key vectors are quantised to FP8 and the keys
are cached together with their scaling factor.  The pages do not fix the FP8 variant or the
rounding, so this module uses the OCP e4m3fn format (largest finite value 448), one fp32
scale per row equal to amax/448 (1 when the row is all zero), and round-to-nearest-even
through torch's float8_e4m3fn cast after clamping to +-448.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

__all__ = ["Dims", "PROD", "TINY", "quantize_e4m3_rows", "prefill_inputs", "decode_inputs"]


@dataclass(frozen=True)
class Dims:
    """Shape constants of one DSA layer."""

    n_idx_heads: int  # H_I, indexer heads
    idx_dim: int  # d_I, indexer head dim
    topk: int  # k, selected keys per query
    n_heads: int  # H, main attention heads (MQA mode)
    qk_dim: int  # latent key dim (latent + rope part)
    v_dim: int  # value dim = leading part of the latent row
    sm_scale: float  # softmax scale
    w_std: float = 1.0  # standard deviation of the indexer head weights w


# DeepSeek-V3.2-Exp shape: 64 indexer heads of dim 128, k = 2048, 128 MQA heads over a
# 576-wide latent row (512 latent + 64 rope), value = the 512 latent dims.
PROD = Dims(64, 128, 2048, 128, 576, 512, 1.0 / math.sqrt(192.0), w_std=0.125)
# Tiny shape used for exhaustive parity: 4 indexer heads of dim 32, k = 32, 8 heads,
# 80-wide key (64 + 16 rope), value 64.
TINY = Dims(4, 32, 32, 8, 80, 64, 1.0 / math.sqrt(80.0), w_std=1.0)


def quantize_e4m3_rows(x: torch.Tensor):
    """Quantise the last axis of ``x`` (float32) to e4m3fn codes with one scale per row.

    Returns (codes uint8 [..., d], scale float32 [...]); x ~= decode(codes) * scale.
    """
    x = x.float()
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp_(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def _randn(g, shape, device, std=1.0, chunk_rows=8192, dtype=torch.float32):
    """Row-chunked normal draws (bounded temporary memory for the 128K shapes)."""
    out = torch.empty(shape, dtype=dtype, device=device)
    n = shape[0]
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        t = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device)
        if std != 1.0:
            t.mul_(std)
        out[r0:r1] = t.to(dtype)
    return out


def _plant_needles(L, n_rows_q, block, per_block, gcpu, query_pos=None):
    """Needle placement: per block of ``block`` keys, ``per_block`` distinct key positions s,
    each aligned to one query position t >= s (uniform in [s, L-1]) or to ``query_pos``."""
    pairs = []
    for b0 in range(0, L, block):
        b1 = min(L, b0 + block)
        m = min(per_block, b1 - b0)
        s = b0 + torch.randperm(b1 - b0, generator=gcpu)[:m]
        for sv in s.tolist():
            if query_pos is None:
                t = sv + int(torch.randint(0, L - sv, (1,), generator=gcpu))
            else:
                t = query_pos
            pairs.append((t, sv))
    return pairs


def prefill_inputs(L: int, dims: Dims = PROD, seed: int = 0, device="cpu", needles: bool = True,
                   needle_block: int = 4096, needles_per_block: int = 64, keep_fp32: bool = False):
    """One causal prefill sequence of length L (T = S = L query and key rows).

    Draw order on ``device``: indexer q, indexer k, w, main q, latent c, all N(0,1) except
    w ~ N(0, w_std^2).  Needle positions come from a CPU generator with the same seed.
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(seed)
    gcpu = torch.Generator().manual_seed(seed)
    H_I, d_I, H, Dq = dims.n_idx_heads, dims.idx_dim, dims.n_heads, dims.qk_dim
    q_idx = _randn(g, (L, H_I, d_I), dev)
    k_idx = _randn(g, (L, d_I), dev)
    w = _randn(g, (L, H_I), dev, std=dims.w_std)
    q = _randn(g, (L, H, Dq), dev, dtype=torch.bfloat16, chunk_rows=2048)
    c = _randn(g, (L, Dq), dev)
    pairs = []
    if needles:
        pairs = _plant_needles(L, L, needle_block, needles_per_block, gcpu)
        ts = torch.tensor([p[0] for p in pairs], dtype=torch.long)
        ss = torch.tensor([p[1] for p in pairs], dtype=torch.long)
        hstar = torch.randint(0, H, (len(pairs),), generator=gcpu)
        ts_d, ss_d, h_d = ts.to(dev), ss.to(dev), hstar.to(dev)
        jstar = w[ts_d].argmax(dim=1)
        k_idx[ss_d] = 4.0 * q_idx[ts_d, jstar]
        c[ss_d] = q[ts_d, h_d].float()
    q8, q_scale = quantize_e4m3_rows(q_idx)
    k8, k_scale = quantize_e4m3_rows(k_idx)
    out = dict(q8=q8, q_scale=q_scale, w=w.contiguous(), k8=k8, k_scale=k_scale,
               q=q.contiguous(), kv=c.to(torch.bfloat16).contiguous(), needles=pairs,
               cu_q=[0, L], cu_k=[0, L], dims=dims)
    if keep_fp32:
        out.update(q_idx_f32=q_idx, k_idx_f32=k_idx)
    return out


def decode_inputs(B: int = 32, dims: Dims = PROD, seed: int = 0, device="cpu", lo: int = 32768,
                  hi: int = 131072, lens=None, needles: bool = True, needle_block: int = 4096,
                  needles_per_block: int = 64):
    """Batched decode: B sequences with context lengths uniform in [lo, hi] (the cache
    already holds the query token, so the query sits at position n_b - 1), one query each.
    Key caches are packed back to back; cu_k holds the offsets."""
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(seed)
    gcpu = torch.Generator().manual_seed(seed)
    if lens is None:
        lens = torch.randint(lo, hi + 1, (B,), generator=gcpu).tolist()
    lens = [int(x) for x in lens]
    B = len(lens)
    cu_k = [0]
    for n in lens:
        cu_k.append(cu_k[-1] + n)
    NS = cu_k[-1]
    H_I, d_I, H, Dq = dims.n_idx_heads, dims.idx_dim, dims.n_heads, dims.qk_dim
    q_idx = _randn(g, (B, H_I, d_I), dev)
    k_idx = _randn(g, (NS, d_I), dev, chunk_rows=65536)
    w = _randn(g, (B, H_I), dev, std=dims.w_std)
    q = _randn(g, (B, H, Dq), dev, dtype=torch.bfloat16)
    c = _randn(g, (NS, Dq), dev, chunk_rows=65536)
    pairs = []
    if needles:
        for b in range(B):
            pb = _plant_needles(lens[b], 1, needle_block, needles_per_block, gcpu, query_pos=lens[b] - 1)
            if not pb:
                continue
            ss = torch.tensor([p[1] for p in pb], dtype=torch.long)
            hstar = torch.randint(0, H, (len(pb),), generator=gcpu)
            jstar = int(w[b].argmax())
            rows = (ss + cu_k[b]).to(dev)
            k_idx[rows] = 4.0 * q_idx[b, jstar]
            c[rows] = q[b, hstar.to(dev)].float()
            pairs.extend((b, s) for s in ss.tolist())
    q8, q_scale = quantize_e4m3_rows(q_idx)
    k8, k_scale = quantize_e4m3_rows(k_idx)
    return dict(q8=q8, q_scale=q_scale, w=w.contiguous(), k8=k8, k_scale=k_scale,
                q=q.contiguous(), kv=c.to(torch.bfloat16).contiguous(), needles=pairs,
                cu_q=list(range(B + 1)), cu_k=cu_k, lens=lens, dims=dims)
