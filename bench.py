"""Benchmark of the DSA hot path on one MI355X.

A step is one dsa_forward over the whole workload (lightning indexer -> top-k -> sparse MQA)
with every input already resident in HBM.  Default workload: causal prefill of one
131072-token sequence (k = 2048, 64 FP8 indexer heads of dim 128, 128 MQA heads over the
576-wide latent cache).  Prints one JSON line.

Besides the end-to-end rate the line carries:
  step_stats    median, spread and percentiles of the per-step times of the timed region;
  stages        per-stage time of the same launches (each stage entry point called on the
                same row passes as dsa_forward makes), measured with HIP events on the stream
                the kernels run on, the median over repetitions, and each stage's algorithmic
                rate against the published peak and against the peak measured on this device;
  prefill_by_length  the same for the 16,384- and 65,536-token prefills;
  measured_peaks     sustained bf16 / FP8 MFMA and HBM read rates of this device (probe kernels);
  roofline      the dominant stage's achieved rate against its MI355X peak;
  k_sweep       the whole forward on the same prefill for k = 512 .. 8192 (k = 2048 is the
                headline configuration; the pages leave the choice of k open);
  decode        batched decode (32 sequences, lengths uniform in [32768, 131072]): the
                forward step (median of 30), its stages (µs and GB/s), the cache producer
                (RoPE + FP8 codes of the new tokens, cache append) alone, and both together;
  cpu_baseline  the CPU oracle on a bounded, uniformly spaced sample of query rows of the
                same workload, timed on the host (rank 0 only), plus the tiny configuration
                through the oracle on one core.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import dsa_inputs  # noqa: E402
import sparse_attention_long_lightning_amd as dsa  # noqa: E402

METRIC = "DSA prefill tokens/s at 128K (+ indexer FP8 TFLOP/s); decode µs/token"
PEAK = {"fp8": 5000.0, "bf16": 2500.0, "hbm": 8000.0}  # TFLOP/s, TFLOP/s, GB/s (MI355X)
FLOP_INDEXER_PAIR = 2 * 64 * 128       # per causal (query, key) pair
FLOP_MQA_PAIR = 2 * 128 * (576 + 512)  # per selected (query, key) pair
FLOP_KL_PAIR = 2 * 128 * 576           # per slot of the indexer KL target (logits only)


# HBM traffic per launch of a kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded in
# profiles/traffic.json together with a hash of the kernel's sources; reported only while the
# sources are unchanged.
KERNEL_SOURCES = {
    "sparse_mqa_kernel": ["sparse_attention_long_lightning_amd/csrc/mqa.hip",
                          "sparse_attention_long_lightning_amd/csrc/common.hpp"],
    "indexer_prefill_kernel": ["sparse_attention_long_lightning_amd/csrc/indexer.hip",
                               "sparse_attention_long_lightning_amd/csrc/common.hpp"],
    "topk_hist_kernel": ["sparse_attention_long_lightning_amd/csrc/topk.hip",
                    "sparse_attention_long_lightning_amd/csrc/common.hpp"],
}


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel):
    """HBM bytes per launch (fetched + written) if recorded for the current sources, else None."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
            rec = json.load(fh).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_hash(kernel):
        return None
    return int(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timer:
    """HIP-event timing on torch's current stream (the stream the library launches on)."""

    def __init__(self):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()

    def ms(self):
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def stats(ms):
    """Median, min, max and 10th/90th percentiles of a list of times (ms)."""
    a = np.asarray(ms, np.float64)
    return dict(n=int(a.size), median_ms=round(float(np.median(a)), 3), min_ms=round(float(a.min()), 3),
                max_ms=round(float(a.max()), 3), p10_ms=round(float(np.percentile(a, 10)), 3),
                p90_ms=round(float(np.percentile(a, 90)), 3))


def timed_steps(fn, steps):
    """Runs fn steps times back to back with an event between steps; returns the total and the
    per-step times (ms) from the same events."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    ev[-1].synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[-1]), per


class Peaks:
    """Sustained rates of this device from the probe kernels of libpeak.so (bf16 and FP8 MFMA
    chains, streaming HBM read), each the best of a few timed runs."""

    def __init__(self, dev):
        import ctypes

        self.lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_long_lightning_amd", "libpeak.so"))
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_double)
        for fn in (self.lib.dsa_peak_mfma_bf16, self.lib.dsa_peak_mfma_fp8):
            fn.argtypes, fn.restype = [I, P, P, D], I
        self.lib.dsa_peak_read.argtypes, self.lib.dsa_peak_read.restype = [P, ctypes.c_size_t, P, P], I
        self.ct = ctypes
        self.dev = dev
        self.sink = torch.zeros(1 << 16, dtype=torch.float32, device=dev)

    def _mfma(self, fn, iters=4000, reps=5):
        flops = self.ct.c_double(0)
        stream = self.ct.c_void_p(torch.cuda.current_stream().cuda_stream)
        best = None
        for _ in range(reps + 1):
            with Timer() as tm:
                rc = fn(iters, self.ct.c_void_p(self.sink.data_ptr()), stream, self.ct.byref(flops))
            ms = tm.ms()
            assert rc == 0, "peak probe launch failed"
            best = ms if best is None else min(best, ms)
        return flops.value / (best / 1e3) / 1e12

    def measure(self):
        bf16 = self._mfma(self.lib.dsa_peak_mfma_bf16)
        fp8 = self._mfma(self.lib.dsa_peak_mfma_fp8)
        nbytes = 4 << 30
        buf = torch.empty(nbytes, dtype=torch.uint8, device=self.dev)
        buf.fill_(1)
        stream = self.ct.c_void_p(torch.cuda.current_stream().cuda_stream)
        best = None
        for _ in range(6):
            with Timer() as tm:
                rc = self.lib.dsa_peak_read(self.ct.c_void_p(buf.data_ptr()), nbytes,
                                            self.ct.c_void_p(self.sink.data_ptr()), stream)
            assert rc == 0, "peak probe launch failed"
            ms = tm.ms()
            best = ms if best is None else min(best, ms)
        del buf
        torch.cuda.empty_cache()
        return dict(bf16_tflops=round(bf16, 1), fp8_tflops=round(fp8, 1), hbm_read_gbps=round(nbytes / (best / 1e3) / 1e9, 1),
                    note="sustained rates of probe kernels on this device: independent MFMA chains in every wave "
                         "(4 workgroups of 512 threads per CU) and a streaming 4 GiB read; the published peaks "
                         "assume 2.4 GHz, the device settles near 2.0 GHz under MFMA load")


def prefill_case(L, dev):
    dims = dsa_inputs.PROD
    t0 = time.time()
    inp = dsa_inputs.prefill_inputs(L, dims, seed=0, device=dev)
    torch.cuda.synchronize()
    log(f"generated prefill L={L} inputs in {time.time() - t0:.1f}s")
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=dev)
    out = torch.empty(L, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(L, dims.n_heads, dtype=torch.float32, device=dev)
    ws = torch.empty(dsa.workspace_size(dims, batch), dtype=torch.uint8, device=dev)
    return dict(dims=dims, inp=inp, batch=batch, out=out, lse=lse, ws=ws, L=L)


def run_forward(c):
    i = c["inp"]
    dsa.forward(c["dims"], c["batch"], i["q8"], i["q_scale"], i["w"], i["k8"], i["k_scale"], i["q"],
                i["kv"], c["out"], c["lse"], None, c["ws"])


def chunk_rows(c):
    """Row passes of dsa_forward in the bench's workspace.  The library sizes each pass by area:
    R rows ending at row r1 take R x round4(r1) fp32 scores plus R index rows and R count rows
    (each area rounded up to 256 bytes) from the start of the workspace, and a pass takes as
    many rows as fit (a multiple of 8, or the rest of the sequence)."""
    L, k = c["L"], c["dims"].topk
    ws = c["ws"].numel()

    def al(x):
        return (x + 255) // 256 * 256

    def fits(r0, rows):
        s = (r0 + rows + 3) // 4 * 4
        return al(rows * s * 4) + al(rows * k * 4) + al(rows * dsa.COUNT_BINS * 4) <= ws

    passes, r0 = [], 0
    while r0 < L:
        rows = L - r0
        if not fits(r0, rows):
            lo, hi = 1, rows - 1
            while lo < hi:
                mid = lo + (hi - lo + 1) // 2
                if fits(r0, mid):
                    lo = mid
                else:
                    hi = mid - 1
            rows = lo - lo % 8 if lo > 8 else lo
        passes.append((r0, r0 + rows))
        r0 += rows
    return passes


def stage_breakdown(c, reps=1):
    """Runs the stage entry points on the same row passes dsa_forward makes (the indexer that
    also counts each row's scores, the top-k that starts from those counts, the sparse MQA)
    and times every call with HIP events.  Returns per-stage totals (ms) and algorithmic
    work."""
    dims, inp, L = c["dims"], c["inp"], c["L"]
    k = dims.topk
    dev = inp["q8"].device
    passes = chunk_rows(c)
    ch = max(r1 - r0 for r0, r1 in passes)
    idx_all = torch.empty(ch, k, dtype=torch.int32, device=dev)
    counts_all = torch.empty(ch, dsa.COUNT_BINS, dtype=torch.int32, device=dev)
    kl = torch.empty(L, dtype=torch.float32, device=dev)
    t_kl, n_kl = 0.0, 0
    t = {"indexer": 0.0, "topk": 0.0, "mqa": 0.0}
    launches = {"indexer": 0, "topk": 0, "mqa": 0}
    per_rep = []
    pairs_idx = 0
    pairs_mqa = 0
    for _ in range(reps):
        t0 = dict(t)
        for r0, r1 in passes:
            n = r1 - r0
            # the pass's score rows at its own stride (its last row's length), as in dsa_forward
            stride = (r1 + 3) // 4 * 4
            scores = c["ws"][: n * stride * 4].view(torch.float32).view(n, stride)
            idx, counts = idx_all[:n], counts_all[:n]
            # the pass as its own batch: queries r0..r1-1 are the last n of keys 0..r1-1
            b = dsa.Batch([0, n], [0, r1], device=dev)
            rsel = max(r0, k)  # rows with p + 1 <= k need no scores
            if rsel < r1:
                bs = dsa.Batch([0, r1 - rsel], [0, r1], device=dev)
                with Timer() as tm:
                    dsa.indexer_scores_counted(dims, bs, inp["q8"][rsel:], inp["q_scale"][rsel:], inp["w"][rsel:],
                                               inp["k8"], inp["k_scale"], scores[rsel - r0:], stride,
                                               counts[rsel - r0:])
                t["indexer"] += tm.ms()
                launches["indexer"] += 1
                pairs_idx += sum_range(rsel + 1, r1)
            with Timer() as tm:
                dsa.topk_counted(dims, b, scores, stride, counts, idx)
            t["topk"] += tm.ms()
            launches["topk"] += 1
            with Timer() as tm:
                dsa.sparse_mqa(dims, b, inp["q"][r0:r1], inp["kv"], idx, c["out"][r0:r1], c["lse"][r0:r1],
                               c["ws"])
            t["mqa"] += tm.ms()
            launches["mqa"] += 1
            # indexer KL target of the pass (training only; not part of the forward step)
            with Timer() as tm:
                dsa.indexer_kl(dims, b, inp["q"][r0:r1], inp["kv"], c["lse"][r0:r1], idx, scores, stride,
                               kl[r0:r1])
            t_kl += tm.ms()
            n_kl += 1
            pairs_mqa += sum(min(p + 1, k) for p in range(r0, r1))
        per_rep.append({s: t[s] - t0[s] for s in t})
    # the median repetition of each stage
    for s in t:
        t[s] = float(np.median([r[s] for r in per_rep]))
    for s in launches:
        launches[s] //= reps
    pairs_idx //= reps
    pairs_mqa //= reps
    topk_rows = sum(1 for p in range(L) if p + 1 > k)
    topk_bytes = 4 * pairs_idx + 8 * 1024 * L  # one read of every valid score + the index rows
    spread = {s: dict(min_ms=round(min(r[s] for r in per_rep), 3), max_ms=round(max(r[s] for r in per_rep), 3))
              for s in t}
    return t, launches, dict(indexer_pairs=pairs_idx, mqa_pairs=pairs_mqa, topk_rows=topk_rows,
                             topk_bytes=topk_bytes, kl_ms=t_kl / reps, kl_launches=n_kl // reps, reps=reps,
                             spread=spread)


def sum_range(lo, hi):
    """Sum of the integers lo..hi (inclusive)."""
    return (lo + hi) * (hi - lo + 1) // 2 if hi >= lo else 0


def decode_case(dev, steps):
    dims = dsa_inputs.PROD
    inp = dsa_inputs.decode_inputs(32, dims, seed=0, device=dev)
    batch = dsa.Batch(inp["cu_q"], inp["cu_k"], device=dev)
    B = 32
    out = torch.empty(B, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, dims.n_heads, dtype=torch.float32, device=dev)
    ws = torch.empty(dsa.workspace_size(dims, batch), dtype=torch.uint8, device=dev)

    # the cache producer of the step: the new tokens' indexer query and key (before RoPE and
    # quantisation) and latent rows, rotary tables for every position
    g = torch.Generator(device=dev).manual_seed(1)
    q_idx = torch.randn(B, dims.n_idx_heads, dims.idx_dim, generator=g, device=dev)
    k_idx = torch.randn(B, dims.idx_dim, generator=g, device=dev)
    kv_new = torch.randn(B, dims.qk_dim, generator=g, device=dev).to(torch.bfloat16)
    n_pos = max(inp["lens"])
    rd = dims.idx_dim // 2
    ang = torch.arange(n_pos, dtype=torch.float64)[:, None] * \
        10000.0 ** (-2.0 * torch.arange(rd // 2, dtype=torch.float64) / rd)[None, :]
    cos, sin = ang.cos().float().to(dev), ang.sin().float().to(dev)

    def append():
        dsa.cache_append(dims, batch, q_idx, k_idx, kv_new, cos, sin, inp["q8"], inp["q_scale"],
                         inp["k8"], inp["k_scale"], inp["kv"])

    def step():
        dsa.forward(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"],
                    inp["q"], inp["kv"], out, lse, None, ws)

    # stage entry points on the same batch: the decode indexer, the split top-k, the split
    # sparse MQA with its combine (the forward runs the same kernels, the indexer also counting
    # its scores and the top-k starting from those counts)
    nkeys = int(inp["cu_k"][-1])
    stride = (batch.max_len_k + 3) // 4 * 4
    sc = torch.empty(B, stride, dtype=torch.float32, device=dev)
    idx = torch.empty(B, dims.topk, dtype=torch.int32, device=dev)
    tws = torch.empty(max(dsa.topk_workspace_size(dims, batch), 16), dtype=torch.uint8, device=dev)

    def st_indexer():
        dsa.indexer_scores(dims, batch, inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], sc, stride)

    def st_topk():
        dsa.topk(dims, batch, sc, stride, idx, tws)

    def st_mqa():
        dsa.sparse_mqa(dims, batch, inp["q"], inp["kv"], idx, out, lse, ws)

    def timed(fn, n=steps):
        # 20 untimed calls first: right after the 128K prefill the first decode steps of a
        # loop ran ~10% slower than a loop measured later in the same process
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        total, per = timed_steps(fn, n)
        return float(np.median(per)) * 1e3, per

    us_app, _ = timed(append)
    us, per = timed(step)
    us_all, _ = timed(lambda: (append(), step()))
    sel = sum(min(n, dims.topk) for n in inp["lens"])
    work = {"indexer": nkeys * (128 + 4 + 4), "topk": nkeys * 4 + B * dims.topk * 4,
            "mqa": sel * 1152 + B * dims.n_heads * (576 + 512) * 2}
    stages = {}
    for name, fn in (("indexer", st_indexer), ("topk", st_topk), ("mqa", st_mqa)):
        t, _ = timed(fn)
        stages[name] = dict(us=round(t, 2), gbps=round(work[name] / (t / 1e6) / 1e9, 1),
                            frac_hbm_peak=round(work[name] / (t / 1e6) / 1e9 / PEAK["hbm"], 4))
    stages["note"] = ("stage entry points on the same batch, median of %d; bytes: indexer 136 per key "
                      "(codes, scale, score), top-k 4 per score + the index rows, sparse MQA the gathered "
                      "latent rows (1,152 B per selected slot) + q and out" % steps)
    return dict(us_per_step=round(us, 2), us_per_token=round(us / B, 3), step_stats=stats(per), batch=B,
                mean_context=round(nkeys / B), hbm_floor_mb=round((nkeys * 132 + B * 2048 * 1152) / 1e6, 1),
                stages=stages, cache_append_us=round(us_app, 2), us_per_step_with_append=round(us_all, 2))


def k_sweep(c, ks, steps=2):
    """The whole forward at the same length and inputs for several k (the inputs do not depend
    on k): ms per step and tokens/s for each."""
    import dataclasses

    res = {}
    for k in ks:
        dims = dataclasses.replace(c["dims"], topk=k)
        n = dsa.workspace_size(dims, c["batch"])
        ws = c["ws"] if c["ws"].numel() >= n else torch.empty(n, dtype=torch.uint8, device=c["ws"].device)
        i = c["inp"]

        def fwd():
            dsa.forward(dims, c["batch"], i["q8"], i["q_scale"], i["w"], i["k8"], i["k_scale"], i["q"],
                        i["kv"], c["out"], c["lse"], None, ws)

        fwd()
        torch.cuda.synchronize()
        with Timer() as tm:
            for _ in range(steps):
                fwd()
        ms = tm.ms() / steps
        res[str(k)] = dict(ms_per_step=round(ms, 3), tokens_per_s=round(c["L"] / (ms / 1e3), 1))
        del ws
        log(f"k={k}: {ms:.2f} ms/step")
    return res


def cpu_baseline(c, budget_s=20.0, max_rows=192):
    """The oracle on uniformly spaced query rows of the same prefill (indexer over every
    earlier key, top-k, MQA).  Rows are processed in growing batches until ~budget_s."""
    import oracle

    inp, L = c["inp"], c["L"]
    host = {"cu_q": inp["cu_q"], "cu_k": inp["cu_k"], "dims": inp["dims"],
            "k8": inp["k8"].cpu().numpy(), "k_scale": inp["k_scale"].cpu().numpy(),
            "kv": inp["kv"].view(torch.int16).cpu().numpy().view(np.uint16)}
    done = 0
    spent = 0.0
    n = oracle.num_threads()
    rng = np.random.default_rng(0)
    while spent < budget_s and done < max_rows:
        m = min(max_rows - done, max(1, n))
        rows = np.sort(rng.integers(0, L, m))
        # only the sampled rows of the query side are copied to the host
        rq = torch.from_numpy(rows).to(inp["q8"].device)
        q8 = inp["q8"][rq].cpu().numpy()
        qs = inp["q_scale"][rq].cpu().numpy()
        w = inp["w"][rq].cpu().numpy()
        q = inp["q"][rq].view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        scores = oracle.indexer_rows(q8, qs, w, host["k8"], host["k_scale"], np.arange(m), rows)
        sel = oracle.topk_rows(scores, inp["dims"].topk)
        oracle.sparse_mqa(q, host["kv"], sel, inp["dims"].v_dim, inp["dims"].sm_scale)
        spent += time.perf_counter() - t0
        done += m
    res = dict(value=round(done / spent, 3), unit="tokens/s", cores=n, kind="oracle",
               sample=f"{done} query rows drawn uniformly from the L={L} prefill (positions "
                      f"seeded), each through the oracle's indexer over all earlier keys, "
                      f"top-k and sparse MQA; {spent:.1f}s of host time")
    # the tiny configuration (L = 256, 4 indexer heads of 32, k = 32, 8 heads over 80-wide rows)
    # through the whole oracle path on a single core
    tiny = dsa_inputs.prefill_inputs(256, dsa_inputs.TINY, seed=0, device="cpu", needles=False)
    th = {k: (v.view(torch.int16).numpy().view(np.uint16) if torch.is_tensor(v) and v.dtype == torch.bfloat16
              else v.numpy() if torch.is_tensor(v) else v) for k, v in tiny.items()}
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.forward_rows(th, np.arange(256))
        t1 = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(n)
    res["tiny_one_core"] = dict(value=round(256 / t1, 1), unit="tokens/s", cores=1,
                                sample="tiny prefill L=256 (indexer 4 heads x 32, k=32, MQA 8 heads x 80/64), "
                                       f"every row through the oracle on one thread: {t1 * 1e3:.1f} ms")
    return res


def stage_objects(t, launches, work, L, peaks):
    """Per-stage records (median ms over repetitions, rates, fractions of the published and of
    the measured peaks) from stage_breakdown's output."""
    tf_idx = work["indexer_pairs"] * FLOP_INDEXER_PAIR / (t["indexer"] / 1e3) / 1e12
    tf_mqa = work["mqa_pairs"] * FLOP_MQA_PAIR / (t["mqa"] / 1e3) / 1e12
    gb_topk = work["topk_bytes"] / (t["topk"] / 1e3) / 1e9
    sp = work["spread"]
    st = {}
    st["indexer"] = dict(ms=round(t["indexer"], 3), launches=launches["indexer"], tflops=round(tf_idx, 1),
                         frac_fp8_peak=round(tf_idx / PEAK["fp8"], 4), tokens_per_s=round(L / (t["indexer"] / 1e3), 1),
                         **sp["indexer"])
    st["topk"] = dict(ms=round(t["topk"], 3), launches=launches["topk"], gbps=round(gb_topk, 1),
                      frac_hbm_peak=round(gb_topk / PEAK["hbm"], 4), tokens_per_s=round(L / (t["topk"] / 1e3), 1),
                      **sp["topk"])
    st["mqa"] = dict(ms=round(t["mqa"], 3), launches=launches["mqa"], tflops=round(tf_mqa, 1),
                     frac_bf16_peak=round(tf_mqa / PEAK["bf16"], 4), tokens_per_s=round(L / (t["mqa"] / 1e3), 1),
                     **sp["mqa"])
    if peaks:
        st["indexer"]["frac_measured_fp8"] = round(tf_idx / peaks["fp8_tflops"], 4)
        st["topk"]["frac_measured_hbm"] = round(gb_topk / peaks["hbm_read_gbps"], 4)
        st["mqa"]["frac_measured_bf16"] = round(tf_mqa / peaks["bf16_tflops"], 4)
    st["reps"] = work["reps"]
    return st, tf_idx, tf_mqa


def forward_rate(c, steps, warmup):
    for _ in range(warmup):
        run_forward(c)
    torch.cuda.synchronize()
    total, per = timed_steps(lambda: run_forward(c), steps)
    return total / steps, per


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--seq-len", type=int, default=131072)
    ap.add_argument("--stage-reps", type=int, default=10, help="repetitions of the per-stage timing (median)")
    ap.add_argument("--lengths", default="16384,65536",
                    help="other prefill lengths timed per stage ('' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-stages", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--k-sweep", default="512,1024,2048,4096,8192",
                    help="comma-separated k values timed on the same prefill ('' to skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="first copy BYTES between two device buffers (a plain copy of known size "
                         "that calibrates the HBM byte counters of a profiled run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.copy_calibration} bytes done")
        del src, dst
    peaks = None
    if not args.no_peaks:
        peaks = Peaks(dev).measure()
        log(f"measured peaks {peaks}")
    L = args.seq_len
    c = prefill_case(L, dev)
    log(f"workspace {c['ws'].numel() / 2**30:.2f} GiB")
    for _ in range(args.warmup):
        run_forward(c)
    torch.cuda.synchronize()
    log("timed region")
    total, per = timed_steps(lambda: run_forward(c), args.steps)
    torch.cuda.synchronize()
    ms = total / args.steps
    tok_s = L / (ms / 1e3)
    log(f"prefill L={L}: {ms:.2f} ms/step, {tok_s:,.0f} tokens/s")

    line = {"metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "fp8-e4m3 indexer + bf16 attention (fp32 accumulate)", "data": "synthetic",
            "config": {"workload": f"DSA causal prefill, one sequence L={L}, k=2048, indexer 64 heads x 128 "
                                   f"(FP8 e4m3), MQA 128 heads over a 576-wide bf16 latent cache (value 512), "
                                   f"64 planted needles per 4K block, seed 0",
                       "seq_len": L, "topk": 2048, "global_batch": 1},
            "step_stats": stats(per)}
    if peaks:
        line["measured_peaks"] = peaks
    if not args.no_stages:
        t, launches, work = stage_breakdown(c, reps=args.stage_reps)
        stages, tf_idx, tf_mqa = stage_objects(t, launches, work, L, peaks)
        line["stages"] = stages
        tf_kl = work["mqa_pairs"] * FLOP_KL_PAIR / (work["kl_ms"] / 1e3) / 1e12
        line["kl_target"] = dict(ms=round(work["kl_ms"], 3), launches=work["kl_launches"],
                                 tflops=round(tf_kl, 1), frac_bf16_peak=round(tf_kl / PEAK["bf16"], 4),
                                 note="indexer KL target over the top-k slots, forward only")
        line["indexer_fp8_tflops"] = round(tf_idx, 1)
        dom = max(("indexer", "topk", "mqa"), key=lambda s: t[s])
        if dom == "indexer":
            per_l = work["indexer_pairs"] * FLOP_INDEXER_PAIR / launches["indexer"] / 1e12
            avg = t["indexer"] / launches["indexer"] / 1e3
            roof = dict(kernel="indexer_prefill_kernel", bound="mfma", achieved=round(per_l / avg, 1),
                        peak=PEAK["fp8"], unit="TFLOP/s")
        elif dom == "mqa":
            per_l = work["mqa_pairs"] * FLOP_MQA_PAIR / launches["mqa"] / 1e12
            avg = t["mqa"] / launches["mqa"] / 1e3
            roof = dict(kernel="sparse_mqa_kernel", bound="mfma", achieved=round(per_l / avg, 1),
                        peak=PEAK["bf16"], unit="TFLOP/s")
        else:
            per_l = work["topk_bytes"] / launches["topk"] / 1e9
            avg = t["topk"] / launches["topk"] / 1e3
            roof = dict(kernel="topk_hist_kernel", bound="hbm", achieved=round(per_l / avg, 1),
                        peak=PEAK["hbm"], unit="GB/s")
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
        roof["traffic"] = recorded_traffic(roof["kernel"])
        roof["avg_launch_ms"] = round(avg * 1e3, 3)
        if peaks:
            mp = peaks["fp8_tflops"] if dom == "indexer" else peaks["bf16_tflops"] if dom == "mqa" else peaks["hbm_read_gbps"]
            roof["measured_peak"] = mp
            roof["frac_measured"] = round(roof["achieved"] / mp, 4)
        line["roofline"] = roof
        log(f"stages {json.dumps(stages)}")
    if args.k_sweep:
        line["k_sweep"] = k_sweep(c, [int(x) for x in args.k_sweep.split(",")])
    if args.lengths and not args.no_stages:
        del c["out"], c["lse"], c["ws"]
        torch.cuda.empty_cache()
        by_len = {}
        for Lx in [int(x) for x in args.lengths.split(",")]:
            cx = prefill_case(Lx, dev)
            msx, perx = forward_rate(cx, steps=args.steps, warmup=2)
            tx, lx, wx = stage_breakdown(cx, reps=max(3, args.stage_reps // 2))
            stx, _, _ = stage_objects(tx, lx, wx, Lx, peaks)
            by_len[str(Lx)] = dict(ms_per_step=round(msx, 3), tokens_per_s=round(Lx / (msx / 1e3), 1),
                                   step_stats=stats(perx), stages=stx)
            log(f"prefill L={Lx}: {msx:.2f} ms/step")
            del cx
            torch.cuda.empty_cache()
        if "stages" in line:
            by_len[str(L)] = dict(ms_per_step=round(ms, 3), tokens_per_s=round(tok_s, 1), stages=line["stages"])
        line["prefill_by_length"] = by_len
    if not args.no_decode:
        for key in ("out", "lse", "ws"):
            c.pop(key, None)
        torch.cuda.empty_cache()
        line["decode"] = decode_case(dev, steps=30)
        log(f"decode {line['decode']}")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(c)
        log(f"cpu baseline {line['cpu_baseline']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
