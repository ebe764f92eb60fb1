#!/usr/bin/env python3
"""Throughput of the fused indexer + sparse latent attention hot path.

Headline workload: the long prefill, one causal sequence of 65,536
positions processed in 16 query chunks of 4,096 (contiguous bf16 latent
cache of 576 per row and index-key cache of 128 per row), 64 indexer heads,
Top-K 2048, 128 attention heads.  One step is the 16
idx_sparse_attn_prefill calls: score every causal position of every query,
select the Top-K, gather the selected latent rows and attend.  Inputs are
seeded synthetic data resident in HBM before timing starts; a 1 GiB write
flushes the caches before every timed step.

Prints one JSON line.  `roofline` describes the step's dominant kernel (the
sparse attention, MFMA-bound): its algorithmic flops per launch over its
average launch time, measured with HIP events the library records on the
launch stream during the timed steps.  `secondary` holds the prefill
indexer's MFMA fraction and the other four workloads (tokens/s, per-kernel
times, the decode attention's HBM fraction).  `cpu_baseline` is the CPU
oracle timed on a bounded row sample of the long prefill (one thread) and
extrapolated.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run this many steps with no timing or oracle (for rocprofv3)")
    ap.add_argument("--workload", type=int, default=0,
                    help="1..5: time another workload (all of its calls per step) and print per-kernel "
                         "figures instead of the headline JSON line")
    ap.add_argument("--kv-write", action="store_true",
                    help="time the FP8 latent-cache and index-key writers on 1,048,576 rows each and print "
                         "their own figures instead of the headline JSON line")
    ap.add_argument("--mxfp8", action="store_true",
                    help="time the decode indexer (scores + Top-K) on the 64 x 32768 decode batch with MXFP8 "
                         "key rows and with bf16 keys, and print their own figures instead of the headline line")
    ap.add_argument("--multi-token", action="store_true",
                    help="time multi-token decode rows (2, 4 and 8 query tokens per request, the speculative "
                         "verification shape) on the decode batch's caches and print their own figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy 3 times (reference for HBM byte counters)")
    return ap.parse_args()


def measure_workload(n, steps, warmup):
    """Per-call and per-kernel times of workload n (a step = every call)."""
    import numpy as np
    import torch
    import indexer_selected_sparse_idx_amd as lib
    from workloads import config, generate

    dev = torch.device("cuda:0")
    wl = config(n)
    inp = generate(wl, dev)
    scale = 1.0 / math.sqrt(576.0)
    calls = []
    ws_bytes = 0
    for call in inp.calls:
        ctx = torch.from_numpy(call.ctx_len.astype(np.int32)).to(dev)
        cu = None if call.cu_q is None else torch.from_numpy(call.cu_q.astype(np.int32)).to(dev)
        bt_np = inp.call_block_table(call)
        bt = None if bt_np is None else torch.from_numpy(bt_np.astype(np.int32)).to(dev)
        s = lib.Seqs(ctx, cu, max_q_len=call.max_q_len, max_ctx_len=int(call.ctx_len.max()),
                     num_tokens=call.num_tokens, block_table=bt, page_size=wl.page_size,
                     seq_stride=inp.seq_stride if not wl.paged else 0)
        s._keep = (ctx, cu, bt)
        ws_bytes = max(ws_bytes, lib.idx_sparse_attn_workspace(s, wl.H_I, wl.d_I, wl.H, wl.top_k))
        calls.append((call, s))
    T_max = max(c.num_tokens for c, _ in calls)
    out = torch.empty((T_max, wl.H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((T_max, wl.H), dtype=torch.float32, device=dev)
    idx = torch.empty((T_max, wl.top_k), dtype=torch.int32, device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def run(call, s):
        sl = slice(call.tok_lo, call.tok_hi)
        fn = lib.idx_sparse_attn_decode if call.is_decode else lib.idx_sparse_attn_prefill
        fn(s, inp.q_idx[sl], inp.k_idx, inp.head_w[sl], wl.top_k, inp.q[sl], inp.kv, scale, k_scale=inp.k_scale,
           out=out[:call.num_tokens], lse=lse[:call.num_tokens], out_idx=idx[:call.num_tokens], ws=ws)

    for _ in range(warmup):
        for c, s in calls:
            run(c, s)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        for c, s in calls:
            run(c, s)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    names = {lib.IDX_KERNEL_SCORE: "score", lib.IDX_KERNEL_TOPK: "topk", lib.IDX_KERNEL_ATTN: "attn",
             lib.IDX_KERNEL_COMBINE: "combine"}
    per_call = []
    tot = {v: 0.0 for v in names.values()}
    for c, s in calls:
        ev = {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in names}
        for e0, e1 in ev.values():
            e0.record()
            e1.record()
        torch.cuda.synchronize()
        for k, (e0, e1) in ev.items():
            lib.idx_timer_arm(k, e0, e1)
        run(c, s)
        torch.cuda.synchronize()
        kt = {}
        for k, (e0, e1) in ev.items():
            kt[names[k]] = e0.elapsed_time(e1) * 1e3 if (k != lib.IDX_KERNEL_COMBINE or e1.query()) else 0.0
        per_call.append({"tokens": c.num_tokens, "max_ctx": int(c.ctx_len.max()), "kernels_us": kt})
        for k in tot:
            tot[k] += kt[k]
    # algorithmic flops of the whole step (causal pairs for the indexer, selected rows for attention)
    idx_flops = attn_flops = 0.0
    for c, _ in calls:
        qlen = [1] * len(c.ctx_len) if c.cu_q is None else list(np.diff(c.cu_q))
        for ctx, ql in zip(c.ctx_len, qlen):
            ts = np.arange(int(ctx) - ql, int(ctx))
            idx_flops += 2.0 * wl.H_I * wl.d_I * float((ts + 1).sum())
            attn_flops += 2176.0 * wl.H * float(np.minimum(wl.top_k, ts + 1).sum())
    tokens = sum(c.num_tokens for c, _ in calls)
    print(json.dumps({"workload": wl.name, "ms_per_step": ms, "tokens_per_s": tokens / (ms * 1e-3),
                      "kernels_us_total": tot,
                      "indexer_tflops": idx_flops / (tot["score"] * 1e-6) / 1e12 if tot["score"] else None,
                      "attn_tflops": attn_flops / ((tot["attn"] + tot["combine"]) * 1e-6) / 1e12,
                      "per_call": per_call}), flush=True)


KV_WRITE_ROWS = 1 << 20   # 8 sequences x 131,072 positions


def measure_kv_write(steps, warmup):
    """FP8 latent-cache writer: quantise 1,048,576 standard-normal bf16 latent
    rows into a packed FP8 cache, as a paged cache's slots are written:
    consecutive rows within pages of 64, the pages in a shuffled order.
    Algorithmic bytes per row: 1152 read, 656 written, 4 of row index; the
    kernel is HBM-bound."""
    import torch
    import indexer_selected_sparse_idx_amd as lib
    dev = torch.device("cuda:0")
    n = KV_WRITE_ROWS
    g = torch.Generator(device=dev).manual_seed(6)
    src = torch.randn((n, 576), generator=g, device=dev).to(torch.bfloat16)
    pages = torch.randperm(n // 64, generator=g, device=dev).to(torch.int32)
    perm = (pages[:, None] * 64 + torch.arange(64, dtype=torch.int32, device=dev)[None, :]).reshape(-1)
    kv = torch.empty((n, 656), dtype=torch.uint8, device=dev)
    for _ in range(max(1, warmup)):
        lib.idx_kv_fp8_write(src, perm, kv)
    torch.cuda.synchronize()
    times = []
    for _ in range(max(1, steps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        e1.record()   # (torch creates the HIP events on first record)
        torch.cuda.synchronize()
        lib.idx_timer_arm(lib.IDX_KERNEL_KV_WRITE, e0, e1)
        lib.idx_kv_fp8_write(src, perm, kv)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    us = sorted(times)[len(times) // 2]
    nbytes = n * (1152 + 656 + 4)
    print(json.dumps({"kernel": "FP8 latent-cache writer", "rows": n, "median_us": us,
                      "algorithmic_bytes": nbytes, "achieved_GBs": nbytes / us / 1e3,
                      "hbm_frac": nbytes / us / 1e3 / HBM_PEAK_GBS, "rows_per_s": n / us * 1e6}), flush=True)
    # index keys: 128 bf16 per row -> 128 e4m3 codes and one fp32 scale
    keys = torch.randn((n, 128), generator=g, device=dev).to(torch.bfloat16)
    kc = torch.empty((n, 128), dtype=torch.uint8, device=dev)
    ks = torch.empty((n,), dtype=torch.float32, device=dev)
    for _ in range(max(1, warmup)):
        lib.idx_key_fp8_write(keys, perm, kc, ks)
    torch.cuda.synchronize()
    times = []
    for _ in range(max(1, steps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        lib.idx_key_fp8_write(keys, perm, kc, ks)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    us = sorted(times)[len(times) // 2]
    nbytes = n * (256 + 128 + 4 + 4)
    print(json.dumps({"kernel": "FP8 index-key writer (per-row scales)", "rows": n, "median_us": us,
                      "algorithmic_bytes": nbytes, "achieved_GBs": nbytes / us / 1e3,
                      "hbm_frac": nbytes / us / 1e3 / HBM_PEAK_GBS, "rows_per_s": n / us * 1e6}), flush=True)


def measure_mxfp8(steps, warmup):
    """Decode indexer (scores + Top-K) on the decode batch (64 requests x
    32768 positions, 64 index heads of 128, Top-K 2048) with MXFP8 key rows
    (128 E4M3 codes and 4 E8M0 block exponents, 132 bytes per position) and,
    for comparison, with the workload's bf16 keys (256 bytes per position).
    The score kernel streams the keys once: algorithmic bytes per launch are
    the key rows plus the queries and head weights, HBM-bound."""
    import numpy as np
    import torch
    import indexer_selected_sparse_idx_amd as lib
    from workloads import config, generate, gen
    dev = torch.device("cuda:0")
    wl = config(2)
    inp = generate(wl, dev)
    call = inp.calls[0]
    T = call.num_tokens
    g = torch.Generator(device=dev).manual_seed(8)
    codes_mx, exps_mx = gen.mxfp8_keys(g, inp.k_idx.shape[0], dev)
    ctx_t = torch.from_numpy(call.ctx_len.astype(np.int32)).to(dev)
    seqs = lib.Seqs(ctx_t, None, max_q_len=1, max_ctx_len=int(call.ctx_len.max()), seq_stride=inp.seq_stride)
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
    ws = torch.empty(lib.idx_score_topk_workspace(seqs, wl.H_I, wl.d_I, wl.top_k), dtype=torch.uint8, device=dev)
    positions = int(call.ctx_len.sum())
    for label, keys, exps, row_bytes in (("MXFP8 keys", codes_mx, exps_mx, 132), ("bf16 keys", inp.k_idx, None, 256)):
        def run():
            lib.idx_score_topk(seqs, inp.q_idx, keys, inp.head_w, wl.top_k, k_scale=exps, out_idx=idx, ws=ws)
        for _ in range(max(1, warmup)):
            run()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(max(1, steps)):
            run()
        b.record()
        torch.cuda.synchronize()
        call_us = a.elapsed_time(b) * 1e3 / max(1, steps)
        times = []
        for _ in range(max(1, steps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            e1.record()
            torch.cuda.synchronize()
            lib.idx_timer_arm(lib.IDX_KERNEL_SCORE, e0, e1)
            run()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        us = sorted(times)[len(times) // 2]
        nbytes = positions * row_bytes + T * wl.H_I * (wl.d_I * 2 + 4)
        print(json.dumps({"kernel": "decode indexer score, " + label, "tokens": T, "positions": positions,
                          "score_median_us": us, "algorithmic_bytes": nbytes, "achieved_GBs": nbytes / us / 1e3,
                          "hbm_frac": nbytes / us / 1e3 / HBM_PEAK_GBS, "score_topk_call_us": call_us}),
              flush=True)
    # a prefill chunk: the last 4096 positions of the first sequence as query
    # tokens (both key formats through the prefill kernel, key tiles shared by
    # 8 tokens; MXFP8: one scaled fp8 MFMA per 128 dims)
    Q = 4096
    ctx0 = int(call.ctx_len[0])
    ctx1 = torch.tensor([ctx0], dtype=torch.int32, device=dev)
    cu = torch.tensor([0, Q], dtype=torch.int32, device=dev)
    pseqs = lib.Seqs(ctx1, cu, max_q_len=Q, max_ctx_len=ctx0, num_tokens=Q, seq_stride=inp.seq_stride)
    pq = torch.randint(-wl.q_range, wl.q_range + 1, (Q, wl.H_I, wl.d_I), generator=g, device=dev).to(torch.bfloat16)
    pw = torch.pow(2.0, -torch.randint(0, 4, (Q, wl.H_I), generator=g, device=dev).float())
    pidx = torch.empty((Q, wl.top_k), dtype=torch.int32, device=dev)
    pws = torch.empty(lib.idx_score_topk_workspace(pseqs, wl.H_I, wl.d_I, wl.top_k), dtype=torch.uint8, device=dev)
    pairs = float(sum(ctx0 - Q + i + 1 for i in range(Q)))
    for label, keys, exps in (("MXFP8 keys", codes_mx, exps_mx), ("bf16 keys", inp.k_idx, None)):
        def prun():
            lib.idx_score_topk(pseqs, pq, keys, pw, wl.top_k, k_scale=exps, out_idx=pidx, ws=pws)
        prun()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(3):
            prun()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / 3
        flops = 2.0 * wl.H_I * wl.d_I * pairs
        print(json.dumps({"kernel": "prefill chunk scores + Top-K, " + label, "tokens": Q, "ctx": ctx0,
                          "causal_pairs": pairs, "call_ms": ms, "tflops": flops / (ms * 1e-3) / 1e12}), flush=True)


def measure_multi_token(steps, warmup):
    """Multi-token decode rows: the decode batch's caches (64 requests x
    32768 positions, bf16 keys and latent rows) with Q = 2, 4, 8 query tokens
    per request at its last Q positions (a speculative verification step),
    through the fused prefill entry point (cu_q batches).  Queries are drawn
    like the workload's (integer index queries, standard-normal latent
    queries)."""
    import numpy as np
    import torch
    import indexer_selected_sparse_idx_amd as lib
    from workloads import config, generate
    dev = torch.device("cuda:0")
    wl = config(2)
    inp = generate(wl, dev)
    call = inp.calls[0]
    B = call.num_tokens
    g = torch.Generator(device=dev).manual_seed(9)
    scale = 1.0 / math.sqrt(576.0)
    names = {lib.IDX_KERNEL_SCORE: "score", lib.IDX_KERNEL_TOPK: "topk", lib.IDX_KERNEL_ATTN: "attn",
             lib.IDX_KERNEL_COMBINE: "combine"}
    ctx_t = torch.from_numpy(call.ctx_len.astype(np.int32)).to(dev)
    for Q in (2, 4, 8):
        T = B * Q
        cu = torch.arange(0, T + 1, Q, dtype=torch.int32, device=dev)
        seqs = lib.Seqs(ctx_t, cu, max_q_len=Q, max_ctx_len=int(call.ctx_len.max()), num_tokens=T,
                        seq_stride=inp.seq_stride)
        q_idx = torch.randint(-wl.q_range, wl.q_range + 1, (T, wl.H_I, wl.d_I), generator=g,
                              device=dev).to(torch.bfloat16)
        head_w = torch.pow(2.0, -torch.randint(0, 4, (T, wl.H_I), generator=g, device=dev).float())
        q = torch.randn((T, wl.H, 576), generator=g, device=dev).to(torch.bfloat16)
        out = torch.empty((T, wl.H, 512), dtype=torch.float32, device=dev)
        lse = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
        idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
        ws = torch.empty(lib.idx_sparse_attn_workspace(seqs, wl.H_I, wl.d_I, wl.H, wl.top_k), dtype=torch.uint8,
                         device=dev)

        def run():
            lib.idx_sparse_attn_prefill(seqs, q_idx, inp.k_idx, head_w, wl.top_k, q, inp.kv, scale, out=out,
                                        lse=lse, out_idx=idx, ws=ws)
        for _ in range(max(1, warmup)):
            run()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(max(1, steps)):
            run()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / max(1, steps)
        ev = {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in names}
        for e0, e1 in ev.values():
            e0.record()
            e1.record()
        torch.cuda.synchronize()
        for k, (e0, e1) in ev.items():
            lib.idx_timer_arm(k, e0, e1)
        run()
        torch.cuda.synchronize()
        kt = {names[k]: e0.elapsed_time(e1) * 1e3 for k, (e0, e1) in ev.items()}
        print(json.dumps({"workload": "multi-token decode: %d requests x %d tokens, ctx %d" % (B, Q, int(call.ctx_len.max())),
                          "tokens": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "kernels_us": kt}),
              flush=True)


FLUSH_BYTES = 1 << 30   # more than the L2s and the 256 MB MALL together


class Flusher:
    """Evicts the caches between timed steps: writes one 1 GiB buffer, then
    reads another, so that the caches hold clean lines of the second when
    the step starts.  (A write alone leaves them full of dirty lines, whose
    write-back then lands inside the step: on the decode batch it slowed
    the index-key stream from 104 to 155 us.)"""

    def __init__(self, dev):
        import torch
        self.wbuf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
        self.rbuf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
        self.n = 0

    def __call__(self):
        import torch
        self.n += 1
        self.wbuf.fill_(self.n)
        torch.sum(self.rbuf, dtype=torch.int64)


def prepared_calls(wl, inp, dev):
    """Batch descriptions and reusable outputs / workspace for every call of
    a generated workload."""
    import numpy as np
    import torch
    import indexer_selected_sparse_idx_amd as lib
    calls = []
    ws_bytes = 0
    for call in inp.calls:
        ctx = torch.from_numpy(call.ctx_len.astype(np.int32)).to(dev)
        cu = None if call.cu_q is None else torch.from_numpy(call.cu_q.astype(np.int32)).to(dev)
        bt_np = inp.call_block_table(call)
        bt = None if bt_np is None else torch.from_numpy(bt_np.astype(np.int32)).to(dev)
        s = lib.Seqs(ctx, cu, max_q_len=call.max_q_len, max_ctx_len=int(call.ctx_len.max()),
                     num_tokens=call.num_tokens, block_table=bt, page_size=wl.page_size,
                     seq_stride=inp.seq_stride if not wl.paged else 0)
        s._keep = (ctx, cu, bt)
        ws_bytes = max(ws_bytes, lib.idx_sparse_attn_workspace(s, wl.H_I, wl.d_I, wl.H, wl.top_k))
        calls.append((call, s))
    T_max = max(c.num_tokens for c, _ in calls)
    bufs = dict(out=torch.empty((T_max, wl.H, 512), dtype=torch.float32, device=dev),
                lse=torch.empty((T_max, wl.H), dtype=torch.float32, device=dev),
                idx=torch.empty((T_max, wl.top_k), dtype=torch.int32, device=dev),
                ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev))
    return calls, bufs


def run_call(lib, wl, inp, call, s, bufs, scale):
    sl = slice(call.tok_lo, call.tok_hi)
    fn = lib.idx_sparse_attn_decode if call.is_decode else lib.idx_sparse_attn_prefill
    T = call.num_tokens
    fn(s, inp.q_idx[sl], inp.k_idx, inp.head_w[sl], wl.top_k, inp.q[sl], inp.kv, scale, k_scale=inp.k_scale,
       out=bufs["out"][:T], lse=bufs["lse"][:T], out_idx=bufs["idx"][:T], ws=bufs["ws"])


def workload_units(wl, calls):
    """Algorithmic work of one step over every call: indexer flops (causal
    pairs), attention flops (selected rows), and the HBM bytes a decode call
    must move (index keys, and the selected latent rows, queries, outputs and
    index rows of the attention)."""
    import numpy as np
    key_bytes = 2 if wl.k_dtype == "bf16" else 1
    row_bytes = 1152 if wl.kv_dtype == "bf16" else 656
    u = dict(idx_flops=0.0, attn_flops=0.0, score_bytes=0.0, attn_bytes=0.0, tokens=0)
    for c, _ in calls:
        qlen = [1] * len(c.ctx_len) if c.cu_q is None else list(np.diff(c.cu_q))
        for ctx, ql in zip(c.ctx_len, qlen):
            ts = np.arange(int(ctx) - int(ql), int(ctx)).astype(np.float64)
            sel = np.minimum(wl.top_k, ts + 1)
            u["idx_flops"] += 2.0 * wl.H_I * wl.d_I * float((ts + 1).sum())
            u["attn_flops"] += 2176.0 * wl.H * float(sel.sum())
            u["score_bytes"] += float((ts + 1).sum()) * wl.d_I * key_bytes + ql * wl.H_I * (wl.d_I * 2 + 4)
            u["attn_bytes"] += float(sel.sum()) * row_bytes + ql * (wl.H * (576 * 2 + 512 * 4 + 4) + wl.top_k * 4)
        u["tokens"] += c.num_tokens
    return u


def pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def event_pairs(n):
    import torch
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in pairs:          # create the underlying HIP events before handing them over
        a.record()
        b.record()
    return pairs


KERNEL_NAMES = {0: "score", 1: "topk", 2: "attn", 3: "combine"}


def timed_steps(lib, wl, inp, calls, bufs, scale, steps, flush, bracket=True):
    """`steps` steps (every call of the workload), each after a cache flush.
    With `bracket`, each step is bracketed by device synchronisations and
    its flush runs before the opening one, outside the bracket; without it
    (steps of a fraction of a millisecond, whose launches would then show
    as gaps) flushes and steps are queued back to back and the wall clock
    spans the whole region.  Returns per-step GPU milliseconds (events
    around the step on the stream), the wall-clock seconds of the timed
    steps, and per-kernel launch microseconds summed per step from the
    events the library records around every launch of each kernel."""
    import torch
    # the split merge runs only in calls whose index lists are split (those
    # need an attention workspace); its timer is armed for those calls only
    merges = [lib.sparse_mla_attn_workspace(s, wl.H, wl.top_k) > 0 for _, s in calls]
    step_ev = event_pairs(steps)
    kev = {k: [event_pairs(len(calls)) for _ in range(steps)] for k in KERNEL_NAMES}
    wall = 0.0
    torch.cuda.synchronize()
    region0 = time.perf_counter()
    for i in range(steps):
        flush()
        if bracket:
            torch.cuda.synchronize()
            wall0 = time.perf_counter()
        step_ev[i][0].record()
        for j, (c, s) in enumerate(calls):
            for k in KERNEL_NAMES:
                if k != lib.IDX_KERNEL_COMBINE or merges[j]:
                    lib.idx_timer_arm(k, kev[k][i][j][0], kev[k][i][j][1])
            run_call(lib, wl, inp, c, s, bufs, scale)
        step_ev[i][1].record()
        if bracket:
            torch.cuda.synchronize()
            wall += time.perf_counter() - wall0
    torch.cuda.synchronize()
    if not bracket:
        wall = time.perf_counter() - region0
    ms = [a.elapsed_time(b) for a, b in step_ev]
    kern = {}
    for k, name in KERNEL_NAMES.items():
        kern[name] = [sum(kev[k][i][j][0].elapsed_time(kev[k][i][j][1]) * 1e3
                          for j in range(len(calls)) if k != lib.IDX_KERNEL_COMBINE or merges[j])
                      for i in range(steps)]
    # (a prefill call whose score kernel selects records its Top-K pair back
    # to back: about zero)
    return ms, wall, kern


def measure_config(n, steps, warmup, flush, dev):
    """One workload: per-step median / p10 / p90 and per-kernel medians."""
    import numpy as np
    import torch
    import indexer_selected_sparse_idx_amd as lib
    from workloads import config, generate
    wl = config(n)
    inp = generate(wl, dev)
    calls, bufs = prepared_calls(wl, inp, dev)
    scale = 1.0 / math.sqrt(576.0)
    for _ in range(warmup):
        for c, s in calls:
            run_call(lib, wl, inp, c, s, bufs, scale)
    torch.cuda.synchronize()
    ms, wall, kern = timed_steps(lib, wl, inp, calls, bufs, scale, steps, flush, bracket=False)
    u = workload_units(wl, calls)
    med = pct(ms, 50)
    km = {k: float(np.median(v)) for k, v in kern.items()}
    res = dict(workload=wl.name, tokens=u["tokens"], steps=steps, median_ms=med, p10_ms=pct(ms, 10),
               p90_ms=pct(ms, 90), tokens_per_s=u["tokens"] / (med * 1e-3), kernels_median_us=km)
    attn_us = km["attn"] + km["combine"]
    if all(c.is_decode for c, _ in calls):
        res["score_hbm_frac"] = u["score_bytes"] / (km["score"] * 1e-6) / 1e9 / HBM_PEAK_GBS
        res["attention_hbm_frac"] = u["attn_bytes"] / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBS
        res["attention_algorithmic_bytes"] = u["attn_bytes"]
    res["indexer_mfma_frac"] = u["idx_flops"] / (km["score"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS
    res["attention_mfma_frac"] = u["attn_flops"] / (attn_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS
    del inp, calls, bufs
    torch.cuda.empty_cache()
    return res


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return model, os.cpu_count(), avail


def cpu_baseline_long_prefill(inp, rows_per_chunk=8, min_seconds=10.0):
    """The oracle, on one thread, on a seeded sample of the long prefill's
    rows, extrapolated to the whole step.  Per chunk: the chunk's keys are
    decoded once (as the oracle's batch driver does), then each sampled row
    is scored, selected and attended with the oracle's single-row functions.
    The full step's time is estimated with the cost model of the work: per
    chunk, decode time + sum over its rows of (t + 1) x (the chunk's
    measured indexer seconds per position) + min(K, t + 1) x (its attention
    seconds per selected row)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import torch
    import oracle
    from oracle import reference as R

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    wl = inp.wl
    K = wl.top_k
    scale = 1.0 / math.sqrt(576.0)
    k_bits = bits(inp.k_idx)
    kv_bits = bits(inp.kv)
    model, ncpu, avail = cpu_info()
    while True:
        rng = np.random.default_rng(3)
        est = 0.0
        spent = 0.0
        nrows = 0
        with threadpool_limits(limits=1):
            for call in inp.calls:
                ctx = int(call.ctx_len[0])
                T = call.num_tokens
                t_first = ctx - T
                pick = sorted({0, T - 1} | set(int(x) for x in rng.choice(T, size=rows_per_chunk - 2, replace=False)))
                g = [call.tok_lo + i for i in pick]
                q_idx = bits(inp.q_idx[g])
                q = bits(inp.q[g])
                w = inp.head_w[g].cpu().numpy().astype(np.float64)
                t0 = time.perf_counter()
                keys = R.decode_rows(k_bits, "bf16", np.arange(ctx))
                t_dec = time.perf_counter() - t0
                t_idx = t_att = 0.0
                pos_sum = sel_sum = 0.0
                for r, i in enumerate(pick):
                    t = t_first + i
                    a = time.perf_counter()
                    sc = oracle.indexer_scores(oracle.bf16_bits_to_f64(q_idx[r]), keys[:t + 1], w[r])
                    idx = oracle.topk_select(sc, K)
                    b = time.perf_counter()
                    sel = idx[idx >= 0].astype(np.int64)
                    rows = R.decode_rows(kv_bits, "bf16", sel)
                    oracle.sparse_attention(oracle.bf16_bits_to_f64(q[r]), rows, scale)
                    c = time.perf_counter()
                    t_idx += b - a
                    t_att += c - b
                    pos_sum += t + 1
                    sel_sum += min(K, t + 1)
                ts = np.arange(t_first, ctx, dtype=np.float64)
                est += t_dec + t_idx * (ts + 1).sum() / pos_sum + t_att * np.minimum(K, ts + 1).sum() / sel_sum
                spent += t_dec + t_idx + t_att
                nrows += len(pick)
        if spent >= min_seconds or rows_per_chunk >= 64:
            break
        # one more pass, sized from this one to about min_seconds
        rows_per_chunk = min(64, int(math.ceil(rows_per_chunk * 1.1 * min_seconds / max(spent, 1e-3))))
    tokens = sum(c.num_tokens for c in inp.calls)
    return dict(value=tokens / est, unit="tokens/s", cores=1, kind="oracle",
                sample="%d seeded rows (%d per 4096-token chunk, each chunk's first and last included) of the "
                       "long prefill, indexer + Top-K + attention with the oracle's functions on 1 thread "
                       "(BLAS pinned to 1): %.1f s measured in the final pass; the whole 65,536-token step extrapolated to %.0f s "
                       "with the cost model (indexer ~ t + 1 per row, attention ~ min(K, t + 1)); host %s, "
                       "%d logical CPUs (%d available to this process)"
                       % (nrows, rows_per_chunk, spent, est, model, ncpu, avail),
                cpu_model=model, nproc=ncpu, extrapolated=True, measured_s=spent, estimated_step_s=est)


def attn_source_digest():
    """Digest of what the attention kernels are built from: attn.hip,
    common.h, and the attention parameter block and tile size of
    kernels.h (the rest of kernels.h belongs to other kernels)."""
    csrc = os.path.join(ROOT, "indexer_selected_sparse_idx_amd", "csrc")
    h = hashlib.sha256()
    for name in ("attn.hip", "common.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    kh = open(os.path.join(csrc, "kernels.h")).read()
    a = kh.index("struct AttnParams {")
    h.update(kh[a:kh.index("};", a) + 2].encode())
    h.update(re.search(r"constexpr int ATTN_TILE = \d+;", kh).group(0).encode())
    return h.hexdigest()[:16]


def attn_counter_traffic():
    """HBM bytes per launch of the prefill attention kernel over the long
    prefill, from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source."""
    path = os.path.join(PROFILE_DIR, "attn_long_prefill_65536_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_digest") != attn_source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(requests would shard across GPUs with no exchange; see DESIGN.md). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import indexer_selected_sparse_idx_amd as lib
    from workloads import config, generate

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        src = torch.full((1 << 30,), 7, dtype=torch.uint8, device="cuda:0")
        dst = torch.zeros_like(src)
        torch.cuda.synchronize()
        for i in range(3):
            dst.copy_(src)
            torch.cuda.synchronize()
            print("copy %d: %d bytes read, %d bytes written" % (i, src.numel(), dst.numel()), flush=True)
        return
    lib.lib()
    dev = torch.device("cuda:0")
    if args.workload:
        measure_workload(args.workload, args.steps, args.warmup)
        return
    if args.kv_write:
        measure_kv_write(args.steps, args.warmup)
        return
    if args.mxfp8:
        measure_mxfp8(args.steps, args.warmup)
        return
    if args.multi_token:
        measure_multi_token(args.steps, args.warmup)
        return

    # ---- headline: the long prefill, 65,536 positions in 16 chunks of 4,096 ----
    wl = config(3)
    inp = generate(wl, dev)
    calls, bufs = prepared_calls(wl, inp, dev)
    scale = 1.0 / math.sqrt(576.0)
    torch.cuda.synchronize()
    if args.profile_steps:
        for i in range(args.profile_steps):
            for c, s in calls:
                run_call(lib, wl, inp, c, s, bufs, scale)
            torch.cuda.synchronize()
            print("profile step %d done" % i, flush=True)
        return
    flush = Flusher(dev)
    for _ in range(args.warmup):
        for c, s in calls:
            run_call(lib, wl, inp, c, s, bufs, scale)
    torch.cuda.synchronize()
    K = args.steps
    ms, wall, kern = timed_steps(lib, wl, inp, calls, bufs, scale, K, flush)
    u = workload_units(wl, calls)
    ms_per_step = wall * 1e3 / K             # the K step brackets / K (flushes outside them)
    attn_us = float(np.mean(kern["attn"]))   # summed over the 16 launches of a step
    score_us = float(np.mean(kern["score"]))
    n_launch = len(calls)
    attn_tflops = u["attn_flops"] / (attn_us * 1e-6) / 1e12
    score_tflops = u["idx_flops"] / (score_us * 1e-6) / 1e12
    print("headline: %.2f ms per step (median %.2f), attention %.2f ms, indexer %.2f ms"
          % (ms_per_step, pct(ms, 50), attn_us / 1e3, score_us / 1e3), file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_long_prefill(inp)
    del inp, calls, bufs
    torch.cuda.empty_cache()

    # ---- the other workloads (secondary figures) ---------------------------------
    others = {}
    names = {1: "tiny_prefill", 2: "decode_batch", 4: "fp8_decode", 5: "mixed_paged"}
    for n in (1, 2, 4, 5):
        nsteps = 20 if n in (1, 2, 4) else 5
        others[names[n]] = measure_config(n, nsteps, 3, flush, dev)
        print("%s: %s" % (names[n], json.dumps(others[names[n]])), file=sys.stderr, flush=True)

    # reference: a plain 1 GiB device-to-device copy (read + write bytes per second)
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    torch.cuda.synchronize()
    ca, cb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ca.record()
    for _ in range(5):
        cdst.copy_(csrc)
    cb.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * (1 << 30) * 5 / (ca.elapsed_time(cb) * 1e-3) / 1e9
    del csrc, cdst, flush

    tokens = u["tokens"]
    result = {
        "metric": "fused indexer+sparse-attn tokens/sec; achieved HBM GB/s & MFMA % of peak",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "long prefill: one causal sequence of 65,536 positions in 16 query chunks of 4,096 "
                               "(one idx_sparse_attn_prefill call per chunk), bf16 caches, indexer 64 heads "
                               "d_I=128, Top-K 2048, 128 attention heads, latent 576",
                   "seq_len": 65536, "chunk": 4096, "H_I": wl.H_I, "d_I": wl.d_I, "top_k": wl.top_k, "H": wl.H,
                   "parallelism": "none (1 GPU)"},
        "step_ms": {"median": pct(ms, 50), "p10": pct(ms, 10), "p90": pct(ms, 90),
                    "note": "GPU events around each step, after a 1 GiB cache-flushing write; ms_per_step is "
                            "the wall time of the K step brackets / K (each step between two device "
                            "synchronisations, its cache flush before the first)"},
        "roofline": {"bound": "mfma", "kernel": "sparse latent attention (prefill, bf16)",
                     "achieved": attn_tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / BF16_PEAK_TFLOPS, "traffic": attn_counter_traffic(),
                     "algorithmic_flops_per_launch": u["attn_flops"] / n_launch,
                     "avg_launch_us": attn_us / n_launch, "launches_per_step": n_launch},
        "kernels_per_step_us": {k: float(np.mean(v)) for k, v in kern.items()},
        "secondary": {
            "indexer_prefill": {"ms_per_step": score_us / 1e3, "tflops": score_tflops,
                                "mfma_frac": score_tflops / BF16_PEAK_TFLOPS,
                                "note": "score kernel with its in-kernel Top-K, 16 launches per step"},
            "target_fractions": {
                "decode_attention_hbm_decode_batch": others["decode_batch"]["attention_hbm_frac"],
                "decode_attention_hbm_fp8_decode": others["fp8_decode"]["attention_hbm_frac"],
                "indexer_prefill_mfma_long_prefill": score_tflops / BF16_PEAK_TFLOPS},
            "workloads": others,
            "copy_kernel_gbs": copy_gbs,
            "wall_s_timed_region": wall,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
