#!/usr/bin/env python3
"""Throughput of the fused indexer + sparse latent attention hot path.

Workload: the decode batch of 64 requests, one new token each, 32768 cached
positions per request (contiguous latent cache of 576 bf16 per row and
index-key cache of 128 bf16 per row), 64 indexer heads, Top-K 2048,
128 attention heads.  One step is one idx_sparse_attn_decode call over the
batch: score every cached position, select the Top-K, gather the selected
latent rows and attend.  Inputs are seeded synthetic data resident in HBM
before timing starts.

Prints one JSON line.  `roofline` describes the dominant kernel (the
indexer score, HBM-bound): its algorithmic bytes per launch over its average
launch time, measured with HIP events the library records on the launch
stream during the timed steps.  `cpu_baseline` is the CPU oracle timed on a
bounded sample of the same workload (one thread).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import hashlib
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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-sample", type=int, default=64, help="decode tokens timed on the CPU oracle")
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


def algorithmic_units(wl, ctx, T):
    """Bytes / flops the method must move or compute (per step)."""
    H_I, d_I, H, K = wl.H_I, wl.d_I, wl.H, wl.top_k
    key_bytes = 2 if wl.k_dtype == "bf16" else 1
    row_bytes = 1152 if wl.kv_dtype == "bf16" else 656
    n_cand = ctx                                   # t + 1 = ctx for a decode token
    sel = min(K, n_cand)
    score_bytes = T * (n_cand * d_I * key_bytes + H_I * d_I * 2 + H_I * 4)
    score_flops = T * 2 * H_I * d_I * n_cand
    topk_bytes = T * K * 4
    attn_bytes = T * (sel * row_bytes + H * 576 * 2 + H * 512 * 4 + H * 4 + K * 4)
    attn_flops = T * 2176 * H * sel
    return dict(score_bytes=score_bytes, score_flops=score_flops, topk_bytes=topk_bytes,
                attn_bytes=attn_bytes, attn_flops=attn_flops)


def score_source_digest():
    h = hashlib.sha256()
    for name in ("score.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "indexer_selected_sparse_idx_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per launch of the score kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    path = os.path.join(PROFILE_DIR, "score_kernel_decode_b64_ctx32768_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_digest") != score_source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, call, n_tokens, min_seconds=10.0):
    """Time the oracle (indexer + Top-K + attention) on the first n_tokens
    decode tokens, one BLAS thread, inputs already on the host."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from oracle import reference as R
    import torch

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    n_tokens = max(1, min(n_tokens, call.num_tokens))
    seq_ids = list(range(n_tokens))
    stride = inp.seq_stride
    k_host = bits(inp.k_idx[: n_tokens * stride])
    kv_host = bits(inp.kv[: n_tokens * stride])
    q_idx = bits(inp.q_idx[:n_tokens])
    q = bits(inp.q[:n_tokens])
    w = inp.head_w[:n_tokens].cpu().numpy()
    seqs = R.Seqs(ctx_len=call.ctx_len[:n_tokens].astype(np.int64), seq_stride=stride)
    with threadpool_limits(limits=1):
        reps, dt = 0, 0.0
        while reps == 0 or (dt < min_seconds and reps < 50):   # bounded: about min_seconds of CPU work
            t0 = time.perf_counter()
            idx = oracle.score_topk(seqs, q_idx, k_host, "bf16", w, inp.wl.top_k)
            oracle.attention(seqs, q, kv_host, "bf16", idx, 1.0 / math.sqrt(576.0))
            dt += time.perf_counter() - t0
            reps += 1
    return dict(value=reps * n_tokens / dt, unit="tokens/s", cores=1, kind="oracle",
                sample="%d pass(es) over %d of the %d decode tokens of one step (each token: indexer over %d "
                       "positions, Top-%d, attention over %d rows x %d heads); %.1f s on 1 thread"
                       % (reps, n_tokens, call.num_tokens, int(call.ctx_len[0]), inp.wl.top_k, inp.wl.top_k,
                          inp.wl.H, dt))


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
    # tokens (MXFP8 keys: every token streams its causal range; bf16 keys: the
    # prefill kernel, key tiles shared by 8 tokens)
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
    wl = config(2)
    inp = generate(wl, dev)
    call = inp.calls[0]
    T = call.num_tokens
    ctx_t = torch.from_numpy(call.ctx_len.astype(np.int32)).to(dev)
    seqs = lib.Seqs(ctx_t, None, max_q_len=1, max_ctx_len=int(call.ctx_len.max()), seq_stride=inp.seq_stride)
    out = torch.empty((T, wl.H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
    ws = torch.empty(lib.idx_sparse_attn_workspace(seqs, wl.H_I, wl.d_I, wl.H, wl.top_k), dtype=torch.uint8,
                     device=dev)
    scale = 1.0 / math.sqrt(576.0)

    def step():
        lib.idx_sparse_attn_decode(seqs, inp.q_idx, inp.k_idx, inp.head_w, wl.top_k, inp.q, inp.kv, scale,
                                   out=out, lse=lse, out_idx=idx, ws=ws)

    torch.cuda.synchronize()
    if args.profile_steps:
        for i in range(args.profile_steps):
            step()
            torch.cuda.synchronize()
            print("profile step %d done" % i, flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    names = {lib.IDX_KERNEL_SCORE: "score", lib.IDX_KERNEL_TOPK: "topk", lib.IDX_KERNEL_ATTN: "attn",
             lib.IDX_KERNEL_COMBINE: "combine"}

    def event_pairs(n):
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in pairs:          # create the underlying HIP events before handing them over
            a.record()
            b.record()
        return pairs

    # timed region: K steps; the library records an event pair around every
    # launch of the dominant (score) kernel on its launch stream
    score_ev = event_pairs(K)
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(K):
        lib.idx_timer_arm(lib.IDX_KERNEL_SCORE, score_ev[i][0], score_ev[i][1])
        step()
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = t_start.elapsed_time(t_stop)
    ms_per_step = gpu_ms / K

    # per-kernel breakdown in a separate (untimed) pass with every kernel armed
    KB = min(K, 20)
    ev = {k: event_pairs(KB) for k in names}
    torch.cuda.synchronize()
    for i in range(KB):
        for k, pairs in ev.items():
            lib.idx_timer_arm(k, pairs[i][0], pairs[i][1])
        step()
    torch.cuda.synchronize()
    kern_ms = {names[k]: sum(a.elapsed_time(b) for a, b in pairs) / KB for k, pairs in ev.items()}
    score_ms = sum(a.elapsed_time(b) for a, b in score_ev) / K

    # reference: a plain 1 GiB device-to-device copy on the same GPU, after the
    # timed region (read + write bytes per second)
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
    del csrc, cdst

    u = algorithmic_units(wl, int(call.ctx_len[0]), T)
    score_us = score_ms * 1e3
    achieved = u["score_bytes"] / (score_ms * 1e-3) / 1e9
    traffic = counter_traffic()
    attn_s = (kern_ms["attn"] + kern_ms["combine"]) * 1e-3

    result = {
        "metric": "fused indexer+sparse-attn tokens/sec; achieved HBM GB/s & MFMA % of peak",
        "value": T / (ms_per_step * 1e-3),
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
        "config": {"workload": "decode batch: 64 requests x 1 token, 32768-position contiguous bf16 caches, "
                               "indexer 64 heads d_I=128, Top-K 2048, 128 attention heads, latent 576",
                   "batch": T, "ctx": int(call.ctx_len[0]), "H_I": wl.H_I, "d_I": wl.d_I, "top_k": wl.top_k,
                   "H": wl.H, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "indexer score", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": u["score_bytes"], "avg_launch_us": score_us},
        "kernels_avg_us": {k: v * 1e3 for k, v in kern_ms.items()},
        "secondary": {
            "attention_hbm_gbs": u["attn_bytes"] / attn_s / 1e9,
            "attention_hbm_frac": u["attn_bytes"] / attn_s / 1e9 / HBM_PEAK_GBS,
            "attention_mfma_frac": u["attn_flops"] / attn_s / 1e12 / BF16_PEAK_TFLOPS,
            "score_mfma_frac": u["score_flops"] / (score_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "step_hbm_gbs": (u["score_bytes"] + u["topk_bytes"] + u["attn_bytes"]) / (ms_per_step * 1e-3) / 1e9,
            "wall_s_timed_region": wall,
            "copy_kernel_gbs": copy_gbs,
            "score_frac_of_copy": achieved / copy_gbs,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, call, args.cpu_sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
