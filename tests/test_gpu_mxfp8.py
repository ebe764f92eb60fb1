"""GPU parity of the MXFP8 indexer (IDX_MXFP8 keys) through the C
ABI against the oracle.

Keys are MXFP8 codes whose blocks take different E8M0 exponents
(workloads.gen.mxfp8_keys); queries are integers times a power of two that
varies per head and block of 32, so both operands' block scales take part
and a scale applied to the wrong block or head changes the scores.  The
oracle quantises the query with the MX rule (oracle/writer.py), decodes the
keys exactly and scores in float64; with these values every fp32 partial
sum is exact, so the Top-K sets must match bit for bit.
"""
import numpy as np
import pytest
import torch

import indexer_selected_sparse_idx_amd as lib
import oracle
from oracle import formats as F
from oracle import writer as W
from workloads import gen

import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.lib()


def _q_oracle(q):
    """MX-quantise then dequantise queries [H_I, 128] per head and block of 32."""
    out = np.zeros_like(q)
    for h in range(q.shape[0]):
        for b in range(4):
            codes, e8 = W.mx_block_quantize(q[h, 32 * b:32 * (b + 1)])
            out[h, 32 * b:32 * (b + 1)] = F.E4M3_TABLE[codes] * 2.0 ** (e8 - 127)
    return out


def _run(ctx, H_I, K, seed, paged=False, qlen=None, k_range=8):
    """One idx_score_topk call over sequences with context lengths ctx and
    qlen[b] query tokens each (the last qlen[b] positions; default 1: a
    decode batch), checked token by token against the oracle."""
    B = len(ctx)
    qlen = [1] * B if qlen is None else list(qlen)
    T = sum(qlen)
    g = torch.Generator(device="cuda").manual_seed(seed)
    stride = max(ctx)
    if paged:
        page = 64
        npg = [-(-c // page) for c in ctx]
        perm = torch.randperm(sum(npg), generator=g, device="cuda").to(torch.int32)
        bt = torch.full((B, max(npg)), 0, dtype=torch.int32, device="cuda")
        o = 0
        for b in range(B):
            bt[b, :npg[b]] = perm[o:o + npg[b]]
            o += npg[b]
        keys, exps = gen.mxfp8_keys(g, sum(npg) * page, "cuda", k_range=k_range)
    else:
        keys, exps = gen.mxfp8_keys(g, B * stride, "cuda", k_range=k_range)
    qi = torch.randint(-4, 5, (T, H_I, 128), generator=g, device="cuda").float()
    shift = torch.randint(0, 2, (T, H_I, 4), generator=g, device="cuda").float()
    q_idx = (qi * torch.pow(2.0, shift).repeat_interleave(32, dim=2)).to(torch.bfloat16)
    head_w = torch.pow(2.0, -torch.randint(0, 4, (T, H_I), generator=g, device="cuda").float())
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    cu_h = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    cu = None if max(qlen) == 1 else torch.from_numpy(cu_h).to("cuda")
    if paged:
        s = lib.Seqs(ctx_t, cu, max_q_len=max(qlen), max_ctx_len=max(ctx), num_tokens=T, block_table=bt,
                     page_size=64)
    else:
        s = lib.Seqs(ctx_t, cu, max_q_len=max(qlen), max_ctx_len=max(ctx), num_tokens=T, seq_stride=stride)
    idx = lib.idx_score_topk(s, q_idx, keys, head_w, K, k_scale=exps)
    torch.cuda.synchronize()
    kf = F.mxfp8_to_f64(keys.cpu().numpy(), exps.cpu().numpy())
    qf = oracle.bf16_bits_to_f64(U.bits16(q_idx))
    w = head_w.cpu().numpy().astype(np.float64)
    bt_h = bt.cpu().numpy() if paged else None
    want = []
    for b in range(B):
        pos = np.arange(ctx[b])
        rows = (bt_h[b, pos // 64].astype(np.int64) * 64 + pos % 64) if paged else b * stride + pos
        for i in range(qlen[b]):
            tok = cu_h[b] + i
            t = ctx[b] - qlen[b] + i
            sc = oracle.indexer_scores(_q_oracle(qf[tok]), kf[rows[:t + 1]], w[tok])
            want.append(oracle.topk_select(sc, K))
    U.check_indices(idx.cpu().numpy(), np.stack(want), "mxfp8")
    return exps


def test_mxfp8_decode_indexer_contiguous():
    exps = _run([5000, 7777, 130, 2049, 9000, 3000], 64, 512, 70)
    e8 = exps.cpu().numpy()
    assert len(np.unique(e8)) == 3                             # the exponents do vary


def test_mxfp8_decode_indexer_paged_fewer_heads_small_k():
    _run([4100, 64, 1, 1500], 40, 100, 71, paged=True)


def test_mxfp8_fused_decode_matches_separate_calls():
    """The fused decode entry point with MXFP8 keys selects the rows the
    indexer entry point selects and attends over them like the attention
    entry point (same kernels, so equal bit for bit)."""
    ctx = [3000, 700, 1]
    B, H_I, K, H = len(ctx), 64, 512, 16
    g = torch.Generator(device="cuda").manual_seed(72)
    stride = max(ctx)
    keys, exps = gen.mxfp8_keys(g, B * stride, "cuda")
    q_idx = torch.randint(-4, 5, (B, H_I, 128), generator=g, device="cuda").to(torch.bfloat16)
    head_w = torch.pow(2.0, -torch.randint(0, 4, (B, H_I), generator=g, device="cuda").float())
    q = torch.randn((B, H, 576), generator=g, device="cuda").to(torch.bfloat16)
    kv = torch.randn((B * stride, 576), generator=g, device="cuda").to(torch.bfloat16)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    s = lib.Seqs(ctx_t, None, max_q_len=1, max_ctx_len=max(ctx), num_tokens=B, seq_stride=stride)
    idx = torch.empty((B, K), dtype=torch.int32, device="cuda")
    out, lse, idx = lib.idx_sparse_attn_decode(s, q_idx, keys, head_w, K, q, kv, U.SCALE, k_scale=exps,
                                               out_idx=idx)
    idx2 = lib.idx_score_topk(s, q_idx, keys, head_w, K, k_scale=exps)
    out2, lse2 = lib.sparse_mla_attn(s, q, kv, idx2, U.SCALE)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert int((idx[2] >= 0).sum()) == 1 and int((idx[1] >= 0).sum()) == K
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_mxfp8_prefill_chunks_contiguous():
    # chunks of 37 and 1 tokens and a whole-context chunk of 300 (rows with
    # t + 1 <= K and a ragged tail), contiguous cache
    _run([6000, 2500, 300], 64, 256, 73, qlen=[37, 1, 300])


def test_mxfp8_prefill_chunks_paged_fewer_heads():
    _run([5000, 130], 24, 512, 74, paged=True, qlen=[70, 130])


def test_mxfp8_largest_top_k_one_head_tile():
    # K = 2048 (the largest), 16 heads (one MFMA row tile); rows with
    # t + 1 = K, t + 1 = K + 1 and a single position
    _run([3000, 2048, 2049, 1], 16, 2048, 75)


def test_mxfp8_top_1_short_multi_token_rows():
    # K = 1; 3 and 5 query tokens (the second sequence's chunk is its whole
    # context), 8 heads
    _run([700, 5], 8, 1, 76, qlen=[3, 5])


def test_mxfp8_all_equal_scores_take_lowest_positions():
    # every code 0: all scores are 0, so each row takes its lowest positions
    _run([4000, 300, 2100], 64, 256, 77, k_range=0, qlen=[1, 2, 1])
