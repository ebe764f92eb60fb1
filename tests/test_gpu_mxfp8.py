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


def _block_ranged_queries(g, T, H_I):
    """Integer queries whose range differs per head and block of 32 (63,
    20, 7 or 2): the blocks' shared exponents differ, most values fall
    between E4M3 codes after the division by 2^e (q / 2^e = 8 q, 16 q, ...)
    and round, and blocks whose largest |q| / 2^e exceeds 448 saturate."""
    ranges = torch.tensor([63.0, 20.0, 7.0, 2.0], device="cuda")
    r = ranges[torch.randint(0, 4, (T, H_I, 4), generator=g, device="cuda")].repeat_interleave(32, dim=2)
    u = torch.rand((T, H_I, 128), generator=g, device="cuda")
    return torch.floor(u * (2.0 * r + 1.0)) - r


def _run(ctx, H_I, K, seed, paged=False, qlen=None, k_range=8, rounding=False):
    """One idx_score_topk call over sequences with context lengths ctx and
    qlen[b] query tokens each (the last qlen[b] positions; default 1: a
    decode batch), checked token by token against the oracle.

    rounding=False: queries are integers in [-4, 4] times a power of two per
    head and block (exactly representable after MX quantisation).
    rounding=True: block-ranged integer queries (see _block_ranged_queries)
    that the MX rule must round and saturate, with head weights in {1/2, 1};
    callers keep k_range and H_I small enough that every fp32 partial sum
    stays exact (quantised queries are integers of at most 63, keys
    multiples of 1/2 of at most 2 k_range)."""
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
    if rounding:
        q_idx = _block_ranged_queries(g, T, H_I).to(torch.bfloat16)
        head_w = torch.pow(2.0, -torch.randint(0, 2, (T, H_I), generator=g, device="cuda").float())
    else:
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
    if rounding:
        # the case is what it claims: the quantiser rounds and saturates
        rounded = saturated = 0
        for tok in range(T):
            qh = _q_oracle(qf[tok])
            rounded += int(np.sum(qh != qf[tok]))
            blocks = np.abs(qf[tok]).reshape(H_I, 4, 32)
            amax = blocks.max(axis=2, keepdims=True)
            e = np.frexp(np.where(amax > 0, amax, 1.0))[1] - 9     # floor(log2 amax) - 8
            saturated += int(np.sum(blocks / 2.0 ** e > 448.0))
        U.log("mxfp8 rounding case: %d query values rounded, %d saturated (of %d)"
              % (rounded, saturated, qf.size))
        assert rounded > qf.size // 10 and saturated > 0
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


def test_mxfp8_query_rounding_and_saturation_64_heads():
    # queries that round (values between E4M3 codes after the division by
    # the block's power of two) and saturate (|q| / 2^e in (448, 512)),
    # keys in [-2, 2] per block exponent, 64 heads: every partial sum is a
    # multiple of 1/4 below 2^21, so the scores are exact in fp32
    _run([5000, 7777, 130, 2049], 64, 512, 78, k_range=1, rounding=True)


def test_mxfp8_query_rounding_and_saturation_prefill_paged():
    # the same query rule through a paged prefill call, 16 heads (one MFMA
    # row tile), keys in [-4, 4] per block exponent
    _run([3000, 900], 16, 256, 79, paged=True, qlen=[40, 9], k_range=2, rounding=True)
