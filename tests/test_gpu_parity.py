"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Top-K index sets must match bit for bit (integer-valued indexer inputs make
the fp32 scores exact); attention must be within max-abs error <= tol * RMS
of the oracle output (tol 2e-2 for a bf16 cache, 6e-2 for an FP8 cache).
Sizes here keep the oracle to seconds while spanning several key blocks,
several attention tiles, ragged tails and every code path (decode/prefill,
bf16/e4m3 keys, bf16/FP8 latent rows, contiguous/paged caches).
"""
import numpy as np
import pytest
import torch

import workloads
from workloads import Workload, config, generate

import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import indexer_selected_sparse_idx_amd as lib
    lib.lib()
    torch.manual_seed(0)


def _parity_all(inp, tol, label):
    """Every token of every call of `inp`, through the fused entry points."""
    for ci, call in enumerate(inp.calls):
        U.log("%s call %d: %d tokens, ctx max %d" % (label, ci, call.num_tokens, int(call.ctx_len.max())))
        out, lse, idx = U.run_fused(inp, call)
        torch.cuda.synchronize()
        tokens = list(range(call.num_tokens))
        w_idx, w_out, w_lse = U.oracle_rows(inp, call, tokens)
        U.check_indices(idx.cpu().numpy(), w_idx, "%s call %d" % (label, ci))
        err = U.check_attention(out.cpu().numpy(), lse.cpu().numpy(), w_out, w_lse, tol,
                                "%s call %d" % (label, ci))
        U.log("  ok: attention err/RMS %.2e" % err)


def test_tiny_prefill_scaled():
    inp = generate(config(1, scale=1 / 8), "cuda")          # L = 256, K = 128, H = 8, H_I = 4
    _parity_all(inp, U.TOL_BF16, "tiny-prefill/8")


def test_decode_ragged_contexts():
    wl = Workload("decode ragged", [2000, 64, 1, 3001, 2048, 2049], [{"seqs": list(range(6)), "q_len": None}],
                  top_k=2048, seed=21)
    _parity_all(generate(wl, "cuda"), U.TOL_BF16, "decode-ragged")


def test_decode_small_topk():
    wl = Workload("decode K=100", [5000, 777, 130], [{"seqs": [0, 1, 2], "q_len": None}], top_k=100, seed=22)
    _parity_all(generate(wl, "cuda"), U.TOL_BF16, "decode-K100")


def test_chunked_prefill_scaled():
    inp = generate(config(3, scale=1 / 32), "cuda")          # L = 2048 in chunks of 128
    for call in inp.calls[::5] + [inp.calls[-1]]:
        sub = workloads.Inputs(inp.wl, [call], inp.q_idx, inp.head_w, inp.q, inp.k_idx, inp.k_scale,
                               inp.kv, inp.seq_stride, inp.block_table)
        _parity_all(sub, U.TOL_BF16, "long-prefill/32")


def test_prefill_small_topk_many_ties():
    # K = 64 over a 700-long causal sequence with keys in {-1, 0, 1}: heavy ties
    wl = Workload("prefill ties", [700], [{"seqs": [0], "q_len": [700]}], top_k=64, H_I=20, d_I=64,
                  H=20, k_range=1, q_range=1, seed=23)
    _parity_all(generate(wl, "cuda"), U.TOL_BF16, "prefill-ties")


def test_attention_three_waves_of_heads():
    # 65 to 96 attention heads run three waves of 32 heads per workgroup (at
    # 72 the third wave has 8 live heads); with FP8 rows each wave gathers
    # and dequantises rows of its own, 11, 11 and 10 of a 32-row tile.  bf16
    # and FP8 rows; decode rows split across workgroups, and a prefill chunk.
    for H in (72, 96):
        for kv_dtype, tol in (("bf16", U.TOL_BF16), ("fp8_656", U.TOL_FP8)):
            wl = Workload("H=%d %s" % (H, kv_dtype), [3000, 900, 2049, 1200],
                          [{"seqs": [0, 1, 2], "q_len": None}, {"seqs": [3], "q_len": [100]}],
                          H=H, top_k=512, kv_dtype=kv_dtype, seed=50 + H)
            _parity_all(generate(wl, "cuda"), tol, "H=%d %s" % (H, kv_dtype))


def test_fp8_decode_scaled():
    inp = generate(config(4, scale=1 / 32), "cuda")          # B = 4, ctx = 4096, e4m3 keys, FP8 rows
    _parity_all(inp, U.TOL_FP8, "fp8-decode/32")


def test_paged_mixed_scaled():
    inp = generate(config(5, scale=1 / 16), "cuda")          # paged, prefill + decode calls
    _parity_all(inp, U.TOL_BF16, "mixed-paged/16")


def test_multi_token_decode_rows_paged():
    # speculative verification: every request scores and attends 2 to 8 new
    # tokens at once (q_len > 1 through cu_q), over a paged cache, with
    # contexts on both sides of K and of the 64-position page
    ctx = [5000, 2100, 64, 130, 7777, 2049, 3000, 9000]
    q_len = [4, 8, 2, 3, 5, 8, 2, 7]
    wl = Workload("spec decode", ctx, [{"seqs": list(range(8)), "q_len": q_len}], top_k=2048, H=32,
                  paged=True, page_size=64, seed=33)
    _parity_all(generate(wl, "cuda"), U.TOL_BF16, "spec-decode")


def test_key_scale_and_d64():
    wl = Workload("k_scale", [900, 333], [{"seqs": [0, 1], "q_len": [40, 7]}], top_k=96, d_I=64, H_I=33,
                  H=48, k_scale=True, seed=24)
    _parity_all(generate(wl, "cuda"), U.TOL_BF16, "k_scale")


def test_prefill_e4m3_keys_small_pages_and_scales():
    # e4m3 index keys and FP8 latent rows in a prefill call, paged with 16-row
    # pages (several pages per key tile), per-row key scales, ragged q_len
    wl = Workload("prefill e4m3 paged", [1500, 600, 77], [{"seqs": [0, 1, 2], "q_len": [37, 300, 77]}],
                  top_k=256, k_dtype="e4m3", kv_dtype="fp8_656", paged=True, page_size=16, k_scale=True,
                  k_range=8, seed=29)
    _parity_all(generate(wl, "cuda"), U.TOL_FP8, "prefill e4m3 paged")


def test_multi_token_all_equal_scores_take_lowest_positions():
    # 5 query tokens: the multi-token score kernel and the decode-style Top-K
    wl = Workload("zeros", [3000], [{"seqs": [0], "q_len": [5]}], top_k=256, seed=25)
    inp = generate(wl, "cuda")
    inp.q_idx.zero_()                                          # every score is exactly 0
    call = inp.calls[0]
    out, lse, idx = U.run_fused(inp, call)
    got = np.sort(idx.cpu().numpy(), axis=1)
    assert np.array_equal(got, np.tile(np.arange(256, dtype=np.int32), (5, 1)))


def test_prefill_all_equal_scores_overflow_the_wave_list():
    # 16 query tokens (the prefill kernel, which selects on its own) over
    # about 5000 equal scores: the threshold key's 22-bit prefix holds every
    # key of a row, more than the 2048-word LDS list of a wave (d_I = 128),
    # so the selection takes its two-pass form over the compacted pairs
    wl = Workload("zeros prefill", [5000], [{"seqs": [0], "q_len": [16]}], top_k=256, H=16, seed=35)
    inp = generate(wl, "cuda")
    inp.q_idx.zero_()
    call = inp.calls[0]
    out, lse, idx = U.run_fused(inp, call)
    got = np.sort(idx.cpu().numpy(), axis=1)
    assert np.array_equal(got, np.tile(np.arange(256, dtype=np.int32), (16, 1)))
    w_idx, w_out, w_lse = U.oracle_rows(inp, call, list(range(16)))
    U.check_indices(idx.cpu().numpy(), w_idx, "zeros prefill")
    U.check_attention(out.cpu().numpy(), lse.cpu().numpy(), w_out, w_lse, U.TOL_BF16, "zeros prefill")


def _three_level_keys(inp, b, n, n_top, n_mid, rng):
    """Index keys of sequence b that give scores of three values only: every
    head's query is the unit vector on dimension 0 and every head weight is
    1, so S = H_I * ReLU(k[0]); k[0] is 2 on n_top positions, 1 on n_mid and
    0 elsewhere (the other dimensions do not count)."""
    k0 = np.zeros(n, np.float32)
    perm = rng.permutation(n)
    k0[perm[:n_top]] = 2.0
    k0[perm[n_top:n_top + n_mid]] = 1.0
    rows = torch.arange(b * inp.seq_stride, b * inp.seq_stride + n, device="cuda")
    inp.k_idx[rows, 0] = torch.from_numpy(k0).to("cuda").to(torch.bfloat16)


@pytest.mark.parametrize("d_I", [128, 64])
def test_prefill_threshold_ties_overflow_the_wave_list(d_I):
    # prefill kernel (20 query tokens); scores take three values, the K-th
    # largest is the middle one and about 3000 keys share it: more than the
    # wave's LDS list (2048 words at d_I = 128, 1024 at d_I = 64), so the
    # selection's two-pass form picks the 150 keys above the threshold and
    # the lowest positions among the ties
    n = 9000
    wl = Workload("ties prefill", [n], [{"seqs": [0], "q_len": [20]}], top_k=512, H=16, d_I=d_I, seed=36)
    inp = generate(wl, "cuda")
    inp.q_idx.zero_()
    inp.q_idx[:, :, 0] = 1.0
    inp.head_w.fill_(1.0)
    _three_level_keys(inp, 0, n, 150, 3000, np.random.default_rng(36))
    _parity_all(inp, U.TOL_BF16, "ties prefill d_I=%d" % d_I)


def test_prefill_bound_jumps_beyond_the_bucket_window():
    # prefill kernel (16 query tokens over 6144 keys): the keys' scale grows
    # by 2^17 every 1024 positions (scores H_I * k[0], k[0] = (1 + s % 7) *
    # 2^(17 (s // 1024)), exact in fp32), so at each refresh of the running
    # bound the bucket of the K-th largest key moves up by about 68 buckets:
    # more than the 64-bucket window above the last one, and the refresh
    # falls back to a pick over the whole histogram; ties (7 values per
    # block) go to the lowest positions
    n = 6144
    wl = Workload("bound jumps", [n], [{"seqs": [0], "q_len": [16]}], top_k=256, H_I=16, H=16, seed=41)
    inp = generate(wl, "cuda")
    inp.q_idx.zero_()
    inp.q_idx[:, :, 0] = 1.0
    inp.head_w.fill_(1.0)
    s = np.arange(n)
    k0 = (1.0 + (s % 7)) * np.exp2(17.0 * (s // 1024))
    rows = torch.arange(0, n, device="cuda")
    inp.k_idx[rows, 0] = torch.from_numpy(k0.astype(np.float32)).to("cuda").to(torch.bfloat16)
    _parity_all(inp, U.TOL_BF16, "bound jumps")


def test_prefill_block_table_beyond_the_staged_pages():
    # pages of 1 position: 5000 pages for the longest sequence, more than the
    # 4096 block-table entries the prefill kernel stages, so the call takes
    # the multi-token score kernel and the decode-style Top-K
    wl = Workload("pages > 4096", [5000, 300], [{"seqs": [0, 1], "q_len": [12, 40]}], top_k=256, H=32,
                  paged=True, page_size=1, seed=37)
    _parity_all(generate(wl, "cuda"), U.TOL_BF16, "pages > 4096")


def test_prefill_rows_longer_than_the_packed_positions():
    # rows of more than 2^22 positions: the prefill selection cannot pack a
    # position beside the key's low bits in its LDS list and takes the
    # two-pass form over the compacted pairs
    n = (1 << 22) + 3000
    wl = Workload("rows > 2^22", [n], [{"seqs": [0], "q_len": [10]}], top_k=256, H_I=4, d_I=64, H=8, seed=38)
    _parity_all(generate(wl, "cuda"), U.TOL_BF16, "rows > 2^22")


def test_prefill_many_sequences_more_blocks_than_workgroups():
    # 300 sequences, q_len 9 .. 24 (2 or 3 token blocks each): more token
    # blocks than the 256 workgroups of the prefill kernel, so workgroups take
    # several blocks from the counter and reuse their candidate rows, and
    # items past a sequence's blocks are skipped
    rng = np.random.default_rng(39)
    B = 300
    ql = [int(x) for x in rng.integers(9, 25, B)]
    ctx = [int(q + x) for q, x in zip(ql, rng.integers(0, 500, B))]
    wl = Workload("prefill items", ctx, [{"seqs": list(range(B)), "q_len": ql}], top_k=64, H_I=8, d_I=64, H=8,
                  seed=39)
    _parity_all(generate(wl, "cuda"), U.TOL_BF16, "prefill items")


def test_prefill_one_sequence_more_blocks_than_workgroups():
    # 263 token blocks of one sequence over 256 workgroups
    wl = Workload("prefill 263 blocks", [2500], [{"seqs": [0], "q_len": [2100]}], top_k=128, H_I=8, d_I=64, H=8,
                  seed=40)
    _parity_all(generate(wl, "cuda"), U.TOL_BF16, "prefill 263 blocks")


def test_decode_all_equal_scores_whole_row_select():
    # every score 0: the threshold bucket holds the whole row (40,000 and 33,000
    # keys, more than the 24,576-entry candidate list), so decode selection
    # runs over the whole row
    wl = Workload("zeros decode", [40000, 33000], [{"seqs": [0, 1], "q_len": None}], top_k=512, H=32, seed=30)
    inp = generate(wl, "cuda")
    inp.q_idx.zero_()
    call = inp.calls[0]
    out, lse, idx = U.run_fused(inp, call)
    got = np.sort(idx.cpu().numpy(), axis=1)
    assert np.array_equal(got, np.tile(np.arange(512, dtype=np.int32), (2, 1)))
    w_idx, w_out, w_lse = U.oracle_rows(inp, call, [0, 1])
    U.check_indices(idx.cpu().numpy(), w_idx, "zeros decode")
    U.check_attention(out.cpu().numpy(), lse.cpu().numpy(), w_out, w_lse, U.TOL_BF16, "zeros decode")


def _top11(scores):
    """Top 11 bits of the order of non-negative fp32 scores (sign, exponent,
    two mantissa bits): the buckets of the score kernel's row histogram."""
    s = np.asarray(scores, np.float32)
    assert np.all(s >= 0)
    return s.view(np.uint32) >> 21


def test_decode_wide_threshold_bucket():
    # Scores built so that 20,000 (request 0) and 24,000 (request 1) keys share
    # the histogram bucket of the K-th largest score, above the 12,288 keys of
    # the older candidate list and within the 24,576 of the packed one; the
    # bucket holds 32 distinct values, so the radix select and the tie rule
    # both take part.  Every head's query is the unit vector on dimension 0
    # and every head weight is 1, so S = 64 * ReLU(k[0]).
    wl = Workload("wide bucket", [131072, 70000], [{"seqs": [0, 1], "q_len": None}], top_k=2048, H=32, seed=32)
    inp = generate(wl, "cuda")
    inp.q_idx.zero_()
    inp.q_idx[:, :, 0] = 1.0
    inp.head_w.fill_(1.0)
    rng = np.random.default_rng(32)
    for b, (n, n_mid) in enumerate([(131072, 20000), (70000, 24000)]):
        k0 = rng.integers(-4, 5, n).astype(np.float32)       # scores 0 .. 256
        perm = rng.permutation(n)
        k0[perm[:1000]] = 100.0                              # score 6400: above the bucket
        k0[perm[1000:1000 + n_mid]] = 64.0 + 0.5 * rng.integers(0, 32, n_mid)  # 4096 .. 5088
        rows = torch.arange(b * inp.seq_stride, b * inp.seq_stride + n, device="cuda")
        inp.k_idx[rows, 0] = torch.from_numpy(k0).to("cuda").to(torch.bfloat16)
    call = inp.calls[0]
    out, lse, idx = U.run_fused(inp, call)
    torch.cuda.synchronize()
    w_idx, w_out, w_lse = U.oracle_rows(inp, call, [0, 1])
    # the case is what it claims: the K-th largest score's bucket size
    import oracle
    for b, n_mid in enumerate([20000, 24000]):
        keys = oracle.bf16_bits_to_f64(U.bits16(inp.k_idx[b * inp.seq_stride:b * inp.seq_stride + int(call.ctx_len[b])]))
        s = 64.0 * np.maximum(keys[:, 0], 0.0)
        kth = np.sort(s)[::-1][2047]
        cnt = int(np.sum(_top11(s) == _top11([kth])[0]))
        U.log("wide bucket request %d: %d keys in the threshold bucket" % (b, cnt))
        assert cnt == n_mid and 12288 < cnt <= 24576
    U.check_indices(idx.cpu().numpy(), w_idx, "wide bucket")
    U.check_attention(out.cpu().numpy(), lse.cpu().numpy(), w_out, w_lse, U.TOL_BF16, "wide bucket")


def test_multi_token_rows_of_140000_positions():
    # 3 query tokens per sequence (the multi-token score kernel and the
    # decode-style Top-K) over rows of 140,000 positions: 69 compaction
    # chunks per row
    wl = Workload("long rows", [140000], [{"seqs": [0], "q_len": [3]}], top_k=256, H_I=4, d_I=64, H=8, seed=31)
    _parity_all(generate(wl, "cuda"), U.TOL_BF16, "long rows")


def test_prefill_rows_of_140000_positions():
    # the same rows through the prefill kernel (10 query tokens): candidate
    # lists of rows of 140,000 keys
    wl = Workload("long rows prefill", [140000], [{"seqs": [0], "q_len": [10]}], top_k=256, H_I=4, d_I=64, H=8,
                  seed=39)
    _parity_all(generate(wl, "cuda"), U.TOL_BF16, "long rows prefill")


def test_separate_entry_points_match_fused():
    import indexer_selected_sparse_idx_amd as lib
    inp = generate(config(2, scale=1 / 16), "cuda")
    call = inp.calls[0]
    s = U.lib_seqs(inp, call)
    out, lse, idx = U.run_fused(inp, call)
    idx2 = lib.idx_score_topk(s, inp.q_idx, inp.k_idx, inp.head_w, inp.wl.top_k)
    out2, lse2 = lib.sparse_mla_attn(s, inp.q, inp.kv, idx2, U.SCALE)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("kv_dtype,H", [("bf16", 32), ("fp8_656", 32), ("fp8_656", 128)])
def test_attention_skips_invalid_entries_and_empty_rows(kv_dtype, H):
    # a row of 6 valid entries (one tile, partly filled) among invalid ones,
    # and a row with none; FP8 rows at 32 heads (one wave gathers every row
    # of a tile) and 128 (four waves, 8 rows each)
    import indexer_selected_sparse_idx_amd as lib
    wl = Workload("attn-only", [100, 50], [{"seqs": [0, 1], "q_len": None}], H=H, top_k=70, kv_dtype=kv_dtype,
                  seed=26)
    inp = generate(wl, "cuda")
    call = inp.calls[0]
    s = U.lib_seqs(inp, call)
    idx = torch.full((2, 70), -1, dtype=torch.int32)
    idx[0, :5] = torch.tensor([3, 99, 100, 5000, 0])          # 100 and 5000 are outside ctx = 100
    idx[0, 40:43] = torch.tensor([-7, 17, 3])                 # duplicates count twice
    # row 1: no valid entry at all
    idx = idx.cuda()
    out, lse = lib.sparse_mla_attn(s, inp.q, inp.kv, idx, U.SCALE)
    torch.cuda.synchronize()
    osq = U.oracle_seqs(inp, call)
    import oracle
    w_out, w_lse = oracle.attention(osq, U.bits16(inp.q), U.host_raw(inp.kv), kv_dtype, idx.cpu().numpy(), U.SCALE)
    tol = U.TOL_BF16 if kv_dtype == "bf16" else U.TOL_FP8
    U.check_attention(out.cpu().numpy(), lse.cpu().numpy(), w_out, w_lse, tol, "invalid entries %s H=%d" % (kv_dtype, H))
    assert torch.all(out[1] == 0) and torch.all(torch.isneginf(lse[1]))


def test_attention_score_growth_far_beyond_first_tile():
    """The softmax runs against the first tile's maximum; when later tiles
    score ~150 (base 2) higher, the p values would overflow fp32, and the
    kernel must fall back to its second pass with the true maximum."""
    import indexer_selected_sparse_idx_amd as lib
    import oracle
    wl = Workload("growth", [256, 256], [{"seqs": [0, 1], "q_len": None}], H=64, top_k=128, seed=28)
    inp = generate(wl, "cuda")
    call = inp.calls[0]
    s = U.lib_seqs(inp, call)
    # query: 12 along latent dim 0 for every head; rows: dim 0 = 200 for the
    # later entries, every value of the first 32 entries scaled to ~0
    q = torch.zeros_like(inp.q)
    q[:, :, 0] = 12.0
    q[:, :, 1:] = inp.q[:, :, 1:] * 0.1
    kv = inp.kv.clone()
    idx = torch.stack([torch.arange(0, 256, 2, dtype=torch.int32), torch.arange(1, 256, 2, dtype=torch.int32)])
    for b in range(2):
        rows = b * inp.seq_stride + idx[b].long()
        first, later = rows[:32].cuda(), rows[32:].cuda()
        kv[first] = (kv[first].float() * 1e-3).to(kv.dtype)
        big = kv[later].float()
        big[:, 0] = 200.0 + torch.arange(big.shape[0], device="cuda", dtype=torch.float32) * 0.25
        kv[later] = big.to(kv.dtype)
    idx = idx.cuda()
    out, lse = lib.sparse_mla_attn(s, q, kv, idx, U.SCALE)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    osq = U.oracle_seqs(inp, call)
    w_out, w_lse = oracle.attention(osq, U.bits16(q), U.host_raw(kv), "bf16", idx.cpu().numpy(), U.SCALE)
    # scores here reach ~100 (natural log units): compare lse relative to its size
    U.check_attention(out.cpu().numpy(), lse.cpu().numpy() / 100.0, w_out, w_lse / 100.0, U.TOL_BF16,
                      "score growth")


def test_paged_equals_contiguous_bitwise():
    wl_c = Workload("c", [1500, 700], [{"seqs": [0, 1], "q_len": None}], top_k=512, seed=27)
    inp = generate(wl_c, "cuda")
    call = inp.calls[0]
    out_c, lse_c, idx_c = U.run_fused(inp, call)
    # scatter the same rows into shuffled pages of 32
    page = 32
    rng = np.random.default_rng(5)
    npg = [-(-int(c) // page) for c in wl_c.ctx_len]
    perm = rng.permutation(sum(npg)).astype(np.int32)
    bt = np.zeros((2, max(npg)), np.int32)
    k_p = torch.zeros((sum(npg) * page, inp.k_idx.shape[1]), dtype=inp.k_idx.dtype, device="cuda")
    kv_p = torch.zeros((sum(npg) * page, inp.kv.shape[1]), dtype=inp.kv.dtype, device="cuda")
    k = 0
    for b in range(2):
        for j in range(npg[b]):
            bt[b, j] = perm[k]
            k += 1
            lo, hi = j * page, min((j + 1) * page, wl_c.ctx_len[b])
            src = b * inp.seq_stride
            k_p[bt[b, j] * page: bt[b, j] * page + hi - lo] = inp.k_idx[src + lo: src + hi]
            kv_p[bt[b, j] * page: bt[b, j] * page + hi - lo] = inp.kv[src + lo: src + hi]
    import indexer_selected_sparse_idx_amd as lib
    ctx = torch.tensor(wl_c.ctx_len, dtype=torch.int32, device="cuda")
    btt = torch.from_numpy(bt).cuda()
    s = lib.Seqs(ctx, None, max_q_len=1, max_ctx_len=1500, block_table=btt, page_size=page)
    out_p, lse_p, idx_p = lib.idx_sparse_attn_decode(s, inp.q_idx, k_p, inp.head_w, 512, inp.q, kv_p, U.SCALE,
                                                     out_idx=torch.empty_like(idx_c))
    torch.cuda.synchronize()
    assert torch.equal(idx_c, idx_p)
    assert torch.equal(out_c, out_p) and torch.equal(lse_c, lse_p)


def test_deterministic():
    inp = generate(config(5, scale=1 / 32), "cuda")
    for call in inp.calls:
        a = U.run_fused(inp, call)
        b = U.run_fused(inp, call)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_two_token_rows_split_keys():
    # at most 2 query tokens per sequence: the multi-token kernel gives each
    # token two waves, over the two halves of a workgroup's keys
    ctx = [5000, 2100, 65, 2, 9000]
    q_len = [2, 2, 1, 2, 2]
    wl = Workload("two-token rows", ctx, [{"seqs": list(range(5)), "q_len": q_len}], top_k=2048, H=16,
                  seed=34)
    _parity_all(generate(wl, "cuda"), U.TOL_BF16, "two-token")


def test_attention_values_beyond_fp16_range():
    """The attention computes in fp16 unless an operand leaves its range:
    rows holding values beyond fp16's 65,504 make the split's scores or
    output non-finite in fp16 (+inf scores where the query value is
    positive, 0 x inf in P.V where it is negative), and the workgroup must
    recompute it in bf16.  bf16 rows hold 70,000 (stored as 70,144); FP8
    rows get a tile scale of 2^9, so their values (up to 448 x 512) stay
    exact in the bf16 recomputation (with a scale that is not a power of
    two the bf16 rounding of such large values moves scores by several
    units, see the design notes).  Decode splits, bf16 and FP8 rows."""
    import indexer_selected_sparse_idx_amd as lib
    import oracle
    from oracle import formats as Fm
    for kv_dtype, tol in (("bf16", U.TOL_BF16), ("fp8_656", U.TOL_FP8)):
        wl = Workload("beyond fp16", [3000, 700], [{"seqs": [0, 1], "q_len": None}], H=64, top_k=512,
                      kv_dtype=kv_dtype, seed=40)
        inp = generate(wl, "cuda")
        call = inp.calls[0]
        s = U.lib_seqs(inp, call)
        rng = np.random.default_rng(40)
        idx = torch.from_numpy(np.stack([np.sort(rng.choice(c, 512, replace=False)) for c in (3000, 700)])
                               .astype(np.int32)).cuda()
        kv = inp.kv.clone()
        for b in range(2):
            rows = (b * inp.seq_stride + idx[b, [7, 300]].long())
            if kv_dtype == "bf16":
                big = kv[rows].float()
                big[:, 5] = 70000.0
                kv[rows] = big.to(torch.bfloat16)
            else:
                # tile 0 of the row: a code of 448 at dim 5, the tile's fp32 scale 2^9
                raw = kv[rows]
                raw[:, 5] = 0x7E
                raw[:, 512:516] = torch.from_numpy(np.array([512.0], np.float32).view(np.uint8)).cuda()
                kv[rows] = raw
        out, lse = lib.sparse_mla_attn(s, inp.q, kv, idx, U.SCALE)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
        osq = U.oracle_seqs(inp, call)
        w_out, w_lse = oracle.attention(osq, U.bits16(inp.q), U.host_raw(kv), kv_dtype, idx.cpu().numpy(), U.SCALE)
        assert np.abs(w_out).max() > 65504.0       # the case is what it claims
        # scores reach thousands (natural log units): lse compared relative to that scale
        U.check_attention(out.cpu().numpy(), lse.cpu().numpy() / 1e4, w_out, w_lse / 1e4, tol,
                          "beyond fp16 %s" % kv_dtype)


def test_attention_values_below_fp16_normals():
    """Rows whose latent values are all far below fp16's smallest normal
    (2^-14): in fp16 they would be subnormals with an absolute spacing of
    2^-24, coarse against values of about 1e-6, so every head's output is
    tiny and the workgroup must recompute the split in bf16.  bf16 rows
    times 2^-20; FP8 rows with tile scales of 2^-27 (values up to 448 x
    2^-27, exact in bf16).  A decode batch with split rows and a prefill
    chunk (one split per row)."""
    import indexer_selected_sparse_idx_amd as lib
    import oracle
    for kv_dtype, tol in (("bf16", U.TOL_BF16), ("fp8_656", U.TOL_FP8)):
        for q_len in (None, [40]):
            calls = [{"seqs": [0, 1], "q_len": None}] if q_len is None else [{"seqs": [0], "q_len": q_len}]
            wl = Workload("below fp16 normals", [3000, 700], calls, H=64, top_k=512, kv_dtype=kv_dtype, seed=41)
            inp = generate(wl, "cuda")
            call = inp.calls[0]
            kv = inp.kv.clone()
            if kv_dtype == "bf16":
                kv = (kv.float() * 2.0 ** -20).to(torch.bfloat16)
            else:
                tiny = torch.from_numpy(np.full(4, 2.0 ** -27, np.float32).view(np.uint8)).cuda()
                kv[:, 512:528] = tiny
            inp.kv = kv
            out, lse, idx = U.run_fused(inp, call)
            torch.cuda.synchronize()
            tokens = list(range(call.num_tokens))
            w_idx, w_out, w_lse = U.oracle_rows(inp, call, tokens)
            U.check_indices(idx.cpu().numpy(), w_idx, "tiny %s" % kv_dtype)
            rms = float(np.sqrt(np.mean(w_out ** 2)))
            assert 0.0 < rms < 2.0 ** -16                   # the case is what it claims
            err = U.check_attention(out.cpu().numpy(), lse.cpu().numpy(), w_out, w_lse, tol,
                                    "tiny %s q_len %s" % (kv_dtype, q_len))
            U.log("  tiny %s q_len %s: err/RMS %.2e" % (kv_dtype, q_len, err))
