"""Pins of the CPU oracle against facts fixed outside it.

Each check compares the oracle with something it does not share code with:
hand-derived worked examples (tests/golden), brute-force enumeration on tiny
inputs, closed forms, special cases that reduce to a library routine
(torch's scaled-dot-product attention in float64, torch's float8/bf16
casts) and invariants.  The checks are plain functions taking the oracle's
entry points as arguments, so test_oracle_mutants.py can plant mistakes in
copies of the oracle and confirm that some check catches each one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import reference as R

from conftest import GOLDEN

RNG = np.random.default_rng(1234)


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# checks (return None on success, raise AssertionError on failure)
# --------------------------------------------------------------------------

def check_indexer_golden(indexer_scores, topk_select):
    for case in _load("indexer_hand_example.json")["cases"]:
        q = np.array(case["q"], dtype=np.float64)
        k = np.array(case["keys"], dtype=np.float64)
        w = np.array(case["w"], dtype=np.float64)
        ks = None if case["k_scale"] is None else np.array(case["k_scale"])
        s = indexer_scores(q, k, w, ks)
        np.testing.assert_array_equal(s, np.array(case["scores"]), err_msg=case["name"])
        for kk, want in case["topk"].items():
            got = topk_select(s, int(kk))
            np.testing.assert_array_equal(got, np.array(want, dtype=np.int32),
                                          err_msg=f"{case['name']} K={kk}")


def _brute_scores(q, k, w, ks):
    """Triple loop, straight from the definition."""
    n, H, d = k.shape[0], q.shape[0], q.shape[1]
    out = []
    for s in range(n):
        tot = 0.0
        for h in range(H):
            dot = 0.0
            for j in range(d):
                dot += float(q[h, j]) * float(k[s, j])
            if ks is not None:
                dot *= float(ks[s])
            tot += float(w[h]) * (dot if dot > 0.0 else 0.0)
        out.append(tot)
    return np.array(out)


def check_indexer_bruteforce(indexer_scores):
    rng = np.random.default_rng(7)
    for trial in range(12):
        H = int(rng.integers(1, 5))
        d = int(rng.integers(1, 9))
        n = int(rng.integers(1, 17))
        q = rng.integers(-4, 5, size=(H, d)).astype(np.float64)
        k = rng.integers(-4, 5, size=(n, d)).astype(np.float64)
        w = (2.0 ** -rng.integers(0, 4, size=H)) * rng.choice([-1.0, 1.0], size=H)
        ks = None if trial % 2 else 2.0 ** rng.integers(-2, 3, size=n)
        got = indexer_scores(q, k, w, ks)
        want = _brute_scores(q, k, w, ks)
        np.testing.assert_array_equal(got, want)


def _brute_topk(scores, K):
    """Full sort by (-score, position); first min(K, n) positions, -1 padded."""
    order = sorted(range(len(scores)), key=lambda s: (-scores[s], s))
    m = min(K, len(scores))
    sel = sorted(order[:m])
    return np.array(sel + [-1] * (K - m), dtype=np.int32)


def check_topk_bruteforce(topk_select):
    rng = np.random.default_rng(11)
    for _ in range(200):
        n = int(rng.integers(0, 40))
        levels = int(rng.integers(1, 6))          # few distinct values: heavy ties
        scores = rng.integers(0, levels, size=n).astype(np.float64) * 0.125
        for K in range(1, n + 3):
            np.testing.assert_array_equal(topk_select(scores, K), _brute_topk(list(scores), K))


def check_topk_exchange_property(topk_select):
    """Definition by exchange: i selected, j not => S[i] > S[j] or (== and i < j)."""
    rng = np.random.default_rng(13)
    for n in range(1, 9):
        for _ in range(20):
            scores = rng.integers(0, 3, size=n).astype(np.float64)
            for K in range(1, n + 1):
                got = topk_select(scores, K)
                sel = set(int(x) for x in got if x >= 0)
                assert len(sel) == min(K, n)
                for i, j in itertools.product(sel, set(range(n)) - sel):
                    assert scores[i] > scores[j] or (scores[i] == scores[j] and i < j)


def check_topk_special_cases(topk_select):
    # all equal -> the first m positions
    for n, K in [(1, 1), (5, 3), (64, 64), (100, 7)]:
        got = topk_select(np.full(n, 2.5), K)
        m = min(n, K)
        assert list(got[:m]) == list(range(m)) and all(got[m:] == -1)
    # strictly increasing -> the last m positions
    for n, K in [(10, 3), (50, 50), (9, 12)]:
        got = topk_select(np.arange(n, dtype=np.float64), K)
        m = min(n, K)
        assert list(got[:m]) == list(range(n - m, n)) and all(got[m:] == -1)
    # -0.0 and +0.0 are the same score
    got = topk_select(np.array([0.0, -0.0, 0.0, 1.0]) + 0.0, 3)
    assert list(got) == [0, 1, 3]


def check_attention_golden(sparse_attention):
    g = _load("attention_closed_form.json")
    scale = 1.0 / g["scale_inv"]
    for case in g["cases"]:
        q = np.zeros((1, 576))
        for j, v in case["q_nonzero"].items():
            q[0, int(j)] = v
        rows = np.zeros((len(case["rows_nonzero"]), 576))
        for r, nz in enumerate(case["rows_nonzero"]):
            for j, v in nz.items():
                rows[r, int(j)] = v
        out, lse = sparse_attention(q, rows, scale)
        want = np.zeros(512)
        for j, v in case["out_nonzero"].items():
            want[int(j)] = v
        assert out.shape == (1, 512)
        np.testing.assert_allclose(out[0], want, rtol=1e-13, atol=1e-15, err_msg=case["name"])
        assert abs(lse[0] - case["lse"]) < 1e-13


def check_attention_special_cases(sparse_attention):
    rng = np.random.default_rng(17)
    # one row: the softmax weight is exactly 1
    q = rng.standard_normal((4, 576))
    row = rng.standard_normal((1, 576))
    out, lse = sparse_attention(q, row, 1 / 24)
    np.testing.assert_allclose(out, np.repeat(row[:, :512], 4, axis=0), rtol=1e-14, atol=0)
    np.testing.assert_allclose(lse, (q @ row[0]) / 24, rtol=1e-13)
    # zero query: uniform weights -> mean of the rows, lse = log m
    rows = rng.standard_normal((9, 576))
    out, lse = sparse_attention(np.zeros((3, 576)), rows, 1 / 24)
    np.testing.assert_allclose(out, np.repeat(rows[:, :512].mean(0, keepdims=True), 3, 0), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, np.log(9.0), rtol=1e-14)
    # empty selection
    out, lse = sparse_attention(q, np.zeros((0, 576)), 1 / 24)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    # row order does not matter
    perm = rng.permutation(9)
    q = rng.standard_normal((5, 576))
    a, la = sparse_attention(q, rows, 1 / 24)
    b, lb = sparse_attention(q, rows[perm], 1 / 24)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-13)


def check_dense_equivalence(score_topk_fn, attention_fn):
    """K >= t + 1 selects every causal position, so the sparse path must equal
    dense causal softmax attention (torch's float64 SDPA on the CPU)."""
    rng = np.random.default_rng(19)
    L, H, Hi, di = 37, 3, 2, 8
    q_idx = _bf16_bits(rng.integers(-4, 5, size=(L, Hi, di)).astype(np.float32))
    k_idx = _bf16_bits(rng.integers(-4, 5, size=(L, di)).astype(np.float32))
    w = np.ones((L, Hi), dtype=np.float32)
    q = _bf16_bits(rng.standard_normal((L, H, 576)).astype(np.float32))
    kv = _bf16_bits(rng.standard_normal((L, 576)).astype(np.float32))
    seqs = R.Seqs(ctx_len=np.array([L]), cu_q=np.array([0, L]), seq_stride=L)
    idx = score_topk_fn(seqs, q_idx, k_idx, "bf16", w, top_k=L)
    out, lse = attention_fn(seqs, q, kv, "bf16", idx, 1 / 24)
    qt = torch.from_numpy(oracle.bf16_bits_to_f64(q)).permute(1, 0, 2)          # [H, L, 576]
    kt = torch.from_numpy(oracle.bf16_bits_to_f64(kv))[None].expand(H, L, 576)
    vt = kt[..., :512]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=True, scale=1 / 24).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    logits = torch.einsum("hld,hsd->hls", qt, kt) / 24
    mask = torch.ones(L, L, dtype=torch.bool).tril()
    ref_lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1).permute(1, 0).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12)


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
# tests
# --------------------------------------------------------------------------

def test_indexer_golden():
    check_indexer_golden(R.indexer_scores, R.topk_select)


def test_indexer_bruteforce():
    check_indexer_bruteforce(R.indexer_scores)


def test_topk_bruteforce():
    check_topk_bruteforce(R.topk_select)


def test_topk_exchange_property():
    check_topk_exchange_property(R.topk_select)


def test_topk_special_cases():
    check_topk_special_cases(R.topk_select)


def test_attention_golden():
    check_attention_golden(R.sparse_attention)


def test_attention_special_cases():
    check_attention_special_cases(R.sparse_attention)


def test_dense_equivalence():
    check_dense_equivalence(R.score_topk, R.attention)


def test_e4m3_golden_values():
    g = _load("e4m3_ocp_values.json")
    for code, val in g["codes"].items():
        got = oracle.e4m3_value(int(code, 16))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in g["nan_codes"]:
        assert math.isnan(oracle.e4m3_value(int(code, 16)))


def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))


def test_bf16_decode_matches_torch():
    x = torch.randn(4096, dtype=torch.float32) * 100
    b = x.to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(bits), b.to(torch.float64).numpy())


def test_fp8_row_decode_hand_example():
    row = np.zeros(656, dtype=np.uint8)
    row[0] = 0x38       # 1.0 in tile 0
    row[130] = 0x40     # 2.0 in tile 1
    row[300] = 0xB8     # -1.0 in tile 2
    row[511] = 0x48     # 4.0 in tile 3
    row[512:528] = np.array([0.5, 3.0, 0.25, 1.5], dtype="<f4").view(np.uint8)
    row[528:530] = np.array([0x3FC0], dtype="<u2").view(np.uint8)   # bf16 1.5 at rope 0
    row[654:656] = np.array([0xC000], dtype="<u2").view(np.uint8)   # bf16 -2.0 at rope 63
    dec = oracle.fp8_rows_to_f64(row[None])[0]
    want = np.zeros(576)
    want[0], want[130], want[300], want[511] = 0.5, 6.0, -0.25, 6.0
    want[512], want[575] = 1.5, -2.0
    np.testing.assert_array_equal(dec, want)


def test_score_topk_invariants():
    rng = np.random.default_rng(23)
    B, Hi, di, K = 3, 4, 16, 24
    ctx = np.array([40, 1, 77])
    qlen = np.array([5, 1, 9])
    cu = np.concatenate([[0], np.cumsum(qlen)])
    T = int(cu[-1])
    stride = 80
    q_idx = _bf16_bits(rng.integers(-4, 5, size=(T, Hi, di)))
    k_idx = _bf16_bits(rng.integers(-4, 5, size=(B * stride, di)))
    w = (2.0 ** -rng.integers(0, 4, size=(T, Hi))).astype(np.float32)
    seqs = R.Seqs(ctx_len=ctx, cu_q=cu, seq_stride=stride)
    idx = R.score_topk(seqs, q_idx, k_idx, "bf16", w, K)
    for r, (b, t) in enumerate(seqs.token_positions()):
        valid = idx[r][idx[r] >= 0]
        m = min(K, t + 1)
        assert valid.size == m
        assert np.all(idx[r][m:] == -1) and np.all(idx[r][:m] >= 0)
        assert np.unique(valid).size == m
        assert valid.max() <= t


def _paged_copy(rng, seqs, raw, page_size):
    """Scatter a contiguous cache into randomly numbered pages."""
    B = seqs.num_seqs
    n_pages = [-(-int(c) // page_size) for c in seqs.ctx_len]
    total = sum(n_pages)
    perm = rng.permutation(total)
    width = max(n_pages)
    bt = np.full((B, width), -1, dtype=np.int64)
    paged = np.zeros((total * page_size,) + raw.shape[1:], dtype=raw.dtype)
    k = 0
    for b in range(B):
        for p in range(n_pages[b]):
            bt[b, p] = perm[k]
            k += 1
            lo = p * page_size
            hi = min(lo + page_size, int(seqs.ctx_len[b]))
            dst = bt[b, p] * page_size
            paged[dst: dst + hi - lo] = raw[b * seqs.seq_stride + lo: b * seqs.seq_stride + hi]
    return R.Seqs(ctx_len=seqs.ctx_len, cu_q=seqs.cu_q, block_table=bt, page_size=page_size), paged


def test_paged_equals_contiguous():
    rng = np.random.default_rng(29)
    B, Hi, di, H, K = 3, 2, 8, 2, 10
    ctx = np.array([19, 64, 33])
    stride = 64
    seqs = R.Seqs(ctx_len=ctx, cu_q=np.array([0, 2, 5, 6]), seq_stride=stride)
    T = 6
    q_idx = _bf16_bits(rng.integers(-4, 5, size=(T, Hi, di)))
    k_idx = _bf16_bits(rng.integers(-4, 5, size=(B * stride, di)))
    w = np.ones((T, Hi), np.float32)
    q = _bf16_bits(rng.standard_normal((T, H, 576)))
    kv = _bf16_bits(rng.standard_normal((B * stride, 576)))
    idx_c = R.score_topk(seqs, q_idx, k_idx, "bf16", w, K)
    o_c, l_c = R.attention(seqs, q, kv, "bf16", idx_c, 1 / 24)
    pseqs, k_pg = _paged_copy(np.random.default_rng(3), seqs, k_idx, 16)
    pseqs2, kv_pg = _paged_copy(np.random.default_rng(3), seqs, kv, 16)
    assert np.array_equal(pseqs.block_table, pseqs2.block_table)
    idx_p = R.score_topk(pseqs, q_idx, k_pg, "bf16", w, K)
    o_p, l_p = R.attention(pseqs, q, kv_pg, "bf16", idx_p, 1 / 24)
    np.testing.assert_array_equal(idx_c, idx_p)
    np.testing.assert_array_equal(o_c, o_p)
    np.testing.assert_array_equal(l_c, l_p)


def test_attention_skips_out_of_range_entries():
    rng = np.random.default_rng(31)
    q = _bf16_bits(rng.standard_normal((1, 2, 576)))
    kv = _bf16_bits(rng.standard_normal((8, 576)))
    seqs = R.Seqs(ctx_len=np.array([5]), seq_stride=8)
    a, la = R.attention(seqs, q, kv, "bf16", np.array([[3, 0, 1]]), 1 / 24)
    b, lb = R.attention(seqs, q, kv, "bf16", np.array([[-1, 3, 7, 0, 5, 1]]), 1 / 24)
    np.testing.assert_allclose(a, b, rtol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-14)
