"""Planted mistakes: each mutant is a copy of an oracle function with one
plausible error (a dropped term, a wrong index or sign, a swapped operand).
Every mutant must be caught by at least one pin in test_oracle_pins.py;
otherwise the pins would not protect the oracle against that mistake.
Everything here runs on the CPU and changes nothing outside this module."""
import numpy as np
import pytest

from oracle import formats
from oracle import reference as R

import test_oracle_pins as P


# ---- indexer mutants -----------------------------------------------------

def scores_no_relu(q, k, w, ks=None):
    d = k @ q.T
    if ks is not None:
        d = d * ks[:, None]
    return d @ w + 0.0


def scores_relu_after_sum(q, k, w, ks=None):
    d = k @ q.T
    if ks is not None:
        d = d * ks[:, None]
    return np.maximum(d @ w, 0.0) + 0.0


def scores_ignore_scale(q, k, w, ks=None):
    return R.indexer_scores(q, k, w, None)


def scores_unweighted(q, k, w, ks=None):
    return R.indexer_scores(q, k, np.ones_like(np.asarray(w, dtype=np.float64)), ks)


# ---- top-k mutants -------------------------------------------------------

def topk_ties_high(scores, K):
    scores = np.asarray(scores, np.float64)
    n = scores.size
    m = min(K, n)
    out = np.full(K, -1, np.int32)
    if m == 0:
        return out
    tau = np.partition(scores, n - m)[n - m]
    above = np.flatnonzero(scores > tau)
    ties = np.flatnonzero(scores == tau)[::-1][: m - above.size]
    out[:m] = np.sort(np.concatenate([above, ties]))
    return out


def topk_off_by_one(scores, K):
    out = R.topk_select(scores, max(K - 1, 0))
    return np.concatenate([out, -np.ones(K - out.size, np.int32)])


def topk_smallest(scores, K):
    return R.topk_select(-np.asarray(scores, np.float64), K)


# ---- attention mutants ---------------------------------------------------

def attn_values_wrong_slice(q, rows, scale):
    out, lse = R.sparse_attention(q, rows, scale)
    if rows.shape[0]:
        logits = scale * (q @ rows.T)
        p = np.exp(logits - logits.max(1, keepdims=True))
        out = (p @ rows[:, 64:]) / p.sum(1, keepdims=True)
    return out, lse


def attn_no_rope_in_logits(q, rows, scale):
    q = np.array(q, dtype=np.float64)
    q[:, 512:] = 0.0
    return R.sparse_attention(q, rows, scale)


def attn_no_scale(q, rows, scale):
    return R.sparse_attention(q, rows, 1.0)


def attn_lse_max_only(q, rows, scale):
    out, lse = R.sparse_attention(q, rows, scale)
    if rows.shape[0]:
        lse = (scale * (q @ rows.T)).max(1)
    return out, lse


# ---- batch-driver mutants -----------------------------------------------

def score_topk_strict_causal(seqs, q_idx, k_idx, k_dtype, head_w, top_k, k_scale=None, tokens=None):
    """Candidates s < t instead of s <= t."""
    pos = seqs.token_positions()
    out = np.empty((len(pos), top_k), np.int32)
    for r, (b, t) in enumerate(pos):
        phys = seqs.physical_rows(b, np.arange(t))
        keys = R.decode_rows(k_idx, k_dtype, phys)
        s = R.indexer_scores(formats.bf16_bits_to_f64(q_idx[r]), keys, head_w[r].astype(np.float64))
        out[r] = R.topk_select(s, top_k)
    return out


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("mutant", [scores_no_relu, scores_relu_after_sum,
                                    scores_ignore_scale, scores_unweighted])
def test_indexer_mutants_caught(mutant):
    assert (_fails(P.check_indexer_golden, mutant, R.topk_select)
            or _fails(P.check_indexer_bruteforce, mutant))


@pytest.mark.parametrize("mutant", [topk_ties_high, topk_off_by_one, topk_smallest])
def test_topk_mutants_caught(mutant):
    assert (_fails(P.check_indexer_golden, R.indexer_scores, mutant)
            or _fails(P.check_topk_bruteforce, mutant)
            or _fails(P.check_topk_exchange_property, mutant)
            or _fails(P.check_topk_special_cases, mutant))


@pytest.mark.parametrize("mutant", [attn_values_wrong_slice, attn_no_rope_in_logits,
                                    attn_no_scale, attn_lse_max_only])
def test_attention_mutants_caught(mutant):
    assert (_fails(P.check_attention_golden, mutant)
            or _fails(P.check_attention_special_cases, mutant))


def test_strict_causal_mutant_caught():
    assert _fails(P.check_dense_equivalence, score_topk_strict_causal, R.attention)
