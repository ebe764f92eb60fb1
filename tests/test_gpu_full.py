"""GPU parity at the workloads' full sizes, in the launch configuration the
bench uses (the fused entry points over whole batches).

The oracle recomputes, on the host, every row it can afford and a seeded
sample of rows elsewhere:
- tiny prefill (L = 2048): every row;
- decode batch (64 x 32768): every row;
- long prefill (65,536 positions in 16 chunks of 4096): 64 rows of every
  chunk (its first and last rows and 62 seeded ones), and every row of the
  first chunk with t < K (the rows whose selection is the whole history);
- FP8 decode (128 x 131072): every row;
- mixed paged batch: every decode row, and every prefill sequence's first
  and last token plus seeded tokens.
Indices are compared bit for bit as sets, attention within tol * RMS of the
oracle's output over the compared rows.
"""
import numpy as np
import pytest
import torch

from workloads import config, generate

import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import indexer_selected_sparse_idx_amd as lib
    lib.lib()


def _check_rows(inp, call, out, lse, idx, tokens, tol, label):
    with U.Timer("%s oracle on %d rows" % (label, len(tokens))):
        w_idx, w_out, w_lse = U.oracle_rows(inp, call, tokens)
    t = torch.tensor(tokens, dtype=torch.long, device=out.device)
    U.check_indices(idx.index_select(0, t).cpu().numpy(), w_idx, label)
    err = U.check_attention(out.index_select(0, t).cpu().numpy(), lse.index_select(0, t).cpu().numpy(),
                            w_out, w_lse, tol, label)
    U.log("  %s: %d rows ok, attention err/RMS %.2e" % (label, len(tokens), err))


def _sample(n, k, rng):
    """k distinct rows of n: the first, the last and k - 2 seeded others."""
    pick = {0, n - 1}
    rest = [int(x) for x in rng.permutation(np.arange(1, n - 1))]
    for x in rest:
        if len(pick) >= min(k, n):
            break
        pick.add(x)
    return sorted(pick)


def test_full_tiny_prefill_all_rows():
    inp = generate(config(1), "cuda")
    call = inp.calls[0]
    out, lse, idx = U.run_fused(inp, call)
    torch.cuda.synchronize()
    _check_rows(inp, call, out, lse, idx, list(range(call.num_tokens)), U.TOL_BF16, "tiny-prefill L=2048")


def test_full_decode_batch_all_rows():
    inp = generate(config(2), "cuda")
    call = inp.calls[0]
    out, lse, idx = U.run_fused(inp, call)
    torch.cuda.synchronize()
    _check_rows(inp, call, out, lse, idx, list(range(call.num_tokens)), U.TOL_BF16, "decode-batch 64x32768")


# ---- long prefill: one generated workload for its tests ---------------------

@pytest.fixture(scope="module")
def long_prefill():
    inp = generate(config(3), "cuda")
    yield inp
    inp.extra.clear()


def _long_prefill_chunks(inp, chunks):
    for ci in chunks:
        call = inp.calls[ci]
        U.log("long-prefill chunk %d: ctx %d" % (ci, int(call.ctx_len[0])))
        out, lse, idx = U.run_fused(inp, call)
        torch.cuda.synchronize()
        rng = np.random.default_rng(3300 + ci)
        _check_rows(inp, call, out, lse, idx, _sample(call.num_tokens, 64, rng), U.TOL_BF16,
                    "long-prefill chunk %d" % ci)
        del out, lse, idx


def test_full_long_prefill_chunk0_rows_below_k(long_prefill):
    inp = long_prefill
    call = inp.calls[0]
    K = inp.wl.top_k
    out, lse, idx = U.run_fused(inp, call)
    torch.cuda.synchronize()
    _check_rows(inp, call, out, lse, idx, list(range(K)), U.TOL_BF16, "long-prefill chunk 0, rows t < K")


def test_full_long_prefill_chunks_0_to_3(long_prefill):
    _long_prefill_chunks(long_prefill, range(0, 4))


def test_full_long_prefill_chunks_4_to_7(long_prefill):
    _long_prefill_chunks(long_prefill, range(4, 8))


def test_full_long_prefill_chunks_8_to_11(long_prefill):
    _long_prefill_chunks(long_prefill, range(8, 12))


def test_full_long_prefill_chunks_12_to_15(long_prefill):
    _long_prefill_chunks(long_prefill, range(12, 16))


# ---- FP8 decode: every request ---------------------------------------------------

@pytest.fixture(scope="module")
def fp8_decode():
    inp = generate(config(4), "cuda")
    call = inp.calls[0]
    out, lse, idx = U.run_fused(inp, call)
    torch.cuda.synchronize()
    yield inp, call, out, lse, idx
    inp.extra.clear()


def test_full_fp8_decode_requests_0_to_63(fp8_decode):
    inp, call, out, lse, idx = fp8_decode
    _check_rows(inp, call, out, lse, idx, list(range(0, 64)), U.TOL_FP8, "fp8-decode 128x131072, requests 0-63")


def test_full_fp8_decode_requests_64_to_127(fp8_decode):
    inp, call, out, lse, idx = fp8_decode
    _check_rows(inp, call, out, lse, idx, list(range(64, 128)), U.TOL_FP8,
                "fp8-decode 128x131072, requests 64-127")


# ---- mixed paged batch ---------------------------------------------------------

def test_full_mixed_paged_rows():
    inp = generate(config(5), "cuda")
    rng = np.random.default_rng(55)
    for ci, call in enumerate(inp.calls):
        out, lse, idx = U.run_fused(inp, call)
        torch.cuda.synchronize()
        if call.is_decode:
            toks = list(range(call.num_tokens))
        else:
            # every prefill request's first and last token, plus seeded tokens
            toks = sorted(set(int(x) for x in call.cu_q[:-1]) | set(int(x) - 1 for x in call.cu_q[1:])
                          | set(_sample(call.num_tokens, 64, rng)))
        _check_rows(inp, call, out, lse, idx, toks, U.TOL_BF16,
                    "mixed-paged %s call" % ("decode" if call.is_decode else "prefill"))
        del out, lse, idx
    inp.extra.clear()
