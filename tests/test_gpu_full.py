"""GPU parity at the workloads' full sizes, in the launch configuration the
bench uses (the fused entry points over whole batches).

The oracle recomputes, on the host, every row it can afford and a seeded
sample of rows elsewhere: all rows of the tiny prefill (L = 2048) and of the
64-request decode batch; sampled rows (first, last and random) of every
long-prefill chunk checked; sampled requests of the FP8 decode batch; and
sampled prefill and decode tokens of the mixed paged batch.  Indices are
compared bit for bit as sets, attention within tol * RMS of the oracle's
output over the compared rows.
"""
import numpy as np
import pytest
import torch

import workloads
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
    pick = {0, n - 1}
    pick.update(int(x) for x in rng.choice(n, size=min(k, n), replace=False))
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


def test_full_long_prefill_sampled_rows():
    inp = generate(config(3), "cuda")
    rng = np.random.default_rng(33)
    for ci, call in enumerate(inp.calls):
        U.log("long-prefill chunk %d: ctx %d" % (ci, int(call.ctx_len[0])))
        out, lse, idx = U.run_fused(inp, call)
        torch.cuda.synchronize()
        if ci in (0, 1, 7, 15):
            _check_rows(inp, call, out, lse, idx, _sample(call.num_tokens, 6, rng), U.TOL_BF16,
                        "long-prefill chunk %d" % ci)
        del out, lse, idx


def test_full_fp8_decode_sampled_requests():
    inp = generate(config(4), "cuda")
    call = inp.calls[0]
    out, lse, idx = U.run_fused(inp, call)
    torch.cuda.synchronize()
    rng = np.random.default_rng(44)
    _check_rows(inp, call, out, lse, idx, _sample(call.num_tokens, 10, rng), U.TOL_FP8, "fp8-decode 128x131072")


def test_full_mixed_paged_sampled_rows():
    inp = generate(config(5), "cuda")
    rng = np.random.default_rng(55)
    for ci, call in enumerate(inp.calls):
        out, lse, idx = U.run_fused(inp, call)
        torch.cuda.synchronize()
        if call.is_decode:
            toks = _sample(call.num_tokens, 16, rng)
        else:
            # every prefill request's first and last token, plus random tokens
            toks = sorted(set(int(x) for x in call.cu_q[:-1]) | set(int(x) - 1 for x in call.cu_q[1:])
                          | set(_sample(call.num_tokens, 8, rng)))
        _check_rows(inp, call, out, lse, idx, toks, U.TOL_BF16,
                    "mixed-paged %s call" % ("decode" if call.is_decode else "prefill"))
        del out, lse, idx
