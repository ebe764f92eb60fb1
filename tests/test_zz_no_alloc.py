"""The allocation-free fused decode (idx_sparse_attn_decode_static) against
the entry point that takes a workspace: the same kernels on the same batch,
so the results must be equal bit for bit.  Two calls in a row, the second on
a smaller batch, so the second runs over what the first left in the
library's static buffer."""
import math

import numpy as np
import pytest
import torch

import indexer_selected_sparse_idx_amd as lib
from workloads import Workload, generate

import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.lib()


def _both(inp):
    call = inp.calls[0]
    s = U.lib_seqs(inp, call)
    T, K = call.num_tokens, inp.wl.top_k
    idx_a = torch.empty((T, K), dtype=torch.int32, device="cuda")
    idx_b = torch.empty((T, K), dtype=torch.int32, device="cuda")
    out_b, lse_b, _ = lib.idx_sparse_attn_decode_static(s, inp.q_idx, inp.k_idx, inp.head_w, K, inp.q, inp.kv,
                                                        U.SCALE, k_scale=inp.k_scale, out_idx=idx_b)
    out_a, lse_a, _ = lib.idx_sparse_attn_decode(s, inp.q_idx, inp.k_idx, inp.head_w, K, inp.q, inp.kv, U.SCALE,
                                                 k_scale=inp.k_scale, out_idx=idx_a)
    torch.cuda.synchronize()
    U.log("static-scratch decode: %d tokens, ctx max %d, workspace %.1f MiB of %d MiB"
          % (T, int(call.ctx_len.max()),
             lib.idx_sparse_attn_workspace(s, inp.wl.H_I, inp.wl.d_I, inp.wl.H, K) / 2 ** 20,
             lib.IDX_STATIC_SCRATCH_BYTES >> 20))
    assert torch.equal(idx_a, idx_b)
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    return call, out_b, lse_b, idx_b


def test_static_scratch_decode_equals_workspace_decode_twice():
    # first call: 64 requests x 32768 positions (about 34 MiB of scratch)
    big = generate(Workload("static big", [32768] * 64, [{"seqs": list(range(64)), "q_len": None}], seed=61),
                   "cuda")
    _both(big)
    # second call, smaller (ragged contexts, fewer heads, smaller K): runs
    # over the first call's leftovers in the static buffer
    small = generate(Workload("static small", [5000, 700, 1, 2049, 130], [{"seqs": list(range(5)), "q_len": None}],
                              top_k=512, H=32, seed=62), "cuda")
    call, out, lse, idx = _both(small)
    # and the small call is right, not only equal
    w_idx, w_out, w_lse = U.oracle_rows(small, call, list(range(call.num_tokens)))
    U.check_indices(idx.cpu().numpy(), w_idx, "static small")
    U.check_attention(out.cpu().numpy(), lse.cpu().numpy(), w_out, w_lse, U.TOL_BF16, "static small")


def test_static_scratch_decode_rejects_a_batch_beyond_its_size():
    # 128 requests x 131072 positions need about 68 MiB of scratch
    ctx = torch.full((128,), 131072, dtype=torch.int32, device="cuda")
    s = lib.Seqs(ctx, None, max_q_len=1, max_ctx_len=131072, seq_stride=131072)
    need = lib.idx_sparse_attn_workspace(s, 64, 128, 128, 2048)
    assert need > lib.IDX_STATIC_SCRATCH_BYTES
    q_idx = torch.zeros((128, 64, 128), dtype=torch.bfloat16, device="cuda")
    k_idx = torch.zeros((1024, 128), dtype=torch.bfloat16, device="cuda")     # never read: rejected first
    w = torch.ones((128, 64), dtype=torch.float32, device="cuda")
    q = torch.zeros((128, 128, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1024, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.IdxError) as e:
        lib.idx_sparse_attn_decode_static(s, q_idx, k_idx, w, 2048, q, kv, U.SCALE)
    assert e.value.status == -5
