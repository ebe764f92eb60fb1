"""The fused decode call captured in a HIP graph (torch.cuda.CUDAGraph over
the library's launches on the capturing stream): every replay, with eager
work on the same buffers between replays, reproduces the eager call bit for
bit.  The call records no memset node (its histogram clearing is a kernel)
and allocates nothing once its workspace is given."""
import math

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


@pytest.mark.parametrize("n,scale", [(2, 1 / 16), (4, 1 / 32)])
def test_decode_call_replays_from_a_graph(n, scale):
    import indexer_selected_sparse_idx_amd as lib
    wl = config(n, scale=scale)
    inp = generate(wl, "cuda")
    call = inp.calls[0]
    s = U.lib_seqs(inp, call)
    sl = slice(call.tok_lo, call.tok_hi)
    T = call.num_tokens
    out = torch.empty((T, wl.H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, wl.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device="cuda")
    ws = torch.empty(lib.idx_sparse_attn_workspace(s, wl.H_I, wl.d_I, wl.H, wl.top_k), dtype=torch.uint8,
                     device="cuda")

    def step():
        lib.idx_sparse_attn_decode(s, inp.q_idx[sl], inp.k_idx, inp.head_w[sl], wl.top_k, inp.q[sl], inp.kv,
                                   1.0 / math.sqrt(576.0), k_scale=inp.k_scale, out=out, lse=lse, out_idx=idx, ws=ws)

    step()
    torch.cuda.synchronize()
    want = (out.clone(), lse.clone(), idx.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(7.0)
        lse.zero_()
        idx.fill_(-7)
        ws.fill_(0xA5)  # the workspace holds nothing across calls
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, want[2]), "replay %d: indices" % r
        assert torch.equal(out, want[0]) and torch.equal(lse, want[1]), "replay %d: attention" % r
        U.log("%s replay %d equals the eager call" % (wl.name, r))
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(idx, want[2]) and torch.equal(out, want[0])
    del g
