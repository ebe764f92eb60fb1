"""Entry points called from two host threads at once, each on its own
stream with its own workspace and outputs (the library keeps no state
between calls): every result equals the one computed alone."""
import math
import threading

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


def test_two_host_threads_two_streams():
    import indexer_selected_sparse_idx_amd as lib
    jobs = []
    for n, scale in ((2, 1 / 16), (4, 1 / 32)):
        wl = config(n, scale=scale)
        inp = generate(wl, "cuda")
        call = inp.calls[0]
        jobs.append((wl, inp, call, U.lib_seqs(inp, call)))

    def run(job):
        wl, inp, call, s = job
        sl = slice(call.tok_lo, call.tok_hi)
        idx = torch.empty((call.num_tokens, wl.top_k), dtype=torch.int32, device="cuda")
        return lib.idx_sparse_attn_decode(s, inp.q_idx[sl], inp.k_idx, inp.head_w[sl], wl.top_k, inp.q[sl], inp.kv,
                                          1.0 / math.sqrt(576.0), k_scale=inp.k_scale, out_idx=idx)

    want = []
    for job in jobs:
        out, lse, idx = run(job)
        torch.cuda.synchronize()
        want.append((out.clone(), lse.clone(), idx.clone()))

    got = [[None] * 8 for _ in jobs]
    errors = []

    def worker(j):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for r in range(8):
                    got[j][r] = run(jobs[j])
            stream.synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for j, job in enumerate(jobs):
        for r in range(8):
            out, lse, idx = got[j][r]
            assert torch.equal(idx, want[j][2]), "%s call %d: indices" % (job[0].name, r)
            assert torch.equal(out, want[j][0]) and torch.equal(lse, want[j][1]), "%s call %d" % (job[0].name, r)
        U.log("%s: 8 calls from its own thread equal the call alone" % job[0].name)
