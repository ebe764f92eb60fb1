"""C-ABI contract tests that need no GPU.

The library must load without a device, export every function declared in
include/idxsparse.h, and reject bad arguments with the documented status
BEFORE launching anything.  Every call below carries at least one argument
error, so the fake (never dereferenced) device addresses are never used.
"""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "idxsparse.h")


@pytest.fixture(scope="module")
def L():
    import indexer_selected_sparse_idx_amd as m
    if not os.path.exists(m.lib_path):
        from indexer_selected_sparse_idx_amd import build
        build.build()
    return m.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ["idx_score_topk", "sparse_mla_attn", "idx_sparse_attn_prefill",
                 "idx_sparse_attn_decode", "idx_score_topk_workspace",
                 "sparse_mla_attn_workspace", "idx_sparse_attn_workspace",
                 "idx_status_string", "idx_timer_arm", "idx_kv_fp8_write", "idx_key_fp8_write"]:
        assert want in names


def test_library_exports_every_declared_symbol(L):
    import indexer_selected_sparse_idx_amd as m
    out = subprocess.run(["nm", "-D", "--defined-only", m.lib_path], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_status_strings(L):
    import indexer_selected_sparse_idx_amd as m
    for code in (0, -1, -2, -3, -4, 7):
        s = m.idx_status_string(code)
        assert isinstance(s, str) and s
    assert m.idx_status_string(-3).startswith("IDX_ERR_WORKSPACE")


# ---- argument checks ----------------------------------------------------------

FAKE = 1 << 20          # 16-byte aligned stand-in address, never dereferenced
MIS = FAKE + 2          # misaligned


def seqs(**kw):
    from indexer_selected_sparse_idx_amd._binding import _IdxSeqs
    d = dict(num_seqs=2, num_tokens=2, cu_q=None, ctx_len=FAKE, max_q_len=1, max_ctx_len=100,
             block_table=None, bt_stride=0, page_size=64, seq_stride=128)
    d.update(kw)
    return _IdxSeqs(**d)


def score(L, s, **kw):
    a = dict(q=FAKE, qdt=1, k=FAKE, kdt=1, ks=None, w=FAKE, H_I=64, d_I=128, K=2048,
             out=FAKE, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return L.idx_score_topk(ctypes.byref(s), a["q"], a["qdt"], a["k"], a["kdt"], a["ks"], a["w"],
                            a["H_I"], a["d_I"], a["K"], a["out"], a["ws"], a["wsb"], None)


def attn(L, s, **kw):
    a = dict(q=FAKE, H=128, kv=FAKE, kvdt=1, idx=FAKE, K=2048, scale=1 / 24, out=FAKE, lse=None,
             ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return L.sparse_mla_attn(ctypes.byref(s), a["q"], a["H"], a["kv"], a["kvdt"], a["idx"], a["K"],
                             a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(w=None), -1), (dict(out=None), -1),
    (dict(q=MIS), -1), (dict(k=MIS), -1),
    (dict(H_I=0), -1), (dict(K=0), -1),
    (dict(H_I=65), -2), (dict(d_I=96), -2), (dict(K=2049), -2), (dict(qdt=2), -2), (dict(kdt=3), -2),
    (dict(ws=None), -3), (dict(wsb=10), -3),
])
def test_score_topk_rejects(L, kw, status):
    assert score(L, seqs(), **kw) == status


@pytest.mark.parametrize("skw", [
    dict(num_seqs=0), dict(ctx_len=None), dict(max_q_len=0), dict(max_ctx_len=0),
    dict(num_tokens=3),                               # decode batch must have T == B
    dict(seq_stride=99),                              # contiguous rows shorter than max_ctx_len
    dict(block_table=FAKE, bt_stride=2, page_size=48),  # page size not a power of two
    dict(block_table=FAKE, bt_stride=1, page_size=64),  # block table too narrow for max_ctx_len
    dict(cu_q=FAKE, num_tokens=5, max_q_len=101),     # q_len bound above ctx bound
])
def test_bad_batches_rejected(L, skw):
    assert score(L, seqs(**skw)) == -1
    assert attn(L, seqs(**skw)) == -1


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(kv=None), -1), (dict(idx=None), -1), (dict(out=None), -1),
    (dict(out=MIS), -1), (dict(H=0), -1), (dict(K=0), -1), (dict(scale=float("nan")), -1),
    (dict(scale=0.0), -1), (dict(scale=-0.5), -1), (dict(scale=float("inf")), -1),
    (dict(H=129), -2), (dict(kvdt=2), -2), (dict(K=4096), -2),
    (dict(ws=None), -3), (dict(wsb=100), -3),
])
def test_sparse_mla_attn_rejects(L, kw, status):
    assert attn(L, seqs(), **kw) == status


def test_decode_requires_one_token_per_sequence(L):
    s = seqs(cu_q=FAKE, num_tokens=2)
    rc = L.idx_sparse_attn_decode(ctypes.byref(s), FAKE, 1, FAKE, 1, None, FAKE, 64, 128, 2048,
                                  FAKE, 128, FAKE, 1, 1 / 24, FAKE, None, None, FAKE, 1 << 40, None)
    assert rc == -1


def test_fused_workspace_check(L):
    s = seqs()
    need = L.idx_sparse_attn_workspace(ctypes.byref(s), 64, 128, 128, 2048)
    assert need > 0
    rc = L.idx_sparse_attn_prefill(ctypes.byref(s), FAKE, 1, FAKE, 1, None, FAKE, 64, 128, 2048,
                                   FAKE, 128, FAKE, 1, 1 / 24, FAKE, None, None, FAKE, need - 1, None)
    assert rc == -3


def test_static_decode_rejects_calls_beyond_its_scratch(L):
    # 64 requests x 2,000,000 positions: the score rows alone exceed the
    # 64 MiB static buffer, so the call fails before touching the device
    s = seqs(num_seqs=64, num_tokens=64, max_ctx_len=2_000_000, seq_stride=2_000_000)
    assert L.idx_sparse_attn_workspace(ctypes.byref(s), 64, 128, 128, 2048) > 64 << 20
    rc = L.idx_sparse_attn_decode_static(ctypes.byref(s), FAKE, 1, FAKE, 1, None, FAKE, 64, 128, 2048,
                                         FAKE, 128, FAKE, 1, 1 / 24, FAKE, None, None, None)
    assert rc == -5
    import indexer_selected_sparse_idx_amd as m
    assert m.idx_status_string(-5).startswith("IDX_ERR_TOO_LARGE")
    # argument errors come first, as for the other entry points
    bad = seqs(cu_q=FAKE, num_tokens=2)
    assert L.idx_sparse_attn_decode_static(ctypes.byref(bad), FAKE, 1, FAKE, 1, None, FAKE, 64, 128, 2048,
                                           FAKE, 128, FAKE, 1, 1 / 24, FAKE, None, None, None) == -1


def test_workspace_sizes(L):
    s = seqs(num_seqs=3, num_tokens=3, max_ctx_len=1000, seq_stride=1000)
    # one fp32 score row per token padded to 64 columns, one 2048-bin key
    # histogram per token and two counts per 2048-key chunk of a row, each
    # part rounded to 256 bytes
    up = lambda b: -(-b // 256) * 256
    want = up(3 * 1024 * 4) + up(3 * 2048 * 4) + up(3 * 1 * 8)
    assert L.idx_score_topk_workspace(ctypes.byref(s), 64, 128, 2048) == want
    assert L.sparse_mla_attn_workspace(ctypes.byref(s), 128, 2048) > 0     # decode splits
    big = seqs(num_seqs=1, num_tokens=4096, cu_q=FAKE, max_q_len=4096, max_ctx_len=8192,
               seq_stride=8192)
    assert L.sparse_mla_attn_workspace(ctypes.byref(big), 128, 2048) == 0  # no split needed


def test_prefill_workspace_is_bounded(L):
    # prefill batches (max_q_len >= 9) run the selecting prefill kernel with
    # at most 256 workgroups taking token blocks from a counter: the
    # workspace is 8 candidate rows per workgroup (one (key, position) pair
    # per position plus a spare pair, padded to 64 positions) and the
    # counter, whatever the token count
    up = lambda b: -(-b // 256) * 256
    for T in (4096, 16384):
        s = seqs(num_seqs=1, num_tokens=T, cu_q=FAKE, max_q_len=T, max_ctx_len=65536, seq_stride=65536)
        assert L.idx_score_topk_workspace(ctypes.byref(s), 64, 128, 2048) == up(2048 * 2 * 65600 * 4) + 256
    s = seqs(num_seqs=32, num_tokens=32 * 512, cu_q=FAKE, max_q_len=512, max_ctx_len=131072, seq_stride=131072)
    assert L.idx_score_topk_workspace(ctypes.byref(s), 64, 128, 2048) == up(2048 * 2 * 131136 * 4) + 256
    # a short prefill batch: one workgroup per token block (2 sequences x 3)
    s = seqs(num_seqs=2, num_tokens=40, cu_q=FAKE, max_q_len=20, max_ctx_len=1000, seq_stride=1000)
    assert L.idx_score_topk_workspace(ctypes.byref(s), 64, 128, 2048) == up(6 * 8 * 2 * 1024 * 4) + 256


def test_timer_arm_rejects_bad_kernel(L):
    assert L.idx_timer_arm(9, FAKE, FAKE) == -1
    assert L.idx_timer_arm(0, None, FAKE) == -1


def test_mxfp8_keys_checks(L):
    s = seqs()
    # a bad workspace comes last: every MXFP8 case that passes the argument
    # checks reaches the workspace check (-3), so nothing is launched
    assert score(L, s, kdt=4, ks=FAKE, ws=None, wsb=0) == -3           # accepted: decode, d_I 128
    assert score(L, s, kdt=4, ks=FAKE + 4, ws=None, wsb=0) == -3       # exponent rows: 4-byte alignment
    assert score(L, s, kdt=4, ks=FAKE + 2) == -1                        # exponents not 4-byte aligned
    assert score(L, s, kdt=4) == -1                                     # exponents required
    assert score(L, s, kdt=4, ks=FAKE, k=FAKE + 4) == -1                # codes 16-byte aligned
    assert score(L, s, kdt=4, ks=FAKE, d_I=64) == -2                    # d_I 128 only
    sp = seqs(cu_q=FAKE, num_seqs=1, num_tokens=8, max_q_len=8)
    assert score(L, sp, kdt=4, ks=FAKE, ws=None, wsb=0) == -3           # prefill batches accepted too


def test_kv_fp8_write_rejects(L):
    # host-side checks only: nothing is launched for any of these
    assert L.idx_kv_fp8_write(FAKE, -1, FAKE, FAKE, None) == -1         # negative row count
    assert L.idx_kv_fp8_write(None, 4, FAKE, FAKE, None) == -1          # null source
    assert L.idx_kv_fp8_write(FAKE, 4, None, FAKE, None) == -1          # null row map
    assert L.idx_kv_fp8_write(FAKE, 4, FAKE, None, None) == -1          # null cache
    assert L.idx_kv_fp8_write(FAKE + 8, 4, FAKE, FAKE, None) == -1      # misaligned source
    assert L.idx_kv_fp8_write(FAKE, 4, FAKE, FAKE + 8, None) == -1      # misaligned cache
    assert L.idx_kv_fp8_write(FAKE, 4, FAKE + 2, FAKE, None) == -1      # misaligned row map
    assert L.idx_kv_fp8_write(None, 0, None, None, None) == 0           # no rows: no-op


def test_key_fp8_write_rejects(L):
    assert L.idx_key_fp8_write(FAKE, 4, 96, FAKE, FAKE, None, None) == -1     # d_I not 64 or 128
    assert L.idx_key_fp8_write(FAKE, -1, 128, FAKE, FAKE, None, None) == -1   # negative row count
    assert L.idx_key_fp8_write(None, 4, 128, FAKE, FAKE, None, None) == -1    # null source
    assert L.idx_key_fp8_write(FAKE, 4, 128, None, FAKE, None, None) == -1    # null row map
    assert L.idx_key_fp8_write(FAKE, 4, 128, FAKE, None, None, None) == -1    # null cache
    assert L.idx_key_fp8_write(FAKE + 8, 4, 128, FAKE, FAKE, None, None) == -1
    assert L.idx_key_fp8_write(FAKE, 4, 128, FAKE, FAKE + 4, None, None) == -1
    assert L.idx_key_fp8_write(FAKE, 4, 128, FAKE, FAKE, FAKE + 2, None) == -1  # misaligned scales
    assert L.idx_key_fp8_write(None, 0, 64, None, None, None, None) == 0      # no rows: no-op


def test_empty_batch_is_a_no_op(L):
    # T = 0: every entry point returns IDX_OK without launching anything
    s = seqs(cu_q=FAKE, num_tokens=0)
    assert score(L, s, ws=None, wsb=0) == 0
    assert attn(L, s, ws=None, wsb=0) == 0
    rc = L.idx_sparse_attn_prefill(ctypes.byref(s), FAKE, 1, FAKE, 1, None, FAKE, 64, 128, 2048,
                                   FAKE, 128, FAKE, 1, 1 / 24, FAKE, None, None, None, 0, None)
    assert rc == 0
