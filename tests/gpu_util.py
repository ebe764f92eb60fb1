"""Helpers for the GPU parity tests: run the library through the C ABI on a
generated workload, run the oracle on host copies of the same bytes, and
compare.  Nothing here computes any part of the method itself."""
import math
import sys
import time

import numpy as np
import torch

import oracle
from oracle import reference as R

import indexer_selected_sparse_idx_amd as lib

SCALE = 1.0 / math.sqrt(576.0)
TOL_BF16 = 2e-2
TOL_FP8 = 6e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bits16(t):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_raw(t):
    if t.dtype == torch.bfloat16:
        return bits16(t)
    return t.detach().contiguous().cpu().numpy()


def kdt(inp):
    return inp.wl.k_dtype


def kvdt(inp):
    return inp.wl.kv_dtype


def lib_seqs(inp, call, device="cuda"):
    ctx = torch.from_numpy(call.ctx_len.astype(np.int32)).to(device)
    cu = None if call.cu_q is None else torch.from_numpy(call.cu_q.astype(np.int32)).to(device)
    bt_np = inp.call_block_table(call)
    bt = None if bt_np is None else torch.from_numpy(bt_np.astype(np.int32)).to(device)
    s = lib.Seqs(ctx, cu, max_q_len=call.max_q_len, max_ctx_len=int(call.ctx_len.max()),
                 num_tokens=call.num_tokens, block_table=bt, page_size=inp.wl.page_size,
                 seq_stride=inp.seq_stride if not inp.wl.paged else 0)
    s._keep = (ctx, cu, bt)
    return s


def oracle_seqs(inp, call):
    return R.Seqs(ctx_len=call.ctx_len.astype(np.int64),
                  cu_q=None if call.cu_q is None else call.cu_q.astype(np.int64),
                  block_table=inp.call_block_table(call), page_size=inp.wl.page_size,
                  seq_stride=inp.seq_stride)


def run_fused(inp, call, want_idx=True):
    """Fused library call for one Call; returns (out, lse, idx) on the device."""
    s = lib_seqs(inp, call)
    sl = slice(call.tok_lo, call.tok_hi)
    T = call.num_tokens
    idx = torch.empty((T, inp.wl.top_k), dtype=torch.int32, device="cuda") if want_idx else None
    fn = lib.idx_sparse_attn_decode if call.is_decode else lib.idx_sparse_attn_prefill
    out, lse, idx = fn(s, inp.q_idx[sl], inp.k_idx, inp.head_w[sl], inp.wl.top_k, inp.q[sl], inp.kv,
                       SCALE, k_scale=inp.k_scale, out_idx=idx)
    return out, lse, idx


def token_positions(call):
    pos = []
    for b in range(len(call.ctx_len)):
        ql = 1 if call.cu_q is None else int(call.cu_q[b + 1] - call.cu_q[b])
        for i in range(ql):
            pos.append((b, int(call.ctx_len[b]) - ql + i))
    return pos


DECODED_CACHE_LIMIT = 1 << 30   # bytes of float64 kept decoded on the host per cache
MIRROR_LIMIT = 16 << 30         # raw bytes of a cache copied whole to the host


class _DeviceRows:
    """Rows of a device cache fetched on demand (caches too large to mirror)."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, rows):
        r = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.int64)).to(self.t.device)
        return host_raw(self.t.index_select(0, r))


def _mirror(t):
    return host_raw(t) if t.numel() * t.element_size() <= MIRROR_LIMIT else _DeviceRows(t)


def host_caches(inp):
    """Host copies of the index-key cache, its per-row scales and the latent
    cache (raw stored bytes), made once per generated workload; caches whose
    float64 form fits DECODED_CACHE_LIMIT are also kept decoded."""
    m = inp.extra.get("host")
    if m is None:
        m = {"k": _mirror(inp.k_idx), "kv": _mirror(inp.kv),
             "ks": None if inp.k_scale is None else inp.k_scale.cpu().numpy(), "kf": None, "kvf": None}
        if inp.k_idx.numel() * 8 <= DECODED_CACHE_LIMIT:
            m["kf"] = oracle.bf16_bits_to_f64(m["k"]) if kdt(inp) == "bf16" else oracle.e4m3_bytes_to_f64(m["k"])
        if kvdt(inp) == "bf16" and inp.kv.numel() * 8 <= DECODED_CACHE_LIMIT:
            m["kvf"] = oracle.bf16_bits_to_f64(m["kv"])
        inp.extra["host"] = m
    return m


def oracle_rows(inp, call, tokens):
    """Oracle indices + attention for selected tokens of a call, read from
    host copies of the caches (the stored bytes) and of each token's
    queries."""
    osq = oracle_seqs(inp, call)
    pos = token_positions(call)
    K = inp.wl.top_k
    hc = host_caches(inp)
    idx = np.empty((len(tokens), K), np.int32)
    outs, lses = [], []
    for r, tok in enumerate(tokens):
        b, t = pos[tok]
        g = call.tok_lo + tok
        phys = osq.physical_rows(b, np.arange(t + 1))
        if hc["kf"] is not None:
            keys = hc["kf"][phys]
        else:
            keys_raw = hc["k"][phys]
            keys = oracle.bf16_bits_to_f64(keys_raw) if kdt(inp) == "bf16" else oracle.e4m3_bytes_to_f64(keys_raw)
        ks = None if hc["ks"] is None else hc["ks"][phys]
        qi = oracle.bf16_bits_to_f64(bits16(inp.q_idx[g]))
        w = inp.head_w[g].cpu().numpy().astype(np.float64)
        s = oracle.indexer_scores(qi, keys, w, ks)
        idx[r] = oracle.topk_select(s, K)
        sel = idx[r][idx[r] >= 0].astype(np.int64)
        rphys = osq.physical_rows(b, sel)
        if hc["kvf"] is not None:
            rows = hc["kvf"][rphys]
        else:
            rows = R.decode_rows(hc["kv"][rphys], "bf16" if kvdt(inp) == "bf16" else "fp8_656", np.arange(len(sel)))
        o, l = oracle.sparse_attention(oracle.bf16_bits_to_f64(bits16(inp.q[g])), rows, SCALE)
        outs.append(o)
        lses.append(l)
    return idx, np.stack(outs), np.stack(lses)


def check_indices(got, want, context=""):
    """Valid entries of each row equal as sets; counts and -1 padding exact."""
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (got.shape, want.shape)
    for r in range(got.shape[0]):
        g = got[r]
        m = int((want[r] >= 0).sum())
        assert np.all(g[m:] == -1), "%s row %d: padding %s" % (context, r, g[m:m + 8])
        gs = np.sort(g[:m])
        ws = np.sort(want[r][:m])
        if not np.array_equal(gs, ws):
            diff = np.setxor1d(gs, ws)
            raise AssertionError("%s row %d: index sets differ (%d valid, %d differing, e.g. %s)"
                                 % (context, r, m, diff.size, diff[:8]))


def attn_error(got, want):
    """max |got - want| / RMS(want) over the whole array."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rms = math.sqrt(float(np.mean(want * want)))
    return float(np.max(np.abs(got - want))) / rms if rms > 0 else float(np.max(np.abs(got)))


def check_attention(got_out, got_lse, want_out, want_lse, tol, context=""):
    err = attn_error(got_out, want_out)
    log("%s: attention max-abs error %.3g x RMS (bound %.3g)" % (context, err, tol))
    assert err <= tol, "%s: max-abs error / RMS = %.4g > %.3g" % (context, err, tol)
    finite = np.isfinite(want_lse)
    assert np.array_equal(np.isfinite(got_lse), finite), context + ": lse finiteness"
    if finite.any():
        lerr = float(np.max(np.abs(np.asarray(got_lse)[finite] - want_lse[finite])))
        assert lerr <= tol, "%s: lse error %.3g" % (context, lerr)
    return err


class Timer:
    def __init__(self, label):
        self.label = label

    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        log("  %s: %.1fs" % (self.label, time.time() - self.t))
