"""Seeded synthetic workloads for index-selected sparse latent attention.

Value distributions follow the workload statements that accompany the
method (integer-valued index queries and keys, power-of-two head weights,
standard-normal latent rows and attention queries): integer inputs make the
fp32 indexer scores exact, so Top-K parity can be bit-exact.

Layout of what `generate` returns (all on `device`):

* q_idx  [T, H_I, d_I] bf16          index queries, integers in [-q_range, q_range]
* head_w [T, H_I] fp32               2^-r, r uniform in {0, 1, 2, 3}
* q      [T, H, 576] bf16            attention queries ~ N(0, 1)
* k_idx  [rows, d_I] bf16, or uint8 holding OCP e4m3 codes
* k_scale[rows] fp32 or None         per-row key scale (powers of two)
* kv     [rows, 576] bf16, or uint8 [rows, 656] packed FP8 latent rows:
         512 e4m3 codes, 4 fp32 tile scales (amax / 448 of each 128-wide
         tile), 64 bf16 rope values.

A row of a contiguous cache is `b * seq_stride + s`; a row of a paged cache is
`page * page_size + s % page_size` with `page = block_table[b, s // page_size]`.
Tokens of every call sit consecutively in q_idx / head_w / q.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

LATENT, ROPE, ROW = 512, 64, 576
FP8_ROW_BYTES = 656
E4M3_MAX = 448.0


@dataclass
class Call:
    """One library call: the sequences it covers and their token slice."""
    seq_ids: List[int]
    ctx_len: np.ndarray                 # int32 [B]
    cu_q: Optional[np.ndarray]          # int32 [B + 1]; None => one token per sequence
    tok_lo: int
    tok_hi: int

    @property
    def num_tokens(self):
        return self.tok_hi - self.tok_lo

    @property
    def is_decode(self):
        return self.cu_q is None

    @property
    def max_q_len(self):
        return 1 if self.cu_q is None else int(np.max(np.diff(self.cu_q)))


@dataclass
class Workload:
    name: str
    ctx_len: List[int]                  # cache rows per sequence
    calls: List[dict]                   # {"seqs": [...], "q_len": [...] | None}
    H_I: int = 64
    d_I: int = 128
    H: int = 128
    top_k: int = 2048
    k_dtype: str = "bf16"               # "bf16" | "e4m3"
    kv_dtype: str = "bf16"              # "bf16" | "fp8_656"
    paged: bool = False
    page_size: int = 64
    q_range: int = 4
    k_range: int = 4
    k_scale: bool = False
    seed: int = 0
    note: str = ""

    def tokens(self):
        n = 0
        for c in self.calls:
            n += len(c["seqs"]) if c["q_len"] is None else int(sum(c["q_len"]))
        return n


@dataclass
class Inputs:
    wl: Workload
    calls: List[Call]
    q_idx: torch.Tensor
    head_w: torch.Tensor
    q: torch.Tensor
    k_idx: torch.Tensor
    k_scale: Optional[torch.Tensor]
    kv: torch.Tensor
    seq_stride: int
    block_table: Optional[np.ndarray]   # int32 [n_seqs, width] (global sequence ids)
    extra: dict = field(default_factory=dict)

    def call_block_table(self, call):
        if self.block_table is None:
            return None
        return np.ascontiguousarray(self.block_table[call.seq_ids])


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def lognormal_context_lengths(n, seed, median=8192, sigma=1.0, lo=1024, hi=131072):
    rng = np.random.default_rng(seed)
    x = np.exp(rng.normal(np.log(median), sigma, size=n))
    return np.clip(np.rint(x), lo, hi).astype(np.int64), rng


def config(n, scale=1.0):
    """Workload n (1..5).  `scale` < 1 shrinks context lengths and token
    counts for quick parity runs while keeping the structure."""
    if n == 1:
        L = max(16, int(2048 * scale))
        return Workload("tiny-prefill L=%d" % L, [L], [{"seqs": [0], "q_len": [L]}],
                        H_I=4, d_I=64, H=8, top_k=128, seed=1)
    if n == 2:
        B = 64 if scale >= 1 else max(2, int(64 * scale))
        ctx = max(64, int(32768 * scale))
        return Workload("decode-batch B=%d ctx=%d" % (B, ctx), [ctx] * B,
                        [{"seqs": list(range(B)), "q_len": None}], seed=2)
    if n == 3:
        L = max(256, int(65536 * scale))
        chunk = max(64, int(4096 * scale))
        calls = []
        for lo in range(0, L, chunk):
            hi = min(L, lo + chunk)
            calls.append({"seqs": [0], "q_len": [hi - lo], "ctx": [hi]})
        return Workload("long-prefill L=%d chunk=%d" % (L, chunk), [L], calls, seed=3)
    if n == 4:
        B = 128 if scale >= 1 else max(2, int(128 * scale))
        ctx = max(64, int(131072 * scale))
        return Workload("fp8-decode B=%d ctx=%d" % (B, ctx), [ctx] * B,
                        [{"seqs": list(range(B)), "q_len": None}],
                        k_dtype="e4m3", kv_dtype="fp8_656", k_range=8, seed=4)
    if n == 5:
        n_req, n_pre, q_pre = 256, 32, 512
        ctx, _ = lognormal_context_lengths(n_req, seed=5)
        if scale < 1:
            n_req, n_pre = max(4, int(256 * scale)), max(2, int(32 * scale))
            q_pre = max(8, int(512 * scale))
            ctx = np.maximum(np.rint(ctx[:n_req] * scale).astype(np.int64), q_pre)
        calls = [{"seqs": list(range(n_pre)), "q_len": [q_pre] * n_pre},
                 {"seqs": list(range(n_pre, n_req)), "q_len": None}]
        return Workload("mixed-paged B=%d" % n_req, [int(c) for c in ctx], calls,
                        paged=True, page_size=64, seed=5)
    raise ValueError(n)


CONFIGS = {n: config(n) for n in range(1, 6)}


# --------------------------------------------------------------------------
# generation
# --------------------------------------------------------------------------

def _ints(gen, shape, r, dtype, device):
    x = torch.randint(-r, r + 1, shape, generator=gen, device=device, dtype=torch.int32)
    return x.to(torch.float32).to(dtype)


def _pow2(e):
    """2**e for small integer tensors e, built from the fp32 exponent bits."""
    return ((e + 127) << 23).to(torch.int32).view(torch.float32)


def _fp8_rows(gen, n, device):
    """Packed FP8 latent rows for n positions (see module docstring)."""
    x = torch.randn((n, LATENT), generator=gen, device=device, dtype=torch.float32)
    tiles = x.view(n, LATENT // 128, 128)
    amax = tiles.abs().amax(dim=2)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    codes = (tiles / scale[:, :, None]).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    rope = torch.randn((n, ROPE), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    out = torch.empty((n, FP8_ROW_BYTES), dtype=torch.uint8, device=device)
    out[:, :LATENT] = codes.view(n, LATENT).view(torch.uint8)
    out[:, LATENT:LATENT + 16] = scale.contiguous().view(torch.uint8).view(n, 16)
    out[:, LATENT + 16:] = rope.contiguous().view(torch.uint8).view(n, 128)
    return out




def mxfp8_keys(gen, n, device, k_range=8, e8_lo=121, e8_hi=123):
    """MXFP8 index keys for n positions, as (codes uint8 [n, 128], E8M0
    block exponents uint8 [n, 4]): the codes hold 32 k for
    integers k uniform in [-k_range, k_range] (exact E4M3 values for
    k_range <= 14), and each block of 32 takes an E8M0 byte uniform in
    [e8_lo, e8_hi], so a key decodes to k * 2^(byte - 122).  With the default
    ranges, integer queries in [-4, 4] and head weights 2^-3 .. 1, every
    partial sum of the indexer score fits fp32's 24 bits (at most 2^19 in
    steps of 2^-4), so the scores are exact."""
    k = torch.randint(-k_range, k_range + 1, (n, 128), generator=gen, device=device)
    codes = (k.float() * 32.0).to(torch.float8_e4m3fn).view(torch.uint8)
    e8 = torch.randint(e8_lo, e8_hi + 1, (n, 4), generator=gen, device=device).to(torch.uint8)
    return codes.contiguous(), e8.contiguous()


def generate(wl, device="cpu", chunk_rows=1 << 20):
    """Draw every tensor of workload `wl` on `device` (seeded by wl.seed)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(wl.seed))
    rng = np.random.default_rng(1000 + int(wl.seed))
    n_seqs = len(wl.ctx_len)

    # ---- cache geometry ------------------------------------------------
    block_table = None
    if wl.paged:
        pages_per = [-(-c // wl.page_size) for c in wl.ctx_len]
        total = int(sum(pages_per))
        perm = rng.permutation(total).astype(np.int32)
        width = max(pages_per)
        block_table = np.full((n_seqs, width), -1, dtype=np.int32)
        k = 0
        for b, npg in enumerate(pages_per):
            block_table[b, :npg] = perm[k:k + npg]
            k += npg
        n_rows = total * wl.page_size
        seq_stride = 0
    else:
        seq_stride = int(max(wl.ctx_len))
        n_rows = n_seqs * seq_stride

    # ---- caches ----------------------------------------------------------
    if wl.k_dtype == "bf16":
        k_idx = torch.empty((n_rows, wl.d_I), dtype=torch.bfloat16, device=device)
    else:
        k_idx = torch.empty((n_rows, wl.d_I), dtype=torch.uint8, device=device)
    for lo in range(0, n_rows, chunk_rows):
        hi = min(n_rows, lo + chunk_rows)
        if wl.k_dtype == "bf16":
            k_idx[lo:hi] = _ints(gen, (hi - lo, wl.d_I), wl.k_range, torch.bfloat16, device)
        else:
            v = _ints(gen, (hi - lo, wl.d_I), wl.k_range, torch.float32, device)
            k_idx[lo:hi] = v.to(torch.float8_e4m3fn).view(torch.uint8)
    k_scale = None
    if wl.k_scale:
        r = torch.randint(-2, 3, (n_rows,), generator=gen, device=device, dtype=torch.int32)
        k_scale = _pow2(r)
    if wl.kv_dtype == "bf16":
        kv = torch.empty((n_rows, ROW), dtype=torch.bfloat16, device=device)
        for lo in range(0, n_rows, chunk_rows):
            hi = min(n_rows, lo + chunk_rows)
            kv[lo:hi] = torch.randn((hi - lo, ROW), generator=gen, device=device).to(torch.bfloat16)
    else:
        kv = torch.empty((n_rows, FP8_ROW_BYTES), dtype=torch.uint8, device=device)
        for lo in range(0, n_rows, chunk_rows // 2):
            hi = min(n_rows, lo + chunk_rows // 2)
            kv[lo:hi] = _fp8_rows(gen, hi - lo, device)

    # ---- calls and per-token inputs ----------------------------------------
    calls = []
    tok = 0
    for c in wl.calls:
        seqs = list(c["seqs"])
        ctx = np.array(c.get("ctx", [wl.ctx_len[s] for s in seqs]), dtype=np.int32)
        if c["q_len"] is None:
            cu = None
            ntok = len(seqs)
        else:
            cu = np.concatenate([[0], np.cumsum(c["q_len"])]).astype(np.int32)
            ntok = int(cu[-1])
        calls.append(Call(seqs, ctx, cu, tok, tok + ntok))
        tok += ntok
    T = tok
    q_idx = torch.empty((T, wl.H_I, wl.d_I), dtype=torch.bfloat16, device=device)
    q = torch.empty((T, wl.H, ROW), dtype=torch.bfloat16, device=device)
    step = max(1, chunk_rows // max(1, wl.H * ROW // 64))
    for lo in range(0, T, step):
        hi = min(T, lo + step)
        q_idx[lo:hi] = _ints(gen, (hi - lo, wl.H_I, wl.d_I), wl.q_range, torch.bfloat16, device)
    r = torch.randint(0, 4, (T, wl.H_I), generator=gen, device=device, dtype=torch.int32)
    head_w = _pow2(-r)
    for lo in range(0, T, step):
        hi = min(T, lo + step)
        q[lo:hi] = torch.randn((hi - lo, wl.H, ROW), generator=gen, device=device).to(torch.bfloat16)
    return Inputs(wl, calls, q_idx, head_w, q, k_idx, k_scale, kv, seq_stride, block_table)
