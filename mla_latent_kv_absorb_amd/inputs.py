"""Seeded synthetic inputs for MLA decode.

This module only draws and lays out inputs.  It holds none of the attention
arithmetic, and serves both the GPU path (which receives the paged pool) and
the CPU oracle (which receives the logical per-request arrays).

Workloads (sizes follow DeepSeek-V2's MLA: 128 heads, latent 512, rotary key
64, content/value head dim 128; 64-token pages):

  tiny_fp32     1 request x 64 tokens, 4 heads, latent 16, rope 8, head dim 8,
                float32 everything, scale 1/sqrt(16)
  v2_single     1 request x 4,096 tokens, BF16 cache, pages in random order
  v2_batched    64 requests, lengths uniform in [16,384, 32,768], pages
                shuffled across one shared pool
  v2_long       1 request x 131,072 tokens; one independent seeded draw per
                layer (seed 4000 + layer)
  v2_fp8_topk   32 requests x 65,536 tokens, latent stored as FP8 E4M3 with
                one float32 scale per token, rotary key in BF16, each request
                reads a sorted list of 2,048 distinct positions
  v2_fp8g_topk  the same draw (same seed), the latent stored as FP8 E4M3 with
                one float32 scale per 128 latent channels of each token

Values: latents, rotary keys and queries ~ N(0, 1); W_UK and W_UV ~ N(0, 1/D_C)
(variance 1/D_C).  BF16 configs round every drawn value to BF16 with
round-to-nearest-even; the oracle receives exactly the rounded values.

Draw order (one numpy PCG64 generator per workload and seed): sequence
lengths, page permutation, c_kv, k_rope, q_nope, q_rope, W_UK, W_UV, top-k
lists.

FP8 encoding of the latent (a data-preparation step, not part of decode):
per token (or per group of 128 consecutive channels of a token) the scale is
max|c|/448 over the token (group), and each element is rounded to the nearest
E4M3 value (ties to the even code), saturating at +-448.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

PAGE_TOKENS = 64

DTYPE_F32 = "f32"
DTYPE_BF16 = "bf16"
DTYPE_FP8 = "fp8_e4m3"
DTYPE_FP8_G128 = "fp8_e4m3_g128"
FP8_GROUP = 128
FP8_DTYPES = (DTYPE_FP8, DTYPE_FP8_G128)

WORKLOADS = {
    "tiny_fp32": dict(H=4, D_C=16, D_R=8, D_N=8, D_V=8, B=1, ctx=(64, 64),
                      cache=DTYPE_F32, act=DTYPE_F32, seed=1, topk=0),
    "v2_single": dict(H=128, D_C=512, D_R=64, D_N=128, D_V=128, B=1, ctx=(4096, 4096),
                      cache=DTYPE_BF16, act=DTYPE_BF16, seed=2, topk=0),
    "v2_batched": dict(H=128, D_C=512, D_R=64, D_N=128, D_V=128, B=64, ctx=(16384, 32768),
                       cache=DTYPE_BF16, act=DTYPE_BF16, seed=3, topk=0),
    "v2_long": dict(H=128, D_C=512, D_R=64, D_N=128, D_V=128, B=1, ctx=(131072, 131072),
                    cache=DTYPE_BF16, act=DTYPE_BF16, seed=4000, topk=0, layers=60),
    "v2_fp8_topk": dict(H=128, D_C=512, D_R=64, D_N=128, D_V=128, B=32, ctx=(65536, 65536),
                        cache=DTYPE_FP8, act=DTYPE_BF16, seed=5, topk=2048),
    "v2_fp8g_topk": dict(H=128, D_C=512, D_R=64, D_N=128, D_V=128, B=32, ctx=(65536, 65536),
                         cache=DTYPE_FP8_G128, act=DTYPE_BF16, seed=5, topk=2048),
}


@dataclasses.dataclass
class DecodeInputs:
    """Logical inputs of one decode step (all requests of one layer)."""
    H: int
    D_C: int
    D_R: int
    D_N: int
    D_V: int
    cache_dtype: str
    act_dtype: str
    scale: float
    seq_lens: np.ndarray          # int32 [B]
    offsets: np.ndarray           # int64 [B+1], request b owns rows offsets[b]:offsets[b+1]
    c_kv: np.ndarray              # float32 [sum T, D_C]; for FP8 the pre-quantisation values
    k_rope: np.ndarray            # float32 [sum T, D_R]
    q_nope: np.ndarray            # float32 [B, H, D_N]
    q_rope: np.ndarray            # float32 [B, H, D_R]
    w_uk: np.ndarray              # float32 [H, D_C, D_N]
    w_uv: np.ndarray              # float32 [H, D_V, D_C]
    page_perm: np.ndarray         # int64 [total pages]: logical page -> physical page
    c_codes: Optional[np.ndarray] = None   # uint8 [sum T, D_C] (FP8 cache)
    c_scales: Optional[np.ndarray] = None  # float32 [sum T], or [sum T, D_C / 128] with group scales
    topk_idx: Optional[np.ndarray] = None  # int32 [B, k] sorted, -1 padded

    @property
    def B(self) -> int:
        return int(self.seq_lens.shape[0])

    def request(self, b: int):
        """Logical arrays of request b: (c_kv or (codes, scales), k_rope, q_nope, q_rope)."""
        lo, hi = int(self.offsets[b]), int(self.offsets[b + 1])
        return lo, hi

    def pages_of(self, b: int) -> int:
        return -(-int(self.seq_lens[b]) // PAGE_TOKENS)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest BF16 value (ties to even); returns
    float32 holding exactly the BF16 values.  Inputs are finite.  Uses torch's
    CPU conversion (same rounding, checked in the tests) when available."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    try:
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    u = x.view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) of float32 values that are already BF16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


# E4M3 encode (data preparation only).  Positive finite values of the format,
# indexed by code 0x00..0x7E.
def _e4m3_positive_table() -> np.ndarray:
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        vals[code] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_POS = _e4m3_positive_table()


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """Round values to the nearest E4M3 code (ties to the even code),
    saturating at +-448.  Returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_E4M3_POS, a, side="left")      # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_hi = _E4M3_POS[hi] - a
    d_lo = a - _E4M3_POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == 0, 0, code).astype(np.uint8)
    sign = np.where(np.signbit(x) & (a > 0), 0x80, 0).astype(np.uint8)
    return code | sign


def quantize_fp8_per_token(c: np.ndarray, chunk_rows: int = 1 << 18):
    """Per-token scale = max|c| / 448, codes = E4M3(c / scale) rounded to the
    nearest value (ties to even), quotients clamped to +-448.  The quotient is
    formed in float32.  Uses torch's CPU float8 conversion when torch is
    present (same rounding as encode_e4m3, checked in the tests)."""
    amax = _row_amax(c).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return _encode_scaled(c, scale[:, None], chunk_rows), scale


def _row_amax(c: np.ndarray) -> np.ndarray:
    """max |c| over each row (exact; torch's threaded CPU reduction when torch
    is present)."""
    try:
        import torch
        return torch.from_numpy(np.ascontiguousarray(c)).abs().amax(dim=1).numpy()
    except ImportError:  # pragma: no cover
        return np.max(np.abs(c), axis=1)


def quantize_fp8_per_group(c: np.ndarray, group: int = FP8_GROUP, chunk_rows: int = 1 << 18):
    """As quantize_fp8_per_token, with one scale per group of ``group``
    consecutive channels of a token: scales [T, D_C / group]."""
    T, D = c.shape
    assert D % group == 0
    amax = np.max(np.abs(c.reshape(T, D // group, group)), axis=2).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return _encode_scaled(c, np.repeat(scale, group, axis=1), chunk_rows), scale


def _encode_scaled(c: np.ndarray, scale: np.ndarray, chunk_rows: int):
    """E4M3 codes of c / scale (scale broadcast over rows [T, 1] or given per
    element [T, D]), quotient in float32, clamped to +-448."""
    codes = np.empty(c.shape, dtype=np.uint8)
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    for lo in range(0, c.shape[0], chunk_rows):
        hi = min(lo + chunk_rows, c.shape[0])
        if torch is not None:
            x = torch.from_numpy(np.ascontiguousarray(c[lo:hi])) / torch.from_numpy(np.ascontiguousarray(scale[lo:hi]))
            codes[lo:hi] = x.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        else:
            x = np.clip(c[lo:hi] / scale[lo:hi], -448.0, 448.0)
            codes[lo:hi] = encode_e4m3(x)
    return codes


def make_inputs(name: str, seed: Optional[int] = None, *, batch: Optional[int] = None,
                ctx: Optional[tuple] = None, seq_lens=None, topk: Optional[int] = None,
                layer: int = 0, dims: Optional[dict] = None) -> DecodeInputs:
    """Draw one workload.  ``batch``, ``ctx`` (lo, hi), ``seq_lens``, ``topk``
    and ``dims`` override the named workload to make smaller test cases with the
    same distributions."""
    spec = dict(WORKLOADS[name])
    if dims:
        spec.update(dims)
    H, D_C, D_R, D_N, D_V = spec["H"], spec["D_C"], spec["D_R"], spec["D_N"], spec["D_V"]
    B = spec["B"] if batch is None else batch
    lo, hi = spec["ctx"] if ctx is None else ctx
    k = spec["topk"] if topk is None else topk
    if seed is None:
        seed = spec["seed"] + (layer if name == "v2_long" else 0)
    rng = np.random.default_rng(seed)
    cache, act = spec["cache"], spec["act"]

    # 1. sequence lengths
    if seq_lens is not None:
        T = np.asarray(seq_lens, dtype=np.int64)
        B = T.shape[0]
    elif lo == hi:
        T = np.full(B, lo, dtype=np.int64)
    else:
        T = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(T)
    total = int(offsets[-1])
    n_pages = int(np.sum(-(-T // PAGE_TOKENS)))
    # 2. page permutation
    page_perm = rng.permutation(n_pages).astype(np.int64)
    # 3-8. values
    c = rng.standard_normal((total, D_C), dtype=np.float32)
    kr = rng.standard_normal((total, D_R), dtype=np.float32)
    qn = rng.standard_normal((B, H, D_N), dtype=np.float32)
    qr = rng.standard_normal((B, H, D_R), dtype=np.float32)
    wstd = np.float32(np.sqrt(1.0 / D_C))
    wuk = rng.standard_normal((H, D_C, D_N), dtype=np.float32) * wstd
    wuv = rng.standard_normal((H, D_V, D_C), dtype=np.float32) * wstd
    # 9. top-k lists
    idx = None
    if k:
        idx = np.full((B, k), -1, dtype=np.int32)
        for b in range(B):
            n = min(k, int(T[b]))
            pick = np.sort(rng.choice(int(T[b]), n, replace=False))
            idx[b, :n] = pick
    if cache == DTYPE_BF16:
        c = round_to_bf16(c)
    if cache in (DTYPE_BF16,) + FP8_DTYPES:
        kr = round_to_bf16(kr)
    if act == DTYPE_BF16:
        qn, qr, wuk, wuv = (round_to_bf16(a) for a in (qn, qr, wuk, wuv))
    codes = scales = None
    if cache == DTYPE_FP8:
        codes, scales = quantize_fp8_per_token(c)
    elif cache == DTYPE_FP8_G128:
        codes, scales = quantize_fp8_per_group(c)
    return DecodeInputs(H=H, D_C=D_C, D_R=D_R, D_N=D_N, D_V=D_V, cache_dtype=cache, act_dtype=act,
                        scale=float(1.0 / np.sqrt(D_N + D_R)), seq_lens=T.astype(np.int32),
                        offsets=offsets, c_kv=c, k_rope=kr, q_nope=qn, q_rope=qr, w_uk=wuk, w_uv=wuv,
                        page_perm=page_perm, c_codes=codes, c_scales=scales, topk_idx=idx)


def make_prefill_queries(inp: DecodeInputs, n: int, seed: int):
    """N new queries for prefill of a one-request workload: q_nope [N, H,
    D_N] and q_rope [N, H, D_R] ~ N(0, 1), rounded to BF16 for BF16
    activations (the queries at positions T - N .. T - 1)."""
    rng = np.random.default_rng(seed)
    qn = rng.standard_normal((n, inp.H, inp.D_N), dtype=np.float32)
    qr = rng.standard_normal((n, inp.H, inp.D_R), dtype=np.float32)
    if inp.act_dtype == DTYPE_BF16:
        qn, qr = round_to_bf16(qn), round_to_bf16(qr)
    return qn, qr


def requantize(inp: DecodeInputs, cache_dtype: str) -> DecodeInputs:
    """The same draw with the latent stored in the other FP8 format (from the
    pre-quantisation values the FP8 workloads keep)."""
    assert inp.cache_dtype in FP8_DTYPES and cache_dtype in FP8_DTYPES
    if cache_dtype == DTYPE_FP8:
        codes, scales = quantize_fp8_per_token(inp.c_kv)
    else:
        codes, scales = quantize_fp8_per_group(inp.c_kv)
    return dataclasses.replace(inp, cache_dtype=cache_dtype, c_codes=codes, c_scales=scales)


# ---------------------------------------------------------------------------
# Lightning-indexer inputs: per request one indexer query (H_I heads of width
# d_I, BF16 values), one float32 weight per head, and per cached position one
# search key of width d_I stored as E4M3 with one float32 scale per position.
#
#   v32_indexer   32 requests x 65,536 positions, 64 heads x 128, top-2,048
#                 (the sparse workload's shape: its index lists come from here)
#
# Draw order: lengths, page permutation, keys, queries, head weights.  Keys,
# queries and weights ~ N(0, 1); queries rounded to BF16; keys quantised per
# position as the FP8 latent is (scale = max|k| / 448).
# ---------------------------------------------------------------------------
INDEXER_WORKLOADS = {
    "v32_indexer": dict(B=32, ctx=(65536, 65536), H_I=64, d_I=128, topk=2048, seed=6),
}


@dataclasses.dataclass
class IndexerInputs:
    H_I: int
    d_I: int
    topk: int
    seq_lens: np.ndarray          # int32 [B]
    offsets: np.ndarray           # int64 [B+1]
    q_idx: np.ndarray             # float32 [B, H_I, d_I] (BF16 values)
    w_idx: np.ndarray             # float32 [B, H_I]
    k_codes: np.ndarray           # uint8 [sum T, d_I]
    k_scales: np.ndarray          # float32 [sum T]
    page_perm: np.ndarray         # int64 [total pages]

    @property
    def B(self) -> int:
        return int(self.seq_lens.shape[0])

    def request(self, b: int):
        return int(self.offsets[b]), int(self.offsets[b + 1])

    def pages_of(self, b: int) -> int:
        return -(-int(self.seq_lens[b]) // PAGE_TOKENS)


def make_indexer_inputs(name: str = "v32_indexer", seed: Optional[int] = None, *, batch: Optional[int] = None,
                        ctx: Optional[tuple] = None, seq_lens=None, topk: Optional[int] = None) -> IndexerInputs:
    spec = dict(INDEXER_WORKLOADS[name])
    B = spec["B"] if batch is None else batch
    lo, hi = spec["ctx"] if ctx is None else ctx
    k = spec["topk"] if topk is None else topk
    rng = np.random.default_rng(spec["seed"] if seed is None else seed)
    H_I, d_I = spec["H_I"], spec["d_I"]
    if seq_lens is not None:
        T = np.asarray(seq_lens, dtype=np.int64)
        B = T.shape[0]
    elif lo == hi:
        T = np.full(B, lo, dtype=np.int64)
    else:
        T = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(T)
    n_pages = int(np.sum(-(-T // PAGE_TOKENS)))
    page_perm = rng.permutation(n_pages).astype(np.int64)
    keys = rng.standard_normal((int(offsets[-1]), d_I), dtype=np.float32)
    q = round_to_bf16(rng.standard_normal((B, H_I, d_I), dtype=np.float32))
    w = rng.standard_normal((B, H_I), dtype=np.float32)
    codes, scales = quantize_fp8_per_token(keys)
    return IndexerInputs(H_I=H_I, d_I=d_I, topk=k, seq_lens=T.astype(np.int32), offsets=offsets, q_idx=q,
                         w_idx=w, k_codes=codes, k_scales=scales, page_perm=page_perm)


def key_page_layout(d_I: int):
    """Search-key page: keys [64][d_I] e4m3, then scales [64] f32, each section
    16-byte aligned."""
    s_off = (PAGE_TOKENS * d_I + 15) // 16 * 16
    return {"k_off": 0, "s_off": s_off, "page_bytes": (s_off + PAGE_TOKENS * 4 + 15) // 16 * 16}


def build_key_pool(inp: IndexerInputs, extra_pages: int = 0):
    """Scatter the search keys into a page pool in the order of
    ``inp.page_perm``.  Returns (pool uint8 [P, page_bytes], block_table int32
    [B, max_pages] padded with -1)."""
    lay = key_page_layout(inp.d_I)
    P = int(inp.page_perm.shape[0]) + extra_pages
    pool = np.zeros((P, lay["page_bytes"]), dtype=np.uint8)
    max_pages = max(inp.pages_of(b) for b in range(inp.B))
    table = np.full((inp.B, max(max_pages, 1)), -1, dtype=np.int32)
    first = 0
    for b in range(inp.B):
        lo, hi = inp.request(b)
        np_b = inp.pages_of(b)
        phys = inp.page_perm[first:first + np_b]
        table[b, :np_b] = phys
        first += np_b
        pad = np_b * PAGE_TOKENS - (hi - lo)
        kc = np.concatenate([inp.k_codes[lo:hi], np.zeros((pad, inp.d_I), np.uint8)])
        ks = np.concatenate([inp.k_scales[lo:hi], np.zeros(pad, np.float32)])
        pool[phys, :PAGE_TOKENS * inp.d_I] = kc.reshape(np_b, -1)
        pool[phys, lay["s_off"]:lay["s_off"] + PAGE_TOKENS * 4] = ks.reshape(np_b, -1).view(np.uint8)
    return pool, table


def key_bytes_read(inp: IndexerInputs) -> int:
    """Algorithmic bytes one indexer scan reads: every visible position's key
    and scale once (the pages' 132-byte search-key item)."""
    return int(np.sum(inp.seq_lens.astype(np.int64))) * (inp.d_I + 4)


# ---------------------------------------------------------------------------
# Paged pool layout.  One page = 64 tokens, sections stored one after another
# (structure of arrays inside a page, each section 16-byte aligned):
#   F32 : c_kv [64][D_C] f32, k_rope [64][D_R] f32
#   BF16: c_kv [64][D_C] bf16, k_rope [64][D_R] bf16
#   FP8 : c_kv [64][D_C] e4m3, k_rope [64][D_R] bf16, scale [64] f32
#   FP8 with group scales: the same, scale [64][D_C / 128] f32
# Rows past a request's length in its last page are zero.
# ---------------------------------------------------------------------------
def page_layout(cache_dtype: str, D_C: int, D_R: int):
    """Byte offsets of the sections in one page and the page size."""
    def al16(x):
        return (x + 15) // 16 * 16
    if cache_dtype == DTYPE_F32:
        c_bytes, r_bytes, s_bytes = PAGE_TOKENS * D_C * 4, PAGE_TOKENS * D_R * 4, 0
    elif cache_dtype == DTYPE_BF16:
        c_bytes, r_bytes, s_bytes = PAGE_TOKENS * D_C * 2, PAGE_TOKENS * D_R * 2, 0
    elif cache_dtype == DTYPE_FP8:
        c_bytes, r_bytes, s_bytes = PAGE_TOKENS * D_C, PAGE_TOKENS * D_R * 2, PAGE_TOKENS * 4
    elif cache_dtype == DTYPE_FP8_G128:
        c_bytes, r_bytes, s_bytes = PAGE_TOKENS * D_C, PAGE_TOKENS * D_R * 2, PAGE_TOKENS * (D_C // FP8_GROUP) * 4
    else:
        raise ValueError(cache_dtype)
    r_off = al16(c_bytes)
    s_off = al16(r_off + r_bytes)
    page = al16(s_off + s_bytes)
    return {"c_off": 0, "r_off": r_off, "s_off": s_off, "page_bytes": page}


def build_paged_pool(inp: DecodeInputs, extra_pages: int = 0):
    """Scatter the logical arrays into a page pool in the order given by
    ``inp.page_perm``.  Returns (pool uint8 [P, page_bytes], block_table int32
    [B, max_pages] padded with -1)."""
    lay = page_layout(inp.cache_dtype, inp.D_C, inp.D_R)
    P = int(inp.page_perm.shape[0]) + extra_pages
    pb = lay["page_bytes"]
    pool = np.zeros((P, pb), dtype=np.uint8)
    max_pages = max(inp.pages_of(b) for b in range(inp.B))
    table = np.full((inp.B, max(max_pages, 1)), -1, dtype=np.int32)
    first = 0
    for b in range(inp.B):
        lo, hi = inp.request(b)
        T = hi - lo
        np_b = inp.pages_of(b)
        phys = inp.page_perm[first:first + np_b]
        table[b, :np_b] = phys
        first += np_b
        pad = np_b * PAGE_TOKENS - T

        def paged(a, dtype):
            a = np.ascontiguousarray(a)
            if pad:
                a = np.concatenate([a, np.zeros((pad,) + a.shape[1:], dtype=a.dtype)])
            return a.reshape(np_b, -1).view(np.uint8) if dtype is None else a.reshape(np_b, -1)

        if inp.cache_dtype == DTYPE_F32:
            cb = paged(inp.c_kv[lo:hi].astype(np.float32), None)
            rb = paged(inp.k_rope[lo:hi].astype(np.float32), None)
        elif inp.cache_dtype == DTYPE_BF16:
            cb = paged(bf16_bits(inp.c_kv[lo:hi]), None)
            rb = paged(bf16_bits(inp.k_rope[lo:hi]), None)
        else:
            cb = paged(inp.c_codes[lo:hi], None)
            rb = paged(bf16_bits(inp.k_rope[lo:hi]), None)
            sb = paged(inp.c_scales[lo:hi].astype(np.float32), None)
            pool[phys, lay["s_off"]:lay["s_off"] + sb.shape[1]] = sb
        pool[phys, lay["c_off"]:lay["c_off"] + cb.shape[1]] = cb
        pool[phys, lay["r_off"]:lay["r_off"] + rb.shape[1]] = rb
    return pool, table


def cache_bytes_read(inp: DecodeInputs) -> int:
    """Algorithmic cache bytes one decode step reads: every visible item once
    (latent + rotary key, plus the scale for FP8)."""
    if inp.cache_dtype == DTYPE_F32:
        item = (inp.D_C + inp.D_R) * 4
    elif inp.cache_dtype == DTYPE_BF16:
        item = (inp.D_C + inp.D_R) * 2
    elif inp.cache_dtype == DTYPE_FP8:
        item = inp.D_C + inp.D_R * 2 + 4
    else:
        item = inp.D_C + inp.D_R * 2 + 4 * (inp.D_C // FP8_GROUP)
    if inp.topk_idx is not None:
        n = int(np.sum(inp.topk_idx >= 0))
    else:
        n = int(np.sum(inp.seq_lens))
    return n * item
