"""Seeded synthetic workloads drawn on the GPU, for the benchmark's timing
legs.

The parity tests and the CPU oracle use the host generator in ``inputs.py``.
Some timing legs need far more data than the host can draw in a benchmark's
time budget: 60 independent long-context layers (9.06 GB of cache), or the FP8
pool of 32 x 65,536 positions.  For those, this module draws the same shapes,
value distributions and page structure with torch's device generator
(Philox), seeded per layer.  The values differ from the host draws of the same
seed.  Timing does not depend on them.  Like ``inputs.py`` it holds only the
input preparation: normal draws, rounding to BF16, FP8 quantisation (scale =
max|c| / 448 per position or per 128 channels, nearest E4M3 code), the page
layout and the page permutation.  It holds no attention arithmetic.
"""

from __future__ import annotations

import numpy as np

from . import inputs as I

PAGE = I.PAGE_TOKENS


def _gen(torch, seed: int):
    g = torch.Generator(device="cuda")
    g.manual_seed(int(seed))
    return g


def _randn(torch, shape, g, dtype):
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(dtype)


def _table(torch, seq_lens: np.ndarray, g):
    """Page permutation over one shared pool: logical page i of request b is
    physical page perm[first_b + i]; unused columns are -1."""
    pages = [-(-int(t) // PAGE) for t in seq_lens]
    total = int(sum(pages))
    perm = torch.randperm(total, generator=g, device="cuda").to(torch.int32)
    table = torch.full((len(pages), max(pages)), -1, dtype=torch.int32, device="cuda")
    first = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[first:first + n]
        first += n
    return total, table


def _queries_weights(torch, g, B, H, D_C, D_R, D_N, D_V):
    bf = torch.bfloat16
    q_nope = _randn(torch, (B, H, D_N), g, bf)
    q_rope = _randn(torch, (B, H, D_R), g, bf)
    std = float(np.sqrt(1.0 / D_C))
    w_uk = (torch.randn((H, D_C, D_N), generator=g, device="cuda") * std).to(bf)
    w_uv = (torch.randn((H, D_V, D_C), generator=g, device="cuda") * std).to(bf)
    return q_nope, q_rope, w_uk, w_uv


def draw_bf16_layer(torch, seed: int, seq_lens, H=128, D_C=512, D_R=64, D_N=128, D_V=128):
    """A BF16-cache decode layer: pool uint8 [pages, 73,728] (c [64][D_C] then
    k_rope [64][D_R], BF16 N(0,1)), shuffled block table, BF16 queries N(0,1)
    and weights N(0, 1/D_C).  Returns a dict of device tensors and the
    host-side DecodeInputs shell (dims and lengths, no value arrays)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    g = _gen(torch, seed)
    n_pages, table = _table(torch, seq_lens, g)
    lay = I.page_layout(I.DTYPE_BF16, D_C, D_R)
    pool = torch.empty((n_pages, lay["page_bytes"]), dtype=torch.uint8, device="cuda")
    pv = pool.view(torch.bfloat16)
    pv[:, : PAGE * D_C] = _randn(torch, (n_pages, PAGE * D_C), g, torch.bfloat16)
    r0 = lay["r_off"] // 2
    pv[:, r0: r0 + PAGE * D_R] = _randn(torch, (n_pages, PAGE * D_R), g, torch.bfloat16)
    q_nope, q_rope, w_uk, w_uv = _queries_weights(torch, g, len(seq_lens), H, D_C, D_R, D_N, D_V)
    return _pack(torch, seq_lens, pool, table, q_nope, q_rope, w_uk, w_uv, None, I.DTYPE_BF16,
                 H, D_C, D_R, D_N, D_V)


def _fp8_codes(torch, x, group):
    """E4M3 codes and float32 scales of float32 rows x [n, D]: one scale per
    row (group 0) or per `group` consecutive channels."""
    n, D = x.shape
    if group:
        xg = x.view(n, D // group, group)
        amax = xg.abs().amax(dim=2)
        scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (xg / scale[:, :, None]).clamp_(-448.0, 448.0).view(n, D)
    else:
        amax = x.abs().amax(dim=1)
        scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (x / scale[:, None]).clamp_(-448.0, 448.0)
    return q.to(torch.float8_e4m3fn).view(torch.uint8), scale.contiguous()


def draw_fp8_topk(torch, seed: int, B=32, T=65536, k=2048, group128=False, H=128, D_C=512, D_R=64, D_N=128,
                  D_V=128, chunk_pages=4096):
    """The FP8 sparse workload: B requests x T positions, latent N(0,1)
    quantised to E4M3 (one float32 scale per position, or per 128 channels),
    rotary key BF16, BF16 queries and weights, and per request a sorted list
    of k distinct positions drawn uniformly from its context."""
    seq_lens = np.full(B, T, dtype=np.int32)
    g = _gen(torch, seed)
    n_pages, table = _table(torch, seq_lens, g)
    cache = I.DTYPE_FP8_G128 if group128 else I.DTYPE_FP8
    lay = I.page_layout(cache, D_C, D_R)
    pool = torch.zeros((n_pages, lay["page_bytes"]), dtype=torch.uint8, device="cuda")
    for p0 in range(0, n_pages, chunk_pages):
        p1 = min(n_pages, p0 + chunk_pages)
        n = p1 - p0
        x = torch.randn((n * PAGE, D_C), generator=g, device="cuda")
        codes, scales = _fp8_codes(torch, x, 128 if group128 else 0)
        pool[p0:p1, : PAGE * D_C] = codes.view(n, PAGE * D_C)
        s = scales.view(torch.uint8).view(n, -1)
        pool[p0:p1, lay["s_off"]: lay["s_off"] + s.shape[1]] = s
        r = _randn(torch, (n, PAGE * D_R), g, torch.bfloat16).view(torch.uint8)
        pool[p0:p1, lay["r_off"]: lay["r_off"] + r.shape[1]] = r
        del x, codes, scales
    q_nope, q_rope, w_uk, w_uv = _queries_weights(torch, g, B, H, D_C, D_R, D_N, D_V)
    idx = draw_topk_lists(torch, g, seq_lens, k)
    return _pack(torch, seq_lens, pool, table, q_nope, q_rope, w_uk, w_uv, idx, cache, H, D_C, D_R, D_N, D_V)


def draw_topk_lists(torch, g, seq_lens, k):
    """Per request a sorted list of k distinct positions in [0, T_b)."""
    rows = []
    for t in seq_lens:
        pick = torch.randperm(int(t), generator=g, device="cuda")[:k]
        rows.append(torch.sort(pick).values.to(torch.int32))
    return torch.stack(rows).contiguous()


def _pack(torch, seq_lens, pool, table, q_nope, q_rope, w_uk, w_uv, idx, cache, H, D_C, D_R, D_N, D_V):
    B = len(seq_lens)
    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(seq_lens)
    shell = I.DecodeInputs(H=H, D_C=D_C, D_R=D_R, D_N=D_N, D_V=D_V, cache_dtype=cache, act_dtype=I.DTYPE_BF16,
                           scale=float(1.0 / np.sqrt(D_N + D_R)), seq_lens=seq_lens, offsets=offsets,
                           c_kv=None, k_rope=None, q_nope=None, q_rope=None, w_uk=None, w_uv=None,
                           page_perm=None,
                           topk_idx=None if idx is None else np.zeros((B, idx.shape[1]), np.int32))
    return {"shell": shell, "pool": pool, "table": table, "q_nope": q_nope, "q_rope": q_rope, "w_uk": w_uk,
            "w_uv": w_uv, "topk_idx": idx}
