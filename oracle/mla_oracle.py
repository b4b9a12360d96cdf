"""Plain float64 CPU oracle for MLA decode over a latent KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it, and it imports nothing from the GPU library: it shares no code, table
or constant with the HIP path.

What it computes is the *unabsorbed* definition of Multi-head Latent Attention
decode, written out step by step in float64 with no blocking, fusion or
reordering:

  * every head expands its content key from the cached latent and concatenates
    the shared rotary key ("DeepSeek's KV Cache: From 3.9 MB to 890 B per
    Token", Figure 4 (1) and Figure 5 (1); "What attention stores, and what
    DeepSeek changed", section "Cache a latent, not the keys");
  * every head expands its value from the latent (same page, Figure 6 (1));
  * the score is the dot product of the concatenated query and key, divided by
    sqrt(d_k + d_r), then softmax over the visible positions, then the weighted
    sum of values (Figure 4; "Shared KV Memory: From Transformers to DeepSeek",
    section 1, scaled dot-product attention).

The helpers ``absorb_query``, ``latent_decode`` and ``up_project`` are the plain
definitions of the absorbed forms (Figure 5 (2) and Figure 6 (2)); the tests
use them to check single GPU calls, and pin them against the unabsorbed path.

Layout conventions (shared with the GPU library only through the array shapes
given to both sides, never through code):
  c_kv    [T, D_C]          cached latent, position order
  k_rope  [T, D_R]          cached rotary key (already rotated)
  q_nope  [H, D_N]          per-head content query
  q_rope  [H, D_R]          per-head rotary query
  w_uk    [H, D_C, D_N]     k_nope_j = c_j @ w_uk[h]   (row-vector form, [input, output])
  w_uv    [H, D_V, D_C]     v_j = w_uv[h] @ c_j        (column form)
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "e4m3_to_f64",
    "dequant_fp8_latent",
    "visible_positions",
    "expand_keys_values",
    "decode_unabsorbed",
    "prefill_unabsorbed",
    "absorb_query",
    "latent_decode",
    "up_project",
    "lse_merge",
    "mha_cache_bytes_per_token",
    "mla_cache_bytes_per_token",
    "mla_read_bytes_per_token",
    "fp8_item_bytes",
    "per_token_layer_counts",
]


# ---------------------------------------------------------------------------
# FP8 E4M3 (OCP): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
# infinities, S.1111.111 is NaN, largest finite value 448.  The pages name the
# format as E4M3 ("DeepSeek's KV Cache", section "DeepSeek-V4-Flash", main KV
# entry) and use 448 as its largest value ("DeepSeek V4.1 Flash grows as its KV
# cache shrinks 4x", the FP4 range remark, 448 x 6).
# ---------------------------------------------------------------------------
def e4m3_to_f64(codes) -> np.ndarray:
    """Decode E4M3 byte codes into float64 values, exactly."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    subnormal = man / 8.0 * 2.0 ** -6
    normal = (1.0 + man / 8.0) * np.exp2(exp - 7.0)
    val = np.where(exp == 0, subnormal, normal)
    val = np.where((exp == 15) & (man == 7), np.nan, val)
    return sign * val


def dequant_fp8_latent(codes, scales) -> np.ndarray:
    """Latent stored as E4M3 codes [T, D_C] with float32 scales: one per token
    ([T]), or one per group of consecutive channels of a token ([T, G], group
    g covering channels g * D_C / G .. (g + 1) * D_C / G - 1).

    The stored value times its scale gives the latent ("DeepSeek's KV Cache",
    section "Calculating V3.2's KV cache": the scale brings low-precision values
    back to their original size; the main KV item keeps one float32 scale per
    128 of the 512 latent dimensions).  Exact in float64.
    """
    vals = e4m3_to_f64(codes)
    s = np.asarray(scales, dtype=np.float64)
    if s.ndim == 1:
        return vals * s[:, None]
    T, D = vals.shape
    G = s.shape[1]
    if D % G:
        raise ValueError("latent width must be a multiple of the number of groups")
    out = np.empty_like(vals)
    w = D // G
    for g in range(G):
        out[:, g * w:(g + 1) * w] = vals[:, g * w:(g + 1) * w] * s[:, g:g + 1]
    return out


# ---------------------------------------------------------------------------
# Visible positions.  In decode the single query sees every cached position,
# its own included ("Shared KV Memory", section 1: M_tj = 0 for j <= t).  With a
# sparse selection, only the picked positions keep probability: the selection
# mask is 0 at picked positions and -inf elsewhere ("DeepSeek's KV Cache",
# Figure 10 and the paragraph before it).  Index entries equal to -1 are
# padding ("up to 2,048" picked positions).
# ---------------------------------------------------------------------------
def visible_positions(T: int, picked=None) -> np.ndarray:
    if picked is None:
        return np.arange(T, dtype=np.int64)
    idx = np.asarray(picked, dtype=np.int64).ravel()
    idx = idx[(idx >= 0) & (idx < T)]
    return np.unique(idx)  # a mask has set semantics


def expand_keys_values(c_kv, w_uk, w_uv, h):
    """Head h's content keys and values for every cached latent row, float64:
    k_content_j = c_j W^UK_h (Figure 5 (1): the key built from the latent) and
    v_j = W^UV_h c_j (Figure 6 (1): the value built from the same latent).
    Returns (k_content [T, D_N], values [T, D_V])."""
    c = np.asarray(c_kv, dtype=np.float64)
    k_content = c @ np.asarray(w_uk[h], dtype=np.float64)
    values = c @ np.asarray(w_uv[h], dtype=np.float64).T
    return k_content, values


def decode_unabsorbed(c_kv, k_rope, q_nope, q_rope, w_uk, w_uv, scale, picked=None, heads=None):
    """One decode query of one request, unabsorbed, float64.

    Returns (out [H, D_V], lse [H], o_lat [H, D_C]) where o_lat is the
    probability-weighted latent (the U_h of Figure 6 (2)), returned so single
    kernel calls can be checked; lse = log sum_j exp(s_j).
    ``heads`` restricts the work to a subset of heads (rows of the outputs are
    then in that order).
    """
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_rope = np.asarray(k_rope, dtype=np.float64)
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    T = c_kv.shape[0]
    sel = visible_positions(T, picked)
    if sel.size == 0:
        raise ValueError("no visible position")
    c = c_kv[sel]
    kr = k_rope[sel]
    hs = list(range(q_nope.shape[0])) if heads is None else list(heads)
    out = np.empty((len(hs), w_uv.shape[1]))
    lse = np.empty(len(hs))
    o_lat = np.empty((len(hs), c_kv.shape[1]))
    for i, h in enumerate(hs):
        # Figure 5 (1) and Figure 6 (1): build the per-head content key and
        # value from the latent; concatenate the shared rotary key to the key
        # (Figure 4: the two scores add up to the dot product of the
        # concatenated query and key).
        k_content, values = expand_keys_values(c, w_uk, w_uv, h)  # [n, D_N], [n, D_V]
        keys = np.concatenate([k_content, kr], axis=1)  # [n, D_N + D_R]
        query = np.concatenate([q_nope[h], q_rope[h]])
        s = scale * (keys @ query)                    # [n]
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        p = e / z
        # Figure 6 (1): weight the expanded values.
        out[i] = p @ values
        o_lat[i] = p @ c
        lse[i] = m + np.log(z)
    return out, lse, o_lat


def prefill_unabsorbed(c_kv, k_rope, q_nope, q_rope, w_uk, w_uv, scale, q_start, heads=None):
    """N new queries of one request at positions q_start .. q_start + N - 1,
    each attending causally to the cached positions up to and including its
    own ("Shared KV Memory", section 1: M_tj = 0 for j <= t): query i is the
    decode of position q_start + i over positions 0 .. q_start + i.
    q_nope [N, H, D_N], q_rope [N, H, D_R].  Returns (out [N, H', D_V],
    lse [N, H']) for the heads asked for."""
    q_nope = np.asarray(q_nope)
    N = q_nope.shape[0]
    outs, lses = [], []
    for i in range(N):
        visible = np.arange(q_start + i + 1)
        o, l, _ = decode_unabsorbed(c_kv, k_rope, q_nope[i], q_rope[i], w_uk, w_uv, scale, picked=visible,
                                    heads=heads)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------------------
# Absorbed forms, as plain definitions.
# ---------------------------------------------------------------------------
def absorb_query(q_nope, w_uk) -> np.ndarray:
    """Figure 5 (2): move W^UK to the query side once, q_hat_h = q_h (W^UK_h)^T,
    a D_C-wide vector dotted directly with the cached latent.  With w_uk[h] of
    shape [D_C, D_N] this is w_uk[h] @ q_nope[h].  Works on [H, D_N] or
    [B, H, D_N] queries."""
    q = np.asarray(q_nope, dtype=np.float64)
    w = np.asarray(w_uk, dtype=np.float64)
    if q.ndim == 2:
        return np.einsum("hcn,hn->hc", w, q)
    return np.einsum("hcn,bhn->bhc", w, q)


def latent_decode(q_lat, q_rope, c_kv, k_rope, scale, picked=None):
    """Attention in latent space for one request: every head scores the cached
    latent with its absorbed query plus the rotary part, and weights the latent
    itself (Figure 5 (2) for the score, Figure 6 (2) first step for U_h).
    Returns (o_lat [H, D_C], lse [H])."""
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_rope = np.asarray(k_rope, dtype=np.float64)
    sel = visible_positions(c_kv.shape[0], picked)
    if sel.size == 0:
        raise ValueError("no visible position")
    c = c_kv[sel]
    kr = k_rope[sel]
    s = scale * (q_lat @ c.T + q_rope @ kr.T)         # [H, n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    return p @ c, (m + np.log(z))[:, 0]


def up_project(o_lat, w_uv) -> np.ndarray:
    """Figure 6 (2) second step: multiply the weighted latent by W^UV_h.
    With w_uv[h] of shape [D_V, D_C] this is w_uv[h] @ o_lat[h].  Works on
    [H, D_C] or [B, H, D_C]."""
    o = np.asarray(o_lat, dtype=np.float64)
    w = np.asarray(w_uv, dtype=np.float64)
    if o.ndim == 2:
        return np.einsum("hvc,hc->hv", w, o)
    return np.einsum("hvc,bhc->bhv", w, o)


def lse_merge(o_parts, lse_parts):
    """Merge softmax-normalised partial results over disjoint position sets.

    A partial (o_s, lse_s) over set S_s is o_s = sum_{j in S_s} exp(s_j) v_j /
    exp(lse_s).  Softmax over the union then gives
    o = sum_s exp(lse_s - LSE) o_s with LSE = log sum_s exp(lse_s).  Empty
    partials carry lse = -inf and contribute nothing.
    o_parts [S, ..., D], lse_parts [S, ...]; returns (o [..., D], LSE [...]).
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = np.max(lse_parts, axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_parts - m_safe)
    tot = w.sum(axis=0)
    lse = m_safe + np.log(tot)
    o = np.einsum("s...,s...d->...d", w / tot, o_parts)
    return o, lse


# ---------------------------------------------------------------------------
# Closed-form cache sizes.  The pages count one stored item per token and
# layer; scales inside an item count, heads and the two K/V roles do not
# double-count ("DeepSeek's KV Cache", section "Looking at reads").
# ---------------------------------------------------------------------------
def mha_cache_bytes_per_token(layers, heads, d_k, d_v, bytes_per_elem):
    """Hypothetical MHA stores a key and a value per head per layer
    ("DeepSeek's KV Cache", section "The baseline: MHA that stores every head's
    Key and Value")."""
    return layers * heads * (d_k + d_v) * bytes_per_elem


def mla_cache_bytes_per_token(layers, d_c, d_r, bytes_per_elem):
    """MLA stores the latent plus the shared rotary key per layer (same page,
    section "Calculating V2's KV cache")."""
    return layers * (d_c + d_r) * bytes_per_elem


def mla_read_bytes_per_token(layers, context, item_bytes):
    """A decode step reads every cached item of every layer once (same
    section)."""
    return layers * context * item_bytes


def fp8_item_bytes(d_c, d_r, n_scales, rope_bytes=2, scale_bytes=4):
    """FP8 latent + float32 scales + BF16 rotary key, no padding (section
    "Calculating V3.2's KV cache")."""
    return d_c * 1 + n_scales * scale_bytes + d_r * rope_bytes


def per_token_layer_counts(n_h, d_h, n_g, d_c, d_r):
    """Cached numbers per token per layer for MHA, GQA, MQA and MLA ("What
    attention stores, and what DeepSeek changed", section "The cache table")."""
    return {"MHA": 2 * n_h * d_h, "GQA": 2 * n_g * d_h, "MQA": 2 * d_h, "MLA": d_c + d_r}
