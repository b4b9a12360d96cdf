"""Plain float64 CPU oracle for the sparse-selection step that produces the
index lists of sparse MLA decode: the lightning indexer score and the top-k
pick.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code, table
or constant with the HIP path.

What it follows ("DeepSeek's KV Cache: From 3.9 MB to 890 B per Token"):
  * section "DSA: three things the indexer builds" and Figure 8: per indexer
    head j a query q^I_j of width d^I (64 heads of width 128 in V3.2), one
    search key k^I per cached position shared by all indexer heads, and one
    weight w^I_j per head and query;
  * section "The score that picks positions" and Figure 9: for each head the
    dot product of its query and the key, through ReLU, times the head weight,
    summed over the heads -- I(t, s) = sum_j w^I(t, j) ReLU(q^I(t, j) . k^I(s));
    then each query keeps up to 2,048 of its highest-scoring visible positions
    (itself included);
  * section "Calculating V3.2's KV cache": the search key is stored as FP8
    (128 values) with one float32 scale for all of them (132 bytes).

Readings (the pages leave these open): the stored key is its E4M3 value times
its scale (the same rule as the main latent); among equal scores the lower
position is picked first; the returned list is sorted by position with -1
padding when fewer than k positions are visible.
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import e4m3_to_f64

__all__ = ["dequant_fp8_key", "indexer_scores", "topk_positions", "select_topk_from_scores"]


def dequant_fp8_key(codes, scales) -> np.ndarray:
    """Search keys stored as E4M3 codes [T, d] with one float32 scale per
    position [T]: the stored value times its scale, exact in float64."""
    return e4m3_to_f64(codes) * np.asarray(scales, dtype=np.float64)[:, None]


def indexer_scores(q_idx, w_idx, keys) -> np.ndarray:
    """I(s) = sum_j w[j] * ReLU(q[j] . k[s]) for one query.

    q_idx [H_I, d], w_idx [H_I], keys [T, d] (already dequantised).  Returns
    the score of every position, float64 [T].  No softmax: the score is only
    used to rank positions.
    """
    q = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w_idx, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    dots = k @ q.T                       # [T, H_I]: head j's query against every key
    relu = np.maximum(dots, 0.0)         # negatives become 0
    return relu @ w                      # weighted sum over the heads


def select_topk_from_scores(scores, T: int, k: int) -> np.ndarray:
    """Up to k highest-scoring positions among 0 .. T-1 (the visible ones),
    ties to the lower position, returned in increasing position order and
    padded with -1 to length k."""
    s = np.asarray(scores)[:T]
    n = min(k, T)
    # rank by (score descending, position ascending); a stable sort on the
    # negated score keeps positions in order among equal scores
    order = np.argsort(-s, kind="stable")[:n]
    out = np.full(k, -1, dtype=np.int64)
    out[:n] = np.sort(order)
    return out


def topk_positions(q_idx, w_idx, key_codes, key_scales, k: int) -> np.ndarray:
    """The whole step for one query over its T visible positions: dequantise
    the keys, score them, keep the top k."""
    keys = dequant_fp8_key(key_codes, key_scales)
    return select_topk_from_scores(indexer_scores(q_idx, w_idx, keys), keys.shape[0], k)
