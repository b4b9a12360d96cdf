"""Pins of the CPU oracle to facts outside itself: printed worked examples,
closed forms, a textbook library routine, brute force and invariants.
None of these tests needs a GPU."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from mla_latent_kv_absorb_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _digits_colmajor(s):
    m = np.array([int(ch) for ch in s], dtype=np.float64).reshape(3, 3)
    return m.T  # rows of the result are the columns of the digit grid


def e1_as_mla():
    """Embed the three-token example into an MLA instance with tiny dims.

    One live head; latent dims 0..2 carry the key, dims 8..10 the value and
    dims 12..14 a one-hot marker of the position (so the weighted latent shows
    the softmax weights).  W_UK and W_UV are 0/1 selectors, rotary parts zero.
    """
    g = _load("e1_three_token.json")
    K = _digits_colmajor(g["K_digits"])
    V = _digits_colmajor(g["V_digits"])
    H, D_C, D_R, D_N, D_V = 4, 16, 8, 8, 8
    c = np.zeros((3, D_C))
    c[:, 0:3] = K
    c[:, 8:11] = V
    c[np.arange(3), 12 + np.arange(3)] = 1.0
    kr = np.zeros((3, D_R))
    w_uk = np.zeros((H, D_C, D_N))
    w_uv = np.zeros((H, D_V, D_C))
    for h in range(H):
        for n in range(3):
            w_uk[h, n, n] = 1.0
            w_uv[h, n, 8 + n] = 1.0
    q_nope = np.zeros((H, D_N))
    q_nope[0, 0:3] = g["q3"]
    q_rope = np.zeros((H, D_R))
    scale = 1.0 / math.sqrt(g["d_h"])
    return g, dict(c_kv=c, k_rope=kr, q_nope=q_nope, q_rope=q_rope, w_uk=w_uk, w_uv=w_uv, scale=scale)


def test_e1_worked_example_printed_values():
    g, a = e1_as_mla()
    out, lse, o_lat = oracle.decode_unabsorbed(**a)
    tol = 0.5 * 10 ** -g["printed_decimals"] + 1e-9
    weights = o_lat[0, 12:15]
    scores = np.log(weights) + lse[0]
    np.testing.assert_allclose(scores, g["printed_scores"], atol=tol)
    np.testing.assert_allclose(weights, g["printed_weights"], atol=tol)
    np.testing.assert_allclose(out[0, 0:3], g["printed_out"], atol=tol)
    assert np.all(out[0, 3:] == 0)


def test_e1_row_major_reading_is_rejected():
    """The other reading of the digit strings does not reproduce the page."""
    g = _load("e1_three_token.json")
    K_rows = np.array([int(ch) for ch in g["K_digits"]], dtype=np.float64).reshape(3, 3)
    s = K_rows @ np.array(g["q3"], dtype=np.float64) / math.sqrt(3)
    assert not np.allclose(s, g["printed_scores"], atol=5e-3)


def test_shared_scalar_memory_gives_logistic():
    """Two shared scalar keys 0 and 1 with values 0 and 1 ("Shared KV Memory",
    section 5, 'Shared memory does not mean shared outputs'): for scalar query
    q the output is e^q / (1 + e^q); different queries read the same memory
    and get different outputs."""
    H, D_C, D_R, D_N, D_V = 4, 16, 8, 8, 8
    c = np.zeros((2, D_C))
    c[1, 0] = 1.0
    kr = np.zeros((2, D_R))
    w_uk = np.zeros((H, D_C, D_N))
    w_uk[:, 0, 0] = 1.0
    w_uv = np.zeros((H, D_V, D_C))
    w_uv[:, 0, 0] = 1.0
    qs = np.array([-2.0, 0.0, 0.7, 3.0])
    q_nope = np.zeros((H, D_N))
    q_nope[:, 0] = qs
    out, lse, o_lat = oracle.decode_unabsorbed(c, kr, q_nope, np.zeros((H, D_R)), w_uk, w_uv, 1.0)
    expect = np.exp(qs) / (1 + np.exp(qs))
    np.testing.assert_allclose(out[:, 0], expect, rtol=0, atol=1e-15)
    # the same value from two one-position partials merged by log-sum-exp
    o1, l1 = oracle.latent_decode(q_nope @ w_uk[0].T, np.zeros((H, D_R)), c, kr, 1.0, picked=[0])
    o2, l2 = oracle.latent_decode(q_nope @ w_uk[0].T, np.zeros((H, D_R)), c, kr, 1.0, picked=[1])
    om, lm = oracle.lse_merge(np.stack([o1, o2]), np.stack([l1, l2]))
    np.testing.assert_allclose(om[:, 0], expect, atol=1e-15)
    np.testing.assert_allclose(lm, np.log(1 + np.exp(qs)), atol=1e-15)


def _random_case(rng, H=3, D_C=12, D_R=4, D_N=5, D_V=6, T=9):
    return dict(
        c_kv=rng.standard_normal((T, D_C)), k_rope=rng.standard_normal((T, D_R)),
        q_nope=rng.standard_normal((H, D_N)), q_rope=rng.standard_normal((H, D_R)),
        w_uk=rng.standard_normal((H, D_C, D_N)) / math.sqrt(D_C),
        w_uv=rng.standard_normal((H, D_V, D_C)) / math.sqrt(D_C),
        scale=1.0 / math.sqrt(D_N + D_R))


def test_expansion_by_hand():
    """Figure 5 (1) and Figure 6 (1) of "DeepSeek's KV Cache": the content key
    is the latent times W^UK ([input, output] form) and the value is W^UV
    times the latent.  Two latent rows of width 3, one head, worked by hand:
    rows (1, 2, 0) and (0, 1, -1); W^UK columns (1, 0, 2) and (0, 3, 1) give
    keys (1, 6) and (-2, 2); W^UV rows (2, 0, 1), (0, -1, 4), (1, 1, 1) give
    values (2, -2, 3) and (-1, -5, 0).  A transposed weight or a dropped
    row would change them."""
    c = np.array([[1.0, 2.0, 0.0], [0.0, 1.0, -1.0]])
    w_uk = np.array([[[1.0, 0.0], [0.0, 3.0], [2.0, 1.0]]])   # [H=1, D_C=3, D_N=2]
    w_uv = np.array([[[2.0, 0.0, 1.0], [0.0, -1.0, 4.0], [1.0, 1.0, 1.0]]])  # [H=1, D_V=3, D_C=3]
    k, v = oracle.expand_keys_values(c, w_uk, w_uv, 0)
    np.testing.assert_array_equal(k, [[1.0, 6.0], [-2.0, 2.0]])
    np.testing.assert_array_equal(v, [[2.0, -2.0, 3.0], [-1.0, -5.0, 0.0]])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_absorbed_equals_expanded(seed):
    """Figures 5 and 6 of "DeepSeek's KV Cache": moving W^UK to the query side
    and W^UV after the weighting changes only the order of the products; the
    demo on "What attention stores" shows a difference of 2.8e-17."""
    a = _random_case(np.random.default_rng(seed))
    out, lse, o_lat = oracle.decode_unabsorbed(**a)
    q_lat = oracle.absorb_query(a["q_nope"], a["w_uk"])
    o_lat2, lse2 = oracle.latent_decode(q_lat, a["q_rope"], a["c_kv"], a["k_rope"], a["scale"])
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o_lat2, o_lat, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.up_project(o_lat2, a["w_uv"]), out, rtol=0, atol=1e-12)
    # content score, both orders, one position
    h, j = 1, 4
    k_c = a["c_kv"][j] @ a["w_uk"][h]
    np.testing.assert_allclose(a["q_nope"][h] @ k_c, q_lat[h] @ a["c_kv"][j], atol=1e-13)


def test_latent_attention_is_mqa_sdpa():
    """With absorbed queries, MLA decode is multi-query attention whose single
    shared key is [c ; k_rope] and whose value is c.  Check against torch's
    scaled_dot_product_attention on the CPU in float64."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    H, D_C, D_R, T = 6, 20, 6, 17
    q_lat = rng.standard_normal((H, D_C))
    q_rope = rng.standard_normal((H, D_R))
    c = rng.standard_normal((T, D_C))
    kr = rng.standard_normal((T, D_R))
    scale = 0.37
    o_lat, lse = oracle.latent_decode(q_lat, q_rope, c, kr, scale)
    q = torch.from_numpy(np.concatenate([q_lat, q_rope], 1))[None, :, None, :]
    k = torch.from_numpy(np.concatenate([c, kr], 1))[None, None].expand(1, H, T, D_C + D_R)
    v = torch.from_numpy(c)[None, None].expand(1, H, T, D_C)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, :, 0, :].numpy()
    np.testing.assert_allclose(o_lat, ref, rtol=0, atol=1e-12)
    # lse against a log-sum-exp from torch
    s = torch.from_numpy(scale * (q_lat @ c.T + q_rope @ kr.T))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), atol=1e-12)


def test_decode_is_last_row_of_causal_attention():
    """Appending a token leaves earlier states unchanged, so decoding the last
    position against the cache equals the last row of full causal attention
    ("Shared KV Memory", section 3).  Brute force with Python loops."""
    rng = np.random.default_rng(11)
    T, H, D_C, D_R, D_N, D_V = 6, 2, 5, 3, 4, 3
    a = _random_case(rng, H=H, D_C=D_C, D_R=D_R, D_N=D_N, D_V=D_V, T=T)
    qn_all = rng.standard_normal((T, H, D_N))
    qr_all = rng.standard_normal((T, H, D_R))
    qn_all[-1] = a["q_nope"]
    qr_all[-1] = a["q_rope"]
    out_dec, _, _ = oracle.decode_unabsorbed(**a)
    for h in range(H):
        # keys and values of every position, by explicit sums
        K = [[sum(a["c_kv"][j][d] * a["w_uk"][h][d][n] for d in range(D_C)) for n in range(D_N)]
             + list(a["k_rope"][j]) for j in range(T)]
        V = [[sum(a["w_uv"][h][v][d] * a["c_kv"][j][d] for d in range(D_C)) for v in range(D_V)]
             for j in range(T)]
        rows = []
        for t in range(T):
            q = list(qn_all[t, h]) + list(qr_all[t, h])
            s = [a["scale"] * sum(q[i] * K[j][i] for i in range(D_N + D_R)) if j <= t else -math.inf
                 for j in range(T)]
            m = max(s)
            e = [math.exp(x - m) if x != -math.inf else 0.0 for x in s]
            z = sum(e)
            rows.append([sum(e[j] / z * V[j][v] for j in range(T)) for v in range(D_V)])
        np.testing.assert_allclose(out_dec[h], rows[-1], rtol=0, atol=1e-12)


def test_topk_all_positions_equals_dense_and_padding_ignored():
    a = _random_case(np.random.default_rng(3), T=12)
    dense = oracle.decode_unabsorbed(**a)
    picked = np.concatenate([np.arange(12), [-1, -1, -1]])
    sparse = oracle.decode_unabsorbed(**a, picked=picked)
    for x, y in zip(dense, sparse):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("seed", range(5))
def test_topk_truncation_bound(seed):
    """Restricting the support renormalises the kept weights, and the output
    moves by at most 2*delta*V where delta is the omitted full-attention mass
    and V bounds the value norms ("Shared KV Memory", section 'What is lost by
    restricting the support?'; the printed inequality was lost, this is the
    bound the section's triangle-inequality argument gives)."""
    rng = np.random.default_rng(100 + seed)
    T = 40
    a = _random_case(rng, T=T, H=4)
    out, lse, _ = oracle.decode_unabsorbed(**a)
    picked = np.sort(rng.choice(T, 13, replace=False))
    out_s, _, _ = oracle.decode_unabsorbed(**a, picked=picked)
    for h in range(4):
        k = np.concatenate([a["c_kv"] @ a["w_uk"][h], a["k_rope"]], 1)
        s = a["scale"] * (k @ np.concatenate([a["q_nope"][h], a["q_rope"][h]]))
        alpha = np.exp(s - lse[h])
        delta = 1.0 - alpha[picked].sum()
        vnorm = np.linalg.norm(a["c_kv"] @ a["w_uv"][h].T, axis=1).max()
        assert np.linalg.norm(out[h] - out_s[h]) <= 2 * delta * vnorm + 1e-12


def test_lse_merge_equals_attention_over_union():
    rng = np.random.default_rng(5)
    H, D_C, D_R, T = 4, 10, 3, 23
    q_lat, q_rope = rng.standard_normal((H, D_C)), rng.standard_normal((H, D_R))
    c, kr = rng.standard_normal((T, D_C)), rng.standard_normal((T, D_R))
    full_o, full_l = oracle.latent_decode(q_lat, q_rope, c, kr, 0.5)
    cuts = [0, 5, 6, 15, 23]
    parts = [oracle.latent_decode(q_lat, q_rope, c, kr, 0.5, picked=np.arange(lo, hi))
             for lo, hi in zip(cuts[:-1], cuts[1:])]
    o_parts = np.stack([p[0] for p in parts] + [np.zeros((H, D_C))])
    l_parts = np.stack([p[1] for p in parts] + [np.full(H, -np.inf)])  # one empty partial
    o, l = oracle.lse_merge(o_parts, l_parts)
    np.testing.assert_allclose(o, full_o, atol=1e-13)
    np.testing.assert_allclose(l, full_l, atol=1e-13)


def test_e4m3_decode_matches_torch_and_format_points():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0          # largest finite
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6     # smallest subnormal / normal
    assert ours[0x38] == 1.0 and np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert np.nanmax(ours) == 448.0


def test_fp8_latent_dequant_is_per_token_scale():
    codes = np.array([[0x38, 0x40], [0xB8, 0x00]], dtype=np.uint8)   # 1, 2 ; -1, 0
    got = oracle.dequant_fp8_latent(codes, np.array([0.5, 3.0], dtype=np.float32))
    np.testing.assert_array_equal(got, [[0.5, 1.0], [-3.0, 0.0]])


def test_fp8_latent_dequant_per_128_channel_groups():
    """One float32 scale per 128 latent dimensions ("DeepSeek's KV Cache",
    section "Calculating V3.2's KV cache", the 656-byte main KV item): channel
    d of a token takes scale d // 128.  Values written out by hand."""
    codes = np.full((2, 512), 0x38, dtype=np.uint8)      # 1.0
    codes[1] = 0xC0                                      # -2.0
    scales = np.array([[1.0, 2.0, 4.0, 8.0], [0.5, 0.25, 3.0, 1.0]], dtype=np.float32)
    got = oracle.dequant_fp8_latent(codes, scales)
    want = np.array([[1.0] * 128 + [2.0] * 128 + [4.0] * 128 + [8.0] * 128,
                     [-1.0] * 128 + [-0.5] * 128 + [-6.0] * 128 + [-2.0] * 128])
    np.testing.assert_array_equal(got, want)
    # an interleaved reading of the groups (channel d -> scale d % 4) differs
    assert not np.array_equal(got[0], np.tile([1.0, 2.0, 4.0, 8.0], 128))
    # equal group scales reduce to the per-token form
    rng = np.random.default_rng(4)
    c = rng.integers(0, 256, size=(3, 512)).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0
    s = np.array([0.5, 3.0, 0.01], dtype=np.float32)
    np.testing.assert_array_equal(oracle.dequant_fp8_latent(c, np.repeat(s[:, None], 4, axis=1)),
                                  oracle.dequant_fp8_latent(c, s))


def test_group_scaled_latent_through_attention():
    """With one cached position and a zero query the weighted latent is that
    position's dequantised latent exactly (probability 1); with two positions
    and equal scores it is their mean."""
    codes = np.full((2, 512), 0x38, dtype=np.uint8)
    codes[1, :] = 0x40                                   # 2.0
    scales = np.array([[1.0, 2.0, 4.0, 8.0], [1.0, 1.0, 1.0, 1.0]], dtype=np.float32)
    c = oracle.dequant_fp8_latent(codes, scales)
    q_lat, q_rope = np.zeros((3, 512)), np.zeros((3, 64))
    kr = np.zeros((2, 64))
    o, lse = oracle.latent_decode(q_lat, q_rope, c[:1], kr[:1], 0.1)
    np.testing.assert_array_equal(o[1], [1.0] * 128 + [2.0] * 128 + [4.0] * 128 + [8.0] * 128)
    o, lse = oracle.latent_decode(q_lat, q_rope, c, kr, 0.1)
    np.testing.assert_allclose(o[2], [1.5] * 128 + [2.0] * 128 + [3.0] * 128 + [5.0] * 128, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, np.log(2.0), rtol=0, atol=1e-15)


def test_byte_count_closed_forms_match_pages():
    g = _load("byte_counts.json")
    mha = oracle.mha_cache_bytes_per_token(60, 128, 128, 128, 2)
    v2 = oracle.mla_cache_bytes_per_token(60, 512, 64, 2)
    assert mha == g["mha_bytes_per_token"]
    assert v2 == g["v2_bytes_per_token"]
    assert oracle.mla_cache_bytes_per_token(1, 512, 64, 2) == g["v2_item_bytes"]
    assert oracle.mla_cache_bytes_per_token(61, 512, 64, 2) == g["v3_bytes_per_token"]
    assert round(mha / v2) == g["v2_ratio_vs_mha"]
    assert round(oracle.mla_read_bytes_per_token(60, 131072, 1152) / 1e9, 2) == g["v2_read_per_token_128k_GB"]
    assert round(mha * 131072 / 1e9) == g["mha_read_per_token_128k_GB"]
    assert round(mha * 131072 / 2 ** 30) == g["gib_mha_128k"]
    assert round(oracle.mla_read_bytes_per_token(60, 131072, 1152) / 2 ** 30, 2) == g["gib_mla_128k"]
    item = oracle.fp8_item_bytes(512, 64, 4)
    assert item == g["v32_main_item_bytes"]
    key = oracle.fp8_item_bytes(128, 0, 1)
    assert key == g["v32_search_key_bytes"]
    assert 61 * (item + key) == g["v32_bytes_per_token"]
    assert round(mha / (61 * (item + key))) == g["v32_ratio_vs_mha"]
    assert 61 * (576 + 128) * 2 == g["v32_all_bf16_bytes_per_token"]
    assert round(oracle.mla_read_bytes_per_token(61, 2048, item) / 1e6) == g["v32_kv_read_per_token_MB"]
    assert round(oracle.mla_read_bytes_per_token(61, 131072, key) / 1e9, 2) == g["v32_key_read_per_token_GB"]
    for tag in ("counts_small", "counts_v2"):
        c = g[tag]
        got = oracle.per_token_layer_counts(c["n_h"], c["d_h"], c["n_g"], c["d_c"], c["d_r"])
        assert got == {k: c[k] for k in ("MHA", "GQA", "MQA", "MLA")}
    from fractions import Fraction
    assert Fraction(576, 32768) == Fraction(g["ratio_v2_num"], g["ratio_v2_den"])


def test_oracle_catches_planted_mistakes():
    """Plausible slips in the oracle's arithmetic fail at least one pin."""
    g, a = e1_as_mla()
    # wrong scale (divide by d_h, the page's literal wording)
    out, lse, o_lat = oracle.decode_unabsorbed(**{**a, "scale": 1.0 / 3.0})
    assert not np.allclose(out[0, :3], g["printed_out"], atol=5e-4)
    # dropped rotary term
    b = _random_case(np.random.default_rng(9))
    full = oracle.decode_unabsorbed(**b)
    no_rope = oracle.decode_unabsorbed(**{**b, "k_rope": np.zeros_like(b["k_rope"])})
    assert not np.allclose(full[0], no_rope[0], atol=1e-6)


# ----------------------------------------------------------------------------
# The input generator (shared by both sides) against library conversions.
# ----------------------------------------------------------------------------
def test_generator_bf16_rounding_is_nearest_even():
    """BF16 rounding of the generator against a brute-force nearest search
    (ties to the even pattern) on values including exact ties."""
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * 3).astype(np.float32)
    u = x.view(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)  # exactly halfway
    x = np.concatenate([x, ties[:2000]])
    ours = inputs.round_to_bf16(x)
    lo = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    hi = ((x.view(np.uint32) & np.uint32(0xFFFF0000)) + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    xd = x.astype(np.float64)
    dlo, dhi = np.abs(xd - lo), np.abs(hi - xd)
    lo_even = ((lo.astype(np.float32).view(np.uint32) >> 16) & 1) == 0
    expect = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo_even, lo, hi)))
    assert np.array_equal(ours.astype(np.float64), expect)


def test_generator_e4m3_encode_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(1).standard_normal(100000) * 50
    x = np.clip(x, -448, 448)
    ours = inputs.encode_e4m3(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # float64 vs float32 input only differs on exact float32 rounding ties; none here
    assert np.array_equal(ours, ref)


def test_generator_group_quantiser_uses_full_range():
    """Per 128-channel group the largest magnitude maps to 448 and every
    element is the nearest E4M3 value of x / scale (generator check)."""
    rng = np.random.default_rng(2)
    c = rng.standard_normal((50, 512)).astype(np.float32)
    c[3, 128:256] = 0.0                                   # an all-zero group
    codes, scales = inputs.quantize_fp8_per_group(c)
    assert codes.shape == (50, 512) and scales.shape == (50, 4)
    vals = oracle.e4m3_to_f64(codes).reshape(50, 4, 128)
    amax = np.max(np.abs(vals), axis=2)
    assert np.all((amax == 448.0) | ((amax == 0.0) & (scales == 1.0)))
    np.testing.assert_array_equal(scales[3, 1], 1.0)
    x = (c.reshape(50, 4, 128) / scales[:, :, None]).astype(np.float32).reshape(50, 512)
    np.testing.assert_array_equal(codes, inputs.encode_e4m3(np.clip(x, -448, 448)))
    # dequantised error within half a step of E4M3 (3 mantissa bits) per element
    deq = oracle.dequant_fp8_latent(codes, scales)
    assert np.all(np.abs(deq - c) <= np.abs(c) * 2.0 ** -4 + np.repeat(scales, 128, axis=1) * 2.0 ** -10)


def test_generator_workload_structure():
    inp = inputs.make_inputs("v2_batched", batch=5, ctx=(100, 300))
    assert inp.seq_lens.min() >= 100 and inp.seq_lens.max() <= 300
    pool, table = inputs.build_paged_pool(inp)
    assert pool.shape[0] == sum(inp.pages_of(b) for b in range(5))
    used = table[table >= 0]
    assert np.array_equal(np.sort(used), np.arange(pool.shape[0]))  # every page once
    inp2 = inputs.make_inputs("v2_fp8_topk", batch=2, ctx=(3000, 3000), topk=100)
    assert inp2.topk_idx.shape == (2, 100)
    for b in range(2):
        row = inp2.topk_idx[b]
        assert np.all(np.diff(row) > 0) and row.min() >= 0 and row.max() < 3000


def test_prefill_is_causal_attention_over_expanded_keys():
    """Prefill pin against a library routine: with the keys and values
    expanded per head ([KV] Figure 5 (1), Figure 6 (1)), the N new queries are
    the last N rows of causal scaled-dot-product attention (torch's CPU SDPA,
    float64) over all T positions."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    T, N, H, D_C, D_R, D_N, D_V = 20, 7, 3, 16, 8, 8, 6
    c, kr = rng.standard_normal((T, D_C)), rng.standard_normal((T, D_R))
    qn, qr = rng.standard_normal((N, H, D_N)), rng.standard_normal((N, H, D_R))
    wuk, wuv = rng.standard_normal((H, D_C, D_N)), rng.standard_normal((H, D_V, D_C))
    scale = 1.0 / np.sqrt(D_N + D_R)
    out, lse = oracle.prefill_unabsorbed(c, kr, qn, qr, wuk, wuv, scale, q_start=T - N)
    for h in range(H):
        K = np.concatenate([c @ wuk[h], kr], axis=1)            # [T, D_N + D_R]
        V = c @ wuv[h].T                                         # [T, D_V]
        # full-length causal attention; only the last N query rows are real
        Q = np.zeros((T, D_N + D_R))
        Q[T - N:] = np.concatenate([qn[:, h], qr[:, h]], axis=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
            is_causal=True, scale=scale)[0].numpy()
        np.testing.assert_allclose(out[:, h], ref[T - N:], rtol=1e-12, atol=1e-12)
    # query i sees q_start + i + 1 positions: the first query sees T - N + 1
    o1, _, _ = oracle.decode_unabsorbed(c[:T - N + 1], kr[:T - N + 1], qn[0], qr[0], wuk, wuv, scale)
    np.testing.assert_allclose(out[0], o1, rtol=1e-13, atol=1e-13)
