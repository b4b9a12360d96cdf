"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Tolerances: max |err| <= 2e-2 * max|ref| for BF16 / FP8 caches on out and
o_lat, and max |err| <= 1e-2 (absolute) on the log-sum-exp; max |err| <= 1e-4
(absolute) for the float32 configuration; index handling bit-exact.

Why 1e-2 absolute on the log-sum-exp: lse is a softmax-weighted mean of the
scores plus the log of the mass, so its error is about the score error.  The
scores differ from the float64 ones by the BF16 rounding of q_lat (one
rounding of a 512-term float32 sum) and, for FP8 caches, of the dequantised
latent: about 2^-9 relative per term, a few 1e-3 on unit-variance scores.  A
relative bound on lse would allow ~0.2 at 16K-131K contexts, a 20% error in
the merge weights.
"""

import math

import numpy as np
import pytest

import oracle
from mla_latent_kv_absorb_amd import inputs as I

pytestmark = pytest.mark.gpu

REL_TOL = 2e-2
LSE_ABS_TOL = 1e-2
F32_TOL = 1e-4


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


@pytest.fixture(scope="module")
def R(torch):
    from mla_latent_kv_absorb_amd import runner
    return runner


def _log(msg):
    print(msg, flush=True)


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def oracle_request(inp, b, heads=None):
    lo, hi = inp.request(b)
    if inp.cache_dtype in I.FP8_DTYPES:
        c = oracle.dequant_fp8_latent(inp.c_codes[lo:hi], inp.c_scales[lo:hi])
    else:
        c = inp.c_kv[lo:hi]
    picked = None if inp.topk_idx is None else inp.topk_idx[b]
    return oracle.decode_unabsorbed(c, inp.k_rope[lo:hi], inp.q_nope[b], inp.q_rope[b], inp.w_uk, inp.w_uv,
                                    inp.scale, picked=picked, heads=heads)


def assert_close(got, ref, tol_rel=REL_TOL, abs_tol=None, what=""):
    err = np.max(np.abs(got - ref))
    if abs_tol is not None:
        assert err <= abs_tol, f"{what}: max|err| {err:.3g} > {abs_tol}"
    else:
        bound = tol_rel * np.max(np.abs(ref))
        assert err <= bound, f"{what}: max|err| {err:.3g} > {bound:.3g} (= {tol_rel} x max|ref|)"
    return err


def check_step(torch, R, inp, split=True, num_workers=None, requests=None, heads=None, f32=False, checks=None,
               lse_tol=LSE_ABS_TOL):
    """Run the whole step on the GPU and compare out, o_lat and lse with the
    oracle.  ``checks`` is a list of (requests, heads) pairs to compare (heads
    None = all); by default (requests, heads) as given, every request and head
    when both are None."""
    w = R.DeviceWorkload(inp, split=split, num_workers=num_workers)
    w.step()
    torch.cuda.synchronize()
    o_lat, out, lse = to_np(w.o_lat), to_np(w.out), to_np(w.lse)
    if checks is None:
        checks = [(range(inp.B) if requests is None else requests, heads)]
    # the merge and up-projection in one launch as well (the benchmarked
    # step), on the same partials, where that call exists (BF16, V2 dims)
    fused = None
    if split and inp.act_dtype == I.DTYPE_BF16 and inp.D_V == 128 and inp.D_C == 512 and inp.H == 128:
        w.out.zero_()
        w.combine_up()
        torch.cuda.synchronize()
        fused = to_np(w.out)
    for reqs, hsel in checks:
        hs = list(range(inp.H)) if hsel is None else list(hsel)
        for b in reqs:
            r_out, r_lse, r_olat = oracle_request(inp, b, heads=hs)
            tag = f"b={b}"
            if fused is not None:
                assert_close(fused[b][hs], r_out, what="fused out " + tag)
            if f32:
                assert_close(out[b][hs], r_out, abs_tol=F32_TOL, what="out " + tag)
                assert_close(o_lat[b][hs], r_olat, abs_tol=F32_TOL, what="o_lat " + tag)
                assert_close(lse[b][hs], r_lse, abs_tol=F32_TOL, what="lse " + tag)
            else:
                assert_close(out[b][hs], r_out, what="out " + tag)
                assert_close(o_lat[b][hs], r_olat, what="o_lat " + tag)
                assert_close(lse[b][hs], r_lse, abs_tol=lse_tol, what="lse " + tag)
    return w


def custom_inputs(c_kv, k_rope, q_nope, q_rope, w_uk, w_uv, seq_lens, cache, act, scale, topk_idx=None,
                  codes=None, scales=None, perm_seed=0):
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    offsets = np.zeros(len(seq_lens) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(seq_lens)
    n_pages = int(np.sum(-(-seq_lens // 64)))
    perm = np.random.default_rng(perm_seed).permutation(n_pages)
    H, D_C = w_uk.shape[0], w_uk.shape[1]
    return I.DecodeInputs(H=H, D_C=D_C, D_R=k_rope.shape[1], D_N=w_uk.shape[2], D_V=w_uv.shape[1],
                          cache_dtype=cache, act_dtype=act, scale=float(scale), seq_lens=seq_lens,
                          offsets=offsets, c_kv=np.ascontiguousarray(c_kv, dtype=np.float32),
                          k_rope=np.ascontiguousarray(k_rope, dtype=np.float32),
                          q_nope=np.ascontiguousarray(q_nope, dtype=np.float32),
                          q_rope=np.ascontiguousarray(q_rope, dtype=np.float32),
                          w_uk=np.ascontiguousarray(w_uk, dtype=np.float32),
                          w_uv=np.ascontiguousarray(w_uv, dtype=np.float32), page_perm=perm,
                          c_codes=codes, c_scales=scales, topk_idx=topk_idx)


# ---------------------------------------------------------------------------
# float32 configuration (tiny dims)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("split", [False, True])
def test_tiny_fp32_full_step(torch, R, split):
    _log(f"tiny_fp32 split={split}")
    inp = I.make_inputs("tiny_fp32")
    check_step(torch, R, inp, split=split, f32=True)


def test_tiny_fp32_ragged_multi_request_splits(torch, R):
    _log("tiny_fp32 ragged")
    inp = I.make_inputs("tiny_fp32", seq_lens=[1, 33, 64, 100, 7])
    for nw in (1, 2, 3, 9):
        check_step(torch, R, inp, split=True, num_workers=nw, f32=True)


def test_three_token_worked_example_on_gpu(torch, R):
    """The page's worked example embedded in tiny MLA dims, run on the GPU
    ("What attention stores, and what DeepSeek changed", first section)."""
    _log("E1 on gpu")
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e1_three_token.json")))
    K = np.array([int(c) for c in g["K_digits"]], dtype=np.float64).reshape(3, 3).T
    V = np.array([int(c) for c in g["V_digits"]], dtype=np.float64).reshape(3, 3).T
    H, D_C, D_R, D_N, D_V = 4, 16, 8, 8, 8
    c = np.zeros((3, D_C)); c[:, 0:3] = K; c[:, 8:11] = V; c[np.arange(3), 12 + np.arange(3)] = 1
    w_uk = np.zeros((H, D_C, D_N)); w_uv = np.zeros((H, D_V, D_C))
    for n in range(3):
        w_uk[:, n, n] = 1
        w_uv[:, n, 8 + n] = 1
    q_nope = np.zeros((1, H, D_N)); q_nope[0, 0, 0:3] = g["q3"]
    inp = custom_inputs(c, np.zeros((3, D_R)), q_nope, np.zeros((1, H, D_R)), w_uk, w_uv, [3],
                        I.DTYPE_F32, I.DTYPE_F32, 1 / math.sqrt(g["d_h"]))
    w = R.DeviceWorkload(inp, split=False)
    w.step()
    torch.cuda.synchronize()
    out = to_np(w.out)[0, 0, :3]
    weights = to_np(w.o_lat)[0, 0, 12:15]
    tol = 0.5 * 10 ** -g["printed_decimals"] + 1e-6
    np.testing.assert_allclose(out, g["printed_out"], atol=tol)
    np.testing.assert_allclose(weights, g["printed_weights"], atol=tol)
    scores = np.log(weights) + to_np(w.lse)[0, 0]
    np.testing.assert_allclose(scores, g["printed_scores"], atol=tol)


# ---------------------------------------------------------------------------
# V2 dims, BF16 cache: several tiles, ragged tails, split counts
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def v2_ragged():
    return I.make_inputs("v2_batched", seed=11, seq_lens=[200, 1000, 77])


@pytest.mark.parametrize("mode", ["direct", 1, 2, 7, "auto"])
def test_v2_bf16_ragged(torch, R, v2_ragged, mode):
    _log(f"v2 ragged mode={mode}")
    if mode == "direct":
        check_step(torch, R, v2_ragged, split=False)
    else:
        check_step(torch, R, v2_ragged, split=True, num_workers=None if mode == "auto" else mode)


def test_v2_page_order_is_bit_identical(torch, R, v2_ragged):
    _log("page permutation")
    import dataclasses
    other = dataclasses.replace(v2_ragged, page_perm=np.random.default_rng(99).permutation(v2_ragged.page_perm.size))
    outs = []
    for inp in (v2_ragged, other):
        w = R.DeviceWorkload(inp, split=True, num_workers=5)
        w.step()
        torch.cuda.synchronize()
        outs.append((w.o_lat.clone(), w.out.clone(), w.lse.clone()))
    for x, y in zip(*outs):
        assert torch.equal(x, y)


@pytest.mark.parametrize("case", ["ragged", "many_segments", "many_segments_direct"])
def test_v2_repeat_runs_bit_identical(torch, R, v2_ragged, case):
    """Every work-group exchanges probabilities and rescale factors between
    its waves through LDS: a missing barrier shows up as results that change
    from run to run.  Many segments per work-group and long ones, split and
    direct."""
    _log(f"determinism {case}")
    inp = v2_ragged if case == "ragged" else I.make_inputs("v2_batched", seed=71, batch=12, ctx=(3000, 9000))
    w = R.DeviceWorkload(inp, split=case != "many_segments_direct")
    w.step()
    a = (w.o_lat.clone(), w.out.clone(), w.lse.clone())
    for _ in range(4):
        w.step()
        torch.cuda.synchronize()
        assert torch.equal(a[0], w.o_lat) and torch.equal(a[1], w.out) and torch.equal(a[2], w.lse)


def test_v2_absorb_and_up_projection_alone(torch, R, v2_ragged):
    _log("absorb/out_up alone")
    inp = v2_ragged
    w = R.DeviceWorkload(inp, split=False)
    w.absorb()
    torch.cuda.synchronize()
    ref = oracle.absorb_query(inp.q_nope, inp.w_uk)
    assert_close(to_np(w.q_lat), ref, what="q_lat")
    x = I.round_to_bf16(np.random.default_rng(3).standard_normal((inp.B, inp.H, inp.D_C)).astype(np.float32))
    w.o_lat.copy_(R.to_device_act(x, I.DTYPE_BF16, "cuda"))
    w.up()
    torch.cuda.synchronize()
    assert_close(to_np(w.out), oracle.up_project(x, inp.w_uv), what="out_up")


@pytest.mark.parametrize("batch", [3, 16, 20, 33, 37])
def test_v2_fused_combine_up(torch, R, batch):
    """mla_combine_out_up: against the oracle, and against mla_combine then
    mla_out_up on the same partials.  The merge is the same code, so lse is
    bit-identical; out may differ in the last BF16 bit (GEMM summation order).
    The fused kernel takes requests in blocks of 16 (up to 32 requests) or 32,
    and merges a block of n requests on 16 waves, each request on 16 // n
    waves when n < 16: 3 requests (5 waves each, one wave idle), 16 (one wave
    each), 20 (a full block and one of 4), 33 (a full block of 32, two
    requests per wave, and one lone request on all 16 waves), 37 (32 and 5)."""
    _log(f"fused merge + up-projection, batch {batch}")
    inp = I.make_inputs("v2_batched", seed=31, batch=batch, ctx=(40, 900))
    for nw in (None, 7):
        w = R.DeviceWorkload(inp, split=True, num_workers=nw)
        w.step()
        torch.cuda.synchronize()
        out_sep, lse_sep = w.out.clone(), w.lse.clone()
        w.out.zero_()
        w.lse.zero_()
        w.combine_up()
        torch.cuda.synchronize()
        assert torch.equal(w.lse, lse_sep)
        assert_close(to_np(w.out), to_np(out_sep), tol_rel=1e-2, what=f"fused vs separate, workers {nw}")
        out = to_np(w.out)
        for b in sorted({0, batch // 2, batch - 1}):
            r_out, _, _ = oracle_request(inp, b)
            assert_close(out[b], r_out, what=f"fused out b={b} workers {nw}")


def test_v2_topk_all_positions_equals_dense(torch, R):
    _log("topk == dense")
    dense = I.make_inputs("v2_batched", seed=12, seq_lens=[300, 129])
    import dataclasses
    idx = np.full((2, 300), -1, dtype=np.int32)
    idx[0, :300] = np.arange(300)
    idx[1, :129] = np.arange(129)
    sparse = dataclasses.replace(dense, topk_idx=idx)
    wd = R.DeviceWorkload(dense, split=False)
    ws = R.DeviceWorkload(sparse, split=False)
    wd.step(); ws.step()
    torch.cuda.synchronize()
    assert torch.equal(wd.o_lat, ws.o_lat)
    assert torch.equal(wd.out, ws.out)


def test_rescale_path_with_growing_scores(torch, R):
    """Scores that grow along the context force the online-softmax rescale
    several times: the top head's scaled score grows by about 0.047 log2
    units per position, about 31 over each of the three workers' ranges, so
    every worker crosses the kernels' lazy-rescale threshold (at most 16 log2
    units) at least once after its first tile."""
    _log("rescale path")
    rng = np.random.default_rng(5)
    T, H, D_C, D_R = 2000, 128, 512, 64
    c = rng.standard_normal((T, D_C)).astype(np.float32) * 0.1
    c[:, 0] = np.arange(T) * 0.15
    c = I.round_to_bf16(c)
    kr = I.round_to_bf16(rng.standard_normal((T, D_R)).astype(np.float32) * 0.1)
    q_lat = np.zeros((1, H, D_C), np.float32)
    q_lat[0, :, 0] = np.linspace(0.5, 3.0, H)
    q_lat = I.round_to_bf16(q_lat)
    qr = I.round_to_bf16(rng.standard_normal((1, H, D_R)).astype(np.float32))
    wz = np.zeros((H, D_C, 128), np.float32)
    inp = custom_inputs(c, kr, np.zeros((1, H, 128), np.float32), qr, wz, np.zeros((H, 128, D_C), np.float32),
                        [T], I.DTYPE_BF16, I.DTYPE_BF16, 1 / math.sqrt(192))
    for split in (False, True):
        w = R.DeviceWorkload(inp, split=split, num_workers=3)
        w.attend(q_lat=R.to_device_act(q_lat, I.DTYPE_BF16, "cuda"))
        w.combine()
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.latent_decode(q_lat[0], qr[0], c, kr, inp.scale)
        assert_close(to_np(w.o_lat)[0], ref_o, what=f"o_lat split={split}")
        assert_close(to_np(w.lse)[0], ref_l, what=f"lse split={split}")


# ---------------------------------------------------------------------------
# FP8 latent + index lists
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cache", [I.DTYPE_FP8, I.DTYPE_FP8_G128])
def test_fp8_every_code_converts_exactly(torch, R, cache):
    """Each finite E4M3 code, weighted by probability 1 (zero query, one
    position), comes back as its exact value times its scale.  With group
    scales the two copies of the 256 codes meet four different scales; every
    product has at most 7 significant bits, so BF16 holds it exactly."""
    _log(f"fp8 codes {cache}")
    H, D_C, D_R = 128, 512, 64
    codes = np.tile(np.arange(256, dtype=np.uint8), 2)[None, :]
    codes[:, (codes[0] & 0x7F) == 0x7F] = 0  # NaN codes stay out of the arithmetic
    codes = np.concatenate([codes, codes[:, ::-1]])            # two requests, one position each
    if cache == I.DTYPE_FP8:
        scales = np.array([1.0, 0.375], dtype=np.float32)
        full = np.repeat(scales[:, None], D_C, axis=1)
    else:
        scales = np.array([[1.0, 0.375, 2.0, 0.15625], [0.15625, 4.0, 0.375, 1.0]], dtype=np.float32)
        full = np.repeat(scales, 128, axis=1)
    inp = custom_inputs(np.zeros((2, D_C)), np.zeros((2, D_R)), np.zeros((2, H, 128)), np.zeros((2, H, D_R)),
                        np.zeros((H, D_C, 128)), np.zeros((H, 128, D_C)), [1, 1], cache, I.DTYPE_BF16,
                        0.1, codes=codes, scales=scales)
    w = R.DeviceWorkload(inp, split=False)
    w.attend(q_lat=torch.zeros_like(w.q_lat))
    torch.cuda.synchronize()
    got = to_np(w.o_lat)
    for b in range(2):
        ref = oracle.e4m3_to_f64(codes[b]) * full[b]
        for h in (0, 63, 127):
            assert np.array_equal(got[b, h], ref), f"request {b} head {h}"


def _bit_pattern_case(cache, seed):
    rng = np.random.default_rng(seed)
    H, D_C, D_R, T, B = 128, 512, 64, 4096, 2
    pos = np.arange(T)
    c = np.zeros((B * T, D_C), np.float32)
    for d in range(12):
        c[:, d] = np.tile((pos >> d) & 1, B)
    codes = scales = None
    if cache in I.FP8_DTYPES:
        codes = np.where(c > 0, 0x38, 0).astype(np.uint8)
        scales = np.ones(B * T, np.float32) if cache == I.DTYPE_FP8 else np.ones((B * T, D_C // 128), np.float32)
    idx = np.full((B, 160), -1, np.int32)
    for b in range(B):
        idx[b, :128] = np.sort(rng.choice(T, 128, replace=False))
    inp = custom_inputs(c, np.zeros((B * T, D_R)), np.zeros((B, H, 128)), np.zeros((B, H, D_R)),
                        np.zeros((H, D_C, 128)), np.zeros((H, 128, D_C)), [T] * B, cache, I.DTYPE_BF16, 0.1,
                        topk_idx=idx, codes=codes, scales=scales, perm_seed=seed)
    return inp, idx


@pytest.mark.parametrize("cache", [I.DTYPE_BF16, I.DTYPE_FP8, I.DTYPE_FP8_G128])
def test_topk_index_handling_bit_exact(torch, R, cache):
    """Zero queries give every picked position probability 1; latent dim d of
    position p holds bit d of p.  With one worker the partial is exactly
    (number of picked positions with bit d set) / 128 (a multiple of 2^-7 with
    at most 8 significant bits, so exact in the BF16 partials too), and a
    wrong, missing or repeated index changes its bits."""
    _log(f"topk bit pattern {cache}")
    inp, idx = _bit_pattern_case(cache, seed=7)
    w = R.DeviceWorkload(inp, split=True, num_workers=1)
    w.attend(q_lat=torch.zeros_like(w.q_lat))
    torch.cuda.synchronize()
    part_o, part_l = w.partials()
    part_o = part_o.cpu().numpy()
    for b in range(inp.B):
        sel = idx[b][idx[b] >= 0]
        expect = np.zeros(inp.D_C, np.float32)
        for d in range(12):
            expect[d] = np.float32(np.sum((sel >> d) & 1)) / np.float32(128)
        got = part_o[0 + b]  # worker 0 covers every request: slot = 0 + b
        assert np.array_equal(got, np.broadcast_to(expect, got.shape)), f"request {b}"
        np.testing.assert_allclose(part_l[b].cpu().numpy(), math.log(128), rtol=1e-6)


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
@pytest.mark.parametrize("workers", [3, 11, 40])
def test_tiny_segments_every_head(torch, R, cache, workers):
    """Contexts of 1 to 65 positions over many workers: segments of one or
    two tiles, ragged last tiles, requests split across workers, workers
    with several short segments.  Exercises the segment start (page ids,
    staged queries, the first two tile loads and the loads past the
    segment's end), the first-tile rescale skip and the output staging at
    their smallest.  Every head of every request."""
    _log(f"tiny segments {cache} workers={workers}")
    lens = [1, 31, 32, 33, 64, 65, 2, 17, 40, 5]
    name = "v2_batched" if cache == "bf16" else "v2_fp8_topk"
    inp = I.make_inputs(name, seed=31, seq_lens=lens, **({} if cache == "bf16" else {"topk": 0}))
    check_step(torch, R, inp, split=True, num_workers=workers)


@pytest.mark.parametrize("name", ["v2_fp8_topk", "v2_fp8g_topk"])
def test_fp8_topk_small(torch, R, name):
    _log(f"{name} small")
    inp = I.make_inputs(name, seed=21, batch=2, ctx=(3000, 3000), topk=100)
    inp.topk_idx[1, 96:] = -1  # padding entries
    for split in (False, True):
        check_step(torch, R, inp, split=split)


@pytest.mark.parametrize("name", ["v2_fp8_topk", "v2_fp8g_topk"])
def test_fp8_dense_small(torch, R, name):
    _log(f"{name} dense small")
    inp = I.make_inputs(name, seed=22, batch=2, ctx=(500, 1500), topk=0)
    check_step(torch, R, inp, split=True)
    check_step(torch, R, inp, split=False)


def test_fp8_group_scales_differ_per_group(torch, R):
    """Group scales that differ by up to 2^4 across the four groups of a
    position (and across positions): the per-group dequantisation, not a
    per-position one, is what matches the oracle (one scale for all groups
    would be off by the whole latent).  The spread is kept at 2^-2 .. 2^2:
    at 2^-5 .. 2^5 the BF16 rounding of the absorbed query alone takes the
    output past the 2e-2 bound, whatever the dequantisation
    (test_precision_model.py models it)."""
    _log("fp8 group scales spread")
    inp = I.make_inputs("v2_fp8g_topk", seed=24, batch=3, ctx=(200, 700), topk=0)
    rng = np.random.default_rng(24)
    inp.c_scales[:] = inp.c_scales * np.exp2(rng.integers(-2, 3, size=inp.c_scales.shape)).astype(np.float32)
    # latents up to 4x larger make scores (and their rounding error) up to 4x
    # larger: the lse bound scales with them
    check_step(torch, R, inp, split=True, lse_tol=4 * LSE_ABS_TOL)


def test_fp8_per_position_scales_applied_in_float32(torch, R):
    """Per-position scales spread over 2^-5 .. 2^5, with q_lat given as BF16
    values that the oracle uses too (so the query's own rounding is out of the
    comparison).  The kernel widens the E4M3 codes exactly and multiplies the
    latent scores and the probabilities by each position's scale in float32,
    which keeps o_lat within 4e-3 of the oracle here; rounding code x scale
    to BF16 first gives 2.3-3.5e-2 on these rows (test_precision_model.py
    models both), so the 1e-2 bound tells the two apart."""
    _log("fp8 per-position scales, wide spread")
    inp = I.make_inputs("v2_fp8_topk", seed=24, batch=3, ctx=(200, 700), topk=0)
    rng = np.random.default_rng(24)
    inp.c_scales[:] = inp.c_scales * np.exp2(rng.integers(-5, 6, size=inp.c_scales.shape)).astype(np.float32)
    q_lat = I.round_to_bf16(oracle.absorb_query(inp.q_nope, inp.w_uk).astype(np.float32))
    for split in (False, True):
        w = R.DeviceWorkload(inp, split=split)
        w.attend(q_lat=R.to_device_act(q_lat, I.DTYPE_BF16, "cuda"))
        w.combine()
        torch.cuda.synchronize()
        o_lat, lse = to_np(w.o_lat), to_np(w.lse)
        for b in range(inp.B):
            lo, hi = inp.request(b)
            c = oracle.dequant_fp8_latent(inp.c_codes[lo:hi], inp.c_scales[lo:hi])
            ref_o, ref_l = oracle.latent_decode(q_lat[b], inp.q_rope[b], c, inp.k_rope[lo:hi], inp.scale)
            err = assert_close(o_lat[b], ref_o, tol_rel=1e-2, what=f"o_lat b={b} split={split}")
            _log(f"  b={b} split={split}: o_lat max|err|/max|ref| = {err / np.max(np.abs(ref_o)):.2e}")
            assert_close(lse[b], ref_l, abs_tol=LSE_ABS_TOL, what=f"lse b={b} split={split}")


def test_out_of_range_indices_are_skipped(torch, R):
    _log("out of range indices")
    inp = I.make_inputs("v2_fp8_topk", seed=23, batch=1, ctx=(1000, 1000), topk=40)
    bad = inp.topk_idx.copy()
    bad[0, 10] = 5000      # beyond the context: skipped
    bad[0, 11] = -7        # negative: skipped
    import dataclasses
    w = R.DeviceWorkload(dataclasses.replace(inp, topk_idx=bad), split=False)
    w.step()
    torch.cuda.synchronize()
    ref_out, _, _ = oracle_request(dataclasses.replace(inp, topk_idx=bad), 0)
    assert_close(to_np(w.out)[0], ref_out, what="out")


# ---------------------------------------------------------------------------
# Index lists longer than one list chunk (2,048 entries) and FP8 dense segments
# longer than one page-id chunk (4,000 tiles): the kernel refills its LDS row
# list and carries the online-softmax state across the refill.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cache", [I.DTYPE_BF16, I.DTYPE_FP8, I.DTYPE_FP8_G128])
def test_topk_list_over_several_chunks(torch, R, cache):
    """4,100 picked positions (three list chunks: 2,048 + 2,048 + 4) in one
    request, 3,000 and padding in the other, in direct mode, on one worker
    and with the planner's split."""
    name = {I.DTYPE_BF16: "v2_batched", I.DTYPE_FP8: "v2_fp8_topk", I.DTYPE_FP8_G128: "v2_fp8g_topk"}[cache]
    _log(f"topk 4100 over chunks, {cache}")
    inp = I.make_inputs(name, seed=41, batch=2, ctx=(9000, 9000), topk=4100)
    inp.topk_idx[1, 3000:] = -1
    for mode in ("direct", 1, "auto"):
        _log(f"  mode {mode}")
        if mode == "direct":
            check_step(torch, R, inp, split=False)
        else:
            check_step(torch, R, inp, split=True, num_workers=None if mode == "auto" else mode)


@pytest.mark.parametrize("cache", [I.DTYPE_BF16, I.DTYPE_FP8, I.DTYPE_FP8_G128])
@pytest.mark.parametrize("T, extra_cols", [(1_000_000, 5), (2_500_000, 0), (1_000_000, -15_000)])
def test_topk_long_block_table_rows(torch, R, cache, T, extra_cols):
    """Index lists into contexts of 1,000,000 and 2,500,000 positions, with
    block-table rows of 15,630 and 39,063 entries: picks anywhere in a long
    row resolve to the right page.  The last case's row has 625 entries
    (fewer than the context's pages), so picks past its pages are skipped.
    The logical pages map onto a 48-page pool (logical page j on the physical
    page of page j % 48 of a 3,072-position request), so the oracle reads
    position p at (p / 64 % 48) * 64 + p % 64 of that request."""
    import dataclasses
    name = {I.DTYPE_BF16: "v2_batched", I.DTYPE_FP8: "v2_fp8_topk", I.DTYPE_FP8_G128: "v2_fp8g_topk"}[cache]
    _log(f"topk over a {T}-position context, {cache}, table columns {extra_cols:+d}")
    small = I.make_inputs(name, seed=43, batch=1, ctx=(48 * 64, 48 * 64), topk=0)
    pool, table = I.build_paged_pool(small)
    pages = -(-T // 64)
    cols = pages + extra_cols
    long_table = np.ascontiguousarray(table[0][np.arange(cols) % 48][None, :], dtype=np.int32)
    rng = np.random.default_rng(43)
    k = 600
    idx = np.sort(rng.choice(T, k, replace=False)).astype(np.int32)[None, :]
    inp = dataclasses.replace(small, seq_lens=np.array([T], np.int32), offsets=np.array([0, T], np.int64),
                              topk_idx=idx)
    seen = idx[0][(idx[0] >> 6) < cols]
    src = (seen >> 6) % 48 * 64 + (seen & 63)
    if cache in I.FP8_DTYPES:
        c = oracle.dequant_fp8_latent(small.c_codes[src], small.c_scales[src])
    else:
        c = small.c_kv[src]
    r_out, r_lse, r_olat = oracle.decode_unabsorbed(c, small.k_rope[src], small.q_nope[0], small.q_rope[0],
                                                    small.w_uk, small.w_uv, small.scale)
    for split in (False, True):
        w = R.DeviceWorkload(inp, split=split, pool=pool, table=long_table)
        w.step()
        torch.cuda.synchronize()
        assert_close(to_np(w.out)[0], r_out, what=f"out split={split}")
        assert_close(to_np(w.o_lat)[0], r_olat, what=f"o_lat split={split}")
        assert_close(to_np(w.lse)[0], r_lse, abs_tol=LSE_ABS_TOL, what=f"lse split={split}")


@pytest.mark.parametrize("name", ["v2_fp8_topk", "v2_fp8g_topk"])
def test_fp8_dense_over_one_page_chunk(torch, R, name):
    """One dense FP8 request of 130,000 positions (4,063 tiles: one full chunk
    of 4,000 tiles and a second one) in direct mode and on one worker."""
    _log(f"{name} dense 130000 positions")
    inp = I.make_inputs(name, seed=42, batch=1, ctx=(130000, 130000), topk=0)
    for mode in ("direct", 1):
        _log(f"  mode {mode}")
        if mode == "direct":
            check_step(torch, R, inp, split=False)
        else:
            check_step(torch, R, inp, split=True, num_workers=1)


# ---------------------------------------------------------------------------
# Index handling at the full list length, through the planner's split
# ---------------------------------------------------------------------------
LOW, HIGH, REQ, ONE = 0, 64, 128, 136  # latent dims of the count pattern


def _count_pattern_case(cache, B=32, T=4096, k=2048, seed=8):
    """Zero queries (every picked position gets probability 1).  Latent dim
    p % 64 and dim 64 + p // 64 of position p hold 1 (a one-hot code of the
    position), dims 128..132 hold the bits of the request index, dim 136 holds
    1, every other dim 0.  All values are 0 or 1: exact in BF16 and in E4M3
    (code 0x38) with unit scales."""
    rng = np.random.default_rng(seed)
    H, D_C, D_R = 128, 512, 64
    pos = np.tile(np.arange(T), B)
    rows = np.arange(B * T)
    c = np.zeros((B * T, D_C), np.float32)
    c[rows, LOW + pos % 64] = 1
    c[rows, HIGH + pos // 64] = 1
    req = np.repeat(np.arange(B), T)
    for j in range(5):
        c[:, REQ + j] = (req >> j) & 1
    c[:, ONE] = 1
    codes = scales = None
    if cache in I.FP8_DTYPES:
        codes = np.where(c > 0, 0x38, 0).astype(np.uint8)
        scales = np.ones(B * T, np.float32) if cache == I.DTYPE_FP8 else np.ones((B * T, D_C // 128), np.float32)
    idx = np.stack([np.sort(rng.choice(T, k, replace=False)) for _ in range(B)]).astype(np.int32)
    inp = custom_inputs(c, np.zeros((B * T, D_R)), np.zeros((B, H, 128)), np.zeros((B, H, D_R)),
                        np.zeros((H, D_C, 128)), np.zeros((H, 128, D_C)), [T] * B, cache, I.DTYPE_BF16, 0.1,
                        topk_idx=idx, codes=codes, scales=scales, perm_seed=seed)
    return inp, idx


# one picked position more or less moves the merged lse by ln(2049/2048) = 4.9e-4
LSE_COUNT_TOL = 5e-5


@pytest.mark.parametrize("cache", [I.DTYPE_BF16, I.DTYPE_FP8, I.DTYPE_FP8_G128])
def test_topk_2048_counts_exact_through_split(torch, R, cache):
    """32 requests x 2,048 picks over the planner's worker split (the launch
    shape of the sparse workload).  Each partial (o_s, lse_s) of a worker
    covers count_s picked positions of one request: exp(lse_s) = count_s and
    o_s[d] = n_d / count_s, with n_d the number of its positions whose one-hot
    code sets dim d.  The n_d are small (a few per dim), so the BF16 rounding
    of o_s (at most 2^-8 relative) moves n_d = o_s[d] * count_s by far less
    than 1/2 and both integers are recovered exactly; the request bits say
    which request the partial belongs to.  Summed over the partials of a
    request, the counts must equal the histograms of position % 64 and
    position / 64 of its index list: a missing, repeated or wrong index
    changes one of these integers.  The merged lse must be ln 2,048 for every
    request and head."""
    _log(f"topk 2048 exact counts through the split, {cache}")
    inp, idx = _count_pattern_case(cache)
    w = R.DeviceWorkload(inp, split=True)
    assert w.plan.num_workers > inp.B, "the split must spread requests over several workers"
    w.workspace.fill_(0xFF)                     # unwritten partials read as NaN
    w.attend(q_lat=torch.zeros_like(w.q_lat))
    torch.cuda.synchronize()
    part_o, part_l = (x.cpu().numpy().astype(np.float64) for x in w.partials())
    counts = np.zeros(inp.B, np.int64)
    hist = np.zeros((inp.B, 128), np.int64)
    used = 0
    for s_ in range(part_o.shape[0]):
        l = part_l[s_]
        if not np.isfinite(l[0]):
            continue
        used += 1
        assert np.all(l == l[0]), f"slot {s_}: heads disagree"
        assert np.all(part_o[s_] == part_o[s_][0]), f"slot {s_}: heads disagree"
        o = part_o[s_][0]
        n = float(np.exp(l[0]))
        cnt = int(round(n))
        assert cnt >= 1 and abs(n - cnt) < 1e-3, f"slot {s_}: exp(lse) = {n}"
        assert o[ONE] == 1.0, f"slot {s_}: weights do not sum to one ({o[ONE]})"
        reqbits = o[REQ:REQ + 5]
        assert np.all((reqbits == 0) | (reqbits == 1)), f"slot {s_}: positions of several requests"
        b = int(np.sum(reqbits.astype(np.int64) << np.arange(5)))
        nd = o[:128] * cnt
        assert np.all(np.abs(nd - np.round(nd)) < 0.25), f"slot {s_}: counts not integral"
        counts[b] += cnt
        hist[b] += np.round(nd).astype(np.int64)
    assert used >= inp.B
    for b in range(inp.B):
        sel = idx[b]
        assert counts[b] == sel.size, f"request {b}: {counts[b]} positions weighted, {sel.size} picked"
        expect = np.concatenate([np.bincount(sel % 64, minlength=64), np.bincount(sel // 64, minlength=64)])
        assert np.array_equal(hist[b], expect), f"request {b}: position histograms differ"
    w.combine()
    torch.cuda.synchronize()
    lse = w.lse.cpu().numpy().astype(np.float64)
    err = np.max(np.abs(lse - math.log(2048)))
    assert err <= LSE_COUNT_TOL, f"merged lse off by {err}"
    o_lat = w.o_lat.float().cpu().numpy()
    assert np.all(o_lat[:, :, ONE] == 1.0)


# ---------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------
def test_v2_single_full(torch, R):
    _log("v2_single full")
    check_step(torch, R, I.make_inputs("v2_single"), split=True)


def test_v2_batched_full_size(torch, R):
    """All 128 heads of eight requests (the first and last two, and four
    from the middle, each spread over several workers), and four heads, one
    per wave, of every request."""
    _log("v2_batched full size")
    inp = I.make_inputs("v2_batched")
    check_step(torch, R, inp, split=True,
               checks=[([0, 1, 17, 31, 32, 47, 62, 63], None), (range(inp.B), [0, 40, 77, 127])])


@pytest.mark.parametrize("workers", [16, 32])
def test_v2_xcd_weighted_split(torch, R, workers):
    """The split weighted by XCD (dense batches, a power-of-two worker count,
    at least 64 units per worker: workers on even XCDs take 65/64 of an
    equal share, odd ones 63/64) against the oracle: 5 requests of 6K-12K
    positions (about 1,400 units), 16 workers (weighted) and 32 (equal
    shares), every request and head."""
    _log(f"xcd-weighted split, {workers} workers")
    inp = I.make_inputs("v2_batched", seed=41, batch=5, ctx=(6000, 12000))
    check_step(torch, R, inp, split=True, num_workers=workers)


@pytest.mark.parametrize("layer", [0, 29, 59])
def test_v2_long_layer_full(torch, R, layer):
    """Long context (1 request x 131,072 positions): the first, middle and
    last of the 60 independently drawn layers, every head."""
    _log(f"v2_long layer {layer}")
    inp = I.make_inputs("v2_long", layer=layer)
    check_step(torch, R, inp, split=True)


@pytest.fixture(scope="module")
def fp8_full():
    return I.make_inputs("v2_fp8_topk")


def test_fp8_topk_full_size(torch, R, fp8_full):
    """32 requests x 65,536 positions, 2,048 picked each, one scale per
    position: every request and head."""
    _log("v2_fp8_topk full size")
    check_step(torch, R, fp8_full, split=True)


def test_fp8_group_scales_topk_full_size(torch, R, fp8_full):
    _log("v2_fp8g_topk full size (same draw, per-128-channel scales)")
    inp = I.requantize(fp8_full, I.DTYPE_FP8_G128)
    check_step(torch, R, inp, split=True)


@pytest.mark.parametrize("cache", [I.DTYPE_FP8, I.DTYPE_FP8_G128])
def test_fp8_topk_full_size_count(torch, R, fp8_full, cache):
    """With zero queries every picked position has probability 1, so the
    merged lse is ln 2,048 for every request and head, through the planner's
    split of the full workload, and o_lat is the mean of the picked latents."""
    _log(f"v2 fp8 top-k full size, zero queries, {cache}")
    inp = fp8_full if cache == I.DTYPE_FP8 else I.requantize(fp8_full, I.DTYPE_FP8_G128)
    w = R.DeviceWorkload(inp, split=True)
    w.q_rope.zero_()
    w.attend(q_lat=torch.zeros_like(w.q_lat))
    w.combine()
    torch.cuda.synchronize()
    lse = w.lse.cpu().numpy().astype(np.float64)
    err = np.max(np.abs(lse - math.log(2048)))
    assert err <= LSE_COUNT_TOL, f"lse off by {err}"
    o_lat = to_np(w.o_lat)
    for b in (0, 15, 31):
        lo, hi = inp.request(b)
        c = oracle.dequant_fp8_latent(inp.c_codes[lo:hi], inp.c_scales[lo:hi])
        ref, _ = oracle.latent_decode(np.zeros((inp.H, inp.D_C)), np.zeros((inp.H, inp.D_R)), c, inp.k_rope[lo:hi],
                                      inp.scale, picked=inp.topk_idx[b])
        assert_close(o_lat[b], ref, what=f"o_lat b={b}")
