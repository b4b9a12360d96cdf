"""GPU parity of the lightning indexer and the top-k pick, through the C ABI,
against the float64 oracle (oracle/dsa_indexer.py).

Tolerances:
  * scores: max |err| <= 1e-4 * max |ref| per request.  Derived from the
    arithmetic: the BF16 queries and the E4M3 keys (exact in BF16) multiply
    exactly in float32, the 128-term dot products and the 64-term weighted
    ReLU sum accumulate in float32 (relative error ~1e-6 for these sizes),
    and the scale is one float32 multiply.
  * pick on given float32 scores: bit-exact (both sides rank the same float32
    values, ties to the lower position).
  * pick on the kernel's own scores: where float rounding decides the order,
    the picked set is checked for validity against the oracle's scores (every
    picked position scores at least the best unpicked one, within the score
    tolerance), and everything unique (count, order, range) exactly.
"""

import numpy as np
import pytest

from oracle import dsa_indexer as X
from mla_latent_kv_absorb_amd import inputs as I

pytestmark = pytest.mark.gpu

SCORE_TOL = 1e-4


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


def oracle_scores(inp, b):
    lo, hi = inp.request(b)
    keys = X.dequant_fp8_key(inp.k_codes[lo:hi], inp.k_scales[lo:hi])
    return X.indexer_scores(inp.q_idx[b], inp.w_idx[b], keys)


def check_scores(got_row, ref, what):
    err = np.max(np.abs(got_row.astype(np.float64) - ref))
    bound = SCORE_TOL * np.max(np.abs(ref))
    assert err <= bound, f"{what}: max|err| {err:.3g} > {bound:.3g}"


def check_pick_valid(idx_row, ref, T, k, what):
    """Unique parts exactly; the choice among near-equal scores by validity."""
    n = min(k, T)
    picked = idx_row[:n]
    assert np.all(idx_row[n:] == -1), what
    assert np.all(np.diff(picked) > 0) and picked.min() >= 0 and picked.max() < T, what
    if n == T:
        return
    band = 2 * SCORE_TOL * np.max(np.abs(ref))
    mask = np.zeros(T, bool)
    mask[picked] = True
    assert ref[mask].min() >= ref[~mask].max() - band, what
    # positions the oracle ranks clearly inside (outside) are picked (not picked)
    thr = np.sort(ref)[::-1][n - 1]
    assert np.all(mask[ref > thr + band]), what
    assert not np.any(mask[ref < thr - band]), what


@pytest.mark.parametrize("ctx", [(100, 2500), (4097, 9000)])
def test_indexer_scores_ragged(torch, R, ctx):
    """Lengths inside one work-group's 4,096-position chunk, and lengths that
    span two or three chunks with a partial last one."""
    _log(f"indexer scores, ragged lengths {ctx}")
    inp = I.make_indexer_inputs(seed=61, batch=3, ctx=ctx, topk=64)
    w = R.IndexerWorkload(inp, score_stride=int(inp.seq_lens.max()) + 77)
    w.scores.fill_(12345.0)
    w.score()
    torch.cuda.synchronize()
    got = w.scores.cpu().numpy()
    for b in range(inp.B):
        T = int(inp.seq_lens[b])
        check_scores(got[b, :T], oracle_scores(inp, b), f"b={b}")
        assert np.all(got[b, T:] == 12345.0), "entries past the length are left alone"


def test_indexer_invalid_page_scores_minus_inf(torch, R):
    _log("indexer invalid page")
    inp = I.make_indexer_inputs(seed=62, batch=1, ctx=(300, 300), topk=16)
    pool, table = I.build_key_pool(inp)
    table = table.copy()
    table[0, 2] = pool.shape[0] + 5      # positions 128..191 sit on a page that does not exist
    w = R.IndexerWorkload(inp, pool=pool, table=table)
    w.score()
    torch.cuda.synchronize()
    got = w.scores.cpu().numpy()[0]
    assert np.all(np.isneginf(got[128:192]))
    ref = oracle_scores(inp, 0)
    keep = np.r_[0:128, 192:300]
    check_scores(got[keep], ref[keep], "valid pages")


def _score_rows(rng, B, stride):
    s = rng.standard_normal((B, stride)).astype(np.float32)
    s[1] = np.round(s[1] * 4) / 4                     # many exact ties
    s[2, ::7] = -0.0                                  # signed zeros among zeros
    s[2, 3::7] = 0.0
    s[3, 5:40] = np.nan                               # NaN ranks below everything
    s[3, 40:60] = -np.inf
    s[4] = 1.0                                        # one value everywhere
    return s


@pytest.mark.parametrize("k", [1, 5, 2048])
def test_topk_select_bit_exact(torch, R, k):
    _log(f"topk select k={k}")
    from mla_latent_kv_absorb_amd import binding as B
    rng = np.random.default_rng(70 + k)
    stride = 9000
    s = _score_rows(rng, 6, stride)
    lens = np.array([9000, 8191, 2049, 5000, 4096, 1500], np.int32)
    lens[5] = max(1, min(lens[5], k - 1)) if k > 1 else 1   # a row with fewer positions than k
    scores = torch.from_numpy(s).cuda()
    seq = torch.from_numpy(lens).cuda()
    idx = torch.full((6, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(B.topk_workspace_bytes(6, stride), dtype=torch.uint8, device="cuda")
    for rep in range(2):  # the workspace is reused: the call clears it itself
        B.mla_topk_select(scores, seq, k, idx, ws)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        for b in range(6):
            want = X.select_topk_from_scores(s[b], int(lens[b]), k)
            assert np.array_equal(got[b], want), f"row {b} rep {rep}"


def test_topk_select_long_row_and_zero_length(torch, R):
    _log("topk select long row")
    from mla_latent_kv_absorb_amd import binding as B
    rng = np.random.default_rng(80)
    stride = 140000
    s = rng.standard_normal((2, stride)).astype(np.float32) * 50
    lens = np.array([131072, 0], np.int32)
    k = 2048
    idx = torch.empty((2, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(B.topk_workspace_bytes(2, stride), dtype=torch.uint8, device="cuda")
    B.mla_topk_select(torch.from_numpy(s).cuda(), torch.from_numpy(lens).cuda(), k, idx, ws)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert np.array_equal(got[0], X.select_topk_from_scores(s[0], 131072, k))
    assert np.all(got[1] == -1)


def test_indexer_then_pick_small(torch, R):
    _log("indexer + pick, small")
    inp = I.make_indexer_inputs(seed=63, batch=4, ctx=(200, 5000), topk=256)
    w = R.IndexerWorkload(inp)
    w.step()
    torch.cuda.synchronize()
    idx = w.idx.cpu().numpy()
    for b in range(inp.B):
        T = int(inp.seq_lens[b])
        check_pick_valid(idx[b], oracle_scores(inp, b), T, inp.topk, f"b={b}")


def _two_calls_then_fused(torch, w):
    """(scores, idx) of the two calls, then of the one-call form, on w."""
    w.step()
    torch.cuda.synchronize()
    s2, i2 = w.scores.cpu().numpy().copy(), w.idx.cpu().numpy().copy()
    w.scores.fill_(777.0)
    w.idx.fill_(-7)
    w.score_and_select()
    torch.cuda.synchronize()
    return s2, i2, w.scores.cpu().numpy(), w.idx.cpu().numpy()


@pytest.mark.parametrize("stride", ["wide", 5000, 5001])
def test_fused_indexer_topk_equals_two_calls(torch, R, stride):
    """mla_indexer_topk builds the pick's first histogram inside the score
    kernel: same float32 scores, same picks (bit-exact), on ragged rows that
    span several chunks, with some rows at or below k.  With score rows of
    5,000 entries the longer requests are cut to the row width in both
    paths; with 5,001 the rows after the first start off a 16-byte boundary,
    so the pick reads them with scalar loads."""
    _log(f"indexer + pick in one call, ragged, stride {stride}")
    # request 1 has exactly k positions and request 3 fewer: every position
    # is picked and no histogram is built for them
    inp = I.make_indexer_inputs(seed=64, seq_lens=[3000, 2048, 9500, 1500, 7001], topk=2048)
    width = int(inp.seq_lens.max()) + 50 if stride == "wide" else stride
    w = R.IndexerWorkload(inp, score_stride=width)
    s2, i2, s1, i1 = _two_calls_then_fused(torch, w)
    for b in range(inp.B):
        T = min(int(inp.seq_lens[b]), width)
        assert np.array_equal(s1[b, :T].view(np.uint32), s2[b, :T].view(np.uint32)), f"scores b={b}"
    assert np.array_equal(i1, i2)
    check_pick_valid(i1[0], oracle_scores(inp, 0), int(inp.seq_lens[0]), inp.topk, "b=0")
    if stride != "wide":
        # request 2 (9,500 positions) is picked among its first 5,000 (5,001)
        check_pick_valid(i1[2], oracle_scores(inp, 2)[:width], width, inp.topk, "b=2 cut to the row")


def test_fused_indexer_topk_caps_at_block_table(torch, R):
    """Positions past 64 * block_table_stride have no page: the one-call form
    scores and picks among min(seq_len, 64 * stride) positions, which is what
    the two calls give with the lengths capped there."""
    _log("indexer + pick in one call, short block table")
    inp = I.make_indexer_inputs(seed=65, batch=3, ctx=(6000, 9000), topk=512)
    pool, table = I.build_key_pool(inp)
    n = 80                                        # 5,120 positions reachable
    short = np.ascontiguousarray(table[:, :n])
    w = R.IndexerWorkload(inp, pool=pool, table=short, score_stride=int(inp.seq_lens.max()))
    w.score_and_select()
    torch.cuda.synchronize()
    i1 = w.idx.cpu().numpy().copy()
    w.seq_lens.copy_(torch.from_numpy(np.minimum(inp.seq_lens, 64 * n).astype(np.int32)))
    w.step()
    torch.cuda.synchronize()
    assert np.array_equal(i1, w.idx.cpu().numpy())


def test_indexer_then_pick_full_size_sampled(torch, R):
    """32 requests x 65,536 positions, top-2,048: the sizes and launch shape
    the benchmark times; scores and picks checked on sampled requests, and the
    one-call form equal to the two calls on every request."""
    _log("indexer full size")
    inp = I.make_indexer_inputs()
    w = R.IndexerWorkload(inp)
    scores, idx, s1, i1 = _two_calls_then_fused(torch, w)
    assert np.array_equal(s1.view(np.uint32), scores.view(np.uint32))
    assert np.array_equal(i1, idx)
    for b in (0, 13, 31):
        ref = oracle_scores(inp, b)
        check_scores(scores[b], ref, f"b={b}")
        check_pick_valid(idx[b], ref, int(inp.seq_lens[b]), inp.topk, f"b={b}")
