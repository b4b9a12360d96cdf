"""GPU parity of mla_cache_append through the C ABI against the oracle
(oracle/cache_append.py).

Bars: latent bytes exact (BF16 / F32 copies; FP8 codes and scales are integer
and float32 decisions taken in float32 on both sides, so bit-exact); rotated
keys within one BF16 step (the kernel rotates in float32, the oracle in
float64, then both round); every byte outside the written rows unchanged.
After the append, the decode step over T + 1 positions matches the oracle
with the stored token.
"""

import numpy as np
import pytest

import oracle
from oracle import cache_append as A
from mla_latent_kv_absorb_amd import inputs as I

pytestmark = pytest.mark.gpu

CACHE_NAME = {I.DTYPE_F32: "f32", I.DTYPE_BF16: "bf16", I.DTYPE_FP8: "fp8", I.DTYPE_FP8_G128: "fp8_g128"}


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


def rope_tables(rows, d_r):
    theta = 10000.0 ** (-np.arange(0, d_r, 2) / d_r)
    ang = np.arange(rows)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def make_case(name, seed, batch, ctx, cache=None):
    inp = I.make_inputs(name, seed=seed, batch=batch, ctx=ctx, topk=0)
    if cache is not None and cache != inp.cache_dtype:
        inp = I.requantize(inp, cache)
    pool, table = I.build_paged_pool(inp, extra_pages=batch)
    # room for one more position: a fresh page where the next position starts one
    table = np.concatenate([table, np.full((batch, 1), -1, np.int32)], axis=1)
    nxt = int(inp.page_perm.shape[0])
    for b in range(batch):
        T = int(inp.seq_lens[b])
        if table[b, T // 64] < 0:
            table[b, T // 64] = nxt
            nxt += 1
    rng = np.random.default_rng(seed + 1)
    act = inp.act_dtype
    c_new = rng.standard_normal((batch, inp.D_C)).astype(np.float32)
    k_new = rng.standard_normal((batch, inp.D_R)).astype(np.float32)
    if act == I.DTYPE_BF16:
        c_new, k_new = I.round_to_bf16(c_new), I.round_to_bf16(k_new)
    return inp, pool, table, c_new, k_new


def expected_rows(inp, c_new, k_new, cos, sin, positions):
    out = []
    for b in range(inp.B):
        p = positions[b]
        out.append(A.append_token(c_new[b], k_new[b], cos[p], sin[p], CACHE_NAME[inp.cache_dtype]))
    return out


def check_pool(inp, before, after, table, positions, rows, skip=()):
    lay = I.page_layout(inp.cache_dtype, inp.D_C, inp.D_R)
    changed = np.zeros(after.shape, bool)
    for b in range(inp.B):
        if b in skip:
            continue
        p = positions[b]
        page, slot = table[b, p // 64], p % 64
        payload, krot, scales = rows[b]
        if inp.cache_dtype == I.DTYPE_F32:
            c_sec = after[page, :lay["r_off"]].view(np.float32).reshape(64, inp.D_C)
            r_sec = after[page, lay["r_off"]:lay["r_off"] + 64 * inp.D_R * 4].view(np.float32).reshape(64, inp.D_R)
            np.testing.assert_array_equal(c_sec[slot], payload)
            np.testing.assert_allclose(r_sec[slot], krot, rtol=1e-6, atol=1e-7)
            w = 4
        else:
            r_sec = after[page, lay["r_off"]:lay["r_off"] + 64 * inp.D_R * 2].view(np.uint16).reshape(64, inp.D_R)
            got_r = (r_sec[slot].astype(np.uint32) << 16).view(np.float32)
            assert np.all(np.abs(got_r - krot) <= np.abs(krot) * 2.0 ** -7 + 1e-30), f"rope b={b}"
            if inp.cache_dtype == I.DTYPE_BF16:
                c_sec = after[page, :lay["r_off"]].view(np.uint16).reshape(64, inp.D_C)
                got_c = (c_sec[slot].astype(np.uint32) << 16).view(np.float32)
                np.testing.assert_array_equal(got_c, payload)
            else:
                c_sec = after[page, :64 * inp.D_C].reshape(64, inp.D_C)
                np.testing.assert_array_equal(c_sec[slot], payload, err_msg=f"codes b={b}")
                g = scales.shape[0]
                s_sec = after[page, lay["s_off"]:lay["s_off"] + 64 * g * 4].view(np.float32).reshape(64, g)
                np.testing.assert_array_equal(s_sec[slot], scales, err_msg=f"scales b={b}")
            w = 2
        # the bytes of this token's rows
        changed[page, slot * inp.D_C * (1 if inp.cache_dtype in I.FP8_DTYPES else w):
                (slot + 1) * inp.D_C * (1 if inp.cache_dtype in I.FP8_DTYPES else w)] = True
        changed[page, lay["r_off"] + slot * inp.D_R * w:lay["r_off"] + (slot + 1) * inp.D_R * w] = True
        if inp.cache_dtype in I.FP8_DTYPES:
            g = scales.shape[0]
            changed[page, lay["s_off"] + slot * 4 * g:lay["s_off"] + (slot + 1) * 4 * g] = True
    assert np.array_equal(before[~changed], after[~changed]), "bytes outside the written rows changed"


def run_append(torch, B, inp, pool, table, c_new, k_new, positions, cos, sin):
    R_cfg = B.make_config(inp.H, inp.D_C, inp.D_R, inp.D_N, inp.D_V, inp.scale,
                          {I.DTYPE_F32: B.MLA_F32, I.DTYPE_BF16: B.MLA_BF16, I.DTYPE_FP8: B.MLA_FP8_E4M3,
                           I.DTYPE_FP8_G128: B.MLA_FP8_E4M3_G128}[inp.cache_dtype],
                          B.MLA_F32 if inp.act_dtype == I.DTYPE_F32 else B.MLA_BF16)
    from mla_latent_kv_absorb_amd import runner
    dev_pool = torch.from_numpy(pool).cuda()
    B.mla_cache_append(R_cfg, runner.to_device_act(c_new, inp.act_dtype, "cuda"),
                       runner.to_device_act(k_new, inp.act_dtype, "cuda"),
                       torch.from_numpy(np.asarray(positions, np.int32)).cuda(), dev_pool,
                       torch.from_numpy(table).cuda(),
                       None if cos is None else torch.from_numpy(cos).cuda(),
                       None if sin is None else torch.from_numpy(sin).cuda())
    torch.cuda.synchronize()
    return dev_pool.cpu().numpy()


@pytest.mark.parametrize("cache", [I.DTYPE_BF16, I.DTYPE_FP8, I.DTYPE_FP8_G128, I.DTYPE_F32])
def test_append_rows_exact(torch, R, cache):
    _log(f"append {cache}")
    from mla_latent_kv_absorb_amd import binding as B
    if cache == I.DTYPE_F32:
        inp, pool, table, c_new, k_new = make_case("tiny_fp32", 41, 3, (60, 200))
    else:
        name = "v2_batched" if cache == I.DTYPE_BF16 else "v2_fp8_topk"
        inp, pool, table, c_new, k_new = make_case(name, 42, 5, (63, 700), cache=cache)
    positions = inp.seq_lens.astype(np.int64)
    cos, sin = rope_tables(int(positions.max()) + 1, inp.D_R)
    after = run_append(torch, B, inp, pool, table, c_new, k_new, positions, cos, sin)
    check_pool(inp, pool, after, table, positions, expected_rows(inp, c_new, k_new, cos, sin, positions))


def test_append_skips_bad_rows_and_stores_unrotated_without_tables(torch, R):
    _log("append edge cases")
    from mla_latent_kv_absorb_amd import binding as B
    inp, pool, table, c_new, k_new = make_case("v2_fp8_topk", 43, 4, (100, 300), cache=I.DTYPE_FP8_G128)
    positions = inp.seq_lens.astype(np.int64).copy()
    positions[1] = -1                              # negative: nothing written
    table = table.copy()
    table[2, positions[2] // 64] = pool.shape[0] + 3   # page id out of range: nothing written
    positions[3] = table.shape[1] * 64             # beyond the block table: nothing written
    after = run_append(torch, B, inp, pool, table, c_new, k_new, positions, None, None)
    zeros = np.zeros((1, inp.D_R // 2), np.float32)
    ident_cos, ident_sin = np.ones((1, inp.D_R // 2), np.float32), zeros
    rows = [A.append_token(c_new[b], k_new[b], None, None, "fp8_g128") for b in range(inp.B)]
    check_pool(inp, pool, after, table, np.maximum(positions, 0), rows, skip=(1, 2, 3))
    # tables that hold the identity rotation give the same bytes as no tables
    pos0 = np.zeros(inp.B, np.int64)
    t2 = table.copy()
    for b in range(inp.B):
        t2[b, 0] = table[0, 0]
    a1 = run_append(torch, B, inp, pool, t2[:1], c_new[:1], k_new[:1], pos0[:1], ident_cos, ident_sin)
    a2 = run_append(torch, B, inp, pool, t2[:1], c_new[:1], k_new[:1], pos0[:1], None, None)
    assert np.array_equal(a1, a2)


@pytest.mark.parametrize("cache", [I.DTYPE_BF16, I.DTYPE_FP8_G128])
def test_append_then_decode(torch, R, cache):
    """The decode step after the append sees T + 1 positions, the new token as
    stored: matches the oracle over the logical arrays with that token."""
    _log(f"append then decode {cache}")
    from mla_latent_kv_absorb_amd import binding as B
    name = "v2_batched" if cache == I.DTYPE_BF16 else "v2_fp8_topk"
    inp, pool, table, c_new, k_new = make_case(name, 44, 3, (200, 900), cache=cache)
    positions = inp.seq_lens.astype(np.int64)
    cos, sin = rope_tables(int(positions.max()) + 1, inp.D_R)
    after = run_append(torch, B, inp, pool, table, c_new, k_new, positions, cos, sin)
    rows = expected_rows(inp, c_new, k_new, cos, sin, positions)
    new_lens = inp.seq_lens + 1
    import dataclasses
    grown = dataclasses.replace(inp, seq_lens=new_lens.astype(np.int32))
    w = R.DeviceWorkload(grown, split=True, pool=after, table=table)
    w.step()
    torch.cuda.synchronize()
    out = w.out.float().cpu().numpy().astype(np.float64)
    for b in range(inp.B):
        lo, hi = inp.request(b)
        payload, krot, scales = rows[b]
        if cache == I.DTYPE_BF16:
            c = np.vstack([inp.c_kv[lo:hi], payload[None, :]])
        else:
            c = np.vstack([oracle.dequant_fp8_latent(inp.c_codes[lo:hi], inp.c_scales[lo:hi]),
                           oracle.dequant_fp8_latent(payload[None, :], scales[None, :])])
        kr = np.vstack([inp.k_rope[lo:hi], krot[None, :]])
        ref, _, _ = oracle.decode_unabsorbed(c, kr, inp.q_nope[b], inp.q_rope[b], inp.w_uk, inp.w_uv, inp.scale)
        err = np.max(np.abs(out[b] - ref))
        assert err <= 2e-2 * np.max(np.abs(ref)), f"b={b}: {err}"
