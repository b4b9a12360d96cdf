"""GPU parity of prefill on the expanded path (mla_prepare_w_uk_t,
mla_prefill_expand, mla_prefill_attn) through the C ABI against the float64
oracle, from BF16 and FP8 caches.

Bars: the rotary keys are copies (bit-exact); the expanded keys and values
are one GEMM each with float32 accumulation and one BF16 rounding (max |err|
<= 1e-2 * max |ref| per head); the attention output is the BF16 bound of the
decode path (max |err| <= 2e-2 * max |ref|), lse within 2e-2 absolute.
"""

import numpy as np
import pytest

import oracle
from mla_latent_kv_absorb_amd import inputs as I

pytestmark = pytest.mark.gpu


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


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def latent_of(inp):
    """The cached latent as the oracle reads it: the BF16 values, or the E4M3
    codes times their scales in float64."""
    if inp.cache_dtype in I.FP8_DTYPES:
        return oracle.dequant_fp8_latent(inp.c_codes, inp.c_scales)
    return inp.c_kv


def check_queries(w, inp, qn, qr, queries, heads):
    out, lse = _np(w.out), w.lse.cpu().numpy()
    T, N = w.T, w.N
    c = latent_of(inp)
    for i in queries:
        pos = T - N + i
        ref_o, ref_l, _ = oracle.decode_unabsorbed(c[:pos + 1], inp.k_rope[:pos + 1], qn[i], qr[i],
                                                   inp.w_uk, inp.w_uv, inp.scale, heads=heads)
        err = np.max(np.abs(out[i][heads] - ref_o))
        assert err <= 2e-2 * np.max(np.abs(ref_o)), f"query {i}: {err}"
        assert np.max(np.abs(lse[i][heads] - ref_l)) <= 2e-2, f"lse query {i}"


def test_prefill_expand(torch, R):
    _log("prefill expand")
    inp = I.make_inputs("v2_single", seed=51, ctx=(300, 300))
    qn, qr = I.make_prefill_queries(inp, 16, seed=52)
    w = R.PrefillWorkload(inp, qn, qr)
    w.expand()
    torch.cuda.synchronize()
    kn, v, kr = _np(w.k_nope), _np(w.v), _np(w.k_rope)
    np.testing.assert_array_equal(kr, inp.k_rope)
    for h in (0, 31, 64, 127):
        ref_k, ref_v = oracle.expand_keys_values(inp.c_kv, inp.w_uk, inp.w_uv, h)
        assert np.max(np.abs(kn[:, h] - ref_k)) <= 1e-2 * np.max(np.abs(ref_k)), f"k head {h}"
        assert np.max(np.abs(v[:, h] - ref_v)) <= 1e-2 * np.max(np.abs(ref_v)), f"v head {h}"


@pytest.mark.parametrize("name", ["v2_fp8_topk", "v2_fp8g_topk"])
def test_prefill_expand_fp8(torch, R, name):
    """FP8 caches, one scale per position and one per 128 channels, with the
    scales spread over 2^-3 .. 2^3 across positions (and groups): the
    expansion reads code x scale.  Bound 1e-2 x max|ref| per head as for
    BF16: with per-position scales the sums run on the exact codes and take
    the scale in float32; group-scaled values are rounded once to BF16."""
    _log(f"prefill expand {name}")
    inp = I.make_inputs(name, seed=56, batch=1, ctx=(333, 333), topk=0)
    rng = np.random.default_rng(56)
    inp.c_scales[:] = inp.c_scales * np.exp2(rng.integers(-3, 4, size=inp.c_scales.shape)).astype(np.float32)
    qn, qr = I.make_prefill_queries(inp, 8, seed=57)
    w = R.PrefillWorkload(inp, qn, qr)
    w.expand()
    torch.cuda.synchronize()
    kn, v, kr = _np(w.k_nope), _np(w.v), _np(w.k_rope)
    np.testing.assert_array_equal(kr, inp.k_rope)
    c = latent_of(inp)
    for h in (0, 33, 64, 127):
        ref_k, ref_v = oracle.expand_keys_values(c, inp.w_uk, inp.w_uv, h)
        assert np.max(np.abs(kn[:, h] - ref_k)) <= 1e-2 * np.max(np.abs(ref_k)), f"k head {h}"
        assert np.max(np.abs(v[:, h] - ref_v)) <= 1e-2 * np.max(np.abs(ref_v)), f"v head {h}"


@pytest.mark.parametrize("name", ["v2_fp8_topk", "v2_fp8g_topk"])
def test_prefill_attn_fp8(torch, R, name):
    _log(f"prefill {name} T=700 N=130")
    inp = I.make_inputs(name, seed=58, batch=1, ctx=(700, 700), topk=0)
    qn, qr = I.make_prefill_queries(inp, 130, seed=59)
    w = R.PrefillWorkload(inp, qn, qr)
    w.step()
    torch.cuda.synchronize()
    check_queries(w, inp, qn, qr, [0, 31, 64, 129], [0, 40, 127])


@pytest.mark.parametrize("T,N", [(300, 300), (300, 77), (97, 1), (1000, 260)])
def test_prefill_attn_small(torch, R, T, N):
    _log(f"prefill T={T} N={N}")
    inp = I.make_inputs("v2_single", seed=53 + T + N, ctx=(T, T))
    qn, qr = I.make_prefill_queries(inp, N, seed=54 + N)
    w = R.PrefillWorkload(inp, qn, qr)
    w.step()
    torch.cuda.synchronize()
    queries = sorted({0, N // 2, N - 1} | ({31, 32, 127, 128} & set(range(N))))
    check_queries(w, inp, qn, qr, queries, [0, 77, 127])


def test_prefill_full_size_sampled(torch, R):
    """The V2 single-request shape: a 4,096-token prompt prefilled at once
    (every query causal over the prompt); sampled queries and heads."""
    _log("prefill 4096 x 4096")
    inp = I.make_inputs("v2_single")
    qn, qr = I.make_prefill_queries(inp, 4096, seed=55)
    w = R.PrefillWorkload(inp, qn, qr)
    w.step()
    torch.cuda.synchronize()
    check_queries(w, inp, qn, qr, [0, 1, 127, 128, 2047, 4095], [0, 64, 127])
