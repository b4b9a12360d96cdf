"""GPU parity of prefill on the expanded path (mla_prepare_w_uk_t,
mla_prefill_expand, mla_prefill_attn) through the C ABI against the float64
oracle.

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


def check_queries(w, inp, qn, qr, queries, heads):
    out, lse = _np(w.out), w.lse.cpu().numpy()
    T, N = w.T, w.N
    for i in queries:
        pos = T - N + i
        ref_o, ref_l, _ = oracle.decode_unabsorbed(inp.c_kv[:pos + 1], inp.k_rope[:pos + 1], qn[i], qr[i],
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
