"""mla_decode_noalloc (partials in the library's static scratch) against the
calls it stands for: mla_decode_attn in split mode with a caller workspace,
then mla_combine or mla_combine_out_up.  The kernels and the plan are the
same, so the outputs must be bit-identical.  Two calls in a row, the second
with a smaller batch and shorter contexts, so the second reads a scratch that
still holds the first call's partials."""

import numpy as np
import pytest

from mla_latent_kv_absorb_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _log(msg):
    print(msg, flush=True)


def _both(torch, inp, form):
    from mla_latent_kv_absorb_amd import binding as B
    from mla_latent_kv_absorb_amd import runner
    w = runner.DeviceWorkload(inp, split=True)
    w.absorb()
    # the existing calls, caller workspace
    w.attend()
    if form == "out":
        w.combine_up()
        ref = (w.out.clone(), w.lse.clone())
    else:
        w.combine()
        ref = (w.o_lat.clone(), w.lse.clone())
    torch.cuda.synchronize()
    # the no-allocation call, into fresh outputs
    got_lse = torch.full_like(w.lse, float("nan"))
    if form == "out":
        got = torch.zeros_like(w.out)
        B.mla_decode_noalloc(w.cfg, w.q_lat, w.q_rope, w.pool, w.table, w.seq_lens, w.plan, topk_idx=w.topk_idx,
                             w_uv=w.w_uv, out=got, lse_out=got_lse)
    else:
        got = torch.zeros_like(w.o_lat)
        B.mla_decode_noalloc(w.cfg, w.q_lat, w.q_rope, w.pool, w.table, w.seq_lens, w.plan, topk_idx=w.topk_idx,
                             o_lat=got, lse_out=got_lse)
    torch.cuda.synchronize()
    assert torch.equal(got, ref[0]), f"{form}: max |diff| {float((got.float() - ref[0].float()).abs().max())}"
    assert torch.equal(got_lse, ref[1])


@pytest.mark.parametrize("form", ["out", "o_lat"])
def test_noalloc_bf16_two_calls_second_smaller(torch, form):
    _log(f"noalloc bf16 {form}")
    big = I.make_inputs("v2_batched", seed=71, batch=12, ctx=(3000, 9000))
    small = I.make_inputs("v2_batched", seed=72, batch=3, ctx=(100, 700))
    _both(torch, big, form)
    _both(torch, small, form)


def test_noalloc_fp8_topk_and_float32(torch):
    _log("noalloc fp8 top-k and float32")
    fp8 = I.make_inputs("v2_fp8g_topk", seed=73, batch=6, ctx=(3000, 5000), topk=300)
    fp8.topk_idx[2, 250:] = -1
    _both(torch, fp8, "out")
    _both(torch, I.make_inputs("tiny_fp32", seq_lens=[1, 33, 64, 100, 7]), "o_lat")


def test_noalloc_largest_batch_that_fits(torch):
    """256 workers and 127 requests: 382 partial slots, the scratch's
    capacity at V2 dims."""
    _log("noalloc at capacity")
    inp = I.make_inputs("v2_batched", seed=74, batch=127, ctx=(100, 400))
    _both(torch, inp, "out")
