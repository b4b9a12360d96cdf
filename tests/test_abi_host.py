"""The C-ABI library on the host: it loads, exports every declared entry
point, and its host-side logic (layout, plan, validation, status codes)
behaves as the header states.  No GPU work is launched."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("mla_absorb.h", "mla_indexer.h")]


@pytest.fixture(scope="module")
def B():
    from mla_latent_kv_absorb_amd import binding
    return binding


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol(B):
    lib = B.raw_lib()
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTED)


def test_abi_version_and_status_strings(B):
    assert B.abi_version() == 1
    for s in (0, 1, 2, 3):
        assert B.status_string(s) not in ("", "unknown status")
    assert B.status_string(99) == "unknown status"


def v2(B, cache=None):
    return B.make_config(128, 512, 64, 128, 128, 1 / np.sqrt(192), B.MLA_BF16 if cache is None else cache, B.MLA_BF16)


def test_page_layout(B):
    assert B.page_layout(v2(B)) == (73728, 65536, 73728)
    pb, ro, so = B.page_layout(v2(B, B.MLA_FP8_E4M3))
    assert (pb, ro, so) == (32768 + 8192 + 256, 32768, 32768 + 8192)
    # per-position bytes actually read: 512 + 128 + 4 = 644
    assert (pb) // 64 == 644
    # one float32 scale per 128 latent channels: the 656-byte item
    pb, ro, so = B.page_layout(v2(B, B.MLA_FP8_E4M3_G128))
    assert (pb, ro, so) == (32768 + 8192 + 1024, 32768, 32768 + 8192)
    assert pb // 64 == 656
    tiny = B.make_config(4, 16, 8, 8, 8, 0.25, B.MLA_F32, B.MLA_F32)
    assert B.page_layout(tiny) == (64 * 24 * 4, 64 * 16 * 4, 64 * 24 * 4)


def test_plan_sizes_workspace(B):
    cfg = v2(B)
    lens = np.array([16384, 32768, 20000], dtype=np.int32)
    plan = B.mla_decode_plan(cfg, 3, lens, 0, 0, 256)
    tiles = int(np.sum((lens + 31) // 32))
    # one worker per CU, at least two tiles each
    assert plan.num_workers == min(256, -(-tiles // 2))
    assert plan.num_slots == plan.num_workers + 2
    assert plan.workspace_bytes == plan.num_slots * 128 * 512 * 4 + (plan.num_slots * 128 * 4 + 15) // 16 * 16
    small = B.mla_decode_plan(cfg, 1, np.array([100], np.int32), 0, 0, 256)
    assert small.num_workers == 2  # 4 tiles
    single = B.mla_decode_plan(cfg, 1, np.array([4096], np.int32), 0, 0, 256)
    assert single.num_workers == 64
    topk = B.mla_decode_plan(cfg, 32, None, 0, 2048, 256)
    assert topk.num_workers == 256
    # index lists: a multiple of the batch, so every worker serves one request
    assert B.mla_decode_plan(cfg, 32, None, 0, 2048, 100).num_workers == 96
    assert B.mla_decode_plan(cfg, 3, None, 0, 300, 256).num_workers == 15   # 30 tiles, two each
    assert B.mla_decode_plan(cfg, 40, None, 0, 64, 256).num_workers == 40   # 80 tiles
    assert B.mla_decode_plan(cfg, 300, None, 0, 64, 256).num_workers == 256  # fewer workers than requests


def test_invalid_arguments_rejected_before_launch(B):
    lib = B.raw_lib()
    cfg = v2(B)
    null = None
    assert lib.mla_absorb_q(ctypes.byref(cfg), null, null, null, 1, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_out_up(ctypes.byref(cfg), null, null, null, 1, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(None, null, null, null, 1, null) == B.MLA_ERR_INVALID_ARG
    # misaligned pointers
    p = ctypes.c_void_p(0x1001)
    assert lib.mla_absorb_q(ctypes.byref(cfg), p, p, p, 1, null) == B.MLA_ERR_INVALID_ARG
    # unsupported dims for the MFMA path
    bad = B.make_config(64, 512, 64, 128, 128, 0.1, B.MLA_BF16, B.MLA_BF16)
    q = ctypes.c_void_p(0x1000)
    assert lib.mla_absorb_q(ctypes.byref(bad), q, q, q, 1, null) == B.MLA_ERR_UNSUPPORTED
    # bad block size / dtype
    bs = v2(B)
    bs.block_size = 32
    assert lib.mla_absorb_q(ctypes.byref(bs), q, q, q, 1, null) == B.MLA_ERR_INVALID_ARG
    mixed = B.make_config(4, 16, 8, 8, 8, 0.25, B.MLA_BF16, B.MLA_F32)
    assert lib.mla_absorb_q(ctypes.byref(mixed), q, q, q, 1, null) == B.MLA_ERR_UNSUPPORTED
    # attention: split mode without workspace, dense with topk > 0, batch < 1
    plan = B.MlaPlan(4, 4, 1 << 20)
    args = [ctypes.byref(cfg), q, q, q, 10, q, 4, q, None, 0, 1, ctypes.byref(plan), None, 0, None, None, None]
    assert lib.mla_decode_attn(*args) == B.MLA_ERR_INVALID_ARG
    args2 = list(args)
    args2[9] = 5
    assert lib.mla_decode_attn(*args2) == B.MLA_ERR_INVALID_ARG
    args3 = list(args)
    args3[10] = 0
    assert lib.mla_decode_attn(*args3) == B.MLA_ERR_INVALID_ARG
    # too small workspace
    args4 = list(args)
    args4[12] = q
    args4[13] = 100
    assert lib.mla_decode_attn(*args4) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_combine(ctypes.byref(cfg), q, 100, q, 0, 1, ctypes.byref(plan), q, None, None) == B.MLA_ERR_INVALID_ARG
    # fused merge + up-projection: null weights, too small workspace, float32 config
    big = 1 << 30
    assert lib.mla_combine_out_up(ctypes.byref(cfg), q, big, q, 0, 1, ctypes.byref(plan), None, q, None,
                                  None) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_combine_out_up(ctypes.byref(cfg), q, 100, q, 0, 1, ctypes.byref(plan), q, q, None,
                                  None) == B.MLA_ERR_INVALID_ARG
    tiny = B.make_config(4, 16, 8, 8, 8, 0.25, B.MLA_F32, B.MLA_F32)
    assert lib.mla_combine_out_up(ctypes.byref(tiny), q, big, q, 0, 1, ctypes.byref(plan), q, q, None,
                                  None) == B.MLA_ERR_UNSUPPORTED


def test_host_metadata_check(B):
    cfg = v2(B)
    lens = np.array([100, 64], np.int32)
    table = np.array([[0, 1], [2, -1]], np.int32)
    assert B.mla_check_decode_inputs_host(cfg, lens, table, 3) == (0, -1)
    assert B.mla_check_decode_inputs_host(cfg, lens, table, 2) == (1, 1)       # page 2 out of range
    assert B.mla_check_decode_inputs_host(cfg, np.array([100, 0], np.int32), table, 3) == (1, 1)
    assert B.mla_check_decode_inputs_host(cfg, np.array([200, 64], np.int32), table, 3) == (1, 0)  # table too short
    good = np.array([[0, 5, 99, -1], [3, 4, 63, -1]], np.int32)
    assert B.mla_check_decode_inputs_host(cfg, lens, table, 3, good) == (0, -1)
    unsorted = np.array([[5, 0, 99, -1], [3, 4, 63, -1]], np.int32)
    assert B.mla_check_decode_inputs_host(cfg, lens, table, 3, unsorted) == (1, 0)
    dup = np.array([[0, 5, 99, -1], [3, 3, 63, -1]], np.int32)
    assert B.mla_check_decode_inputs_host(cfg, lens, table, 3, dup) == (1, 1)
    out_of_range = np.array([[0, 5, 100, -1], [3, 4, 63, -1]], np.int32)
    assert B.mla_check_decode_inputs_host(cfg, lens, table, 3, out_of_range) == (1, 0)
    pad_inside = np.array([[0, -1, 99, -1], [3, 4, 63, -1]], np.int32)
    assert B.mla_check_decode_inputs_host(cfg, lens, table, 3, pad_inside) == (1, 0)


def test_binding_rejects_bad_tensors(B):
    torch = pytest.importorskip("torch")
    cfg = v2(B)
    with pytest.raises(ValueError):
        B.mla_absorb_q(cfg, torch.zeros(1, 128, 128), torch.zeros(128, 512, 128), torch.zeros(1, 128, 512))


def test_indexer_layout_and_validation(B):
    # 128 E4M3 values + one float32 scale per position: 132 B, 8,448 per page
    assert B.indexer_page_layout(128) == (8448, 8192)
    # histogram, control words, 3 counters per 4,096-position chunk, gathered keys and positions
    assert B.topk_workspace_bytes(32, 65536) == 32 * (2048 + 16 + 3 * 16 + 2 * 65536) * 4
    assert B.topk_workspace_bytes(0, 65536) == 0 and B.topk_workspace_bytes(2, 0) == 0
    lib = B.raw_lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.cast(buf, ctypes.c_void_p)
    null = None
    # unsupported dims, then bad arguments: nothing is launched
    assert lib.mla_indexer_scores(32, 128, p, p, p, 1, p, 1, p, 1, p, 1, null) == B.MLA_ERR_UNSUPPORTED
    assert lib.mla_indexer_scores(64, 128, null, p, p, 1, p, 1, p, 1, p, 1, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_indexer_scores(64, 128, p, p, p, 1, p, 1, p, 0, p, 1, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_indexer_scores(64, 128, p, p, p, 1, p, 1, p, 1, p, 0, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_topk_select(p, 16, p, 2, 0, p, p, 1 << 16, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_topk_select(p, 16, p, 2, 4, p, p, 100, null) == B.MLA_ERR_INVALID_ARG   # workspace too small
    assert lib.mla_topk_select(null, 16, p, 2, 4, p, p, 1 << 16, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_topk_select(p, 2048 * 4096 + 1, p, 1, 4, p, p, 1 << 40, null) == B.MLA_ERR_UNSUPPORTED
    # both steps in one call: the checks of the two
    ws = 1 << 16
    assert lib.mla_indexer_topk(32, 128, p, p, p, 1, p, 1, p, 1, p, 16, 4, p, p, ws, null) == B.MLA_ERR_UNSUPPORTED
    assert lib.mla_indexer_topk(64, 128, p, p, p, 1, p, 1, p, 1, p, 16, 0, p, p, ws, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_indexer_topk(64, 128, p, p, p, 1, p, 1, p, 1, p, 16, 4, null, p, ws, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_indexer_topk(64, 128, p, p, p, 1, p, 0, p, 1, p, 16, 4, p, p, ws, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_indexer_topk(64, 128, p, p, p, 1, p, 1, p, 1, p, 16, 4, p, p, 100, null) == B.MLA_ERR_INVALID_ARG
    assert (lib.mla_indexer_topk(64, 128, p, p, p, 1, p, 1, p, 1, p, 2048 * 4096 + 1, 4, p, p, 1 << 40, null)
            == B.MLA_ERR_UNSUPPORTED)


def test_append_and_prefill_validation(B):
    """Host-side checks of mla_cache_append and the prefill calls: bad
    arguments are refused before anything is enqueued."""
    lib = B.raw_lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.c_void_p((ctypes.addressof(buf) + 15) // 16 * 16)
    null = None
    cfg = v2(B)
    c = ctypes.byref(cfg)
    # append: both tables or neither; rows >= 1 with tables; batch >= 1
    assert lib.mla_cache_append(c, p, p, p, null, 4, p, p, 1, p, 1, 1, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_append(c, p, p, p, p, 0, p, p, 1, p, 1, 1, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_append(c, p, p, null, null, 0, p, p, 1, p, 1, 0, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_append(c, null, p, null, null, 0, p, p, 1, p, 1, 1, null) == B.MLA_ERR_INVALID_ARG
    odd = B.make_config(4, 16, 7, 8, 8, 0.25, B.MLA_F32, B.MLA_F32)
    assert lib.mla_cache_append(ctypes.byref(odd), p, p, null, null, 0, p, p, 1, p, 1, 1, null) == B.MLA_ERR_UNSUPPORTED
    # prefill: V2 dims with a BF16 or FP8 cache (float32 refused); counts and ranges checked
    f32 = B.make_config(128, 512, 64, 128, 128, 0.1, B.MLA_F32, B.MLA_F32)
    assert lib.mla_prepare_w_uk_t(ctypes.byref(f32), p, p, null) == B.MLA_ERR_UNSUPPORTED
    assert lib.mla_prefill_expand(ctypes.byref(f32), p, 1, p, 64, p, p, p, p, p, null) == B.MLA_ERR_UNSUPPORTED
    for dt in (B.MLA_FP8_E4M3, B.MLA_FP8_E4M3_G128):
        fp8 = v2(B, dt)
        assert lib.mla_prefill_expand(ctypes.byref(fp8), p, 1, p, 0, p, p, p, p, p, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_prepare_w_uk_t(c, null, p, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_prefill_expand(c, p, 1, p, 0, p, p, p, p, p, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_prefill_expand(c, p, 1, p, 64, p, p, null, p, p, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_prefill_attn(c, p, p, p, p, p, 100, 90, 11, p, null, null) == B.MLA_ERR_INVALID_ARG   # past T
    assert lib.mla_prefill_attn(c, p, p, p, p, p, 100, -1, 10, p, null, null) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_prefill_attn(c, p, p, p, p, p, 100, 0, 0, p, null, null) == B.MLA_ERR_INVALID_ARG
    tiny = B.make_config(4, 16, 8, 8, 8, 0.25, B.MLA_F32, B.MLA_F32)
    assert lib.mla_prefill_attn(ctypes.byref(tiny), p, p, p, p, p, 100, 0, 10, p, null, null) == B.MLA_ERR_UNSUPPORTED


def test_noalloc_checks_before_touching_its_scratch(B):
    """mla_decode_noalloc refuses bad arguments, both or neither output form,
    and a split whose partials would not fit its static scratch, before it
    looks up or touches the scratch (nothing is launched here)."""
    lib = B.raw_lib()
    cfg = v2(B)
    c = ctypes.byref(cfg)
    q = ctypes.c_void_p(0x1000)
    null = None
    plan = B.MlaPlan(256, 256 + 126, 0)
    ok_args = lambda batch, o_lat, w_uv, out: [c, q, q, q, 10, q, 4, q, null, 0, batch, ctypes.byref(plan),
                                               o_lat, w_uv, out, null, null]
    # neither output, both outputs
    assert lib.mla_decode_noalloc(*ok_args(127, null, null, null)) == B.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_noalloc(*ok_args(127, q, q, q)) == B.MLA_ERR_INVALID_ARG
    # up-projection form without weights
    assert lib.mla_decode_noalloc(*ok_args(127, null, null, q)) == B.MLA_ERR_INVALID_ARG
    # 256 workers + 200 requests - 1 = 455 BF16 partial slots of 131,584 B: over 48 MiB
    assert lib.mla_decode_noalloc(*ok_args(200, q, null, null)) == B.MLA_ERR_SCRATCH
    assert lib.mla_decode_noalloc(*ok_args(200, null, q, q)) == B.MLA_ERR_SCRATCH
    # the usual checks of the attention call (misaligned query, no plan)
    args = ok_args(127, q, null, null)
    args[1] = ctypes.c_void_p(0x1008)
    assert lib.mla_decode_noalloc(*args) == B.MLA_ERR_INVALID_ARG
    args = ok_args(127, q, null, null)
    args[11] = None
    assert lib.mla_decode_noalloc(*args) == B.MLA_ERR_INVALID_ARG
    # the largest batch that fits with 256 workers: 382 slots
    assert (382 * (128 * 512 * 2) + 382 * 128 * 4) <= B.NOALLOC_SCRATCH_BYTES < (383 * (128 * 512 * 2) + 383 * 128 * 4)
    assert B.status_string(B.MLA_ERR_SCRATCH) != "unknown status"
