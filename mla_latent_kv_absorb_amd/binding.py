"""ctypes binding of libmla_absorb.so (C ABI in include/mla_absorb.h and
include/mla_indexer.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity (the C ABI receives plain pointers and cannot check sizes), then
their pointers and the current HIP stream are passed to the library.  Every
step of the decode path runs in the library's HIP kernels.  Importing this
module loads the library and raises if it has not been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

LIB_PATH = os.environ.get("MLA_ABSORB_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "libmla_absorb.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_LAUNCH, MLA_ERR_SCRATCH = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 48 << 20
MLA_F32, MLA_BF16, MLA_FP8_E4M3, MLA_FP8_E4M3_G128 = 0, 1, 2, 3
PAGE_TOKENS = 64
TILE_TOKENS = 32

EXPORTED = (
    "mla_abi_version", "mla_status_string", "mla_page_layout", "mla_decode_plan",
    "mla_absorb_q", "mla_decode_attn", "mla_combine", "mla_out_up", "mla_combine_out_up",
    "mla_check_decode_inputs_host", "mla_cache_append",
    "mla_prepare_w_uk_t", "mla_prefill_expand", "mla_prefill_attn",
    "mla_indexer_page_layout", "mla_indexer_scores", "mla_topk_workspace_bytes", "mla_topk_select",
    "mla_indexer_topk", "mla_decode_noalloc",
)
INDEXER_HEADS, INDEXER_DIM = 64, 128


class MlaConfig(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32), ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32),
        ("d_nope", ctypes.c_int32), ("d_v", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("cache_dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
    ]


class MlaPlan(ctypes.Structure):
    _fields_ = [("num_workers", ctypes.c_int32), ("num_slots", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m mla_latent_kv_absorb_amd.build_lib` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp, planp = ctypes.POINTER(MlaConfig), ctypes.POINTER(MlaPlan)
    i32p = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "mla_abi_version": ([], I32),
        "mla_status_string": ([I32], ctypes.c_char_p),
        "mla_page_layout": ([cfgp, ctypes.POINTER(SZ), ctypes.POINTER(SZ), ctypes.POINTER(SZ)], I32),
        "mla_decode_plan": ([cfgp, I32, i32p, I32, I32, I32, planp], I32),
        "mla_absorb_q": ([cfgp, P, P, P, I32, P], I32),
        "mla_decode_attn": ([cfgp, P, P, P, I64, P, I32, P, P, I32, I32, planp, P, SZ, P, P, P], I32),
        "mla_combine": ([cfgp, P, SZ, P, I32, I32, planp, P, P, P], I32),
        "mla_out_up": ([cfgp, P, P, P, I32, P], I32),
        "mla_combine_out_up": ([cfgp, P, SZ, P, I32, I32, planp, P, P, P, P], I32),
        "mla_check_decode_inputs_host": ([cfgp, I32, i32p, i32p, I32, I64, i32p, I32, i32p], I32),
        "mla_cache_append": ([cfgp, P, P, P, P, I32, P, P, I64, P, I32, I32, P], I32),
        "mla_prepare_w_uk_t": ([cfgp, P, P, P], I32),
        "mla_prefill_expand": ([cfgp, P, I64, P, I32, P, P, P, P, P, P], I32),
        "mla_prefill_attn": ([cfgp, P, P, P, P, P, I32, I32, I32, P, P, P], I32),
        "mla_indexer_page_layout": ([I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)], I32),
        "mla_indexer_scores": ([I32, I32, P, P, P, I64, P, I32, P, I32, P, I64, P], I32),
        "mla_topk_workspace_bytes": ([I32, I64], SZ),
        "mla_topk_select": ([P, I64, P, I32, I32, P, P, SZ, P], I32),
        "mla_indexer_topk": ([I32, I32, P, P, P, I64, P, I32, P, I32, P, I64, I32, P, P, SZ, P], I32),
        "mla_decode_noalloc": ([cfgp, P, P, P, I64, P, I32, P, P, I32, I32, planp, P, P, P, P, P], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def status_string(status: int) -> str:
    return _lib.mla_status_string(int(status)).decode()


def abi_version() -> int:
    return int(_lib.mla_abi_version())


def make_config(H, D_C, D_R, D_N, D_V, scale, cache_dtype, act_dtype) -> MlaConfig:
    return MlaConfig(H, D_C, D_R, D_N, D_V, PAGE_TOKENS, float(scale), int(cache_dtype), int(act_dtype))


def _check(fn: str, st: int):
    if st != MLA_OK:
        raise MlaError(fn, st)


def _torch():
    import torch
    return torch


def _dev(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _act(cfg: MlaConfig):
    torch = _torch()
    return torch.float32 if cfg.act_dtype == MLA_F32 else torch.bfloat16


def page_layout(cfg: MlaConfig):
    pb, ro, so = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check("mla_page_layout", _lib.mla_page_layout(ctypes.byref(cfg), ctypes.byref(pb), ctypes.byref(ro),
                                                   ctypes.byref(so)))
    return int(pb.value), int(ro.value), int(so.value)


def mla_decode_plan(cfg: MlaConfig, batch: int, seq_lens_host=None, max_len: int = 0, topk: int = 0,
                    num_cus: int = 256) -> MlaPlan:
    plan = MlaPlan()
    arr = None
    if seq_lens_host is not None:
        arr = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
        if arr.shape != (batch,):
            raise ValueError("seq_lens_host must have one entry per request")
    ptr = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if arr is not None else None
    _check("mla_decode_plan", _lib.mla_decode_plan(ctypes.byref(cfg), batch, ptr, int(max_len), int(topk),
                                                   int(num_cus), ctypes.byref(plan)))
    return plan


def mla_absorb_q(cfg: MlaConfig, q_nope, w_uk, q_lat, stream=None):
    B = q_nope.shape[0]
    dt = _act(cfg)
    H, DC, DN = cfg.num_heads, cfg.d_latent, cfg.d_nope
    st = _lib.mla_absorb_q(ctypes.byref(cfg), _dev(q_nope, "q_nope", dt, (B, H, DN)),
                           _dev(w_uk, "w_uk", dt, (H, DC, DN)), _dev(q_lat, "q_lat", dt, (B, H, DC)),
                           B, _stream(stream))
    _check("mla_absorb_q", st)


def mla_out_up(cfg: MlaConfig, o_lat, w_uv, out, stream=None):
    B = o_lat.shape[0]
    dt = _act(cfg)
    H, DC, DV = cfg.num_heads, cfg.d_latent, cfg.d_v
    st = _lib.mla_out_up(ctypes.byref(cfg), _dev(o_lat, "o_lat", dt, (B, H, DC)),
                         _dev(w_uv, "w_uv", dt, (H, DV, DC)), _dev(out, "out", dt, (B, H, DV)),
                         B, _stream(stream))
    _check("mla_out_up", st)


def mla_decode_attn(cfg: MlaConfig, q_lat, q_rope, kv_pool, block_table, seq_lens, topk_idx=None,
                    plan: Optional[MlaPlan] = None, workspace=None, o_lat=None, lse_out=None, stream=None):
    """Direct mode when o_lat is given (one work-group per request, final
    output); split mode otherwise (plan + workspace, finish with mla_combine)."""
    torch = _torch()
    B = q_lat.shape[0]
    dt = _act(cfg)
    H, DC, DR = cfg.num_heads, cfg.d_latent, cfg.d_rope
    page_bytes, _, _ = page_layout(cfg)
    if kv_pool.dtype != torch.uint8 or kv_pool.dim() != 2 or kv_pool.shape[1] != page_bytes:
        raise ValueError(f"kv_pool must be uint8 [num_pages, {page_bytes}]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [batch, stride]")
    topk = 0
    tp = None
    if topk_idx is not None:
        if topk_idx.dim() != 2 or topk_idx.shape[0] != B:
            raise ValueError("topk_idx must be int32 [batch, k]")
        topk = int(topk_idx.shape[1])
        tp = _dev(topk_idx, "topk_idx", torch.int32)
    ws, wsb = None, 0
    if o_lat is None:
        if plan is None or workspace is None:
            raise ValueError("split mode needs a plan and a workspace")
        ws = _dev(workspace, "workspace", torch.uint8)
        wsb = workspace.numel()
        ol = None
    else:
        ol = _dev(o_lat, "o_lat", dt, (B, H, DC))
    lp = _dev(lse_out, "lse_out", torch.float32, (B, H)) if lse_out is not None else None
    st = _lib.mla_decode_attn(
        ctypes.byref(cfg), _dev(q_lat, "q_lat", dt, (B, H, DC)), _dev(q_rope, "q_rope", dt, (B, H, DR)),
        _dev(kv_pool, "kv_pool"), int(kv_pool.shape[0]), _dev(block_table, "block_table", torch.int32),
        int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, (B,)), tp, topk, B,
        ctypes.byref(plan) if plan is not None else None, ws, wsb, ol, lp, _stream(stream))
    _check("mla_decode_attn", st)


def mla_combine(cfg: MlaConfig, workspace, seq_lens, plan: MlaPlan, o_lat, lse_out=None, topk: int = 0,
                stream=None):
    torch = _torch()
    B = o_lat.shape[0]
    dt = _act(cfg)
    lp = _dev(lse_out, "lse_out", torch.float32, (B, cfg.num_heads)) if lse_out is not None else None
    st = _lib.mla_combine(ctypes.byref(cfg), _dev(workspace, "workspace", torch.uint8), workspace.numel(),
                          _dev(seq_lens, "seq_lens", torch.int32, (B,)), int(topk), B, ctypes.byref(plan),
                          _dev(o_lat, "o_lat", dt, (B, cfg.num_heads, cfg.d_latent)), lp, _stream(stream))
    _check("mla_combine", st)


def mla_combine_out_up(cfg: MlaConfig, workspace, seq_lens, plan: MlaPlan, w_uv, out, lse_out=None, topk: int = 0,
                       stream=None):
    torch = _torch()
    B = out.shape[0]
    dt = _act(cfg)
    H, DC, DV = cfg.num_heads, cfg.d_latent, cfg.d_v
    lp = _dev(lse_out, "lse_out", torch.float32, (B, H)) if lse_out is not None else None
    st = _lib.mla_combine_out_up(ctypes.byref(cfg), _dev(workspace, "workspace", torch.uint8), workspace.numel(),
                                 _dev(seq_lens, "seq_lens", torch.int32, (B,)), int(topk), B, ctypes.byref(plan),
                                 _dev(w_uv, "w_uv", dt, (H, DV, DC)), _dev(out, "out", dt, (B, H, DV)), lp,
                                 _stream(stream))
    _check("mla_combine_out_up", st)


def mla_decode_noalloc(cfg: MlaConfig, q_lat, q_rope, kv_pool, block_table, seq_lens, plan: MlaPlan, topk_idx=None,
                       o_lat=None, w_uv=None, out=None, lse_out=None, stream=None):
    """Split attention and merge in one call, partials in the library's
    static scratch: o_lat given -> merged weighted latent; out and w_uv given
    -> merged up-projection."""
    torch = _torch()
    B = q_lat.shape[0]
    dt = _act(cfg)
    H, DC, DR, DV = cfg.num_heads, cfg.d_latent, cfg.d_rope, cfg.d_v
    page_bytes, _, _ = page_layout(cfg)
    if kv_pool.dtype != torch.uint8 or kv_pool.dim() != 2 or kv_pool.shape[1] != page_bytes:
        raise ValueError(f"kv_pool must be uint8 [num_pages, {page_bytes}]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [batch, stride]")
    topk, tp = 0, None
    if topk_idx is not None:
        if topk_idx.dim() != 2 or topk_idx.shape[0] != B:
            raise ValueError("topk_idx must be int32 [batch, k]")
        topk = int(topk_idx.shape[1])
        tp = _dev(topk_idx, "topk_idx", torch.int32)
    ol = _dev(o_lat, "o_lat", dt, (B, H, DC)) if o_lat is not None else None
    wp = _dev(w_uv, "w_uv", dt, (H, DV, DC)) if w_uv is not None else None
    op = _dev(out, "out", dt, (B, H, DV)) if out is not None else None
    lp = _dev(lse_out, "lse_out", torch.float32, (B, H)) if lse_out is not None else None
    st = _lib.mla_decode_noalloc(
        ctypes.byref(cfg), _dev(q_lat, "q_lat", dt, (B, H, DC)), _dev(q_rope, "q_rope", dt, (B, H, DR)),
        _dev(kv_pool, "kv_pool"), int(kv_pool.shape[0]), _dev(block_table, "block_table", torch.int32),
        int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, (B,)), tp, topk, B, ctypes.byref(plan),
        ol, wp, op, lp, _stream(stream))
    _check("mla_decode_noalloc", st)


def mla_check_decode_inputs_host(cfg: MlaConfig, seq_lens, block_table, num_pages: int, topk_idx=None):
    """Host check of the metadata contract; returns (status, failing request)."""
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    tk = None if topk_idx is None else np.ascontiguousarray(topk_idx, dtype=np.int32)
    err = ctypes.c_int32(-1)
    i32p = ctypes.POINTER(ctypes.c_int32)
    st = _lib.mla_check_decode_inputs_host(
        ctypes.byref(cfg), int(sl.shape[0]), sl.ctypes.data_as(i32p), bt.ctypes.data_as(i32p), int(bt.shape[1]),
        int(num_pages), tk.ctypes.data_as(i32p) if tk is not None else None,
        int(tk.shape[1]) if tk is not None else 0, ctypes.byref(err))
    return int(st), int(err.value)


def raw_lib():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib


def mla_cache_append(cfg: MlaConfig, c_new, k_new, positions, kv_pool, block_table, rope_cos=None, rope_sin=None,
                     stream=None):
    """Write one token per request (row positions[b] of its pages)."""
    torch = _torch()
    B = c_new.shape[0]
    dt = _act(cfg)
    page_bytes = page_layout(cfg)[0]
    if kv_pool.dtype != torch.uint8 or kv_pool.dim() != 2 or kv_pool.shape[1] != page_bytes:
        raise ValueError(f"kv_pool must be uint8 [num_pages, {page_bytes}]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [batch, stride]")
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("give both rope tables or neither")
    rows = 0
    cp = sp = None
    if rope_cos is not None:
        rows = int(rope_cos.shape[0])
        cp = _dev(rope_cos, "rope_cos", torch.float32, (rows, cfg.d_rope // 2))
        sp = _dev(rope_sin, "rope_sin", torch.float32, (rows, cfg.d_rope // 2))
    st = _lib.mla_cache_append(ctypes.byref(cfg), _dev(c_new, "c_new", dt, (B, cfg.d_latent)),
                               _dev(k_new, "k_new", dt, (B, cfg.d_rope)), cp, sp, rows,
                               _dev(positions, "positions", torch.int32, (B,)), _dev(kv_pool, "kv_pool"),
                               int(kv_pool.shape[0]), _dev(block_table, "block_table", torch.int32),
                               int(block_table.shape[1]), B, _stream(stream))
    _check("mla_cache_append", st)


def mla_prepare_w_uk_t(cfg: MlaConfig, w_uk, w_uk_t, stream=None):
    torch = _torch()
    H, DC, DN = cfg.num_heads, cfg.d_latent, cfg.d_nope
    _check("mla_prepare_w_uk_t", _lib.mla_prepare_w_uk_t(
        ctypes.byref(cfg), _dev(w_uk, "w_uk", torch.bfloat16, (H, DC, DN)),
        _dev(w_uk_t, "w_uk_t", torch.bfloat16, (H, DN, DC)), _stream(stream)))


def mla_prefill_expand(cfg: MlaConfig, kv_pool, block_row, T: int, w_uk_t, w_uv, k_nope, v, k_rope, stream=None):
    """Expanded keys / values of positions 0 .. T-1 of one request (its page
    ids in block_row, int32 [>= ceil(T / 64)])."""
    torch = _torch()
    H, DC, DN, DV, DR = cfg.num_heads, cfg.d_latent, cfg.d_nope, cfg.d_v, cfg.d_rope
    page_bytes = page_layout(cfg)[0]
    if kv_pool.dtype != torch.uint8 or kv_pool.dim() != 2 or kv_pool.shape[1] != page_bytes:
        raise ValueError(f"kv_pool must be uint8 [num_pages, {page_bytes}]")
    if block_row.dim() != 1 or block_row.shape[0] < -(-T // PAGE_TOKENS):
        raise ValueError("block_row must hold the request's ceil(T / 64) page ids")
    _check("mla_prefill_expand", _lib.mla_prefill_expand(
        ctypes.byref(cfg), _dev(kv_pool, "kv_pool"), int(kv_pool.shape[0]), _dev(block_row, "block_row", torch.int32),
        int(T), _dev(w_uk_t, "w_uk_t", torch.bfloat16, (H, DN, DC)), _dev(w_uv, "w_uv", torch.bfloat16, (H, DV, DC)),
        _dev(k_nope, "k_nope", torch.bfloat16, (T, H, DN)), _dev(v, "v", torch.bfloat16, (T, H, DV)),
        _dev(k_rope, "k_rope", torch.bfloat16, (T, DR)), _stream(stream)))


def mla_prefill_attn(cfg: MlaConfig, q_nope, q_rope, k_nope, v, k_rope, q_start: int, out, lse_out=None,
                     stream=None):
    torch = _torch()
    N = q_nope.shape[0]
    T = k_nope.shape[0]
    H, DN, DV, DR = cfg.num_heads, cfg.d_nope, cfg.d_v, cfg.d_rope
    _check("mla_prefill_attn", _lib.mla_prefill_attn(
        ctypes.byref(cfg), _dev(q_nope, "q_nope", torch.bfloat16, (N, H, DN)),
        _dev(q_rope, "q_rope", torch.bfloat16, (N, H, DR)), _dev(k_nope, "k_nope", torch.bfloat16, (T, H, DN)),
        _dev(v, "v", torch.bfloat16, (T, H, DV)), _dev(k_rope, "k_rope", torch.bfloat16, (T, DR)), int(T),
        int(q_start), int(N), _dev(out, "out", torch.bfloat16, (N, H, DV)),
        None if lse_out is None else _dev(lse_out, "lse_out", torch.float32, (N, H)), _stream(stream)))


# ---- lightning indexer (include/mla_indexer.h) ------------------------------
def indexer_page_layout(dim: int = INDEXER_DIM):
    pb, so = ctypes.c_size_t(), ctypes.c_size_t()
    _check("mla_indexer_page_layout", _lib.mla_indexer_page_layout(int(dim), ctypes.byref(pb), ctypes.byref(so)))
    return int(pb.value), int(so.value)


def mla_indexer_scores(q_idx, w_idx, key_pool, block_table, seq_lens, scores, stream=None):
    """scores [B, score_stride] float32 <- I(b, s) for the cached positions."""
    torch = _torch()
    B, H, D = q_idx.shape
    page_bytes, _ = indexer_page_layout(D)
    if key_pool.dtype != torch.uint8 or key_pool.dim() != 2 or key_pool.shape[1] != page_bytes:
        raise ValueError(f"key_pool must be uint8 [num_pages, {page_bytes}]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [batch, stride]")
    if scores.dim() != 2 or scores.shape[0] != B:
        raise ValueError("scores must be float32 [batch, stride]")
    st = _lib.mla_indexer_scores(
        H, D, _dev(q_idx, "q_idx", torch.bfloat16), _dev(w_idx, "w_idx", torch.float32, (B, H)),
        _dev(key_pool, "key_pool"), int(key_pool.shape[0]), _dev(block_table, "block_table", torch.int32),
        int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, (B,)), B,
        _dev(scores, "scores", torch.float32), int(scores.shape[1]), _stream(stream))
    _check("mla_indexer_scores", st)


def topk_workspace_bytes(batch: int, score_stride: int) -> int:
    return int(_lib.mla_topk_workspace_bytes(int(batch), int(score_stride)))


def mla_topk_select(scores, seq_lens, k: int, idx_out, workspace, stream=None):
    """idx_out [B, k] int32 <- the k best positions of each score row, in
    increasing order, -1 padded."""
    torch = _torch()
    B = scores.shape[0]
    st = _lib.mla_topk_select(
        _dev(scores, "scores", torch.float32), int(scores.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, (B,)),
        B, int(k), _dev(idx_out, "idx_out", torch.int32, (B, k)), _dev(workspace, "workspace"),
        int(workspace.numel() * workspace.element_size()), _stream(stream))
    _check("mla_topk_select", st)


def mla_indexer_topk(q_idx, w_idx, key_pool, block_table, seq_lens, scores, k: int, idx_out, workspace,
                     stream=None):
    """scores as mla_indexer_scores, then idx_out [B, k] as mla_topk_select,
    in one call."""
    torch = _torch()
    B, H, D = q_idx.shape
    page_bytes, _ = indexer_page_layout(D)
    if key_pool.dtype != torch.uint8 or key_pool.dim() != 2 or key_pool.shape[1] != page_bytes:
        raise ValueError(f"key_pool must be uint8 [num_pages, {page_bytes}]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [batch, stride]")
    if scores.dim() != 2 or scores.shape[0] != B:
        raise ValueError("scores must be float32 [batch, stride]")
    st = _lib.mla_indexer_topk(
        H, D, _dev(q_idx, "q_idx", torch.bfloat16), _dev(w_idx, "w_idx", torch.float32, (B, H)),
        _dev(key_pool, "key_pool"), int(key_pool.shape[0]), _dev(block_table, "block_table", torch.int32),
        int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, (B,)), B,
        _dev(scores, "scores", torch.float32), int(scores.shape[1]), int(k),
        _dev(idx_out, "idx_out", torch.int32, (B, k)), _dev(workspace, "workspace"),
        int(workspace.numel() * workspace.element_size()), _stream(stream))
    _check("mla_indexer_topk", st)
