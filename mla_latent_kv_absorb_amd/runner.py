"""Device-resident workload and the four-call decode step.

Uploads one seeded workload (paged pool, block table, lengths, index lists,
queries, weights) to GPU memory with torch, allocates the outputs and the
split workspace, and runs absorb -> attention -> combine -> up-projection
through the C ABI on the current stream.
"""

from __future__ import annotations

import numpy as np

from . import binding as B
from . import inputs as I


def _dtype_code(name: str) -> int:
    return {I.DTYPE_F32: B.MLA_F32, I.DTYPE_BF16: B.MLA_BF16, I.DTYPE_FP8: B.MLA_FP8_E4M3,
            I.DTYPE_FP8_G128: B.MLA_FP8_E4M3_G128}[name]


def to_device_act(x: np.ndarray, act: str, device):
    import torch
    if act == I.DTYPE_F32:
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    bits = I.bf16_bits(x).view(np.int16)
    return torch.from_numpy(bits).to(device).view(torch.bfloat16)


def workspace_bytes(H: int, D_C: int, slots: int) -> int:
    """Bytes of the split workspace: a partials section sized for float32
    [slots][H][D_C] (the BF16-activation paths store BF16 partials in its first
    half) then float32 log-sum-exps [slots][H], each section 16-byte aligned
    (the layout mla_decode_plan sizes)."""
    al = lambda x: (x + 15) // 16 * 16
    return al(slots * H * D_C * 4) + al(slots * H * 4)


class DeviceWorkload:
    def __init__(self, inp: I.DecodeInputs, device="cuda", split=True, num_workers=None, num_cus=256,
                 pool=None, table=None, tensors=None):
        """Upload ``inp`` (host arrays) to the device, or, with ``tensors``,
        take device tensors already drawn there (pool, table, q_nope,
        q_rope, w_uk, w_uv, topk_idx; ``inp`` then only gives dims and
        lengths)."""
        import torch
        self.inp = inp
        self.device = device
        self.cfg = B.make_config(inp.H, inp.D_C, inp.D_R, inp.D_N, inp.D_V, inp.scale,
                                 _dtype_code(inp.cache_dtype), _dtype_code(inp.act_dtype))
        self.seq_lens = torch.from_numpy(inp.seq_lens.astype(np.int32)).to(device)
        act = inp.act_dtype
        if tensors is not None:
            self.pool, self.table = tensors["pool"], tensors["table"]
            self.q_nope, self.q_rope = tensors["q_nope"], tensors["q_rope"]
            self.w_uk, self.w_uv = tensors["w_uk"], tensors["w_uv"]
            self.topk_idx = tensors.get("topk_idx")
        else:
            if pool is None:
                pool, table = I.build_paged_pool(inp)
            self.pool = torch.from_numpy(pool).to(device)
            self.table = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(device)
            self.topk_idx = None
            if inp.topk_idx is not None:
                self.topk_idx = torch.from_numpy(inp.topk_idx.astype(np.int32)).to(device)
            self.q_nope = to_device_act(inp.q_nope, act, device)
            self.q_rope = to_device_act(inp.q_rope, act, device)
            self.w_uk = to_device_act(inp.w_uk, act, device)
            self.w_uv = to_device_act(inp.w_uv, act, device)
        self.topk = 0 if self.topk_idx is None else int(self.topk_idx.shape[1])
        dt = torch.float32 if act == I.DTYPE_F32 else torch.bfloat16
        Bn, H = inp.B, inp.H
        self.q_lat = torch.empty((Bn, H, inp.D_C), dtype=dt, device=device)
        self.o_lat = torch.empty((Bn, H, inp.D_C), dtype=dt, device=device)
        self.out = torch.empty((Bn, H, inp.D_V), dtype=dt, device=device)
        self.lse = torch.empty((Bn, H), dtype=torch.float32, device=device)
        self.split = split
        self.plan = None
        self.workspace = None
        if split:
            self.plan = B.mla_decode_plan(self.cfg, Bn, inp.seq_lens, 0, self.topk, num_cus)
            if num_workers is not None:
                self.plan.num_workers = int(num_workers)
                self.plan.num_slots = int(num_workers) + Bn - 1
                self.plan.workspace_bytes = workspace_bytes(H, inp.D_C, self.plan.num_slots)
            self.workspace = torch.empty(self.plan.workspace_bytes, dtype=torch.uint8, device=device)

    # the four calls ---------------------------------------------------------
    def absorb(self, stream=None):
        B.mla_absorb_q(self.cfg, self.q_nope, self.w_uk, self.q_lat, stream)

    def attend(self, stream=None, q_lat=None):
        ql = self.q_lat if q_lat is None else q_lat
        if self.split:
            B.mla_decode_attn(self.cfg, ql, self.q_rope, self.pool, self.table, self.seq_lens, self.topk_idx,
                              plan=self.plan, workspace=self.workspace, stream=stream)
        else:
            B.mla_decode_attn(self.cfg, ql, self.q_rope, self.pool, self.table, self.seq_lens, self.topk_idx,
                              o_lat=self.o_lat, lse_out=self.lse, stream=stream)

    def combine(self, stream=None):
        if self.split:
            B.mla_combine(self.cfg, self.workspace, self.seq_lens, self.plan, self.o_lat, self.lse,
                          topk=self.topk, stream=stream)

    def up(self, stream=None):
        B.mla_out_up(self.cfg, self.o_lat, self.w_uv, self.out, stream)

    def combine_up(self, stream=None):
        """Merge and up-projection in one launch (split mode, BF16 V2 dims);
        o_lat is not written."""
        B.mla_combine_out_up(self.cfg, self.workspace, self.seq_lens, self.plan, self.w_uv, self.out,
                             lse_out=self.lse, topk=self.topk, stream=stream)

    def step(self, stream=None):
        self.absorb(stream)
        self.attend(stream)
        self.combine(stream)
        self.up(stream)

    def step_fused(self, stream=None):
        """The same step with the merge and the up-projection in one launch."""
        self.absorb(stream)
        self.attend(stream)
        self.combine_up(stream)

    def partials(self):
        """(o_part [slots, H, D_C], lse_part [slots, H]) of the workspace (split
        mode), both float32; the partials are stored as BF16 when the
        activations are BF16 and widened here."""
        import torch
        slots = self.plan.num_slots
        H, DC = self.inp.H, self.inp.D_C
        n_o = slots * H * DC
        o_bytes = (n_o * 4 + 15) // 16 * 16
        ws = self.workspace
        if self.inp.act_dtype == I.DTYPE_F32:
            o = ws[: n_o * 4].view(torch.float32).view(slots, H, DC)
        else:
            o = ws[: n_o * 2].view(torch.bfloat16).view(slots, H, DC).float()
        l = ws[o_bytes: o_bytes + slots * H * 4].view(torch.float32).view(slots, H)
        return o, l


class IndexerWorkload:
    """Device buffers of one lightning-indexer workload: queries, head
    weights, the paged FP8 search-key pool, the score rows and the picked
    index lists, with the two calls (scores, then top-k pick)."""

    def __init__(self, inp: I.IndexerInputs, device="cuda", score_stride=None, pool=None, table=None):
        import torch
        self.inp = inp
        if pool is None:
            pool, table = I.build_key_pool(inp)
        self.pool = torch.from_numpy(pool).to(device)
        self.table = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(device)
        self.seq_lens = torch.from_numpy(inp.seq_lens.astype(np.int32)).to(device)
        self.q = to_device_act(inp.q_idx, I.DTYPE_BF16, device)
        self.w = torch.from_numpy(np.ascontiguousarray(inp.w_idx, dtype=np.float32)).to(device)
        stride = int(inp.seq_lens.max()) if score_stride is None else int(score_stride)
        self.scores = torch.empty((inp.B, stride), dtype=torch.float32, device=device)
        self.k = int(inp.topk)
        self.idx = torch.empty((inp.B, self.k), dtype=torch.int32, device=device)
        self.workspace = torch.empty(B.topk_workspace_bytes(inp.B, stride), dtype=torch.uint8, device=device)

    def score(self, stream=None):
        B.mla_indexer_scores(self.q, self.w, self.pool, self.table, self.seq_lens, self.scores, stream)

    def select(self, stream=None, scores=None):
        B.mla_topk_select(self.scores if scores is None else scores, self.seq_lens, self.k, self.idx,
                          self.workspace, stream)

    def step(self, stream=None):
        self.score(stream)
        self.select(stream)

    def score_and_select(self, stream=None):
        """Both calls as one (mla_indexer_topk)."""
        B.mla_indexer_topk(self.q, self.w, self.pool, self.table, self.seq_lens, self.scores, self.k, self.idx,
                           self.workspace, stream)


class PrefillWorkload:
    """One request's prefill on the expanded path: the request's cache pages,
    the weights (W_UK transposed once), the N new queries at positions
    T - N .. T - 1, and the expanded keys / values."""

    def __init__(self, inp: I.DecodeInputs, q_nope, q_rope, device="cuda"):
        import torch
        assert inp.B == 1
        self.inp = inp
        self.cfg = B.make_config(inp.H, inp.D_C, inp.D_R, inp.D_N, inp.D_V, inp.scale,
                                 _dtype_code(inp.cache_dtype), B.MLA_BF16)
        pool, table = I.build_paged_pool(inp)
        self.pool = torch.from_numpy(pool).to(device)
        self.block_row = torch.from_numpy(np.ascontiguousarray(table[0], dtype=np.int32)).to(device)
        self.T = int(inp.seq_lens[0])
        self.w_uk = to_device_act(inp.w_uk, I.DTYPE_BF16, device)
        self.w_uv = to_device_act(inp.w_uv, I.DTYPE_BF16, device)
        self.w_uk_t = torch.empty((inp.H, inp.D_N, inp.D_C), dtype=torch.bfloat16, device=device)
        B.mla_prepare_w_uk_t(self.cfg, self.w_uk, self.w_uk_t)
        self.q_nope = to_device_act(q_nope, I.DTYPE_BF16, device)
        self.q_rope = to_device_act(q_rope, I.DTYPE_BF16, device)
        self.N = int(q_nope.shape[0])
        T, H = self.T, inp.H
        self.k_nope = torch.empty((T, H, inp.D_N), dtype=torch.bfloat16, device=device)
        self.v = torch.empty((T, H, inp.D_V), dtype=torch.bfloat16, device=device)
        self.k_rope = torch.empty((T, inp.D_R), dtype=torch.bfloat16, device=device)
        self.out = torch.empty((self.N, H, inp.D_V), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((self.N, H), dtype=torch.float32, device=device)

    def expand(self, stream=None):
        B.mla_prefill_expand(self.cfg, self.pool, self.block_row, self.T, self.w_uk_t, self.w_uv, self.k_nope,
                             self.v, self.k_rope, stream)

    def attend(self, stream=None):
        B.mla_prefill_attn(self.cfg, self.q_nope, self.q_rope, self.k_nope, self.v, self.k_rope, self.T - self.N,
                           self.out, self.lse, stream)

    def step(self, stream=None):
        self.expand(stream)
        self.attend(stream)
