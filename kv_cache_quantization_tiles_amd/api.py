"""Allocate-and-call helpers over the C-ABI binding.

torch provides device memory and the stream; every computation is a libkvq
kernel.  Nothing here falls back to the CPU: without the built library and a
GPU these functions raise.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import (config, kvq_append_and_decode, kvq_append_and_requant, kvq_baseline_page_bytes,  # noqa: F401
                   kvq_baseline_workspace_bytes, kvq_decode_workspace_bytes, kvq_dequantize,
                   kvq_append_pages_fp8, kvq_append_pages_fp16, kvq_fill_pages_fp8,
                   kvq_fill_pages_fp16, kvq_multi_query_workspace_bytes,
                   kvq_paged_decode_attn, kvq_paged_multi_query_attn,
                   kvq_paged_decode_attn_fp8, kvq_paged_decode_attn_fp16, kvq_quantize_tiles,
                   kvq_quantize_to_pages, kvq_rematerialize_fp16_pages, kvq_slot_bytes)

HEAD_DIM = 128
PAGE_TOKENS = 16


def _require_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("libkvq works on device tensors only")


def quantize_tiles(x: torch.Tensor, cfg, bits: int):
    """x fp16 [n, H, 128] on the GPU -> dict(codes, alpha, scale, offset)."""
    _require_cuda(x)
    n, h, d = x.shape
    t = cfg.tile_tokens
    dev = x.device
    out = dict(codes=torch.empty((n, h, d * bits // 8), dtype=torch.uint8, device=dev),
               alpha=torch.empty(((n + t - 1) // t, h, d), dtype=torch.float32, device=dev),
               scale=torch.empty((n, h), dtype=torch.float32, device=dev),
               offset=torch.empty((n, h), dtype=torch.float32, device=dev))
    kvq_quantize_tiles(cfg, x.contiguous(), n, h, bits, out["codes"], out["alpha"], out["scale"],
                       out["offset"])
    return out


def dequantize(q: dict, cfg, bits: int) -> torch.Tensor:
    n, h, _ = q["codes"].shape
    out = torch.empty((n, h, HEAD_DIM), dtype=torch.float16, device=q["codes"].device)
    kvq_dequantize(cfg, q["codes"], q["alpha"], q["scale"], q["offset"], n, h, bits, out)
    return out


class PagedCache:
    """Quantized page pools of one layer plus the fp16 staging of partial tiles."""

    def __init__(self, cfg, num_pages: int, kv_heads: int, block_table: torch.Tensor,
                 num_seqs: int, device="cuda"):
        self.cfg = cfg
        self.kv_heads = kv_heads
        self.num_seqs = num_seqs
        self.block_table = block_table.to(device=device, dtype=torch.int32).contiguous()
        self.max_blocks = self.block_table.shape[1]
        self.slot_k = kvq_slot_bytes(cfg, False)
        self.slot_v = kvq_slot_bytes(cfg, True)
        self.pool_k = torch.zeros((num_pages, kv_heads, self.slot_k), dtype=torch.uint8, device=device)
        self.pool_v = torch.zeros((num_pages, kv_heads, self.slot_v), dtype=torch.uint8, device=device)
        t = cfg.tile_tokens
        self.staging_k = torch.zeros((num_seqs, t, kv_heads, HEAD_DIM), dtype=torch.float16, device=device)
        self.staging_v = torch.zeros_like(self.staging_k)

    def quantize_prefill(self, k, v, cu_seqlens):
        """k, v fp16 [total_tokens, kv_heads, 128] (sequences back to back),
        cu_seqlens int32 [num_seqs + 1] on the device."""
        _require_cuda(k, v, cu_seqlens)
        kvq_quantize_to_pages(self.cfg, k, v, cu_seqlens, self.num_seqs, int(k.shape[0]), self.kv_heads,
                              self.block_table, self.max_blocks, self.pool_k, self.pool_v,
                              self.staging_k, self.staging_v)

    def append(self, k_new, v_new, lens_before):
        _require_cuda(k_new, v_new, lens_before)
        kvq_append_and_requant(self.cfg, k_new, v_new, lens_before, self.num_seqs, self.kv_heads,
                               self.staging_k, self.staging_v, self.block_table, self.max_blocks,
                               self.pool_k, self.pool_v)

    def workspace(self, q_heads, max_seq_len):
        nbytes = kvq_decode_workspace_bytes(self.cfg, self.num_seqs, q_heads, self.kv_heads, int(max_seq_len))
        return torch.empty(max(nbytes, 4), dtype=torch.uint8, device=self.pool_k.device)

    def decode(self, q, seq_lens, max_seq_len, out=None, workspace=None, sm_scale=None):
        _require_cuda(q, seq_lens)
        s, hq, d = q.shape
        if out is None:
            out = torch.empty((s, hq, d), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = self.workspace(hq, max_seq_len)
        sm = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
        kvq_paged_decode_attn(self.cfg, q.contiguous(), s, hq, self.kv_heads, self.block_table,
                              self.max_blocks, seq_lens, int(max_seq_len), self.pool_k, self.pool_v, sm,
                              out, workspace, workspace.numel())
        return out

    def append_decode(self, k_new, v_new, lens_before, q, max_seq_len, out=None, workspace=None, sm_scale=None):
        """Append one token per sequence and attend over every cached token, in one
        launch (max_seq_len bounds the lengths after the append)."""
        _require_cuda(k_new, v_new, lens_before, q)
        s, hq, d = q.shape
        if out is None:
            out = torch.empty((s, hq, d), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = self.workspace(hq, max_seq_len)
        sm = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
        kvq_append_and_decode(self.cfg, k_new, v_new, lens_before, self.num_seqs, self.kv_heads, self.staging_k,
                              self.staging_v, self.block_table, self.max_blocks, self.pool_k, self.pool_v,
                              q.contiguous(), hq, int(max_seq_len), sm, out, workspace, workspace.numel())
        return out

    def multi_query(self, q, seq_lens, max_seq_len, out=None, workspace=None, sm_scale=None):
        """q fp16 [S, n_q, Hq, 128]: the n_q newest cached tokens of each sequence,
        each attending causally up to its own position; returns fp32 [S, n_q, Hq, 128]."""
        _require_cuda(q, seq_lens)
        s, n_q, hq, d = q.shape
        if out is None:
            out = torch.empty((s, n_q, hq, d), dtype=torch.float32, device=q.device)
        if workspace is None:
            nbytes = kvq_multi_query_workspace_bytes(self.cfg, s, n_q, hq, self.kv_heads, int(max_seq_len))
            workspace = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=q.device)
        sm = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
        kvq_paged_multi_query_attn(self.cfg, q.contiguous(), s, n_q, hq, self.kv_heads, self.block_table,
                                   self.max_blocks, seq_lens, int(max_seq_len), self.pool_k, self.pool_v, sm,
                                   out, workspace, workspace.numel())
        return out

    def rematerialize_into(self, base: "BaselineCache", seq_lens, max_seq_len):
        """Restore every cached token into the fp16 pools of `base` (same page ids),
        the read path that re-materializes fp16 before attention."""
        _require_cuda(seq_lens)
        if base.fp8:
            raise ValueError("re-materialization writes fp16 pools")
        kvq_rematerialize_fp16_pages(self.cfg, self.pool_k, self.pool_v, self.block_table, self.max_blocks, seq_lens,
                                     self.num_seqs, int(max_seq_len), self.kv_heads, base.pool_k, base.pool_v)


class BaselineCache:
    """fp16 or fp8 (E4M3, one scale per tensor) page pools of one layer, the
    uncompressed and 8-bit modes the quantized cache is compared with."""

    def __init__(self, num_pages: int, kv_heads: int, block_table: torch.Tensor, num_seqs: int,
                 fp8: bool = False, k_scale: float = 1.0, v_scale: float = 1.0, device="cuda"):
        self.cfg = config()
        self.fp8 = fp8
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.kv_heads = kv_heads
        self.num_seqs = num_seqs
        self.block_table = block_table.to(device=device, dtype=torch.int32).contiguous()
        self.max_blocks = self.block_table.shape[1]
        dt = torch.uint8 if fp8 else torch.float16
        self.pool_k = torch.zeros((num_pages, kv_heads, PAGE_TOKENS * HEAD_DIM), dtype=dt, device=device)
        self.pool_v = torch.zeros_like(self.pool_k)

    def fill(self, k, v, cu_seqlens, max_seq_len):
        _require_cuda(k, v, cu_seqlens)
        args = (self.cfg, k.contiguous(), v.contiguous(), cu_seqlens, self.num_seqs, int(max_seq_len),
                self.kv_heads, self.block_table, self.max_blocks, self.pool_k, self.pool_v)
        if self.fp8:
            kvq_fill_pages_fp8(*args, self.k_scale, self.v_scale)
        else:
            kvq_fill_pages_fp16(*args)

    def append(self, k_new, v_new, lens_before):
        """Write one token per sequence at position lens_before[s]."""
        _require_cuda(k_new, v_new, lens_before)
        args = (self.cfg, k_new.contiguous(), v_new.contiguous(), lens_before, self.num_seqs, self.kv_heads,
                self.block_table, self.max_blocks, self.pool_k, self.pool_v)
        if self.fp8:
            kvq_append_pages_fp8(*args, self.k_scale, self.v_scale)
        else:
            kvq_append_pages_fp16(*args)

    def workspace(self, q_heads, max_seq_len):
        nbytes = kvq_baseline_workspace_bytes(self.cfg, self.num_seqs, q_heads, self.kv_heads, int(max_seq_len))
        return torch.empty(max(nbytes, 4), dtype=torch.uint8, device=self.pool_k.device)

    def decode(self, q, seq_lens, max_seq_len, out=None, workspace=None, sm_scale=None):
        _require_cuda(q, seq_lens)
        s, hq, d = q.shape
        if out is None:
            out = torch.empty((s, hq, d), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = self.workspace(hq, max_seq_len)
        sm = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
        args = (self.cfg, q.contiguous(), s, hq, self.kv_heads, self.block_table, self.max_blocks, seq_lens,
                int(max_seq_len), self.pool_k, self.pool_v)
        if self.fp8:
            kvq_paged_decode_attn_fp8(*args, self.k_scale, self.v_scale, sm, out, workspace, workspace.numel())
        else:
            kvq_paged_decode_attn_fp16(*args, sm, out, workspace, workspace.numel())
        return out
