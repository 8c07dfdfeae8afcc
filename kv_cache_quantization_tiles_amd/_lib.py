"""ctypes binding of libkvq.so: the C-ABI functions under the same names.

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the method runs in the library's kernels.
The library must have been built (kv_cache_quantization_tiles_amd/build.py);
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_HIP, KVQ_ERR_WORKSPACE = 0, -1, -2, -3, -4

EXPORTED = (
    "kvq_last_error", "kvq_version", "kvq_slot_bytes", "kvq_quantize_tiles", "kvq_dequantize",
    "kvq_quantize_to_pages", "kvq_append_and_requant", "kvq_decode_workspace_bytes",
    "kvq_paged_decode_attn", "kvq_bandwidth_probe", "kvq_baseline_page_bytes", "kvq_fill_pages_fp16",
    "kvq_fill_pages_fp8", "kvq_baseline_workspace_bytes", "kvq_paged_decode_attn_fp16",
    "kvq_paged_decode_attn_fp8", "kvq_append_and_decode", "kvq_rematerialize_fp16_pages",
    "kvq_multi_query_workspace_bytes", "kvq_paged_multi_query_attn", "kvq_append_and_decode_noalloc",
    "kvq_append_pages_fp16", "kvq_append_pages_fp8",
)

KVQ_NOALLOC_SCRATCH_BYTES = 32 << 20


class KvqConfig(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
                ("tile_tokens", ctypes.c_int32), ("bits_k", ctypes.c_int32),
                ("bits_v", ctypes.c_int32), ("sinkhorn_iters", ctypes.c_int32),
                ("hadamard_signs", ctypes.c_uint32 * 4), ("meta_fp16", ctypes.c_int32),
                ("k_per_channel", ctypes.c_int32)]


def config(tile_tokens=64, bits_k=4, bits_v=4, sinkhorn_iters=3, head_dim=128, page_tokens=16,
           hadamard_signs=None, meta_fp16=False, k_per_channel=False):
    """hadamard_signs: None (plain rotation) or 4 32-bit words, bit c mod 32 of
    word c // 32 set = channel c negated before the Hadamard.  meta_fp16: slot
    metadata in fp16 instead of fp32.  k_per_channel: K tiles rounded per
    channel (page pools only)."""
    signs = (ctypes.c_uint32 * 4)(*[int(w) & 0xFFFFFFFF for w in (hadamard_signs if hadamard_signs is not None
                                                                   else (0, 0, 0, 0))])
    return KvqConfig(head_dim, page_tokens, tile_tokens, bits_k, bits_v, sinkhorn_iters, signs, int(bool(meta_fp16)),
                     int(bool(k_per_channel)))


class KvqError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"kvq status {status}: {msg}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_CFG = ctypes.POINTER(KvqConfig)


def load():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m "
                           "kv_cache_quantization_tiles_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.kvq_last_error.restype = ctypes.c_char_p
    lib.kvq_version.restype = ctypes.c_char_p
    lib.kvq_slot_bytes.argtypes = [_CFG, _I]
    lib.kvq_slot_bytes.restype = ctypes.c_size_t
    lib.kvq_quantize_tiles.argtypes = [_CFG, _P, _I, _I, _I, _P, _P, _P, _P, _P]
    lib.kvq_dequantize.argtypes = [_CFG, _P, _P, _P, _P, _I, _I, _I, _P, _P]
    lib.kvq_quantize_to_pages.argtypes = [_CFG, _P, _P, _P, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P]
    lib.kvq_append_and_requant.argtypes = [_CFG, _P, _P, _P, _I, _I, _P, _P, _P, _I, _P, _P, _P]
    lib.kvq_decode_workspace_bytes.argtypes = [_CFG, _I, _I, _I, _I]
    lib.kvq_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.kvq_paged_decode_attn.argtypes = [_CFG, _P, _I, _I, _I, _P, _I, _P, _I, _P, _P,
                                          ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
    lib.kvq_bandwidth_probe.argtypes = [_P, _P, ctypes.c_size_t, _P]
    lib.kvq_multi_query_workspace_bytes.argtypes = [_CFG, _I, _I, _I, _I, _I]
    lib.kvq_multi_query_workspace_bytes.restype = ctypes.c_size_t
    lib.kvq_paged_multi_query_attn.argtypes = [_CFG, _P, _I, _I, _I, _I, _P, _I, _P, _I, _P, _P,
                                               ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
    _F = ctypes.c_float
    lib.kvq_append_and_decode.argtypes = [_CFG, _P, _P, _P, _I, _I, _P, _P, _P, _I, _P, _P, _P, _I, _I, _F, _P,
                                          _P, ctypes.c_size_t, _P]
    lib.kvq_append_and_decode_noalloc.argtypes = [_CFG, _P, _P, _P, _I, _I, _P, _P, _P, _I, _P, _P, _P, _I, _I,
                                                  _F, _P, _P]
    lib.kvq_rematerialize_fp16_pages.argtypes = [_CFG, _P, _P, _P, _I, _P, _I, _I, _I, _P, _P, _P]
    lib.kvq_baseline_page_bytes.argtypes = [_I]
    lib.kvq_baseline_page_bytes.restype = ctypes.c_size_t
    lib.kvq_fill_pages_fp16.argtypes = [_CFG, _P, _P, _P, _I, _I, _I, _P, _I, _P, _P, _P]
    lib.kvq_fill_pages_fp8.argtypes = [_CFG, _P, _P, _P, _I, _I, _I, _P, _I, _P, _P, _F, _F, _P]
    lib.kvq_append_pages_fp16.argtypes = [_CFG, _P, _P, _P, _I, _I, _P, _I, _P, _P, _P]
    lib.kvq_append_pages_fp8.argtypes = [_CFG, _P, _P, _P, _I, _I, _P, _I, _P, _P, _F, _F, _P]
    lib.kvq_baseline_workspace_bytes.argtypes = [_CFG, _I, _I, _I, _I]
    lib.kvq_baseline_workspace_bytes.restype = ctypes.c_size_t
    lib.kvq_paged_decode_attn_fp16.argtypes = [_CFG, _P, _I, _I, _I, _P, _I, _P, _I, _P, _P, _F, _P, _P,
                                               ctypes.c_size_t, _P]
    lib.kvq_paged_decode_attn_fp8.argtypes = [_CFG, _P, _I, _I, _I, _P, _I, _P, _I, _P, _P, _F, _F, _F, _P,
                                              _P, ctypes.c_size_t, _P]
    for name in ("kvq_quantize_tiles", "kvq_dequantize", "kvq_quantize_to_pages",
                 "kvq_append_and_requant", "kvq_paged_decode_attn", "kvq_bandwidth_probe",
                 "kvq_fill_pages_fp16", "kvq_fill_pages_fp8", "kvq_paged_decode_attn_fp16",
                 "kvq_paged_decode_attn_fp8", "kvq_append_and_decode", "kvq_rematerialize_fp16_pages",
                 "kvq_paged_multi_query_attn", "kvq_append_and_decode_noalloc", "kvq_append_pages_fp16",
                 "kvq_append_pages_fp8"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status):
    if status != KVQ_OK:
        raise KvqError(status, load().kvq_last_error().decode())


def kvq_last_error() -> str:
    return load().kvq_last_error().decode()


def kvq_version() -> str:
    return load().kvq_version().decode()


def kvq_slot_bytes(cfg: KvqConfig, is_v: bool) -> int:
    return int(load().kvq_slot_bytes(ctypes.byref(cfg), int(is_v)))


def kvq_quantize_tiles(cfg, x, n_tokens, heads, bits, codes, alpha, tok_scale, tok_offset, stream=None):
    _check(load().kvq_quantize_tiles(ctypes.byref(cfg), _ptr(x), n_tokens, heads, bits, _ptr(codes),
                                     _ptr(alpha), _ptr(tok_scale), _ptr(tok_offset), _stream(stream)))


def kvq_dequantize(cfg, codes, alpha, tok_scale, tok_offset, n_tokens, heads, bits, out, stream=None):
    _check(load().kvq_dequantize(ctypes.byref(cfg), _ptr(codes), _ptr(alpha), _ptr(tok_scale),
                                 _ptr(tok_offset), n_tokens, heads, bits, _ptr(out), _stream(stream)))


def kvq_quantize_to_pages(cfg, k, v, cu_seqlens, num_seqs, total_tokens, kv_heads, block_table,
                          max_blocks, pool_k, pool_v, staging_k=None, staging_v=None, stream=None):
    _check(load().kvq_quantize_to_pages(ctypes.byref(cfg), _ptr(k), _ptr(v), _ptr(cu_seqlens), num_seqs,
                                        total_tokens, kv_heads, _ptr(block_table), max_blocks,
                                        _ptr(pool_k), _ptr(pool_v), _ptr(staging_k), _ptr(staging_v),
                                        _stream(stream)))


def kvq_append_and_requant(cfg, k_new, v_new, seq_lens_before, num_seqs, kv_heads, staging_k,
                           staging_v, block_table, max_blocks, pool_k, pool_v, stream=None):
    _check(load().kvq_append_and_requant(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new),
                                         _ptr(seq_lens_before), num_seqs, kv_heads, _ptr(staging_k),
                                         _ptr(staging_v), _ptr(block_table), max_blocks, _ptr(pool_k),
                                         _ptr(pool_v), _stream(stream)))


def kvq_decode_workspace_bytes(cfg, num_seqs, q_heads, kv_heads, max_seq_len) -> int:
    return int(load().kvq_decode_workspace_bytes(ctypes.byref(cfg), num_seqs, q_heads, kv_heads,
                                                 max_seq_len))


def kvq_paged_decode_attn(cfg, q, num_seqs, q_heads, kv_heads, block_table, max_blocks, seq_lens,
                          max_seq_len, pool_k, pool_v, sm_scale, out, workspace, workspace_bytes,
                          stream=None):
    _check(load().kvq_paged_decode_attn(ctypes.byref(cfg), _ptr(q), num_seqs, q_heads, kv_heads,
                                        _ptr(block_table), max_blocks, _ptr(seq_lens), max_seq_len,
                                        _ptr(pool_k), _ptr(pool_v), float(sm_scale), _ptr(out),
                                        _ptr(workspace), workspace_bytes, _stream(stream)))


def kvq_multi_query_workspace_bytes(cfg, num_seqs, n_q, q_heads, kv_heads, max_seq_len) -> int:
    return int(load().kvq_multi_query_workspace_bytes(ctypes.byref(cfg), num_seqs, n_q, q_heads, kv_heads,
                                                      max_seq_len))


def kvq_paged_multi_query_attn(cfg, q, num_seqs, n_q, q_heads, kv_heads, block_table, max_blocks, seq_lens,
                               max_seq_len, pool_k, pool_v, sm_scale, out, workspace, workspace_bytes,
                               stream=None):
    _check(load().kvq_paged_multi_query_attn(ctypes.byref(cfg), _ptr(q), num_seqs, n_q, q_heads, kv_heads,
                                             _ptr(block_table), max_blocks, _ptr(seq_lens), max_seq_len,
                                             _ptr(pool_k), _ptr(pool_v), float(sm_scale), _ptr(out),
                                             _ptr(workspace), workspace_bytes, _stream(stream)))


def kvq_bandwidth_probe(src, dst, nbytes, stream=None):
    _check(load().kvq_bandwidth_probe(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def kvq_rematerialize_fp16_pages(cfg, pool_k, pool_v, block_table, max_blocks, seq_lens, num_seqs, max_seq_len,
                                 kv_heads, base_k, base_v, stream=None):
    _check(load().kvq_rematerialize_fp16_pages(ctypes.byref(cfg), _ptr(pool_k), _ptr(pool_v), _ptr(block_table),
                                               max_blocks, _ptr(seq_lens), num_seqs, max_seq_len, kv_heads,
                                               _ptr(base_k), _ptr(base_v), _stream(stream)))


def kvq_baseline_page_bytes(fp8: bool) -> int:
    return int(load().kvq_baseline_page_bytes(int(fp8)))


def kvq_fill_pages_fp16(cfg, k, v, cu_seqlens, num_seqs, max_seq_len, kv_heads, block_table, max_blocks,
                        pool_k, pool_v, stream=None):
    _check(load().kvq_fill_pages_fp16(ctypes.byref(cfg), _ptr(k), _ptr(v), _ptr(cu_seqlens), num_seqs,
                                      max_seq_len, kv_heads, _ptr(block_table), max_blocks, _ptr(pool_k),
                                      _ptr(pool_v), _stream(stream)))


def kvq_fill_pages_fp8(cfg, k, v, cu_seqlens, num_seqs, max_seq_len, kv_heads, block_table, max_blocks,
                       pool_k, pool_v, k_scale, v_scale, stream=None):
    _check(load().kvq_fill_pages_fp8(ctypes.byref(cfg), _ptr(k), _ptr(v), _ptr(cu_seqlens), num_seqs,
                                     max_seq_len, kv_heads, _ptr(block_table), max_blocks, _ptr(pool_k),
                                     _ptr(pool_v), float(k_scale), float(v_scale), _stream(stream)))


def kvq_baseline_workspace_bytes(cfg, num_seqs, q_heads, kv_heads, max_seq_len) -> int:
    return int(load().kvq_baseline_workspace_bytes(ctypes.byref(cfg), num_seqs, q_heads, kv_heads,
                                                   max_seq_len))


def kvq_paged_decode_attn_fp16(cfg, q, num_seqs, q_heads, kv_heads, block_table, max_blocks, seq_lens,
                               max_seq_len, pool_k, pool_v, sm_scale, out, workspace, workspace_bytes,
                               stream=None):
    _check(load().kvq_paged_decode_attn_fp16(ctypes.byref(cfg), _ptr(q), num_seqs, q_heads, kv_heads,
                                             _ptr(block_table), max_blocks, _ptr(seq_lens), max_seq_len,
                                             _ptr(pool_k), _ptr(pool_v), float(sm_scale), _ptr(out),
                                             _ptr(workspace), workspace_bytes, _stream(stream)))


def kvq_paged_decode_attn_fp8(cfg, q, num_seqs, q_heads, kv_heads, block_table, max_blocks, seq_lens,
                              max_seq_len, pool_k, pool_v, k_scale, v_scale, sm_scale, out, workspace,
                              workspace_bytes, stream=None):
    _check(load().kvq_paged_decode_attn_fp8(ctypes.byref(cfg), _ptr(q), num_seqs, q_heads, kv_heads,
                                            _ptr(block_table), max_blocks, _ptr(seq_lens), max_seq_len,
                                            _ptr(pool_k), _ptr(pool_v), float(k_scale), float(v_scale),
                                            float(sm_scale), _ptr(out), _ptr(workspace), workspace_bytes,
                                            _stream(stream)))


def kvq_append_and_decode(cfg, k_new, v_new, seq_lens_before, num_seqs, kv_heads, staging_k, staging_v,
                          block_table, max_blocks, pool_k, pool_v, q, q_heads, max_seq_len, sm_scale, out,
                          workspace, workspace_bytes, stream=None):
    _check(load().kvq_append_and_decode(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new), _ptr(seq_lens_before),
                                        num_seqs, kv_heads, _ptr(staging_k), _ptr(staging_v), _ptr(block_table),
                                        max_blocks, _ptr(pool_k), _ptr(pool_v), _ptr(q), q_heads, max_seq_len,
                                        float(sm_scale), _ptr(out), _ptr(workspace), workspace_bytes,
                                        _stream(stream)))



def kvq_append_and_decode_noalloc(cfg, k_new, v_new, seq_lens_before, num_seqs, kv_heads, staging_k, staging_v,
                                  block_table, max_blocks, pool_k, pool_v, q, q_heads, max_seq_len, sm_scale, out,
                                  stream=None):
    _check(load().kvq_append_and_decode_noalloc(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new),
                                                _ptr(seq_lens_before), num_seqs, kv_heads, _ptr(staging_k),
                                                _ptr(staging_v), _ptr(block_table), max_blocks, _ptr(pool_k),
                                                _ptr(pool_v), _ptr(q), q_heads, max_seq_len, float(sm_scale),
                                                _ptr(out), _stream(stream)))


def kvq_append_pages_fp16(cfg, k_new, v_new, seq_lens_before, num_seqs, kv_heads, block_table, max_blocks, pool_k,
                          pool_v, stream=None):
    _check(load().kvq_append_pages_fp16(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new), _ptr(seq_lens_before),
                                        num_seqs, kv_heads, _ptr(block_table), max_blocks, _ptr(pool_k),
                                        _ptr(pool_v), _stream(stream)))


def kvq_append_pages_fp8(cfg, k_new, v_new, seq_lens_before, num_seqs, kv_heads, block_table, max_blocks, pool_k,
                         pool_v, k_scale, v_scale, stream=None):
    _check(load().kvq_append_pages_fp8(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new), _ptr(seq_lens_before),
                                       num_seqs, kv_heads, _ptr(block_table), max_blocks, _ptr(pool_k),
                                       _ptr(pool_v), float(k_scale), float(v_scale), _stream(stream)))
