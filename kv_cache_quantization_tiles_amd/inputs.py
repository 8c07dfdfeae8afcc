"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and lays out page tables. It holds none
of the quantizer's arithmetic, so both the CPU oracle and the HIP path may use
it without sharing any of the method.

The five workloads mirror the shapes the pages talk about (there is no dataset
to load):

* the Qwen3-32B 16K-context burst at TP=2 on the axbrief KVarN page
  ("Huawei's KVarN boosts vLLM KV-cache capacity by 5x without accuracy loss",
  untitled lede), of which one GPU holds half the KV heads;
* the A100 run with 128K context per user and 1024 decode tokens on the
  aitrends.kr page (article 74976, TL;DR).

Value recipe: K ~ N(0, 1) with a few channels scaled up (the pages say that
KV outliers concentrate in particular channels: axbrief KVarN page, section
"기존 방식과 달라진 지점"), V ~ N(0, 1), Q ~ N(0, 1).  Values are drawn in
float64, clamped to the fp16 range and rounded to fp16.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

HEAD_DIM = 128
PAGE_TOKENS = 16
FP16_MAX = 65504.0

_ROLE_IDS = {"K": 1, "V": 2, "Q": 3, "outlier": 4, "lens": 5, "table": 6, "decode_k": 7,
             "decode_v": 8, "decode_q": 9, "multi_q": 10}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes and quantizer parameters."""

    name: str
    index: int
    seq_lens: tuple          # context length of each sequence before decoding
    hkv: int                 # KV heads
    hq: int                  # query heads (a multiple of hkv)
    tile_tokens: int
    bits_k: int
    bits_v: int
    iters: int               # Sinkhorn-like iterations
    decode_steps: int        # tokens appended per sequence after the prefill
    k_recipe: str            # "outlier_fixed4x20", "outlier_2pct_10_50", "student_t3_loguniform"
    layers: int = 1
    head_dim: int = HEAD_DIM
    page_tokens: int = PAGE_TOKENS

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))

    def cu_seqlens(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(np.asarray(self.seq_lens, dtype=np.int64))
        return cu

    def scaled(self, num_seqs=None, seq_len=None, name=None) -> "Workload":
        """The same recipe at a smaller size (for tests the oracle finishes in seconds)."""
        lens = list(self.seq_lens)
        if num_seqs is not None:
            lens = lens[:num_seqs]
        if seq_len is not None:
            lens = [min(int(seq_len), l) for l in lens]
        return dataclasses.replace(self, seq_lens=tuple(lens), name=name or self.name + "-small")


def _rng(cfg: int, layer: int, role: str, extra: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([20261202, cfg, layer, _ROLE_IDS[role], extra]))


def workload(index: int) -> Workload:
    """Workloads 1..5 (the first is the small correctness case)."""
    if index == 1:
        return Workload("single-head-1k", 1, (1024,), 1, 8, 64, 4, 4, 3, 1, "outlier_fixed4x20")
    if index == 2:
        return Workload("qwen3-4b-layer-4x16k", 2, (16384,) * 4, 8, 32, 64, 4, 4, 3, 1,
                        "outlier_2pct_10_50")
    if index == 3:
        return Workload("qwen3-32b-tp2-share-32x16k", 3, (16384,) * 32, 4, 32, 64, 4, 4, 3, 256,
                        "outlier_2pct_10_50")
    if index == 4:
        return Workload("qwen3-4b-36l-6x128k", 4, (131072,) * 6, 8, 32, 128, 4, 4, 3, 1024,
                        "outlier_2pct_10_50", layers=36)
    if index == 5:
        rng = _rng(5, 0, "lens")
        lens = tuple(int(x) for x in rng.integers(1024, 32768 + 1, size=64))
        return Workload("mixed-64seq-1k-32k", 5, lens, 8, 64, 32, 4, 2, 5, 1, "student_t3_loguniform")
    raise ValueError(f"unknown workload {index}")


def _to_fp16(x: np.ndarray) -> np.ndarray:
    return np.clip(x, -FP16_MAX, FP16_MAX).astype(np.float16)


def channel_scales(wl: Workload, layer: int = 0) -> np.ndarray:
    """Per (kv head, channel) multiplier applied to K, float64 [hkv, head_dim]."""
    d = wl.head_dim
    scale = np.ones((wl.hkv, d), dtype=np.float64)
    rng = _rng(wl.index, layer, "outlier")
    if wl.k_recipe == "outlier_fixed4x20":
        ch = rng.choice(d, size=4, replace=False)
        scale[:, ch] = 20.0
    elif wl.k_recipe == "outlier_2pct_10_50":
        n_out = int(round(0.02 * d))
        for h in range(wl.hkv):
            ch = rng.choice(d, size=n_out, replace=False)
            scale[h, ch] = rng.uniform(10.0, 50.0, size=n_out)
    elif wl.k_recipe == "student_t3_loguniform":
        scale = np.exp(rng.uniform(math.log(0.1), math.log(50.0), size=(wl.hkv, d)))
    else:
        raise ValueError(wl.k_recipe)
    return scale


def gen_kv(wl: Workload, role: str, layer: int = 0, seqs=None) -> np.ndarray:
    """fp16 K or V for the prefill, packed by sequence: [total_tokens, hkv, head_dim].

    `seqs` restricts generation to a subset of sequences (same values as in the
    full tensor: every sequence has its own stream)."""
    assert role in ("K", "V")
    seqs = range(wl.num_seqs) if seqs is None else seqs
    scale = channel_scales(wl, layer) if role == "K" else None
    out = []
    for i in seqs:
        n = wl.seq_lens[i]
        rng = _rng(wl.index, layer, role, i)
        if role == "K" and wl.k_recipe == "student_t3_loguniform":
            x = rng.standard_t(3.0, size=(n, wl.hkv, wl.head_dim))
        else:
            x = rng.standard_normal(size=(n, wl.hkv, wl.head_dim))
        if scale is not None:
            x = x * scale[None]
        out.append(_to_fp16(x))
    return np.concatenate(out, axis=0) if out else np.zeros((0, wl.hkv, wl.head_dim), np.float16)


def gen_decode_kv(wl: Workload, role: str, step: int, layer: int = 0) -> np.ndarray:
    """fp16 K or V of the token appended at decode `step`: [num_seqs, hkv, head_dim]."""
    assert role in ("K", "V")
    rng = _rng(wl.index, layer, "decode_k" if role == "K" else "decode_v", step)
    if role == "K" and wl.k_recipe == "student_t3_loguniform":
        x = rng.standard_t(3.0, size=(wl.num_seqs, wl.hkv, wl.head_dim))
    else:
        x = rng.standard_normal(size=(wl.num_seqs, wl.hkv, wl.head_dim))
    if role == "K":
        x = x * channel_scales(wl, layer)[None]
    return _to_fp16(x)


def gen_q(wl: Workload, step: int = 0, layer: int = 0) -> np.ndarray:
    """fp16 queries of one decode step: [num_seqs, hq, head_dim]."""
    rng = _rng(wl.index, layer, "decode_q", step)
    return _to_fp16(rng.standard_normal(size=(wl.num_seqs, wl.hq, wl.head_dim)))


def gen_q_multi(wl: Workload, n_q: int, step: int = 0, layer: int = 0) -> np.ndarray:
    """fp16 queries of the n_q newest tokens of each sequence (a verify or
    chunk step): [num_seqs, n_q, hq, head_dim]."""
    rng = _rng(wl.index, layer, "multi_q", step * 1000 + n_q)
    return _to_fp16(rng.standard_normal(size=(wl.num_seqs, n_q, wl.hq, wl.head_dim)))


def hadamard_signs(seed: int) -> np.ndarray:
    """A seeded 128-bit sign mask for the randomized rotation (4 x uint32; bit
    c mod 32 of word c // 32 set = channel c negated).  Random numbers the
    method draws are inputs: the library and the oracle both take this mask."""
    rng = np.random.default_rng(np.random.SeedSequence([20261202, 77, int(seed)]))
    return rng.integers(0, 1 << 32, size=4, dtype=np.uint64).astype(np.uint32)


def block_table(wl: Workload, capacity_tokens=None, layer: int = 0):
    """Shuffled page table, pages allocated in whole tiles.

    Every tile a sequence can reach (its prefill plus its decode tokens, or
    `capacity_tokens` per sequence) owns tile_tokens / page_tokens pages, so a
    partial tile always has a page for each slice of its channel factors.
    Returns (table int32 [num_seqs, max_blocks] with -1 past each sequence's
    pages, num_pages)."""
    t, p = wl.tile_tokens, wl.page_tokens
    caps = [(l + wl.decode_steps) if capacity_tokens is None else int(capacity_tokens)
            for l in wl.seq_lens]
    pages = [int(math.ceil(c / t)) * (t // p) for c in caps]
    total = int(sum(pages))
    perm = _rng(wl.index, layer, "table").permutation(total).astype(np.int32)
    max_blocks = max(pages) if pages else 1
    table = np.full((wl.num_seqs, max_blocks), -1, dtype=np.int32)
    off = 0
    for i, n in enumerate(pages):
        table[i, :n] = perm[off:off + n]
        off += n
    return table, total


def identity_block_table(wl: Workload, capacity_tokens=None):
    """Same allocation as block_table() but pages in order (for layout tests)."""
    table, total = block_table(wl, capacity_tokens)
    out = np.full_like(table, -1)
    off = 0
    for i in range(table.shape[0]):
        n = int((table[i] >= 0).sum())
        out[i, :n] = np.arange(off, off + n, dtype=np.int32)
        off += n
    return out, total


def gen_kv_device(wl: Workload, role: str, layer: int = 0, device="cuda"):
    """fp16 K or V of the whole prefill drawn on the device with a seeded torch
    generator, for workloads too large to draw on the host (the 36-layer 128K
    one, the 64-sequence mixed-length one): [total_tokens, hkv, head_dim].
    Same recipe as gen_kv (normal or Student-t(3) values, K channels scaled by
    channel_scales, clamped, rounded to fp16), a different stream of numbers.
    Student-t(3) is drawn as z / sqrt(c / 3) with z standard normal and c
    chi-square with 3 degrees of freedom (twice a Gamma(3/2) variate)."""
    import torch
    assert role in ("K", "V")
    g = torch.Generator(device=device)
    g.manual_seed(20261202 * 1000 + wl.index * 100 + layer * 10 + _ROLE_IDS[role])
    shape = (wl.total_tokens, wl.hkv, wl.head_dim)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if role == "K" and wl.k_recipe == "student_t3_loguniform":
        c = torch._standard_gamma(torch.full(shape, 1.5, device=device, dtype=torch.float32), generator=g)
        x /= torch.sqrt(c * (2.0 / 3.0))
        del c
    if role == "K":
        x *= torch.from_numpy(channel_scales(wl, layer)).to(device=device, dtype=torch.float32)[None]
    return x.clamp_(-FP16_MAX, FP16_MAX).to(torch.float16)
