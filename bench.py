#!/usr/bin/env python
"""Throughput of the quantized KV-cache hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. quantize every page of the prefill (K and V, all sequences and heads),
  2. one decode step in a single launch (kvq_append_and_decode): append one
     token per sequence, re-quantize its tile, and attend over every cached
     token straight from the pages.
Default workload: a Qwen3-4B-shaped layer, 8 KV heads / 32 query heads,
4 sequences x 16K context, 16-token pages, tile 64, 4-bit K and V, 3
normalization iterations.

Prints one JSON line.  `value` is the step's algorithmic bytes (quantize +
append + decode) over the step time, in GB/s, the K timed steps replayed
from one HIP graph (`value_eager`: the same steps launched call by call).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from kv_cache_quantization_tiles_amd import inputs  # noqa: E402

HBM_PEAK_GBPS = 8000.0
# Non-packed fp32 VALU issue peak of MI355X: 256 CUs x 64 lanes x 2.4 GHz
# (packed fp32 is kept out of the generated code).
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
D = 128


def quantize_valu_ops_per_element(iters: int) -> int:
    """Algorithmic VALU lane-ops per element of the quantizer: the rotation's
    channel bits 0..4 run on the matrix cores (fp16 in, exact products), bits
    5 and 6 are a 4-point butterfly (2); 3 per normalization half-step
    (shifted value, sum, sum of squares) over 2*iters-1 half-steps (the last
    token step cancels); rounding (scale, min/max, affine map, convert: 4)."""
    return 2 + 3 * max(2 * iters - 1, 0) + 4


def measured_traffic(kernel_sources, profile: str):
    """HBM bytes per launch from a committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    measurement, if it was taken on the current kernel sources (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for name in kernel_sources:
        with open(os.path.join(ROOT, "kv_cache_quantization_tiles_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return {"read_bytes": rec["read_bytes"], "write_bytes": rec["write_bytes"],
            "total_bytes": rec["read_bytes"] + rec["write_bytes"], "source": "profiles/" + profile}


# sources the quantize kernel is built from (the traffic record names their hash)
QUANTIZE_SOURCES = ("kvq_quantize.hip", "kvq_tile.h", "kvq_internal.h")


# ----------------------------------------------------------------------------- byte model
def quantize_bytes(n_token_heads: int, bits: int, tile: int, meta16: bool = False) -> float:
    """Algorithmic bytes of quantizing n token-heads of K or V: fp16 read,
    codes + scale + offset written, and the tile's channel factors."""
    return n_token_heads * (2 * D + slot_bytes_per_token(bits, tile, meta16))


def slot_bytes_per_token(bits: int, tile: int, meta16: bool = False, kchan: bool = False) -> float:
    if kchan:   # K rounded per channel: beta per token, channel scale and zero offset per channel of the tile
        return D * bits / 8 + 4 + 8 * D / tile
    m = 2 if meta16 else 4   # bytes per metadata value (fp16 or fp32)
    return D * bits / 8 + 2 * m + m * D / tile


def decode_bytes(wl, lens, meta16: bool = False) -> float:
    """Slot bytes of every page read by one decode step (whole tiles)."""
    t = wl.tile_tokens
    tok = sum(int(math.ceil(l / t)) * t for l in lens) * wl.hkv
    return tok * (slot_bytes_per_token(wl.bits_k, t, meta16) + slot_bytes_per_token(wl.bits_v, t, meta16))


def append_bytes(wl, lens_before) -> float:
    """Staging rows read and the tile's slots rewritten, K and V."""
    t = wl.tile_tokens
    tot = 0.0
    for l in lens_before:
        rows = l % t + 1
        for bits in (wl.bits_k, wl.bits_v):
            tot += wl.hkv * (rows * 2 * D + 2 * D + t * slot_bytes_per_token(bits, t))
    return tot


# ----------------------------------------------------------------------------- CPU oracle leg
def _oracle_quantize_unit(args):
    import oracle as orc
    from oracle import kvq_oracle as orc_impl
    wl, s, h, role = args
    x = inputs.gen_kv(wl, role, seqs=[s])[:, h:h + 1]
    n = x.shape[0]
    table = np.arange(int(math.ceil(n / wl.tile_tokens)) * (wl.tile_tokens // 16), dtype=np.int32)[None]
    bits = wl.bits_k if role == "K" else wl.bits_v
    pool = orc.new_pool(table.shape[1], 1, bits, wl.tile_tokens)
    t0 = time.perf_counter()
    # this unit's role only: every tile through the oracle's quantizer into its pages
    t = wl.tile_tokens
    for j in range((n + t - 1) // t):
        tq = orc.quantize_tile(x[j * t:min(n, (j + 1) * t), 0, :], bits, wl.iters)
        orc_impl._store_tile(pool, table[0], 0, role, bits, t, j, tq)
    return (s, h, role), pool, time.perf_counter() - t0


def _oracle_decode_unit(args):
    import oracle as orc
    wl, s, h, pk, pv, q = args
    n = wl.seq_lens[s]
    table = np.arange(pk.shape[0], dtype=np.int32)[None]
    t0 = time.perf_counter()
    orc.paged_decode_attn(q, table, np.array([n], np.int32), pk, pv, wl.tile_tokens, wl.bits_k, wl.bits_v)
    return time.perf_counter() - t0


def cpu_baseline(wl, max_seqs: int):
    """Time the oracle (as it stands) on the host cores, on a bounded sample:
    the first `max_seqs` sequences of the workload, all heads, K and V
    quantized, then one decode step over them."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    cores = min(len(os.sched_getaffinity(0)), 16)
    seqs = list(range(min(max_seqs, wl.num_seqs)))
    units = [(wl, s, h, role) for s in seqs for h in range(wl.hkv) for role in ("K", "V")]
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        t0 = time.perf_counter()
        res = pool.map(_oracle_quantize_unit, units, chunksize=1)
        tq = time.perf_counter() - t0
        pools = {key: p for key, p, _ in res}
        q = inputs.gen_q(wl)
        dunits = [(wl, s, h, pools[(s, h, "K")], pools[(s, h, "V")],
                   q[s:s + 1, h * wl.group:(h + 1) * wl.group]) for s in seqs for h in range(wl.hkv)]
        t1 = time.perf_counter()
        pool.map(_oracle_decode_unit, dunits, chunksize=1)
        td = time.perf_counter() - t1
    # one unit (sequence 0, kv head 0, K) on one core, in this process
    t2 = time.perf_counter()
    _oracle_quantize_unit(units[0])
    t_unit = time.perf_counter() - t2
    ntok_heads = sum(wl.seq_lens[s] for s in seqs) * wl.hkv
    qb = quantize_bytes(ntok_heads, wl.bits_k, wl.tile_tokens) + quantize_bytes(ntok_heads, wl.bits_v, wl.tile_tokens)
    db = decode_bytes(wl, [wl.seq_lens[s] for s in seqs])
    unit_bytes = quantize_bytes(wl.seq_lens[0], wl.bits_k, wl.tile_tokens)
    ntok = sum(wl.seq_lens[s] for s in seqs)
    return {"value": round((qb + db) / (tq + td) / 1e9, 6), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{wl.name}: {len(seqs)} of {wl.num_seqs} sequences ({ntok} tokens), all {wl.hkv} kv heads: "
                      f"quantize K and V to pages, then one decode step (fp64 NumPy oracle, "
                      f"{cores} worker processes)",
            "decode_tok_per_s": round(len(seqs) / td, 3),
            "quantize_s": round(tq, 3), "decode_s": round(td, 3),
            "single_core_quantize_GBps": round(unit_bytes / t_unit / 1e9, 6),
            "single_core_unit": f"quantize one (sequence, kv head) of K, {wl.seq_lens[0]} tokens: {t_unit:.3f} s",
            "machine_cores": os.cpu_count()}


# ----------------------------------------------------------------------------- long-context comparison
def long_context_leg(n_iter: int = 10):
    """One layer of the 36-layer, 6 x 128K Qwen3-4B-shaped workload (8 kv /
    32 query heads, tile 128): the decode-attention step on fp16 pages, fp8
    (E4M3, per-tensor scale) pages, and 4-, 2- and 8-bit quantized pages, all
    filled from the same inputs, and the 4-bit pages read the other way:
    restored to fp16 pages first, then the fp16 decode (kvq4_rematerialize).
    Attention only (no append), context 131072,
    pages far larger than the 256 MB last-level cache, so every call streams
    from HBM.  tok/s is for all 36 layers (36 such steps per token)."""
    import torch
    from kv_cache_quantization_tiles_amd import api

    wl = inputs.workload(4)
    dev = torch.device("cuda:0")
    table, npages = inputs.block_table(wl, capacity_tokens=max(wl.seq_lens))
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    max_len = max(wl.seq_lens)
    cu = torch.from_numpy(wl.cu_seqlens()).to(dev)
    q = torch.from_numpy(inputs.gen_q(wl)).to(dev)
    out = torch.empty((wl.num_seqs, wl.hq, D), dtype=torch.float32, device=dev)
    k = inputs.gen_kv_device(wl, "K", device=dev)
    v = inputs.gen_kv_device(wl, "V", device=dev)
    token_heads = wl.total_tokens * wl.hkv

    def timed(fn, n):
        for _ in range(2):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    modes = {}
    for name in ("fp16", "fp8", "kvq4", "kvq2", "kvq8", "kvq4_meta16", "kvq2_meta16", "kvq4_kchan"):
        if name in ("fp16", "fp8"):
            fp8 = name == "fp8"
            ks = float(k.abs().max()) / 448.0 if fp8 else 1.0
            vs = float(v.abs().max()) / 448.0 if fp8 else 1.0
            cache = api.BaselineCache(npages, wl.hkv, torch.from_numpy(table), wl.num_seqs, fp8, ks, vs)
            fill_ms = timed(lambda: cache.fill(k, v, cu, max_len), 3)
            per_token_head = 2 * 128 * (1 if fp8 else 2)
            fill_bytes = token_heads * (2 * 2 * D + per_token_head)
        else:
            bits, m16, kch = int(name[3]), name.endswith("meta16"), name.endswith("kchan")
            cfg = api.config(wl.tile_tokens, bits, bits, wl.iters, meta_fp16=m16, k_per_channel=kch)
            cache = api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
            fill_ms = timed(lambda: cache.quantize_prefill(k, v, cu), 3)
            per_token_head = (slot_bytes_per_token(bits, wl.tile_tokens, m16, kch)
                              + slot_bytes_per_token(bits, wl.tile_tokens, m16))
            fill_bytes = token_heads * (4 * D + per_token_head)
        ws = cache.workspace(wl.hq, max_len)
        dec_ms = timed(lambda: cache.decode(q, lens, max_len, out=out, workspace=ws), n_iter)
        dbytes = token_heads * per_token_head
        modes[name] = {"decode_attn_ms": round(dec_ms, 4),
                       "decode_GBps": round(dbytes / (dec_ms * 1e-3) / 1e9, 1),
                       "decode_hbm_frac": round(dbytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                       "kv_bytes_per_layer_GB": round(dbytes / 1e9, 3),
                       "tok_per_s_36_layers_attn_only": round(wl.num_seqs / (wl.layers * dec_ms * 1e-3), 1),
                       "fill_ms": round(fill_ms, 3),
                       "fill_GBps": round(fill_bytes / (fill_ms * 1e-3) / 1e9, 1)}
        if name == "kvq4":
            # the read path the direct decode avoids: restore every page to fp16, then the fp16 decode
            base16 = api.BaselineCache(npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
            ws16 = base16.workspace(wl.hq, max_len)
            restore_ms = timed(lambda: cache.rematerialize_into(base16, lens, max_len), n_iter)
            step_ms = timed(lambda: (cache.rematerialize_into(base16, lens, max_len),
                                     base16.decode(q, lens, max_len, out=out, workspace=ws16)), n_iter)
            rbytes = token_heads * (per_token_head + 2 * 2 * D)   # slots read, fp16 K and V written
            modes["kvq4_rematerialize"] = {
                "decode_attn_ms": round(step_ms, 4), "restore_ms": round(restore_ms, 4),
                "restore_GBps": round(rbytes / (restore_ms * 1e-3) / 1e9, 1),
                "restore_hbm_frac": round(rbytes / (restore_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "kv_bytes_per_layer_GB": round(dbytes / 1e9, 3),
                "tok_per_s_36_layers_attn_only": round(wl.num_seqs / (wl.layers * step_ms * 1e-3), 1)}
            del base16, ws16
        del cache, ws
        torch.cuda.empty_cache()
    del k, v
    torch.cuda.empty_cache()
    base = modes["fp16"]["decode_attn_ms"]
    for m in modes.values():
        m["speedup_vs_fp16"] = round(base / m["decode_attn_ms"], 3)
    for m in modes.values():
        m["bytes_per_token_head"] = round(m["kv_bytes_per_layer_GB"] * 1e9 / token_heads, 2)
    return {"workload": f"{wl.name}, one layer of {wl.layers}", "num_seqs": wl.num_seqs, "context": max_len,
            "kv_heads": wl.hkv, "q_heads": wl.hq, "tile_tokens": wl.tile_tokens, "iters": n_iter,
            "modes": modes,
            "pages_context": "A100-80GB, whole Qwen3-4B at 128K: 66.6 / 105.0 / 140.9 tok/s for "
                             "fp16 / fp8 / compressed KV (other hardware, end-to-end; context only)"}


def cpu_baseline_legs():
    """The oracle beside the other workloads, each on a bounded sample (its
    first sequences; one layer of the long-context one), same byte formulas."""
    out = {}
    for idx, nseq in ((1, 1), (3, 2), (5, 2), (4, 1)):
        wl = inputs.workload(idx)
        if wl.layers > 1:
            wl = dataclasses.replace(wl, layers=1)
        r = cpu_baseline(wl, nseq)
        r["sample"] += " (one layer)" if idx == 4 else ""
        out[wl.name] = r
    return out


def latency_leg(n: int = 50):
    """The single-head 1024-token correctness workload as a latency line:
    quantize its prefill, then one fused append + decode step (8 query heads),
    each launch timed alone (events around one call, inputs resident)."""
    import torch
    from kv_cache_quantization_tiles_amd import api
    wl = inputs.workload(1)
    dev = torch.device("cuda:0")
    table, npages = inputs.block_table(wl)
    cfg = api.config(wl.tile_tokens, wl.bits_k, wl.bits_v, wl.iters)
    cache = api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
    k = torch.from_numpy(inputs.gen_kv(wl, "K")).to(dev)
    v = torch.from_numpy(inputs.gen_kv(wl, "V")).to(dev)
    cu = torch.from_numpy(wl.cu_seqlens()).to(dev)
    kn = torch.from_numpy(inputs.gen_decode_kv(wl, "K", 0)).to(dev)
    vn = torch.from_numpy(inputs.gen_decode_kv(wl, "V", 0)).to(dev)
    q = torch.from_numpy(inputs.gen_q(wl)).to(dev)
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    out = torch.empty((wl.num_seqs, wl.hq, D), dtype=torch.float32, device=dev)
    ws = cache.workspace(wl.hq, max(wl.seq_lens) + 1)

    def one(fn):
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        return float(np.median(ts))
    tq = one(lambda: cache.quantize_prefill(k, v, cu))
    td = one(lambda: cache.append_decode(kn, vn, lens, q, max(wl.seq_lens) + 1, out=out, workspace=ws))
    return {"workload": wl.name, "tokens": wl.total_tokens, "kv_heads": wl.hkv, "q_heads": wl.hq,
            "quantize_latency_us": round(tq, 2), "decode_step_latency_us": round(td, 2),
            "note": "median of single launches (bulk + short-tile quantize; fused decode + merge); launch-bound"}


def rematerialize_leg(idx: int, n_iter: int = 20):
    """The read path the direct decode avoids, on a 16K workload: restore every
    page to fp16 pages, then the fp16 decode, against the direct decode of the
    same quantized pages (both timed as back-to-back batches over rotated
    pools)."""
    import torch
    from kv_cache_quantization_tiles_amd import api
    wl = inputs.workload(idx)
    dev = torch.device("cuda:0")
    table, npages = inputs.block_table(wl)
    max_len = max(wl.seq_lens)
    cu = torch.from_numpy(wl.cu_seqlens()).to(dev)
    k = inputs.gen_kv_device(wl, "K", device=dev)
    v = inputs.gen_kv_device(wl, "V", device=dev)
    cfg = api.config(wl.tile_tokens, wl.bits_k, wl.bits_v, wl.iters)
    pool_bytes = npages * wl.hkv * (api.kvq_slot_bytes(cfg, False) + api.kvq_slot_bytes(cfg, True))
    nc = max(2, int(math.ceil(1.0e9 / pool_bytes)))
    caches = [api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs) for _ in range(nc)]
    for c in caches:
        c.quantize_prefill(k, v, cu)
    del k, v
    base = [api.BaselineCache(npages, wl.hkv, torch.from_numpy(table), wl.num_seqs) for _ in range(2)]
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    q = torch.from_numpy(inputs.gen_q(wl)).to(dev)
    out = torch.empty((wl.num_seqs, wl.hq, D), dtype=torch.float32, device=dev)
    ws = caches[0].workspace(wl.hq, max_len)
    ws16 = base[0].workspace(wl.hq, max_len)

    def batch(fn):
        fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for j in range(n_iter):
            fn(j)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n_iter
    direct = batch(lambda j: caches[j % nc].decode(q, lens, max_len, out=out, workspace=ws))
    remat = batch(lambda j: (caches[j % nc].rematerialize_into(base[j % 2], lens, max_len),
                             base[j % 2].decode(q, lens, max_len, out=out, workspace=ws16)))
    del caches, base
    torch.cuda.empty_cache()
    return {"workload": wl.name, "direct_decode_ms": round(direct, 4), "rematerialize_then_fp16_decode_ms": round(remat, 4),
            "ratio": round(remat / direct, 2)}


def long_context_decode_phase(n_steps: int = 1024):
    """The long-context workload's decode phase on one layer: 6 sequences of
    131072 tokens, 8 kv / 32 query heads, then 1024 decode steps, each an
    append of one token per sequence and the attention that includes it:
    fused append + re-quantize + attend for the 4- and 2-bit pages (tile 128:
    the steps cross 8 tile boundaries), append + decode for the fp16 and fp8
    pages.  The 1024 steps run back to back between two events; per-step
    tokens and queries are resident before timing."""
    import torch
    from kv_cache_quantization_tiles_amd import api
    wl = dataclasses.replace(inputs.workload(4), layers=1, decode_steps=n_steps)
    dev = torch.device("cuda:0")
    table, npages = inputs.block_table(wl)
    max_len = max(wl.seq_lens)
    cu = torch.from_numpy(wl.cu_seqlens()).to(dev)
    k = inputs.gen_kv_device(wl, "K", device=dev)
    v = inputs.gen_kv_device(wl, "V", device=dev)
    kd = torch.from_numpy(np.stack([inputs.gen_decode_kv(wl, "K", i) for i in range(n_steps)])).to(dev)
    vd = torch.from_numpy(np.stack([inputs.gen_decode_kv(wl, "V", i) for i in range(n_steps)])).to(dev)
    qd = torch.from_numpy(np.stack([inputs.gen_q(wl, i) for i in range(n_steps)])).to(dev)
    lens0 = torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    lens = [lens0 + i for i in range(n_steps)]
    out = torch.empty((wl.num_seqs, wl.hq, D), dtype=torch.float32, device=dev)
    res = {}
    for name in ("fp16", "fp8", "kvq4", "kvq2"):
        if name in ("fp16", "fp8"):
            fp8 = name == "fp8"
            ks = max(float(k.abs().max()), float(kd.abs().max())) / 448.0 if fp8 else 1.0
            vs = max(float(v.abs().max()), float(vd.abs().max())) / 448.0 if fp8 else 1.0
            cache = api.BaselineCache(npages, wl.hkv, torch.from_numpy(table), wl.num_seqs, fp8, ks, vs)
            cache.fill(k, v, cu, max_len)
            ws = cache.workspace(wl.hq, max_len + n_steps)

            def step(i):
                cache.append(kd[i], vd[i], lens[i])
                cache.decode(qd[i], lens[i] + 1, max_len + n_steps, out=out, workspace=ws)
            per_tok = 2 * 128 * (1 if fp8 else 2)
        else:
            bits = int(name[3:])
            cfg = api.config(wl.tile_tokens, bits, bits, wl.iters)
            cache = api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
            cache.quantize_prefill(k, v, cu)
            ws = cache.workspace(wl.hq, max_len + n_steps)

            def step(i):
                cache.append_decode(kd[i], vd[i], lens[i], qd[i], max_len + n_steps, out=out, workspace=ws)
            per_tok = 2 * slot_bytes_per_token(bits, wl.tile_tokens)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n_steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n_steps
        mid = max_len + n_steps // 2
        rb = wl.num_seqs * wl.hkv * per_tok * (mid if name in ("fp16", "fp8") else
                                               math.ceil(mid / wl.tile_tokens) * wl.tile_tokens)
        res[name] = {"step_ms": round(ms, 4), "tok_per_s_per_layer": round(wl.num_seqs / (ms * 1e-3), 1),
                     "tok_per_s_36_layers_extrapolated": round(wl.num_seqs / (36 * ms * 1e-3), 1),
                     "read_GBps": round(rb / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(rb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        del cache, ws
        torch.cuda.empty_cache()
    del k, v, kd, vd, qd
    torch.cuda.empty_cache()
    base = res["fp16"]["step_ms"]
    for m in res.values():
        m["speedup_vs_fp16"] = round(base / m["step_ms"], 3)
    return {"workload": f"{wl.name}, one layer, {n_steps} decode steps", "num_seqs": wl.num_seqs,
            "context_start": max_len, "tile_tokens": wl.tile_tokens, "modes": res,
            "note": "step = append of one token per sequence + attention over every cached token (+ merge); "
                    "read GB/s at the middle step's length; 36-layer figures are this layer's time x 36"}


def burst_leg():
    """One GPU's TP=2 share of the Qwen3-32B-shaped 16K burst (32 sequences x
    16384 tokens, 4 kv / 32 query heads, tile 64, 4-bit K and V, 3
    iterations): quantize the burst prefill, then the workload's 256 decode
    steps, each one fused append + re-quantize + attend launch (plus the
    partition merge).  Inputs drawn on the device; the new tokens and queries
    of every step are resident before timing."""
    import torch
    from kv_cache_quantization_tiles_amd import api

    wl = inputs.workload(3)
    dev = torch.device("cuda:0")
    table, npages = inputs.block_table(wl)
    max_len = max(wl.seq_lens)
    cu = torch.from_numpy(wl.cu_seqlens()).to(dev)
    k = inputs.gen_kv_device(wl, "K", device=dev)
    v = inputs.gen_kv_device(wl, "V", device=dev)
    cfg = api.config(wl.tile_tokens, wl.bits_k, wl.bits_v, wl.iters)
    steps = wl.decode_steps
    kn = torch.stack([torch.from_numpy(inputs.gen_decode_kv(wl, "K", i)) for i in range(steps)]).to(dev)
    vn = torch.stack([torch.from_numpy(inputs.gen_decode_kv(wl, "V", i)) for i in range(steps)]).to(dev)
    qs = torch.stack([torch.from_numpy(inputs.gen_q(wl, i)) for i in range(steps)]).to(dev)
    lens0 = torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    lens = [lens0 + i for i in range(steps)]
    out = torch.empty((wl.num_seqs, wl.hq, D), dtype=torch.float32, device=dev)
    caches = [api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs) for _ in range(2)]
    ws = caches[0].workspace(wl.hq, max_len + steps)
    caches[1].quantize_prefill(k, v, cu)   # warm-up
    torch.cuda.synchronize()
    c = caches[0]
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record()
    c.quantize_prefill(k, v, cu)
    e[1].record()
    for i in range(steps):
        c.append_decode(kn[i], vn[i], lens[i], qs[i], max_len + steps, out=out, workspace=ws)
    e[2].record()
    torch.cuda.synchronize()
    q_ms = e[0].elapsed_time(e[1])
    d_ms = e[1].elapsed_time(e[2]) / steps
    th = wl.total_tokens * wl.hkv
    qbytes = quantize_bytes(th, wl.bits_k, wl.tile_tokens) + quantize_bytes(th, wl.bits_v, wl.tile_tokens)
    mid = [l + steps // 2 for l in wl.seq_lens]
    dbytes = decode_bytes(wl, mid)
    del caches, k, v, kn, vn, qs
    torch.cuda.empty_cache()
    return {"workload": wl.name, "num_seqs": wl.num_seqs, "context": max_len, "kv_heads": wl.hkv, "q_heads": wl.hq,
            "tile_tokens": wl.tile_tokens, "decode_steps": steps,
            "quantize_prefill_ms": round(q_ms, 4), "quantize_GBps": round(qbytes / (q_ms * 1e-3) / 1e9, 1),
            "decode_step_ms": round(d_ms, 4),
            "decode_tok_per_s": round(wl.num_seqs / (d_ms * 1e-3), 1),
            "decode_slot_GBps": round(dbytes / (d_ms * 1e-3) / 1e9, 1),
            "decode_hbm_frac": round(dbytes / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": "decode step = fused append + re-quantize of the partial tile + attention + merge; "
                    "slot bytes at the middle step's lengths"}


def mixed_leg(n_iter: int = 10):
    """The mixed-precision stress workload: 64 sequences of 1K-32K tokens
    (seeded lengths), 8 kv / 64 query heads, heavy-tailed K (Student-t(3) times
    log-uniform channel scales), tile 32, 4-bit K / 2-bit V, 5 iterations:
    quantize the prefill, then one fused append + decode step.  Inputs drawn on
    the device."""
    import torch
    from kv_cache_quantization_tiles_amd import api

    wl = inputs.workload(5)
    dev = torch.device("cuda:0")
    table, npages = inputs.block_table(wl)
    max_len = max(wl.seq_lens)
    cu = torch.from_numpy(wl.cu_seqlens()).to(dev)
    k = inputs.gen_kv_device(wl, "K", device=dev)
    v = inputs.gen_kv_device(wl, "V", device=dev)
    cfg = api.config(wl.tile_tokens, wl.bits_k, wl.bits_v, wl.iters)
    caches = [api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs) for _ in range(2)]
    kn = torch.from_numpy(inputs.gen_decode_kv(wl, "K", 0)).to(dev)
    vn = torch.from_numpy(inputs.gen_decode_kv(wl, "V", 0)).to(dev)
    q = torch.from_numpy(inputs.gen_q(wl)).to(dev)
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    out = torch.empty((wl.num_seqs, wl.hq, D), dtype=torch.float32, device=dev)
    ws = caches[0].workspace(wl.hq, max_len + 1)

    def timed(fn, n):
        fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n
    q_ms = timed(lambda i: caches[i % 2].quantize_prefill(k, v, cu), 4)
    for c in caches:
        c.quantize_prefill(k, v, cu)
    # the append re-quantizes the same tile each time (lengths are not advanced)
    d_ms = timed(lambda i: caches[i % 2].append_decode(kn, vn, lens, q, max_len + 1, out=out, workspace=ws), n_iter)
    th = wl.total_tokens * wl.hkv
    qbytes = quantize_bytes(th, wl.bits_k, wl.tile_tokens) + quantize_bytes(th, wl.bits_v, wl.tile_tokens)
    dbytes = decode_bytes(wl, [l + 1 for l in wl.seq_lens])
    del caches, k, v
    torch.cuda.empty_cache()
    return {"workload": wl.name, "num_seqs": wl.num_seqs, "tokens": wl.total_tokens, "kv_heads": wl.hkv,
            "q_heads": wl.hq, "tile_tokens": wl.tile_tokens, "bits_k": wl.bits_k, "bits_v": wl.bits_v,
            "iters": wl.iters,
            "quantize_prefill_ms": round(q_ms, 4), "quantize_GBps": round(qbytes / (q_ms * 1e-3) / 1e9, 1),
            "quantize_hbm_frac": round(qbytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "decode_step_ms": round(d_ms, 4), "decode_tok_per_s": round(wl.num_seqs / (d_ms * 1e-3), 1),
            "decode_slot_GBps": round(dbytes / (d_ms * 1e-3) / 1e9, 1),
            "decode_hbm_frac": round(dbytes / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def context_sweep(contexts=(1024, 4096, 16384, 65536, 131072), num_seqs=6, n_iter=10):
    """Decode-attention time against context length for one layer of the
    Qwen3-4B-shaped long-context workload (8 kv / 32 query heads, tile 128):
    fp16 and fp8 pages, and 4-, 2- and 8-bit quantized pages filled from the
    same inputs.  One JSON line per context."""
    import dataclasses
    import torch
    from kv_cache_quantization_tiles_amd import api

    dev = torch.device("cuda:0")
    out_lines = []
    for ctx in contexts:
        wl = dataclasses.replace(inputs.workload(4), seq_lens=(ctx,) * num_seqs, layers=1)
        table, npages = inputs.block_table(wl, capacity_tokens=ctx)
        lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev)
        cu = torch.from_numpy(wl.cu_seqlens()).to(dev)
        q = torch.from_numpy(inputs.gen_q(wl)).to(dev)
        out = torch.empty((wl.num_seqs, wl.hq, D), dtype=torch.float32, device=dev)
        k = inputs.gen_kv_device(wl, "K", device=dev)
        v = inputs.gen_kv_device(wl, "V", device=dev)
        copies = max(2, int(math.ceil(1.0e9 / (wl.total_tokens * wl.hkv * 512))))   # >= 1 GB of fp16 pools
        rec = {"context": ctx, "num_seqs": num_seqs, "modes": {}}
        for name in ("fp16", "fp8", "kvq4", "kvq2", "kvq8"):
            if name in ("fp16", "fp8"):
                fp8 = name == "fp8"
                ks = float(k.abs().max()) / 448.0 if fp8 else 1.0
                vs = float(v.abs().max()) / 448.0 if fp8 else 1.0
                caches = [api.BaselineCache(npages, wl.hkv, torch.from_numpy(table), wl.num_seqs, fp8, ks, vs)
                          for _ in range(copies)]
                for c in caches:
                    c.fill(k, v, cu, ctx)
                per_tok = 2 * 128 * (1 if fp8 else 2)
            else:
                bits = int(name[3:])
                cfg = api.config(wl.tile_tokens, bits, bits, wl.iters)
                caches = [api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
                          for _ in range(copies)]
                for c in caches:
                    c.quantize_prefill(k, v, cu)
                per_tok = 2 * slot_bytes_per_token(bits, wl.tile_tokens)
            ws = caches[0].workspace(wl.hq, ctx)
            for i in range(2):
                caches[i % copies].decode(q, lens, ctx, out=out, workspace=ws)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(n_iter):
                caches[i % copies].decode(q, lens, ctx, out=out, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / n_iter
            byts = wl.total_tokens * wl.hkv * per_tok
            rec["modes"][name] = {"decode_attn_us": round(ms * 1e3, 2),
                                  "GBps": round(byts / (ms * 1e-3) / 1e9, 1),
                                  "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
            del caches, ws
            torch.cuda.empty_cache()
        base = rec["modes"]["fp16"]["decode_attn_us"]
        for m in rec["modes"].values():
            m["speedup_vs_fp16"] = round(base / m["decode_attn_us"], 3)
        del k, v
        torch.cuda.empty_cache()
        print(json.dumps(rec), flush=True)
        out_lines.append(rec)
    return out_lines


# ----------------------------------------------------------------------------- GPU leg
def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--cpu-seqs", type=int, default=4, help="sequences in the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the fp16 / fp8 / 4-bit / 2-bit comparison at 6 x 128K, the 32 x 16K burst and the mixed-length leg")
    ap.add_argument("--sweep", action="store_true",
                    help="print decode-attention time against context length (fp16, fp8, 4-, 2-, 8-bit pages) "
                         "instead of the bench line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (each GPU would run "
              "this path on its own share of sequences and kv heads, with no communication)", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        import torch
        torch.cuda.set_device(0)
        context_sweep()
        return
    wl = inputs.workload(args.workload)
    if wl.layers != 1:
        raise SystemExit("multi-layer workloads are not bench lines")

    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, args.cpu_seqs)  # before any GPU call
    cpu_legs = None if (args.no_cpu_baseline or args.no_long_context) else cpu_baseline_legs()

    import torch
    from kv_cache_quantization_tiles_amd import api

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = api.config(wl.tile_tokens, wl.bits_k, wl.bits_v, wl.iters)
    table, npages = inputs.block_table(wl)
    k_np, v_np = inputs.gen_kv(wl, "K"), inputs.gen_kv(wl, "V")
    n_in = 2   # input copies, alternated so that inputs stream from HBM
    ks = [torch.from_numpy(k_np).to(dev) for _ in range(n_in)]
    vs = [torch.from_numpy(v_np).to(dev) for _ in range(n_in)]
    del k_np, v_np
    cu = torch.from_numpy(wl.cu_seqlens()).to(dev)
    max_len = max(wl.seq_lens)
    pool_bytes = (npages * wl.hkv * (api.kvq_slot_bytes(cfg, False) + api.kvq_slot_bytes(cfg, True)))
    n_pools = max(3, int(math.ceil(1.0e9 / pool_bytes)))   # >= 1 GB of pools between reuses
    caches = [api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs) for _ in range(n_pools)]
    lens_before = torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    lens_after = lens_before + 1
    kn = torch.from_numpy(inputs.gen_decode_kv(wl, "K", 0)).to(dev)
    vn = torch.from_numpy(inputs.gen_decode_kv(wl, "V", 0)).to(dev)
    q = torch.from_numpy(inputs.gen_q(wl)).to(dev)
    out = torch.empty((wl.num_seqs, wl.hq, D), dtype=torch.float32, device=dev)
    ws = caches[0].workspace(wl.hq, max_len + 1)

    def step(i, ev=None):
        c = caches[i % n_pools]
        if ev is not None:
            ev[0].record()
        c.quantize_prefill(ks[i % n_in], vs[i % n_in], cu)
        if ev is not None:
            ev[1].record()
        c.append_decode(kn, vn, lens_before, q, max_len + 1, out=out, workspace=ws)
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the timed steps carry no events: a timing event between launches leaves
    # the GPU idle (each step would take ~9x its kernel time)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step_eager = wall * 1e3 / args.steps
    # The same K steps recorded into one HIP graph (the launches of a serving
    # loop's step, replayed without per-launch host work; the graph runs the
    # identical kernels on the identical rotation of inputs and pools, and its
    # replays are bit-identical to eager calls: tests/test_gpu_graph.py).
    # Untimed: the capture's side-stream warm-up, the capture and one replay.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(min(args.steps, n_pools)):
            step(args.warmup + i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            step(args.warmup + i)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    del graph
    # per-phase split of the same step, in a separate untimed-for-value loop
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    tq = [e[0].elapsed_time(e[1]) for e in evs]
    tad = [e[1].elapsed_time(e[2]) for e in evs]

    # the same decode step as two calls (append, then decode), for comparison
    n_split = max(20, args.steps)
    sp_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_split)]
    for j in range(n_split):
        c = caches[j % n_pools]
        sp_ev[j][0].record()
        c.append(kn, vn, lens_before)
        sp_ev[j][1].record()
        c.decode(q, lens_after, max_len + 1, out=out, workspace=ws)
        sp_ev[j][2].record()

    # kernels alone, back to back between two events (inputs and pools rotated,
    # so every launch streams from HBM): average launch durations
    def batch_ms(fn, n):
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        for j in range(n):
            fn(j)
        b1.record()
        return b0, b1, n
    n_q = max(20, args.steps)
    q_batch = batch_ms(lambda j: caches[j % n_pools].quantize_prefill(ks[j % n_in], vs[j % n_in], cu), n_q)
    d_batch = batch_ms(lambda j: caches[j % n_pools].decode(q, lens_after, max_len + 1, out=out, workspace=ws), n_q)
    # the fused decode step alone (append + re-quantize + attend, then the merge), back to back
    ad_batch = batch_ms(lambda j: caches[j % n_pools].append_decode(kn, vn, lens_before, q, max_len + 1, out=out,
                                                                    workspace=ws), n_q)
    # the same plain decode at a short context (same batch, heads, tile and
    # widths): the difference to the full-context decode splits the decode's
    # time into a fixed part (launches, the dependent loads before the first
    # chunk, the partition merge) and the streaming of the pages
    short_ctx = 1024
    wl_s = dataclasses.replace(wl, seq_lens=(short_ctx,) * wl.num_seqs)
    table_s, npages_s = inputs.block_table(wl_s)
    cu_s = torch.from_numpy(wl_s.cu_seqlens()).to(dev)
    k_s, v_s = inputs.gen_kv_device(wl_s, "K", device=dev), inputs.gen_kv_device(wl_s, "V", device=dev)
    caches_short = [api.PagedCache(cfg, npages_s, wl.hkv, torch.from_numpy(table_s), wl.num_seqs)
                    for _ in range(n_pools)]
    for c in caches_short:
        c.quantize_prefill(k_s, v_s, cu_s)
    lens_s = torch.full((wl.num_seqs,), short_ctx, dtype=torch.int32, device=dev)
    ws_s = caches_short[0].workspace(wl.hq, short_ctx)
    caches_short[0].decode(q, lens_s, short_ctx, out=out, workspace=ws_s)
    ds_short_batch = batch_ms(lambda j: caches_short[j % n_pools].decode(q, lens_s, short_ctx, out=out,
                                                                       workspace=ws_s), n_q)
    torch.cuda.synchronize()
    del caches_short, k_s, v_s
    # bandwidth probe: plain copy of 1 GiB
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    api._lib.kvq_bandwidth_probe(src, dst, nb)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        api._lib.kvq_bandwidth_probe(src, dst, nb)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * nb * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # the randomized rotation (a seeded +-1 diagonal before H): same kernels, signs on
    cfg_s = api.config(wl.tile_tokens, wl.bits_k, wl.bits_v, wl.iters, hadamard_signs=inputs.hadamard_signs(1))
    caches_s = [api.PagedCache(cfg_s, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs) for _ in range(n_pools)]
    qs_batch = batch_ms(lambda j: caches_s[j % n_pools].quantize_prefill(ks[j % n_in], vs[j % n_in], cu), n_q)
    ds_batch = batch_ms(lambda j: caches_s[j % n_pools].decode(q, lens_after, max_len + 1, out=out, workspace=ws), n_q)
    torch.cuda.synchronize()
    del caches_s
    # 8-bit codes for K and V: same kernels at the wider width
    cfg_8 = api.config(wl.tile_tokens, 8, 8, wl.iters)
    caches_8 = [api.PagedCache(cfg_8, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs) for _ in range(n_pools)]
    q8_batch = batch_ms(lambda j: caches_8[j % n_pools].quantize_prefill(ks[j % n_in], vs[j % n_in], cu), n_q)
    d8_batch = batch_ms(lambda j: caches_8[j % n_pools].decode(q, lens_after, max_len + 1, out=out, workspace=ws), n_q)
    torch.cuda.synchronize()
    q8_ms = q8_batch[0].elapsed_time(q8_batch[1]) / q8_batch[2]
    d8_ms = d8_batch[0].elapsed_time(d8_batch[1]) / d8_batch[2]
    del caches_8
    # fp16 metadata slots (same codes; S, O and the channel factors in fp16)
    cfg_h = api.config(wl.tile_tokens, wl.bits_k, wl.bits_v, wl.iters, meta_fp16=True)
    caches_h = [api.PagedCache(cfg_h, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs) for _ in range(n_pools)]
    qh_batch = batch_ms(lambda j: caches_h[j % n_pools].quantize_prefill(ks[j % n_in], vs[j % n_in], cu), n_q)
    dh_batch = batch_ms(lambda j: caches_h[j % n_pools].decode(q, lens_after, max_len + 1, out=out, workspace=ws), n_q)
    adh_batch = batch_ms(lambda j: caches_h[j % n_pools].append_decode(kn, vn, lens_before, q, max_len + 1, out=out,
                                                                      workspace=ws), n_q)
    torch.cuda.synchronize()
    qh_ms = qh_batch[0].elapsed_time(qh_batch[1]) / qh_batch[2]
    dh_ms = dh_batch[0].elapsed_time(dh_batch[1]) / dh_batch[2]
    adh_ms = adh_batch[0].elapsed_time(adh_batch[1]) / adh_batch[2]
    del caches_h
    # K rounded per channel (V per token as before)
    cfg_c = api.config(wl.tile_tokens, wl.bits_k, wl.bits_v, wl.iters, k_per_channel=True)
    caches_c = [api.PagedCache(cfg_c, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs) for _ in range(n_pools)]
    qc_batch = batch_ms(lambda j: caches_c[j % n_pools].quantize_prefill(ks[j % n_in], vs[j % n_in], cu), n_q)
    dc_batch = batch_ms(lambda j: caches_c[j % n_pools].decode(q, lens_after, max_len + 1, out=out, workspace=ws), n_q)
    adc_batch = batch_ms(lambda j: caches_c[j % n_pools].append_decode(kn, vn, lens_before, q, max_len + 1, out=out,
                                                                      workspace=ws), n_q)
    torch.cuda.synchronize()
    qc_ms = qc_batch[0].elapsed_time(qc_batch[1]) / qc_batch[2]
    dc_ms = dc_batch[0].elapsed_time(dc_batch[1]) / dc_batch[2]
    adc_ms = adc_batch[0].elapsed_time(adc_batch[1]) / adc_batch[2]
    # restore error of K (relative RMS over the layer, fp16 restore through the
    # re-materialize path) for per-token and per-channel K pages
    k_err = {}
    for tag, cc in (("per_token", caches[0]), ("per_channel", caches_c[0])):
        cc.quantize_prefill(ks[0], vs[0], cu)
        b16 = api.BaselineCache(npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
        cc.rematerialize_into(b16, lens_before, max_len)
        tab = torch.from_numpy(table).to(dev).long()
        tok = torch.arange(max_len, device=dev)
        pages = tab[:, tok // 16]                                   # [S, L]
        kr = b16.pool_k.view(npages, wl.hkv, 16, D)[pages, :, tok % 16]   # [S, L, Hkv, D]
        kref = ks[0].view(wl.num_seqs, max_len, wl.hkv, D).float()
        k_err[tag] = round(float(((kr.float() - kref) ** 2).mean().sqrt() / (kref ** 2).mean().sqrt()), 5)
        del b16
    del caches_c
    # several queries per sequence (a speculative verify of 4 and of 16 draft
    # tokens) over the same pages: tokens past the appended one are stale
    # pool bytes (timing only; parity is in the tests)
    mq = {}
    for n_mq in (4, 16):
        qm = torch.from_numpy(inputs.gen_q_multi(wl, n_mq)).to(dev)
        sl = lens_before + n_mq
        mo = torch.empty((wl.num_seqs, n_mq, wl.hq, D), dtype=torch.float32, device=dev)
        nb = api.kvq_multi_query_workspace_bytes(cfg, wl.num_seqs, n_mq, wl.hq, wl.hkv, max_len + n_mq)
        mw = torch.empty(nb, dtype=torch.uint8, device=dev)
        caches[0].multi_query(qm, sl, max_len + n_mq, out=mo, workspace=mw)
        mb = batch_ms(lambda j: caches[j % n_pools].multi_query(qm, sl, max_len + n_mq, out=mo, workspace=mw), n_q)
        torch.cuda.synchronize()
        mq_ms = mb[0].elapsed_time(mb[1]) / mb[2]
        mq_bytes = decode_bytes(wl, [l + n_mq for l in wl.seq_lens])
        mq[f"n_q_{n_mq}"] = {"attn_ms": round(mq_ms, 4), "GBps": round(mq_bytes / (mq_ms * 1e-3) / 1e9, 1),
                             "hbm_frac": round(mq_bytes / (mq_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                             "query_tokens_per_s": round(wl.num_seqs * n_mq / (mq_ms * 1e-3), 1)}
        del mw
    # the dense entry points (one token run [n, H, 128], codes and scale vectors
    # in their own arrays) on the same rows: quantize, then restore to fp16
    n_tok = wl.total_tokens
    dq = [dict(codes=torch.empty((n_tok, wl.hkv, D * wl.bits_k // 8), dtype=torch.uint8, device=dev),
               alpha=torch.empty(((n_tok + wl.tile_tokens - 1) // wl.tile_tokens, wl.hkv, D), dtype=torch.float32,
                                 device=dev),
               scale=torch.empty((n_tok, wl.hkv), dtype=torch.float32, device=dev),
               offset=torch.empty((n_tok, wl.hkv), dtype=torch.float32, device=dev)) for _ in range(n_in)]
    restored = [torch.empty_like(ks[0]) for _ in range(n_in)]

    def dense_q(j):
        o = dq[j % n_in]
        api.kvq_quantize_tiles(cfg, ks[j % n_in], n_tok, wl.hkv, wl.bits_k, o["codes"], o["alpha"], o["scale"],
                               o["offset"])

    def dense_dq(j):
        o = dq[j % n_in]
        api.kvq_dequantize(cfg, o["codes"], o["alpha"], o["scale"], o["offset"], n_tok, wl.hkv, wl.bits_k,
                           restored[j % n_in])
    dense_q(0)
    dense_q(1)
    dqz_batch = batch_ms(dense_q, n_q)
    ddq_batch = batch_ms(dense_dq, n_q)
    torch.cuda.synchronize()
    dqz_ms = dqz_batch[0].elapsed_time(dqz_batch[1]) / dqz_batch[2]
    ddq_ms = ddq_batch[0].elapsed_time(ddq_batch[1]) / ddq_batch[2]
    th_k = n_tok * wl.hkv
    stored = th_k * (D * wl.bits_k / 8 + 8 + 4 * D / wl.tile_tokens)   # codes, scale, offset, alpha share
    dq_bytes = stored + th_k * 2 * D                                   # ... read, fp16 rows written
    dense = {"quantize_ms": round(dqz_ms, 4),
             "quantize_GBps": round(quantize_bytes(th_k, wl.bits_k, wl.tile_tokens) / (dqz_ms * 1e-3) / 1e9, 1),
             "dequantize_ms": round(ddq_ms, 4),
             "dequantize_GBps": round(dq_bytes / (ddq_ms * 1e-3) / 1e9, 1),
             "dequantize_hbm_frac": round(dq_bytes / (ddq_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
             "note": f"K only, one token run of {n_tok} tokens x {wl.hkv} heads, {wl.bits_k}-bit"}
    del dq, restored
    q_kernel_ms = q_batch[0].elapsed_time(q_batch[1]) / q_batch[2]
    td_cold = d_batch[0].elapsed_time(d_batch[1]) / d_batch[2]
    td_short = ds_short_batch[0].elapsed_time(ds_short_batch[1]) / ds_short_batch[2]
    ad_kernel_ms = ad_batch[0].elapsed_time(ad_batch[1]) / ad_batch[2]
    qs_ms = qs_batch[0].elapsed_time(qs_batch[1]) / qs_batch[2]
    ds_ms = ds_batch[0].elapsed_time(ds_batch[1]) / ds_batch[2]
    ta = [e[0].elapsed_time(e[1]) for e in sp_ev]
    td = [e[1].elapsed_time(e[2]) for e in sp_ev]

    ntok_heads = wl.total_tokens * wl.hkv
    qbytes = quantize_bytes(ntok_heads, wl.bits_k, wl.tile_tokens) + quantize_bytes(ntok_heads, wl.bits_v, wl.tile_tokens)
    abytes = append_bytes(wl, wl.seq_lens)
    q8_bytes = 2 * quantize_bytes(ntok_heads, 8, wl.tile_tokens)
    d8_bytes = decode_bytes(dataclasses.replace(wl, bits_k=8, bits_v=8), [l + 1 for l in wl.seq_lens])
    dbytes = decode_bytes(wl, [l + 1 for l in wl.seq_lens])
    q_ms, ad_ms = float(np.mean(tq)), float(np.mean(tad))
    a_ms, d_ms = float(np.mean(ta)), float(np.mean(td))
    q_gbps = qbytes / (q_kernel_ms * 1e-3) / 1e9
    n_elem = 2 * ntok_heads * D
    q_tops = n_elem * quantize_valu_ops_per_element(wl.iters) / (q_kernel_ms * 1e-3) / 1e12
    d_gbps_cold = dbytes / (td_cold * 1e-3) / 1e9
    dbytes_short = decode_bytes(wl_s, wl_s.seq_lens)
    d_marginal_gbps = (dbytes - dbytes_short) / max((td_cold - td_short) * 1e-3, 1e-9) / 1e9
    d_fixed_us = (td_short * 1e-3 - dbytes_short / (d_marginal_gbps * 1e9)) * 1e6
    value = (qbytes + abytes + dbytes) / (ms_step * 1e-3) / 1e9
    rec = {
        "metric": "quantize GB/s + quantized decode-attn tokens/s at 16K; % of HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_timing": "the K steps replayed from one HIP graph (ms_per_step_eager: the same K steps "
                       "launched one call at a time)",
        "ms_per_step_eager": round(ms_step_eager, 4),
        "value_eager": round((qbytes + abytes + dbytes) / (ms_step_eager * 1e-3) / 1e9, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "num_seqs": wl.num_seqs, "context": max_len, "kv_heads": wl.hkv,
                   "q_heads": wl.hq, "head_dim": D, "page_tokens": 16, "tile_tokens": wl.tile_tokens,
                   "bits_k": wl.bits_k, "bits_v": wl.bits_v, "sinkhorn_iters": wl.iters},
        "quantize_ms": round(q_ms, 4), "quantize_kernel_ms": round(q_kernel_ms, 4),
        "quantize_GBps": round(q_gbps, 1),
        "quantize_hbm_frac": round(q_gbps / HBM_PEAK_GBPS, 4),
        "append_decode_ms": round(ad_ms, 4),
        "split_append_ms": round(a_ms, 4), "split_decode_attn_ms": round(d_ms, 4),
        "decode_attn_cold_ms": round(td_cold, 4),
        "decode_attn_GBps_cold": round(d_gbps_cold, 1),
        "decode_hbm_frac_cold": round(d_gbps_cold / HBM_PEAK_GBPS, 4),
        "decode_tok_per_s": round(wl.num_seqs / (ad_kernel_ms * 1e-3), 1),
        "decode_step_ms": round(ad_kernel_ms, 4),
        "decode_attn_only_tok_per_s": round(wl.num_seqs / (td_cold * 1e-3), 1),
        "copy_probe_GBps": round(copy_gbps, 1),
        "multi_query_verify": mq,
        "dense_entry_points": dense,
        "randomized_rotation": {"quantize_kernel_ms": round(qs_ms, 4), "decode_attn_ms": round(ds_ms, 4),
                                "quantize_GBps": round(qbytes / (qs_ms * 1e-3) / 1e9, 1)},
        "meta_fp16": {"bytes_per_token_head_k": slot_bytes_per_token(wl.bits_k, wl.tile_tokens, True),
                      "bytes_per_token_head_k_fp32_meta": slot_bytes_per_token(wl.bits_k, wl.tile_tokens),
                      "quantize_kernel_ms": round(qh_ms, 4), "decode_attn_ms": round(dh_ms, 4),
                      "decode_step_ms": round(adh_ms, 4),
                      "quantize_GBps": round(2 * quantize_bytes(ntok_heads, wl.bits_k, wl.tile_tokens, True)
                                             / (qh_ms * 1e-3) / 1e9, 1),
                      "decode_attn_GBps": round(decode_bytes(wl, [l + 1 for l in wl.seq_lens], True)
                                                / (dh_ms * 1e-3) / 1e9, 1)},
        "k_per_channel": {"bytes_per_token_head_k": slot_bytes_per_token(wl.bits_k, wl.tile_tokens, kchan=True),
                          "quantize_kernel_ms": round(qc_ms, 4), "decode_attn_ms": round(dc_ms, 4),
                          "decode_step_ms": round(adc_ms, 4),
                          "k_restore_rel_rms": k_err,
                          "note": "K restore error over the layer (relative RMS of the fp16 restore against the "
                                  "input K): per-token against per-channel rounding of K"},
        "codes_8bit": {"quantize_kernel_ms": round(q8_ms, 4), "decode_attn_ms": round(d8_ms, 4),
                       "quantize_GBps": round(q8_bytes / (q8_ms * 1e-3) / 1e9, 1),
                       "decode_attn_GBps": round(d8_bytes / (d8_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "kernel": f"quantize_paged_kernel<{wl.tile_tokens},{wl.bits_k},{wl.bits_v},false,false>",
                     "achieved": round(q_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(q_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(QUANTIZE_SOURCES, f"traffic-quantize_paged_kernel-{wl.name}.json"),
                     "algorithmic_bytes_per_launch": int(qbytes), "launch_us": round(q_kernel_ms * 1e3, 2),
                     "timing": "HIP events on the launch stream around a back-to-back batch of quantize calls "
                               "(inputs and pools rotated over >= 1 GB); a call is the bulk kernel plus the "
                               "short-tile pass (sequences' last tiles of fewer than 16 tokens, none here)",
                     "valu_ceiling": {"ops_per_element": quantize_valu_ops_per_element(wl.iters),
                                      "achieved_Tlane_ops": round(q_tops, 3),
                                      "peak_Tlane_ops": round(VALU_PEAK_TOPS, 3),
                                      "frac": round(q_tops / VALU_PEAK_TOPS, 4)}},
        "roofline_decode": {"bound": "hbm", "kernel": f"decode_kernel<{wl.tile_tokens},{wl.bits_k},{wl.bits_v}> "
                                                      "fused with the append, + combine_kernel",
                            "achieved": round((dbytes + abytes) / (ad_kernel_ms * 1e-3) / 1e9, 1),
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round((dbytes + abytes) / (ad_kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                            "algorithmic_bytes_per_launch": int(dbytes + abytes),
                            "launch_us": round(ad_kernel_ms * 1e3, 2),
                            "timing": "HIP events around a back-to-back batch of fused decode steps "
                                      "(pools rotated); slot bytes of every cached token read plus the "
                                      "re-quantized tile's staging rows and slots",
                            "fixed_and_streaming": {
                                "short_context": short_ctx, "short_decode_us": round(td_short * 1e3, 2),
                                "full_decode_us": round(td_cold * 1e3, 2),
                                "marginal_GBps": round(d_marginal_gbps, 1),
                                "marginal_frac": round(d_marginal_gbps / HBM_PEAK_GBPS, 4),
                                "fixed_us": round(d_fixed_us, 2),
                                "note": "plain decode (decode kernel + partition merge) at the full and at a "
                                        "1024-token context, same batch and heads: the slot bytes the longer "
                                        "context adds over the time it adds (marginal), and the time left at "
                                        "zero bytes (fixed)"}},
        "cpu_baseline": cpu,
    }
    del caches, ks, vs, src, dst
    torch.cuda.empty_cache()
    rec["cpu_baseline_legs"] = cpu_legs
    rec["latency_1x1024"] = latency_leg()
    rec["long_context"] = None if args.no_long_context else long_context_leg()
    rec["long_context_decode_phase"] = None if args.no_long_context else long_context_decode_phase()
    rec["rematerialize_16k"] = None if args.no_long_context else [rematerialize_leg(2), rematerialize_leg(3)]
    rec["burst_32x16k"] = None if args.no_long_context else burst_leg()
    rec["mixed_64seq"] = None if args.no_long_context else mixed_leg()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
