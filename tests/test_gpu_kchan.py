"""GPU parity for K pages rounded per channel (kvq_config.k_per_channel = 1):
the prefill, appends across tile boundaries (the float64 short tiles
included), the fused append + decode step (equal to the two calls bit for
bit), decode and multi-query attention and the restore into fp16 pages, each
against the oracle's per-channel K format (codes within the rounding window;
beta within 1e-4; the channel scales and zero offsets through their effect on
the restored values; attention and restores within the usual bars on the
GPU's own pages)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as orc
from kv_cache_quantization_tiles_amd import api, inputs
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

CASES = [
    # (recipe, lens, hkv, hq, tile, bits_k, bits_v, iters)
    (2, (200, 131, 64, 17), 2, 8, 64, 4, 4, 3),
    (5, (300, 97, 33), 2, 16, 32, 4, 2, 5),
    (2, (260, 128, 7), 1, 4, 128, 2, 2, 3),
    (2, (96, 40), 2, 8, 32, 2, 4, 3),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api._lib.load()


def _wl(case, decode_steps=4):
    recipe, lens, hkv, hq, tile, bk, bv, iters = case
    return dataclasses.replace(inputs.workload(recipe), seq_lens=tuple(lens), hkv=hkv, hq=hq, tile_tokens=tile,
                               bits_k=bk, bits_v=bv, iters=iters, decode_steps=decode_steps)


def _prefill(wl):
    k, v = inputs.gen_kv(wl, "K"), inputs.gen_kv(wl, "V")
    table, npages = inputs.block_table(wl)
    cfg = api.config(wl.tile_tokens, wl.bits_k, wl.bits_v, wl.iters, k_per_channel=True)
    cache = api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
    cache.quantize_prefill(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                           torch.from_numpy(wl.cu_seqlens()).cuda())
    torch.cuda.synchronize()
    return k, v, table, npages, cache


def _check_tiles(wl, table, seq, n, rows_of, gpk, gpv, what, tiles=None):
    """Codes and metadata of the tiles of one sequence against the oracle's
    tiles of the fp16 rows rows_of(role, head)."""
    t = wl.tile_tokens
    tot = [0, 0, 0]
    for h in range(wl.hkv):
        _, kc, ka, kb, km = orc.read_sequence(gpk, table[seq], n, h, "K", wl.bits_k, t, kchan=True)
        _, vc, va, vs, vo = orc.read_sequence(gpv, table[seq], n, h, "V", wl.bits_v, t)
        for j in (range((n + t - 1) // t) if tiles is None else tiles):
            sl = slice(j * t, min(n, (j + 1) * t))
            tk = orc.quantize_tile(rows_of("K", h)[sl], wl.bits_k, wl.iters, kchan=True)
            c = pu.compare_codes(kc[sl], tk.codes, tk.pre, f"{what} s{seq} h{h} K tile{j}")
            tot = [a + b for a, b in zip(tot, c)]
            pu.check_tile_metadata_kchan(tk, ka[j], kb[sl], km[j], f"{what} s{seq} h{h} K tile{j}")
            tv = orc.quantize_tile(rows_of("V", h)[sl], wl.bits_v, wl.iters)
            c = pu.compare_codes(vc[sl], tv.codes, tv.pre, f"{what} s{seq} h{h} V tile{j}")
            tot = [a + b for a, b in zip(tot, c)]
            pu.check_tile_metadata(tv.codes, va[j], vs[sl], vo[sl], tv.alpha, tv.scale, tv.offset,
                                   orc.dequantize_tile, f"{what} s{seq} h{h} V tile{j}")
    return tot


@pytest.mark.parametrize("case", CASES)
def test_kchan_prefill_decode_and_multi_query(case):
    wl = _wl(case)
    k, v, table, npages, cache = _prefill(wl)
    assert cache.slot_k == orc.slot_bytes(wl.bits_k, wl.tile_tokens, kchan=True)
    assert cache.slot_v == orc.slot_bytes(wl.bits_v, wl.tile_tokens)
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    cu = wl.cu_seqlens()
    tot = [0, 0, 0]
    for s in range(wl.num_seqs):
        src = {"K": k[cu[s]:cu[s + 1]], "V": v[cu[s]:cu[s + 1]]}
        c = _check_tiles(wl, table, s, wl.seq_lens[s], lambda role, h: src[role][:, h], gpk, gpv, "kchan prefill")
        tot = [a + b for a, b in zip(tot, c)]
    print(f"[codes] kchan prefill {case}: {tot[0]} elements, {tot[1]} in window, {tot[2]} mismatches", flush=True)
    seq_lens = np.array(wl.seq_lens, np.int32)
    q = inputs.gen_q(wl)
    out = cache.decode(torch.from_numpy(q).cuda(), torch.from_numpy(seq_lens).cuda(), max(wl.seq_lens)).cpu().numpy()
    ref, sc = orc.paged_decode_attn(q, table, seq_lens, gpk, gpv, wl.tile_tokens, wl.bits_k, wl.bits_v,
                                    return_scale=True, kchan=True)
    err = pu.assert_attn(out, ref, f"kchan decode {case}", sc)
    errs = []
    for n_q in (2, 5):   # (query, head) rows below and above 16: both multi-query kernels
        qm = inputs.gen_q_multi(wl, n_q)
        outm = cache.multi_query(torch.from_numpy(qm).cuda(), torch.from_numpy(seq_lens).cuda(),
                                 max(wl.seq_lens)).cpu().numpy()
        refm, scm = orc.paged_multi_query_attn(qm, table, seq_lens, gpk, gpv, wl.tile_tokens, wl.bits_k,
                                               wl.bits_v, return_scale=True, kchan=True)
        errs.append(pu.assert_attn(outm, refm, f"kchan multi-query n_q={n_q} {case}", scm))
    print(f"[attn] kchan {case}: decode {err:.2e}, multi-query {errs[0]:.2e} / {errs[1]:.2e}", flush=True)


def _steps(case):
    return case[4] + 3   # one tile plus a few: every sequence crosses a tile boundary


@pytest.mark.parametrize("case", CASES[:3])
def test_kchan_fused_steps_and_restore(case):
    steps = _steps(case)
    wl = _wl(case, decode_steps=steps)
    k, v, table, npages, cache = _prefill(wl)
    t = wl.tile_tokens
    lens = np.array(wl.seq_lens, np.int32)
    max_len = max(wl.seq_lens) + steps
    ws = cache.workspace(wl.hq, max_len)
    cu = wl.cu_seqlens()
    rows = {(s, r): list((k if r == "K" else v)[cu[s]:cu[s + 1]]) for s in range(wl.num_seqs) for r in "KV"}
    for step in range(steps):
        kn, vn = inputs.gen_decode_kv(wl, "K", step), inputs.gen_decode_kv(wl, "V", step)
        q = inputs.gen_q(wl, step)
        out = cache.append_decode(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(),
                                  torch.from_numpy(lens).cuda(), torch.from_numpy(q).cuda(), max_len,
                                  workspace=ws).cpu().numpy()
        for s in range(wl.num_seqs):
            rows[(s, "K")].append(kn[s])
            rows[(s, "V")].append(vn[s])
        lens = lens + 1
        if step in (0, 1, t // 2, steps - 1):
            gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
            for s in range(wl.num_seqs):
                n = int(lens[s])
                xs = {r: np.stack(rows[(s, r)]) for r in "KV"}
                _check_tiles(wl, table, s, n, lambda role, h: xs[role][:, h], gpk, gpv, f"kchan step{step}",
                             tiles=[(n - 1) // t])
            ref, sc = orc.paged_decode_attn(q, table, lens, gpk, gpv, t, wl.bits_k, wl.bits_v, return_scale=True,
                                            kchan=True)
            pu.assert_attn(out, ref, f"kchan fused step {step} {case}", sc)
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    base = api.BaselineCache(npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
    cache.rematerialize_into(base, torch.from_numpy(lens).cuda(), max_len)
    bk_got, bv_got = base.pool_k.cpu().numpy(), base.pool_v.cpu().numpy()
    ref_k, ref_v = np.zeros_like(bk_got), np.zeros_like(bv_got)
    orc.rematerialize_pages(gpk, gpv, table, lens, t, wl.bits_k, wl.bits_v, ref_k, ref_v, kchan=True)
    for s in range(wl.num_seqs):
        for h in range(wl.hkv):
            for role, gp, rp in (("K", bk_got, ref_k), ("V", bv_got, ref_v)):
                pu.assert_dequant(orc.read_baseline_sequence(gp, table[s], int(lens[s]), h, role),
                                  orc.read_baseline_sequence(rp, table[s], int(lens[s]), h, role),
                                  f"kchan restore {case} s{s} h{h} {role}")


@pytest.mark.parametrize("case", [CASES[1], CASES[3]])
def test_kchan_fused_step_equals_append_then_decode(case):
    steps = case[4] + 2
    wl = _wl(case, decode_steps=steps)
    _, _, _, _, fused = _prefill(wl)
    _, _, _, _, split = _prefill(wl)
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    max_len = max(wl.seq_lens) + steps
    ws_f, ws_s = fused.workspace(wl.hq, max_len), split.workspace(wl.hq, max_len)
    for step in range(steps):
        kn = torch.from_numpy(inputs.gen_decode_kv(wl, "K", step)).cuda()
        vn = torch.from_numpy(inputs.gen_decode_kv(wl, "V", step)).cuda()
        q = torch.from_numpy(inputs.gen_q(wl, step)).cuda()
        of = fused.append_decode(kn, vn, lens, q, max_len, workspace=ws_f)
        split.append(kn, vn, lens)
        os_ = split.decode(q, lens + 1, max_len, workspace=ws_s)
        lens = lens + 1
        torch.cuda.synchronize()
        assert torch.equal(fused.pool_k, split.pool_k), step
        assert torch.equal(fused.pool_v, split.pool_v), step
        assert torch.equal(fused.staging_k, split.staging_k), step
        assert torch.equal(of, os_), (step, (of - os_).abs().max().item())


def test_full_size_4x16k_layer_kchan_sampled():
    """The 4 x 16K, 8/32-head layer with K rounded per channel in the launch
    configuration the bench times: quantize every page, one fused append +
    decode step; random whole tiles, every appended one-token tile and three
    (sequence, kv head) attention outputs against the oracle."""
    wl = inputs.workload(2)
    k, v, table, npages, cache = _prefill(wl)
    lens = np.array(wl.seq_lens, np.int32)
    kn, vn = inputs.gen_decode_kv(wl, "K", 0), inputs.gen_decode_kv(wl, "V", 0)
    q = inputs.gen_q(wl)
    out = cache.append_decode(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), torch.from_numpy(lens).cuda(),
                              torch.from_numpy(q).cuda(), int(lens.max()) + 1)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    cu, t = wl.cu_seqlens(), wl.tile_tokens
    rng = np.random.default_rng(11)
    tot = [0, 0, 0]
    for _ in range(6):   # a sequence, then 2 whole tiles of it (every kv head, K and V)
        s = int(rng.integers(wl.num_seqs))
        tiles = sorted(int(x) for x in rng.choice(int(lens[s]) // t, 2, replace=False))
        src = {"K": k[cu[s]:cu[s + 1]], "V": v[cu[s]:cu[s + 1]]}
        c = _check_tiles(wl, table, s, int(lens[s]), lambda role, h: src[role][:, h], gpk, gpv, "kchan 4x16k",
                         tiles=tiles)
        tot = [a + b for a, b in zip(tot, c)]
    for s in range(wl.num_seqs):   # the appended token opens a tile of one row
        new = {"K": kn[s][None], "V": vn[s][None]}
        j = int(lens[s]) // t
        rows = lambda role, h, new=new, j=j: np.concatenate([np.zeros((j * t, 128), np.float16), new[role][:, h]])
        c = _check_tiles(wl, table, s, int(lens[s]) + 1, rows, gpk, gpv, "kchan 4x16k append", tiles=[j])
        tot = [a + b for a, b in zip(tot, c)]
    print(f"[codes] kchan 4x16k sampled: {tot[0]} elements, {tot[1]} in window, {tot[2]} mismatches", flush=True)
    g = wl.group
    for s, kh in ((0, 0), (3, 7), (2, 3)):
        ref, sc = orc.paged_decode_attn(q[s:s + 1, kh * g:(kh + 1) * g], table[s:s + 1], lens[s:s + 1] + 1,
                                        gpk[:, kh:kh + 1], gpv[:, kh:kh + 1], t, wl.bits_k, wl.bits_v,
                                        return_scale=True, kchan=True)
        err = pu.assert_attn(got[s, kh * g:(kh + 1) * g], ref[0], f"kchan 4x16k s{s} kv head {kh}", sc[0])
        print(f"[attn] kchan 4x16k s{s} kv head {kh}: max abs err {err:.2e}", flush=True)
    assert np.isfinite(got).all()
