"""GPU parity: the HIP path through the C-ABI against the CPU oracle, on the
same seeded inputs.  Rules in tests/parity_util.py."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle as orc
from kv_cache_quantization_tiles_amd import api, inputs
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api._lib.load()


def _report(what, counts):
    n, win, mism = counts
    print(f"[codes] {what}: {n} elements, {win} in window ({100.0 * win / max(n, 1):.3f}%), "
          f"{mism} mismatches", flush=True)


def _x(n, heads, recipe=2, role="K", seed=0):
    base = inputs.workload(recipe)
    wl = dataclasses.replace(base, seq_lens=(n,), hkv=heads, hq=heads * base.group,
                             index=base.index * 100 + seed)
    return inputs.gen_kv(wl, role)


DENSE_CASES = [
    # (tile, bits, iters, n_tokens, heads, recipe)
    (64, 4, 3, 1024, 1, 1),     # the single-head 1K correctness workload (K)
    (64, 4, 3, 1000, 2, 2),     # ragged tail, 2 heads, 2% outliers x10-50
    (32, 2, 5, 77, 3, 5),       # heavy-tailed K, 5 iterations
    (128, 4, 0, 300, 1, 2),     # no normalization
    (128, 2, 1, 129, 1, 2),     # one-row last tile
    (64, 4, 3, 1, 1, 2),        # a single token
    (32, 4, 3, 33, 2, 1),
    (64, 8, 3, 1000, 2, 2),     # 8-bit codes, ragged tail
    (32, 8, 5, 77, 3, 5),       # 8-bit, heavy-tailed K
    (128, 8, 0, 129, 1, 2),     # 8-bit, no normalization, one-row last tile
    (64, 4, 16, 200, 2, 5),     # the largest iteration count, heavy-tailed K
]


@pytest.mark.parametrize("tile,bits,iters,n,heads,recipe", DENSE_CASES)
def test_dense_quantize_and_dequantize(tile, bits, iters, n, heads, recipe):
    x = _x(n, heads, recipe)
    cfg = api.config(tile, bits, bits, iters)
    q = api.quantize_tiles(torch.from_numpy(x).cuda(), cfg, bits)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in q.items()}
    ref = orc.quantize_dense(x, tile, bits, iters)
    codes = orc.unpack_codes(got["codes"], bits)
    _report(f"dense T{tile} b{bits} it{iters} n{n} h{heads}",
            pu.compare_codes(codes, ref["codes_raw"], ref["pre"], "dense"))
    pu.assert_rel(got["alpha"], ref["alpha"], pu.META_RTOL, "alpha")
    pu.assert_rel(got["scale"], ref["scale"], pu.META_RTOL, "scale")
    pu.assert_rel(got["offset"], ref["offset"], pu.META_RTOL, "offset")
    # restore: GPU dequantize of the GPU codes vs the oracle restoring the same codes
    deq = api.dequantize(q, cfg, bits).cpu().numpy().astype(np.float64)
    ref_deq = orc.dequantize_dense(got["codes"], got["alpha"], got["scale"], got["offset"], tile, bits)
    pu.assert_dequant(deq, ref_deq, "dequantize")
    # and the round trip stays within the rounding bound of the method
    err = np.linalg.norm(deq - x.astype(np.float64), axis=-1)
    bound = got["scale"] / 2 * np.linalg.norm(got["alpha"], axis=-1)[np.arange(n) // tile]
    assert np.all(err <= bound * 1.01 + 2e-3 * np.linalg.norm(x.astype(np.float64), axis=-1))


def test_dense_quantize_is_deterministic():
    x = torch.from_numpy(_x(4096, 4, 2)).cuda()
    cfg = api.config(64, 4, 4, 3)
    a = api.quantize_tiles(x, cfg, 4)
    b = api.quantize_tiles(x, cfg, 4)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def _paged_workload(recipe, lens, hkv, hq, tile, bits_k, bits_v, iters, decode_steps=4):
    base = inputs.workload(recipe)
    return dataclasses.replace(base, seq_lens=tuple(lens), hkv=hkv, hq=hq, tile_tokens=tile,
                               bits_k=bits_k, bits_v=bits_v, iters=iters, decode_steps=decode_steps)


PAGED_CASES = [
    # (recipe, lens, hkv, hq, tile, bits_k, bits_v, iters)
    (1, (1024,), 1, 8, 64, 4, 4, 3),
    (2, (200, 131, 64, 17), 2, 8, 64, 4, 4, 3),
    (5, (300, 97, 33), 2, 16, 32, 4, 2, 5),
    (2, (260, 128), 1, 4, 128, 2, 2, 3),
    (2, (200, 131, 64, 17), 2, 8, 64, 8, 8, 3),     # 8-bit codes
    (5, (300, 97, 33), 2, 16, 32, 8, 8, 5),
]


def _gpu_prefill(wl, shuffled=True, signs=None):
    k = inputs.gen_kv(wl, "K")
    v = inputs.gen_kv(wl, "V")
    table, npages = (inputs.block_table if shuffled else inputs.identity_block_table)(wl)
    cfg = api.config(wl.tile_tokens, wl.bits_k, wl.bits_v, wl.iters, hadamard_signs=signs)
    cache = api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
    cu = torch.from_numpy(wl.cu_seqlens()).cuda()
    cache.quantize_prefill(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), cu)
    torch.cuda.synchronize()
    return k, v, table, npages, cache


def _compare_pools(wl, table, lens, gpu_pk, gpu_pv, ref_pk, ref_pv, pre, what):
    tot = [0, 0, 0]
    for s in range(wl.num_seqs):
        for h in range(wl.hkv):
            for role, bits, gp, rp in (("K", wl.bits_k, gpu_pk, ref_pk), ("V", wl.bits_v, gpu_pv, ref_pv)):
                _, gc, ga, gs, go = orc.read_sequence(gp, table[s], int(lens[s]), h, role, bits, wl.tile_tokens)
                _, rc, ra, rs, ro = orc.read_sequence(rp, table[s], int(lens[s]), h, role, bits, wl.tile_tokens)
                c = pu.compare_codes(gc, rc, pre[(s, h, role)], f"{what} s{s} h{h} {role}")
                tot = [a + b for a, b in zip(tot, c)]
                t = wl.tile_tokens
                for j in range(ga.shape[0]):
                    sl = slice(j * t, min(int(lens[s]), (j + 1) * t))
                    pu.check_tile_metadata(rc[sl], ga[j], gs[sl], go[sl], ra[j], rs[sl], ro[sl],
                                           orc.dequantize_tile, f"{what} s{s} h{h} {role} tile{j}")
    _report(what, tot)
    # every byte past the sequences' ends inside their last tiles is zero-filled as the
    # layout says, so whole slots agree apart from codes in the window
    return tot


@pytest.mark.parametrize("case", PAGED_CASES)
def test_paged_prefill_parity(case):
    recipe, lens, hkv, hq, tile, bk, bv, iters = case
    wl = _paged_workload(recipe, lens, hkv, hq, tile, bk, bv, iters)
    k, v, table, npages, cache = _gpu_prefill(wl)
    ref_pk = orc.new_pool(npages, hkv, bk, tile)
    ref_pv = orc.new_pool(npages, hkv, bv, tile)
    stg_k = np.zeros((wl.num_seqs, tile, hkv, 128), np.float16)
    stg_v = np.zeros_like(stg_k)
    pre = orc.quantize_to_pages(k, v, wl.cu_seqlens(), table, tile, bk, bv, iters, ref_pk, ref_pv, stg_k, stg_v)
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    _compare_pools(wl, table, wl.seq_lens, gpk, gpv, ref_pk, ref_pv, pre, f"prefill {case}")
    # staging holds the fp16 tail rows of partial tiles
    gsk, gsv = cache.staging_k.cpu().numpy(), cache.staging_v.cpu().numpy()
    for s, n in enumerate(wl.seq_lens):
        tail = n % tile
        np.testing.assert_array_equal(gsk[s, :tail], stg_k[s, :tail])
        np.testing.assert_array_equal(gsv[s, :tail], stg_v[s, :tail])


@pytest.mark.parametrize("case", [PAGED_CASES[1], PAGED_CASES[2], PAGED_CASES[3], PAGED_CASES[4]])
def test_append_and_requant_parity(case):
    recipe, lens, hkv, hq, tile, bk, bv, iters = case
    wl = _paged_workload(recipe, lens, hkv, hq, tile, bk, bv, iters, decode_steps=tile + 3)
    k, v, table, npages, cache = _gpu_prefill(wl)
    ref_pk = orc.new_pool(npages, hkv, bk, tile)
    ref_pv = orc.new_pool(npages, hkv, bv, tile)
    stg_k = np.zeros((wl.num_seqs, tile, hkv, 128), np.float16)
    stg_v = np.zeros_like(stg_k)
    orc.quantize_to_pages(k, v, wl.cu_seqlens(), table, tile, bk, bv, iters, ref_pk, ref_pv, stg_k, stg_v)
    lens_now = np.array(wl.seq_lens, np.int32)
    prefill_k, prefill_v = cache.pool_k.clone(), cache.pool_v.clone()
    steps = [0, 1, 2, tile - 1, tile, tile + 2]   # crosses a tile boundary for every sequence
    for step in range(max(steps) + 1):
        kn = inputs.gen_decode_kv(wl, "K", step)
        vn = inputs.gen_decode_kv(wl, "V", step)
        cache.append(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), torch.from_numpy(lens_now).cuda())
        pre = orc.append_and_requant(kn, vn, lens_now, table, tile, bk, bv, iters, ref_pk, ref_pv, stg_k, stg_v)
        lens_now = lens_now + 1
        if step not in steps:
            continue
        torch.cuda.synchronize()
        gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
        for s in range(wl.num_seqs):
            n = int(lens_now[s])
            t0 = ((n - 1) // tile) * tile          # first row of the re-quantized tile
            for h in range(hkv):
                for role, bits, gp, rp in (("K", bk, gpk, ref_pk), ("V", bv, gpv, ref_pv)):
                    _, gc, ga, gs, go = orc.read_sequence(gp, table[s], n, h, role, bits, tile)
                    _, rc, ra, rs, ro = orc.read_sequence(rp, table[s], n, h, role, bits, tile)
                    pu.compare_codes(gc[t0:], rc[t0:], pre[(s, h, role)], f"append step{step} s{s} h{h} {role}")
                    j = t0 // tile
                    pu.check_tile_metadata(rc[t0:], ga[j], gs[t0:], go[t0:], ra[j], rs[t0:], ro[t0:],
                                           orc.dequantize_tile, f"append step{step} s{s} h{h} {role}")
            # pages of tiles the prefill completed are untouched by the appends
            first_new_tile = wl.seq_lens[s] // tile
            done = table[s, :first_new_tile * (tile // 16)]
            assert torch.equal(cache.pool_k[done], prefill_k[done])
            assert torch.equal(cache.pool_v[done], prefill_v[done])
            r = int(lens_now[s] % tile) or tile
            np.testing.assert_array_equal(cache.staging_k[s, :r].cpu().numpy(), stg_k[s, :r])
            np.testing.assert_array_equal(cache.staging_v[s, :r].cpu().numpy(), stg_v[s, :r])


DECODE_CASES = [
    # (recipe, lens, hkv, hq, tile, bits_k, bits_v, iters)
    (1, (1024,), 1, 8, 64, 4, 4, 3),                 # single-head 1K workload, G = 8
    (2, (700, 513, 64, 1), 2, 8, 64, 4, 4, 3),       # G = 4, ragged, a 1-token sequence
    (5, (611, 200, 33, 96, 1000, 17), 2, 16, 32, 4, 2, 5),  # G = 8, K4/V2, tile 32
    (2, (900, 129), 2, 8, 128, 2, 2, 3),             # 2-bit, tile 128
    (2, (300,), 1, 1, 64, 4, 4, 3),                  # G = 1 (padded)
    (2, (257, 40), 1, 16, 64, 4, 2, 3),              # G = 16
    (2, (700, 513, 64, 1), 2, 8, 64, 8, 8, 3),       # 8-bit codes
    (5, (611, 33, 96), 2, 16, 32, 8, 8, 5),          # 8-bit, tile 32, G = 8
    (2, (900, 129), 1, 16, 128, 8, 8, 3),            # 8-bit, tile 128, G = 16
    (2, (700, 130, 5), 1, 8, 128, 4, 4, 3),          # tile 128, G = 8 (two head groups)
    (2, (500, 33, 64), 2, 8, 32, 4, 4, 3),           # tile 32, G = 4 (one head group)
    (2, (300, 65), 2, 4, 64, 2, 4, 3),               # G = 2 (padded), K2 / V4
]


@pytest.mark.parametrize("case", DECODE_CASES)
def test_paged_decode_parity(case):
    recipe, lens, hkv, hq, tile, bk, bv, iters = case
    wl = _paged_workload(recipe, lens, hkv, hq, tile, bk, bv, iters)
    k, v, table, npages, cache = _gpu_prefill(wl)
    q = inputs.gen_q(wl)
    seq_lens = np.array(wl.seq_lens, np.int32)
    out = cache.decode(torch.from_numpy(q).cuda(), torch.from_numpy(seq_lens).cuda(), max(lens))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    ref, sc = orc.paged_decode_attn(q, table, seq_lens, gpk, gpv, tile, bk, bv, return_scale=True)
    err = pu.assert_attn(got, ref, f"decode {case}", sc)
    # informative: against the oracle's own pages (quantization error included)
    ref_pk = orc.new_pool(npages, hkv, bk, tile)
    ref_pv = orc.new_pool(npages, hkv, bv, tile)
    orc.quantize_to_pages(k, v, wl.cu_seqlens(), table, tile, bk, bv, iters, ref_pk, ref_pv)
    e2e = np.abs(got - orc.paged_decode_attn(q, table, seq_lens, ref_pk, ref_pv, tile, bk, bv)).max()
    print(f"[attn] {case}: max abs err vs oracle on GPU pages {err:.2e}; vs oracle pages {e2e:.2e}", flush=True)


def test_decode_page_order_and_determinism():
    case = DECODE_CASES[1]
    recipe, lens, hkv, hq, tile, bk, bv, iters = case
    wl = _paged_workload(recipe, lens, hkv, hq, tile, bk, bv, iters)
    q = torch.from_numpy(inputs.gen_q(wl)).cuda()
    sl = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    outs = []
    for shuffled in (True, False, True):
        _, _, _, _, cache = _gpu_prefill(wl, shuffled)
        outs.append(cache.decode(q, sl, max(lens)))
    assert torch.equal(outs[0], outs[2])
    assert torch.equal(outs[0], outs[1])


def test_append_then_decode_matches_oracle():
    # a decode step as the bench runs it: append one token, attend over all of them
    wl = _paged_workload(2, (511, 64, 300), 2, 8, 64, 4, 4, 3)
    k, v, table, npages, cache = _gpu_prefill(wl)
    lens = np.array(wl.seq_lens, np.int32)
    kn, vn = inputs.gen_decode_kv(wl, "K", 0), inputs.gen_decode_kv(wl, "V", 0)
    cache.append(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), torch.from_numpy(lens).cuda())
    q = inputs.gen_q(wl, step=0)
    out = cache.decode(torch.from_numpy(q).cuda(), torch.from_numpy(lens + 1).cuda(), int(lens.max()) + 1)
    torch.cuda.synchronize()
    ref, sc = orc.paged_decode_attn(q, table, lens + 1, cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy(),
                                    64, 4, 4, return_scale=True)
    pu.assert_attn(out.cpu().numpy(), ref, "append+decode", sc)


BASELINE_CASES = [
    # (recipe, lens, hkv, hq)
    (1, (1024,), 1, 8),
    (2, (700, 513, 64, 1), 2, 8),
    (5, (611, 200, 33, 96, 1000, 17), 2, 16),
    (2, (300,), 1, 1),
    (2, (257, 40), 1, 16),
    (2, (5000, 37), 2, 8),      # several partitions per sequence
]


def _baseline_prefill(wl, fp8):
    k = inputs.gen_kv(wl, "K")
    v = inputs.gen_kv(wl, "V")
    table, npages = inputs.block_table(wl)
    ks, vs = (orc.fp8_scale(k), orc.fp8_scale(v)) if fp8 else (1.0, 1.0)
    cache = api.BaselineCache(npages, wl.hkv, torch.from_numpy(table), wl.num_seqs, fp8, ks, vs)
    cache.fill(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
               torch.from_numpy(wl.cu_seqlens()).cuda(), max(wl.seq_lens))
    torch.cuda.synchronize()
    return k, v, table, npages, ks, vs, cache


@pytest.mark.parametrize("fp8", [False, True], ids=["fp16", "fp8"])
@pytest.mark.parametrize("case", BASELINE_CASES)
def test_baseline_fill_and_decode_parity(case, fp8):
    recipe, lens, hkv, hq = case
    wl = _paged_workload(recipe, lens, hkv, hq, 64, 4, 4, 3)
    k, v, table, npages, ks, vs, cache = _baseline_prefill(wl, fp8)
    # the pages: byte-exact, unused pages and rows past the ends included
    ref_pk = orc.new_baseline_pool(npages, hkv, fp8)
    ref_pv = orc.new_baseline_pool(npages, hkv, fp8)
    orc.fill_pages_baseline(k, v, wl.cu_seqlens(), table, ref_pk, ref_pv, fp8, ks, vs)
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    np.testing.assert_array_equal(gpk.view(np.uint8), ref_pk.view(np.uint8))
    np.testing.assert_array_equal(gpv.view(np.uint8), ref_pv.view(np.uint8))
    # one decode step over them
    q = inputs.gen_q(wl)
    seq_lens = np.array(wl.seq_lens, np.int32)
    out = cache.decode(torch.from_numpy(q).cuda(), torch.from_numpy(seq_lens).cuda(), max(lens))
    torch.cuda.synchronize()
    ref = orc.paged_decode_attn_baseline(q, table, seq_lens, ref_pk, ref_pv, fp8, ks, vs)
    err = pu.assert_attn(out.cpu().numpy(), ref, f"baseline {'fp8' if fp8 else 'fp16'} {case}")
    print(f"[attn] baseline {'fp8' if fp8 else 'fp16'} {case}: max abs err {err:.2e}", flush=True)


@pytest.mark.parametrize("fp8", [False, True], ids=["fp16", "fp8"])
def test_baseline_append_and_decode_parity(fp8):
    """Decode tokens appended to fp16 / fp8 pages one step at a time: pages
    byte-exact against the oracle's appends, attention within the bar."""
    wl = _paged_workload(2, (200, 63, 16, 1), 2, 8, 64, 4, 4, 3, decode_steps=40)
    k, v = inputs.gen_kv(wl, "K"), inputs.gen_kv(wl, "V")
    table, npages = inputs.block_table(wl)
    kd = [inputs.gen_decode_kv(wl, "K", i) for i in range(40)]
    vd = [inputs.gen_decode_kv(wl, "V", i) for i in range(40)]
    ks = max(orc.fp8_scale(k), orc.fp8_scale(np.stack(kd))) if fp8 else 1.0
    vs = max(orc.fp8_scale(v), orc.fp8_scale(np.stack(vd))) if fp8 else 1.0
    cache = api.BaselineCache(npages, wl.hkv, torch.from_numpy(table), wl.num_seqs, fp8, ks, vs)
    cache.fill(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(wl.cu_seqlens()).cuda(),
               max(wl.seq_lens))
    rk, rv = orc.new_baseline_pool(npages, wl.hkv, fp8), orc.new_baseline_pool(npages, wl.hkv, fp8)
    orc.fill_pages_baseline(k, v, wl.cu_seqlens(), table, rk, rv, fp8, ks, vs)
    lens = np.array(wl.seq_lens, np.int32)
    for i in range(40):
        cache.append(torch.from_numpy(kd[i]).cuda(), torch.from_numpy(vd[i]).cuda(), torch.from_numpy(lens).cuda())
        orc.append_pages_baseline(kd[i], vd[i], lens, table, rk, rv, fp8, ks, vs)
        lens = lens + 1
    gk, gv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    view = np.uint8 if fp8 else np.float16
    np.testing.assert_array_equal(gk.view(view), rk.view(view))
    np.testing.assert_array_equal(gv.view(view), rv.view(view))
    q = inputs.gen_q(wl, 40)
    out = cache.decode(torch.from_numpy(q).cuda(), torch.from_numpy(lens).cuda(), int(lens.max())).cpu().numpy()
    ref = orc.paged_decode_attn_baseline(q, table, lens, gk, gv, fp8, ks, vs)
    err = pu.assert_attn(out, ref, f"baseline append {'fp8' if fp8 else 'fp16'}")
    print(f"[attn] baseline append + decode {'fp8' if fp8 else 'fp16'}: max abs err {err:.2e}", flush=True)


def test_baseline_decode_is_deterministic_and_order_free():
    wl = _paged_workload(2, (700, 513, 64, 1), 2, 8, 64, 4, 4, 3)
    q = torch.from_numpy(inputs.gen_q(wl)).cuda()
    sl = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    k = torch.from_numpy(inputs.gen_kv(wl, "K")).cuda()
    v = torch.from_numpy(inputs.gen_kv(wl, "V")).cuda()
    cu = torch.from_numpy(wl.cu_seqlens()).cuda()
    outs = []
    for tab in (inputs.block_table, inputs.identity_block_table, inputs.block_table):
        table, npages = tab(wl)
        cache = api.BaselineCache(npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
        cache.fill(k, v, cu, max(wl.seq_lens))
        outs.append(cache.decode(q, sl, max(wl.seq_lens)))
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


# ----------------------------------------------------------------------------- full sizes, sampled
def _sampled_tile_checks(wl, k, v, table, gpk, gpv, rng, n_samples, what):
    """Complete prefill tiles drawn at random: GPU slots vs the oracle on that tile alone."""
    cu = wl.cu_seqlens()
    t = wl.tile_tokens
    ppt = t // 16
    tot = [0, 0, 0]
    for _ in range(n_samples):
        s = int(rng.integers(wl.num_seqs))
        h = int(rng.integers(wl.hkv))
        role = ("K", "V")[int(rng.integers(2))]
        j = int(rng.integers(wl.seq_lens[s] // t))
        x = (k if role == "K" else v)[cu[s] + j * t:cu[s] + (j + 1) * t, h]
        bits = wl.bits_k if role == "K" else wl.bits_v
        ref = orc.quantize_tile(x, bits, wl.iters)
        gp = gpk if role == "K" else gpv
        _, gc, ga, gs, go = orc.read_sequence(gp, table[s, j * ppt:(j + 1) * ppt], t, h, role, bits, t)
        c = pu.compare_codes(gc, ref.codes, ref.pre, f"{what} s{s} h{h} {role} tile{j}")
        tot = [a + b for a, b in zip(tot, c)]
        pu.check_tile_metadata(ref.codes, ga[0], gs, go, ref.alpha, ref.scale, ref.offset, orc.dequantize_tile,
                               f"{what} s{s} h{h} {role} tile{j}")
    _report(f"{what} sampled tiles", tot)


def _sampled_decode_checks(wl, q, table, lens, gpk, gpv, got, pairs, what):
    g = wl.group
    for s, kh in pairs:
        ref, sc = orc.paged_decode_attn(q[s:s + 1, kh * g:(kh + 1) * g], table[s:s + 1], lens[s:s + 1],
                                        gpk[:, kh:kh + 1], gpv[:, kh:kh + 1], wl.tile_tokens, wl.bits_k, wl.bits_v,
                                        return_scale=True)
        err = pu.assert_attn(got[s, kh * g:(kh + 1) * g], ref[0], f"{what} s{s} kv head {kh}", sc[0])
        print(f"[attn] {what} s{s} kv head {kh} (L={int(lens[s])}): max abs err {err:.2e}", flush=True)


def test_full_size_qwen3_4b_layer_4x16k_sampled():
    """The 4 x 16K, 8/32-head layer in the launch configuration the bench times:
    quantize every page, append one token, one decode step; tiles, appended
    rows and attention outputs sampled against the oracle."""
    wl = inputs.workload(2)
    k, v, table, npages, cache = _gpu_prefill(wl)
    lens = np.array(wl.seq_lens, np.int32)
    kn, vn = inputs.gen_decode_kv(wl, "K", 0), inputs.gen_decode_kv(wl, "V", 0)
    cache.append(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), torch.from_numpy(lens).cuda())
    q = inputs.gen_q(wl)
    out = cache.decode(torch.from_numpy(q).cuda(), torch.from_numpy(lens + 1).cuda(), int(lens.max()) + 1)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    rng = np.random.default_rng(42)
    _sampled_tile_checks(wl, k, v, table, gpk, gpv, rng, 32, "4x16k")
    # the appended token opens tile 256 of every sequence: a one-row tile
    t = wl.tile_tokens
    for s in range(wl.num_seqs):
        j = int(lens[s]) // t
        for h in range(wl.hkv):
            for role, new, gp, bits in (("K", kn, gpk, wl.bits_k), ("V", vn, gpv, wl.bits_v)):
                ref = orc.quantize_tile(new[s, h][None], bits, wl.iters)
                _, gc, ga, gs, go = orc.read_sequence(gp, table[s, j * 4:(j + 1) * 4], 1, h, role, bits, t)
                pu.compare_codes(gc, ref.codes, ref.pre, f"append s{s} h{h} {role}")
                pu.check_tile_metadata(ref.codes, ga[0], gs, go, ref.alpha, ref.scale, ref.offset,
                                       orc.dequantize_tile, f"append s{s} h{h} {role}")
    _sampled_decode_checks(wl, q, table, lens + 1, gpk, gpv, got, [(0, 0), (3, 7), (1, 4)], "4x16k decode")
    assert np.isfinite(got).all()


def test_full_size_qwen3_32b_tp2_burst_sampled():
    """One GPU's share of the 32 x 16K burst (4 kv heads, 32 query heads):
    quantize the prefill, then the workload's 256 decode steps of append +
    attend (every sequence crosses four tile boundaries); sampled checks at
    the end."""
    wl = inputs.workload(3)
    k, v, table, npages, cache = _gpu_prefill(wl)
    lens = np.array(wl.seq_lens, np.int32)
    q = None
    steps = wl.decode_steps
    assert steps == 256
    d_lens = torch.from_numpy(lens).cuda()
    for step in range(steps):
        kn = torch.from_numpy(inputs.gen_decode_kv(wl, "K", step)).cuda()
        vn = torch.from_numpy(inputs.gen_decode_kv(wl, "V", step)).cuda()
        cache.append(kn, vn, d_lens)
        d_lens = d_lens + 1
        q = inputs.gen_q(wl, step)
        out = cache.decode(torch.from_numpy(q).cuda(), d_lens, int(lens.max()) + step + 1)
    torch.cuda.synchronize()
    lens_now = lens + steps
    got = out.cpu().numpy()
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    rng = np.random.default_rng(43)
    _sampled_tile_checks(wl, k, v, table, gpk, gpv, rng, 24, "32x16k")
    # the last (partial) tile of two sequences, rebuilt by the oracle from its fp16 rows
    t = wl.tile_tokens
    for s in (0, 31):
        j = int(lens_now[s] - 1) // t
        rows = []
        for pos in range(j * t, int(lens_now[s])):
            if pos < lens[s]:
                rows.append(k[wl.cu_seqlens()[s] + pos])
            else:
                rows.append(inputs.gen_decode_kv(wl, "K", pos - int(lens[s]))[s])
        x = np.stack(rows)                                   # [n, hkv, 128]
        for h in range(wl.hkv):
            ref = orc.quantize_tile(x[:, h], wl.bits_k, wl.iters)
            n = x.shape[0]
            _, gc, ga, gs, go = orc.read_sequence(gpk, table[s, j * 4:(j + 1) * 4], n, h, "K", wl.bits_k, t)
            pu.compare_codes(gc, ref.codes, ref.pre, f"burst last tile s{s} h{h}")
            pu.check_tile_metadata(ref.codes, ga[0], gs, go, ref.alpha, ref.scale, ref.offset,
                                   orc.dequantize_tile, f"burst last tile s{s} h{h}")
    _sampled_decode_checks(wl, q, table, lens_now, gpk, gpv, got, [(0, 0), (31, 3)], "32x16k decode")


REMAT_CASES = [
    # (recipe, lens, hkv, hq, tile, bits_k, bits_v, iters)
    (2, (200, 131, 64, 17), 2, 8, 64, 4, 4, 3),
    (5, (300, 97, 33), 2, 16, 32, 4, 2, 5),
    (2, (260, 128, 1000), 1, 4, 128, 2, 2, 3),
    (1, (1024, 1), 1, 8, 64, 2, 4, 3),
    (2, (200, 131, 64, 17), 2, 8, 64, 8, 8, 3),
]


@pytest.mark.parametrize("case", REMAT_CASES)
def test_rematerialized_fp16_pages_match_oracle(case):
    """Quantized pages restored into fp16 pages: each token within the restore
    bar of the oracle's restore of the same (GPU) pages, rows past the ends 0,
    pages past them untouched; the fp16 decode over them matches the oracle's
    fp16 attention over the same pages."""
    recipe, lens, hkv, hq, tile, bk, bv, iters = case
    wl = _paged_workload(recipe, lens, hkv, hq, tile, bk, bv, iters)
    k, v, table, npages, cache = _gpu_prefill(wl)
    seq_lens = np.array(wl.seq_lens, np.int32)
    base = api.BaselineCache(npages, hkv, torch.from_numpy(table), wl.num_seqs)
    base.pool_k.fill_(1.0)   # pages the restore must leave alone keep this
    base.pool_v.fill_(1.0)
    cache.rematerialize_into(base, torch.from_numpy(seq_lens).cuda(), max(lens))
    torch.cuda.synchronize()
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    bk_got, bv_got = base.pool_k.cpu().numpy(), base.pool_v.cpu().numpy()
    ref_k = np.ones_like(bk_got)
    ref_v = np.ones_like(bv_got)
    orc.rematerialize_pages(gpk, gpv, table, seq_lens, tile, bk, bv, ref_k, ref_v)
    for s in range(wl.num_seqs):
        n = int(seq_lens[s])
        for h in range(hkv):
            for role, got_pool, ref_pool in (("K", bk_got, ref_k), ("V", bv_got, ref_v)):
                got = orc.read_baseline_sequence(got_pool, table[s], n, h, role)
                ref = orc.read_baseline_sequence(ref_pool, table[s], n, h, role)
                pu.assert_dequant(got, ref, f"remat {case} s{s} h{h} {role}")
    # every page outside the sequences' tokens, and every row past an end, as the oracle left it
    used = np.zeros((npages, 16), bool)
    for s in range(wl.num_seqs):
        for t in range(int(seq_lens[s])):
            used[table[s][t // 16], t % 16] = True
    kk = bk_got.reshape(npages, hkv, 16, 128)
    vv = bv_got.reshape(npages, hkv, 128, 16)
    rk = ref_k.reshape(npages, hkv, 16, 128)
    rv = ref_v.reshape(npages, hkv, 128, 16)
    for pg in range(npages):
        for t in range(16):
            if not used[pg, t]:
                np.testing.assert_array_equal(kk[pg, :, t], rk[pg, :, t])
                np.testing.assert_array_equal(vv[pg, :, :, t], rv[pg, :, :, t])
    q = inputs.gen_q(wl)
    out = base.decode(torch.from_numpy(q).cuda(), torch.from_numpy(seq_lens).cuda(), max(lens))
    torch.cuda.synchronize()
    ref = orc.paged_decode_attn_baseline(q, table, seq_lens, bk_got, bv_got)
    pu.assert_attn(out.cpu().numpy(), ref, f"remat decode {case}")


FUSED_CASES = [
    # (recipe, lens, hkv, hq, tile, bits_k, bits_v, iters)
    (2, (200, 131, 64, 17), 2, 8, 64, 4, 4, 3),
    (5, (300, 97, 33), 2, 16, 32, 4, 2, 5),
    (2, (260, 128, 1000), 1, 4, 128, 2, 2, 3),
    (1, (1024,), 1, 8, 64, 4, 4, 3),
    (2, (700, 513, 64, 1), 2, 8, 32, 4, 4, 3),
    (2, (300, 97, 33), 2, 8, 64, 8, 8, 3),
    (5, (200, 64, 17), 1, 16, 32, 8, 8, 5),
    (2, (300, 129, 5), 1, 8, 128, 4, 4, 3),    # tile 128, G = 8 (two head groups)
    (2, (90, 200), 2, 4, 64, 2, 4, 3),         # G = 2 (padded), K2 / V4
]


@pytest.mark.parametrize("case", FUSED_CASES)
def test_append_and_decode_fused_matches_two_calls(case):
    """One launch of append + decode equals kvq_append_and_requant followed by
    kvq_paged_decode_attn: identical pages, staging rows and outputs, step after
    step (tiles fill and new ones start), and the outputs match the oracle."""
    recipe, lens, hkv, hq, tile, bk, bv, iters = case
    steps = tile + 2
    wl = _paged_workload(recipe, lens, hkv, hq, tile, bk, bv, iters, decode_steps=steps)
    k, v, table, npages, fused = _gpu_prefill(wl)
    _, _, _, _, split = _gpu_prefill(wl)
    lens_now = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    max_len = max(wl.seq_lens) + steps
    ws_f, ws_s = fused.workspace(hq, max_len), split.workspace(hq, max_len)
    for step in range(steps):
        kn = torch.from_numpy(inputs.gen_decode_kv(wl, "K", step)).cuda()
        vn = torch.from_numpy(inputs.gen_decode_kv(wl, "V", step)).cuda()
        q = torch.from_numpy(inputs.gen_q(wl, step)).cuda()
        of = fused.append_decode(kn, vn, lens_now, q, max_len, workspace=ws_f)
        split.append(kn, vn, lens_now)
        os_ = split.decode(q, lens_now + 1, max_len, workspace=ws_s)
        lens_now = lens_now + 1
        torch.cuda.synchronize()
        assert torch.equal(fused.pool_k, split.pool_k), step
        assert torch.equal(fused.pool_v, split.pool_v), step
        assert torch.equal(fused.staging_k, split.staging_k), step
        assert torch.equal(fused.staging_v, split.staging_v), step
        assert torch.equal(of, os_), (step, (of - os_).abs().max().item())
        if step in (0, tile - 1, steps - 1):
            ref, sc = orc.paged_decode_attn(q.cpu().numpy(), table, lens_now.cpu().numpy(), fused.pool_k.cpu().numpy(),
                                            fused.pool_v.cpu().numpy(), tile, bk, bv, return_scale=True)
            err = pu.assert_attn(of.cpu().numpy(), ref, f"fused {case} step {step}", sc)
            print(f"[attn] fused {case} step {step}: max abs err {err:.2e} (largest output scale {sc.max():.3g})",
                  flush=True)


# ---------------------------------------------------------------- randomized rotation (H diag(s))

SIGNED_CASES = [
    # (recipe, lens, hkv, hq, tile, bits_k, bits_v, iters, mask seed)
    (2, (200, 131, 64, 17), 2, 8, 64, 4, 4, 3, 1),
    (5, (300, 97, 33), 2, 16, 32, 4, 2, 5, 2),
    (2, (260, 128, 1000), 1, 4, 128, 2, 2, 3, 3),
    (2, (200, 64, 17), 2, 8, 64, 8, 8, 3, 4),
]


@pytest.mark.parametrize("case", SIGNED_CASES)
def test_randomized_rotation_paged_decode_fused_and_restore(case):
    """With a random sign mask: pages match the oracle's (codes within the
    window), the decode matches the oracle's attention with the same signs,
    the fused step equals the two calls bit for bit and matches the oracle,
    and the fp16 re-materialization matches the oracle's restore."""
    recipe, lens, hkv, hq, tile, bk, bv, iters, seed = case
    mask = inputs.hadamard_signs(seed)
    wl = _paged_workload(recipe, lens, hkv, hq, tile, bk, bv, iters)
    k, v, table, npages, cache = _gpu_prefill(wl, signs=mask)
    ref_pk, ref_pv = orc.new_pool(npages, hkv, bk, tile), orc.new_pool(npages, hkv, bv, tile)
    pre = orc.quantize_to_pages(k, v, wl.cu_seqlens(), table, tile, bk, bv, iters, ref_pk, ref_pv, signs=mask)
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    _compare_pools(wl, table, wl.seq_lens, gpk, gpv, ref_pk, ref_pv, pre, f"signed prefill {case}")
    lens_np = np.array(wl.seq_lens, np.int32)
    q = inputs.gen_q(wl)
    out = cache.decode(torch.from_numpy(q).cuda(), torch.from_numpy(lens_np).cuda(), max(lens))
    torch.cuda.synchronize()
    ref, sc = orc.paged_decode_attn(q, table, lens_np, gpk, gpv, tile, bk, bv, return_scale=True, signs=mask)
    pu.assert_attn(out.cpu().numpy(), ref, f"signed decode {case}", sc)
    # the mask is in effect: restoring the same pages without it gives other outputs
    plain = orc.paged_decode_attn(q, table, lens_np, gpk, gpv, tile, bk, bv)
    assert np.abs(plain - ref).max() > 1e-2
    # one fused append + decode step against the two calls
    _, _, _, _, split = _gpu_prefill(wl, signs=mask)
    lens_t = torch.from_numpy(lens_np).cuda()
    kn = torch.from_numpy(inputs.gen_decode_kv(wl, "K", 0)).cuda()
    vn = torch.from_numpy(inputs.gen_decode_kv(wl, "V", 0)).cuda()
    q1 = torch.from_numpy(inputs.gen_q(wl, 1)).cuda()
    max_len = max(lens) + 1
    of = cache.append_decode(kn, vn, lens_t, q1, max_len)
    split.append(kn, vn, lens_t)
    os_ = split.decode(q1, lens_t + 1, max_len)
    torch.cuda.synchronize()
    assert torch.equal(cache.pool_k, split.pool_k) and torch.equal(cache.pool_v, split.pool_v)
    assert torch.equal(of, os_)
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    ref1, sc1 = orc.paged_decode_attn(q1.cpu().numpy(), table, lens_np + 1, gpk, gpv, tile, bk, bv,
                                      return_scale=True, signs=mask)
    pu.assert_attn(of.cpu().numpy(), ref1, f"signed fused {case}", sc1)
    # fp16 re-materialization with the signs
    base = api.BaselineCache(npages, hkv, torch.from_numpy(table), wl.num_seqs)
    cache.rematerialize_into(base, lens_t + 1, max_len)
    torch.cuda.synchronize()
    ref_k = np.zeros((npages, hkv, 16 * 128), np.float16)
    ref_v = np.zeros_like(ref_k)
    orc.rematerialize_pages(gpk, gpv, table, lens_np + 1, tile, bk, bv, ref_k, ref_v, signs=mask)
    bk_got, bv_got = base.pool_k.cpu().numpy(), base.pool_v.cpu().numpy()
    for s in range(wl.num_seqs):
        for h in range(hkv):
            for role, got_pool, ref_pool in (("K", bk_got, ref_k), ("V", bv_got, ref_v)):
                pu.assert_dequant(orc.read_baseline_sequence(got_pool, table[s], int(lens_np[s]) + 1, h, role),
                                  orc.read_baseline_sequence(ref_pool, table[s], int(lens_np[s]) + 1, h, role),
                                  f"signed remat {case} s{s} h{h} {role}")


@pytest.mark.parametrize("tile,bits", [(64, 4), (32, 2), (128, 4), (64, 8)])
def test_randomized_rotation_dense(tile, bits):
    mask = inputs.hadamard_signs(7 + tile)
    x = _x(300, 3, 2)
    cfg = api.config(tile, bits, bits, 3, hadamard_signs=mask)
    q = api.quantize_tiles(torch.from_numpy(x).cuda(), cfg, bits)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in q.items()}
    ref = orc.quantize_dense(x, tile, bits, 3, mask)
    _report(f"signed dense T{tile} b{bits}",
            pu.compare_codes(orc.unpack_codes(got["codes"], bits), ref["codes_raw"], ref["pre"], "signed dense"))
    pu.assert_rel(got["alpha"], ref["alpha"], pu.META_RTOL, "alpha")
    pu.assert_rel(got["scale"], ref["scale"], pu.META_RTOL, "scale")
    deq = api.dequantize(q, cfg, bits).cpu().numpy().astype(np.float64)
    ref_deq = orc.dequantize_dense(got["codes"], got["alpha"], got["scale"], got["offset"], tile, bits, mask)
    pu.assert_dequant(deq, ref_deq, "signed dequantize")


MQ_CASES = [
    # (recipe, lens, hkv, hq, tile, bits_k, bits_v, iters, n_q)
    (2, (700, 513, 64, 5), 2, 8, 64, 4, 4, 3, 4),        # G = 4, 4 queries: 16 rows in one workgroup
    (5, (611, 200, 33), 2, 16, 32, 4, 2, 5, 3),          # G = 8, 24 rows: blocks of 16 + 8
    (2, (900, 129), 2, 8, 128, 2, 2, 3, 2),              # 8 rows, 2-bit, tile 128
    (2, (300, 70), 1, 1, 64, 4, 4, 3, 1),                # one row
    (2, (257, 40), 1, 16, 64, 4, 2, 3, 5),               # G = 16, 80 rows in 5 blocks
    (2, (700, 100), 2, 8, 64, 8, 8, 3, 4),               # 8-bit codes
    (2, (400, 300), 1, 4, 64, 4, 4, 3, 70),              # a 70-token chunk: the mask spans two chunks
    (2, (100, 3), 1, 4, 64, 4, 4, 3, 6),                 # a sequence shorter than n_q: zero rows
    (2, (900, 300), 1, 16, 128, 8, 8, 3, 2),             # 8-bit, tile 128, G = 16: 32 rows in 4 blocks
    (5, (300, 65), 2, 8, 32, 8, 8, 5, 5),                # 8-bit, tile 32, heavy-tailed K, 20 rows
]


@pytest.mark.parametrize("case", MQ_CASES)
def test_paged_multi_query_parity(case):
    """Several queries per sequence, causal, against the oracle on the GPU's pages."""
    recipe, lens, hkv, hq, tile, bk, bv, iters, n_q = case
    wl = _paged_workload(recipe, lens, hkv, hq, tile, bk, bv, iters)
    k, v, table, npages, cache = _gpu_prefill(wl)
    q = inputs.gen_q_multi(wl, n_q)
    seq_lens = np.array(wl.seq_lens, np.int32)
    out = cache.multi_query(torch.from_numpy(q).cuda(), torch.from_numpy(seq_lens).cuda(), max(lens))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    ref, sc = orc.paged_multi_query_attn(q, table, seq_lens, gpk, gpv, tile, bk, bv, return_scale=True)
    err = pu.assert_attn(got, ref, f"multi-query {case}", sc)
    assert np.isfinite(got).all()
    print(f"[attn] multi-query {case}: max abs err vs oracle on GPU pages {err:.2e}", flush=True)


def test_multi_query_with_one_query_is_the_decode_bit_for_bit():
    recipe, lens, hkv, hq, tile, bk, bv, iters = DECODE_CASES[2]
    wl = _paged_workload(recipe, lens, hkv, hq, tile, bk, bv, iters)
    _, _, _, _, cache = _gpu_prefill(wl)
    q = torch.from_numpy(inputs.gen_q(wl)).cuda()
    sl = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    dec = cache.decode(q, sl, max(lens))
    mq = cache.multi_query(q[:, None], sl, max(lens))
    torch.cuda.synchronize()
    assert torch.equal(mq[:, 0], dec)


def test_full_size_qwen3_4b_layer_4x16k_verify_4_sampled():
    """The 4 x 16K, 8/32-head layer: 4 draft tokens per sequence appended, then
    verified with one multi-query launch; sampled (sequence, kv head) outputs
    against the oracle."""
    wl = inputs.workload(2)
    k, v, table, npages, cache = _gpu_prefill(wl)
    lens = np.array(wl.seq_lens, np.int32)
    n_q = 4
    for step in range(n_q):
        kn, vn = inputs.gen_decode_kv(wl, "K", step), inputs.gen_decode_kv(wl, "V", step)
        cache.append(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), torch.from_numpy(lens + step).cuda())
    q = inputs.gen_q_multi(wl, n_q)
    out = cache.multi_query(torch.from_numpy(q).cuda(), torch.from_numpy(lens + n_q).cuda(), int(lens.max()) + n_q)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    g = wl.group
    for s, kh in [(0, 0), (3, 7), (2, 3)]:
        ref, sc = orc.paged_multi_query_attn(q[s:s + 1, :, kh * g:(kh + 1) * g], table[s:s + 1], lens[s:s + 1] + n_q,
                                             gpk[:, kh:kh + 1], gpv[:, kh:kh + 1], wl.tile_tokens, wl.bits_k,
                                             wl.bits_v, return_scale=True)
        err = pu.assert_attn(got[s, :, kh * g:(kh + 1) * g], ref[0], f"verify s{s} kv head {kh}", sc[0])
        print(f"[attn] 4x16k verify-4 s{s} kv head {kh}: max abs err {err:.2e}", flush=True)


def _appended_row_checks(wl, kn, vn, lens, table, gpk, gpv, seqs, what):
    """The token appended after a prefill of whole tiles opens a one-row tile."""
    t = wl.tile_tokens
    ppt = t // 16
    for s in seqs:
        j = int(lens[s]) // t
        assert int(lens[s]) % t == 0
        for h in range(wl.hkv):
            for role, new, gp, bits in (("K", kn, gpk, wl.bits_k), ("V", vn, gpv, wl.bits_v)):
                ref = orc.quantize_tile(new[s, h][None], bits, wl.iters)
                _, gc, ga, gs, go = orc.read_sequence(gp, table[s, j * ppt:(j + 1) * ppt], 1, h, role, bits, t)
                pu.compare_codes(gc, ref.codes, ref.pre, f"{what} append s{s} h{h} {role}")
                pu.check_tile_metadata(ref.codes, ga[0], gs, go, ref.alpha, ref.scale, ref.offset,
                                       orc.dequantize_tile, f"{what} append s{s} h{h} {role}")


@pytest.mark.parametrize("bits", [4, 2])
def test_full_size_long_context_layer_6x128k_sampled(bits):
    """One layer of the 6 x 128K long-context workload (8 kv / 32 query heads,
    tile 128, 3 iterations) at 4- and 2-bit codes, in the launch configuration
    the bench times: quantize the prefill (drawn on the device), then one
    fused append + decode step; sampled tiles, the appended rows and attention
    outputs over 131073 tokens against the oracle."""
    wl = dataclasses.replace(inputs.workload(4), bits_k=bits, bits_v=bits)
    max_len = max(wl.seq_lens)
    k = inputs.gen_kv_device(wl, "K")
    v = inputs.gen_kv_device(wl, "V")
    table, npages = inputs.block_table(wl, capacity_tokens=max_len + 1)
    cfg = api.config(wl.tile_tokens, bits, bits, wl.iters)
    cache = api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
    cache.quantize_prefill(k, v, torch.from_numpy(wl.cu_seqlens()).cuda())
    lens = np.array(wl.seq_lens, np.int32)
    kn, vn = inputs.gen_decode_kv(wl, "K", 0), inputs.gen_decode_kv(wl, "V", 0)
    q = inputs.gen_q(wl)
    out = cache.append_decode(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), torch.from_numpy(lens).cuda(),
                              torch.from_numpy(q).cuda(), max_len + 1)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    k_np, v_np = k.cpu().numpy(), v.cpu().numpy()
    del k, v
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    what = f"6x128k b{bits}"
    _sampled_tile_checks(wl, k_np, v_np, table, gpk, gpv, np.random.default_rng(44 + bits), 24, what)
    _appended_row_checks(wl, kn, vn, lens, table, gpk, gpv, (0, 5), what)
    pairs = [(0, 0), (5, 7)] if bits == 4 else [(3, 2)]
    _sampled_decode_checks(wl, q, table, lens + 1, gpk, gpv, got, pairs, f"{what} decode")


def test_full_size_mixed_64_seqs_1k_32k_sampled():
    """The mixed-precision stress workload at full size: 64 sequences of 1K-32K
    tokens, 8 kv / 64 query heads, heavy-tailed K (Student-t(3) times
    log-uniform channel scales, drawn on the device), tile 32, 4-bit K, 2-bit
    V, 5 iterations; quantize, then one fused append + decode step; sampled
    tiles and attention outputs against the oracle."""
    wl = inputs.workload(5)
    max_len = max(wl.seq_lens)
    k = inputs.gen_kv_device(wl, "K")
    v = inputs.gen_kv_device(wl, "V")
    table, npages = inputs.block_table(wl)
    cfg = api.config(wl.tile_tokens, wl.bits_k, wl.bits_v, wl.iters)
    cache = api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
    cache.quantize_prefill(k, v, torch.from_numpy(wl.cu_seqlens()).cuda())
    lens = np.array(wl.seq_lens, np.int32)
    kn, vn = inputs.gen_decode_kv(wl, "K", 0), inputs.gen_decode_kv(wl, "V", 0)
    q = inputs.gen_q(wl)
    out = cache.append_decode(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), torch.from_numpy(lens).cuda(),
                              torch.from_numpy(q).cuda(), max_len + 1)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    k_np, v_np = k.cpu().numpy(), v.cpu().numpy()
    del k, v
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    _sampled_tile_checks(wl, k_np, v_np, table, gpk, gpv, np.random.default_rng(45), 32, "mixed-64")
    # the appended token's tile (partial for most lengths): rebuilt from its fp16 rows
    t = wl.tile_tokens
    cu = wl.cu_seqlens()
    for s in (int(np.argmin(lens)), int(np.argmax(lens)), 17):
        j = int(lens[s]) // t
        n = int(lens[s]) - j * t + 1
        for h in (0, wl.hkv - 1):
            for role, src, new, gp, bits in (("K", k_np, kn, gpk, wl.bits_k), ("V", v_np, vn, gpv, wl.bits_v)):
                x = np.concatenate([src[cu[s] + j * t:cu[s] + int(lens[s]), h], new[s, h][None]])
                ref = orc.quantize_tile(x, bits, wl.iters)
                _, gc, ga, gs, go = orc.read_sequence(gp, table[s, j * (t // 16):(j + 1) * (t // 16)], n, h, role,
                                                      bits, t)
                pu.compare_codes(gc, ref.codes, ref.pre, f"mixed-64 last tile s{s} h{h} {role}")
                pu.check_tile_metadata(ref.codes, ga[0], gs, go, ref.alpha, ref.scale, ref.offset,
                                       orc.dequantize_tile, f"mixed-64 last tile s{s} h{h} {role}")
    _sampled_decode_checks(wl, q, table, lens + 1, gpk, gpv, got,
                           [(int(np.argmin(lens)), 0), (int(np.argmax(lens)), 5), (37, 7)], "mixed-64 decode")


def _degenerate_inputs(wl):
    """K and V with the method's degenerate tiles in sequence 1 (tile 64):
    tile 0 all zero, tile 1 one row repeated, tile 2 rows constant across
    channels, tile 3 a channel riding on an offset 100x its spread, tile 4 one
    row 1000x the others; sequence 0 is empty and sequence 2 random."""
    k, v = inputs.gen_kv(wl, "K").astype(np.float64), inputs.gen_kv(wl, "V").astype(np.float64)
    cu = wl.cu_seqlens()
    rng = np.random.default_rng(7)
    for x in (k, v):
        b = cu[1]
        x[b:b + 64] = 0.0
        x[b + 64:b + 128] = x[b + 64]
        x[b + 128:b + 192] = rng.standard_normal((64, x.shape[1], 1))
        x[b + 192:b + 256, :, 5] += 100.0
        x[b + 300] *= 1000.0
    return np.clip(k, -65504, 65504).astype(np.float16), np.clip(v, -65504, 65504).astype(np.float16)


def test_degenerate_tiles_and_empty_sequence():
    wl = _paged_workload(2, (0, 320, 77), 2, 8, 64, 4, 4, 3)
    k, v = _degenerate_inputs(wl)
    table, npages = inputs.block_table(wl)
    cfg = api.config(64, 4, 4, 3)
    cache = api.PagedCache(cfg, npages, wl.hkv, torch.from_numpy(table), wl.num_seqs)
    cache.quantize_prefill(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                           torch.from_numpy(wl.cu_seqlens()).cuda())
    torch.cuda.synchronize()
    ref_pk, ref_pv = orc.new_pool(npages, wl.hkv, 4, 64), orc.new_pool(npages, wl.hkv, 4, 64)
    stg_k = np.zeros((wl.num_seqs, 64, wl.hkv, 128), np.float16)
    stg_v = np.zeros_like(stg_k)
    pre = orc.quantize_to_pages(k, v, wl.cu_seqlens(), table, 64, 4, 4, 3, ref_pk, ref_pv, stg_k, stg_v)
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    tot = [0, 0, 0]
    for s in (1, 2):
        for h in range(wl.hkv):
            for role, bits, gp, rp in (("K", 4, gpk, ref_pk), ("V", 4, gpv, ref_pv)):
                n = wl.seq_lens[s]
                _, gc, ga, gs, go = orc.read_sequence(gp, table[s], n, h, role, bits, 64)
                _, rc, ra, rs, ro = orc.read_sequence(rp, table[s], n, h, role, bits, 64)
                c = pu.compare_codes(gc, rc, pre[(s, h, role)], f"degenerate s{s} h{h} {role}")
                tot = [a + b for a, b in zip(tot, c)]
                for j in range(ga.shape[0]):
                    sl = slice(j * 64, min(n, (j + 1) * 64))
                    pu.check_tile_metadata(rc[sl], ga[j], gs[sl], go[sl], ra[j], rs[sl], ro[sl],
                                           orc.dequantize_tile, f"degenerate s{s} h{h} {role} tile{j}")
    _report("degenerate tiles", tot)
    # the all-zero tile stores zero codes, zero scales and offsets and unit channel factors
    _, zc, za, zs, zo = orc.read_sequence(gpk, table[1], 64, 0, "K", 4, 64)
    assert not zc.any() and not zs.any() and not zo.any() and np.all(za == 1.0)
    # decode: the empty sequence gives a zero row, the others match the oracle
    lens = np.array(wl.seq_lens, np.int32)
    q = inputs.gen_q(wl)
    out = cache.decode(torch.from_numpy(q).cuda(), torch.from_numpy(lens).cuda(), max(wl.seq_lens)).cpu().numpy()
    assert not out[0].any()
    ref, sc = orc.paged_decode_attn(q[1:], table[1:], lens[1:], gpk, gpv, 64, 4, 4, return_scale=True)
    pu.assert_attn(out[1:], ref, "degenerate decode", sc)
    # one fused append + decode step: the empty sequence now holds one token
    kn, vn = inputs.gen_decode_kv(wl, "K", 0), inputs.gen_decode_kv(wl, "V", 0)
    out1 = cache.append_decode(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), torch.from_numpy(lens).cuda(),
                               torch.from_numpy(q).cuda(), max(wl.seq_lens) + 1).cpu().numpy()
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    ref1, sc1 = orc.paged_decode_attn(q, table, lens + 1, gpk, gpv, 64, 4, 4, return_scale=True)
    pu.assert_attn(out1, ref1, "degenerate fused step", sc1)
    one = orc.quantize_tile(kn[0, 0][None], 4, 3)
    _, gc, ga, gs, go = orc.read_sequence(gpk, table[0], 1, 0, "K", 4, 64)
    pu.compare_codes(gc, one.codes, one.pre, "appended token of the empty sequence")


@pytest.mark.parametrize("case", [(2, (300, 97, 33), 2, 8, 64, 4, 4, 3, 5, 4), (5, (200, 70), 1, 8, 32, 4, 2, 5, 3, 5)])
def test_multi_query_with_randomized_rotation(case):
    """Several causal queries per sequence over pages quantized with a random
    sign mask: the query takes the signs before H and the output after it."""
    recipe, lens, hkv, hq, tile, bk, bv, iters, n_q, seed = case
    mask = inputs.hadamard_signs(seed)
    wl = _paged_workload(recipe, lens, hkv, hq, tile, bk, bv, iters)
    _, _, table, _, cache = _gpu_prefill(wl, signs=mask)
    q = inputs.gen_q_multi(wl, n_q)
    seq_lens = np.array(wl.seq_lens, np.int32)
    out = cache.multi_query(torch.from_numpy(q).cuda(), torch.from_numpy(seq_lens).cuda(), max(lens)).cpu().numpy()
    gpk, gpv = cache.pool_k.cpu().numpy(), cache.pool_v.cpu().numpy()
    ref, sc = orc.paged_multi_query_attn(q, table, seq_lens, gpk, gpv, tile, bk, bv, return_scale=True, signs=mask)
    err = pu.assert_attn(out, ref, f"signed multi-query {case}", sc)
    plain = orc.paged_multi_query_attn(q, table, seq_lens, gpk, gpv, tile, bk, bv)
    assert np.abs(plain - ref).max() > 1e-2   # the mask is in effect
    print(f"[attn] signed multi-query {case}: max abs err {err:.2e}", flush=True)
