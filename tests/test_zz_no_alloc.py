"""kvq_append_and_decode_noalloc (the fused decode step whose partition
partials live in the library's static device scratch) against
kvq_append_and_decode with a caller workspace, through the C ABI: identical
output, pages and staging rows on two calls in a row, the second with a
smaller input (fewer sequences, shorter contexts, a smaller GQA group)."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_tiles_amd import _lib as L
from kv_cache_quantization_tiles_amd import api, inputs
from tests.test_gpu_parity import _gpu_prefill, _paged_workload


def _step(cache, wl, noalloc, ws=None):
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    kn = torch.from_numpy(inputs.gen_decode_kv(wl, "K", 0)).cuda()
    vn = torch.from_numpy(inputs.gen_decode_kv(wl, "V", 0)).cuda()
    q = torch.from_numpy(inputs.gen_q(wl)).cuda()
    out = torch.full((wl.num_seqs, wl.hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    max_len = max(wl.seq_lens) + 1
    args = (cache.cfg, kn, vn, lens, wl.num_seqs, wl.hkv, cache.staging_k, cache.staging_v, cache.block_table,
            cache.max_blocks, cache.pool_k, cache.pool_v, q, wl.hq, max_len, 1.0 / np.sqrt(128.0), out)
    if noalloc:
        L.kvq_append_and_decode_noalloc(*args)
    else:
        L.kvq_append_and_decode(*args, ws, ws.numel())
    return out


@pytest.mark.gpu
def test_noalloc_fused_step_equals_the_workspace_call_twice_then_smaller():
    cases = [
        # (recipe, lens, hkv, hq, tile, bits_k, bits_v, iters): the second call is smaller
        (2, (1500, 700, 64, 1), 4, 32, 64, 4, 4, 3),
        (5, (300, 17), 2, 8, 32, 4, 2, 5),
    ]
    for case in cases:
        wl = _paged_workload(*case, decode_steps=1)
        _, _, _, _, a = _gpu_prefill(wl)
        _, _, _, _, b = _gpu_prefill(wl)
        ws = torch.empty(L.kvq_decode_workspace_bytes(a.cfg, wl.num_seqs, wl.hq, wl.hkv, max(wl.seq_lens) + 1),
                         dtype=torch.uint8, device="cuda")
        oa = _step(a, wl, False, ws)
        ob = _step(b, wl, True)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), (case, (oa - ob).abs().max().item())
        assert not torch.isnan(ob).any()
        for x, y in ((a.pool_k, b.pool_k), (a.pool_v, b.pool_v), (a.staging_k, b.staging_k),
                     (a.staging_v, b.staging_v)):
            assert torch.equal(x, y), case
        print(f"[noalloc] {case}: output, pages and staging identical", flush=True)
