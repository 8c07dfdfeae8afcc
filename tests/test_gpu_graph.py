"""The prefill quantize and the fused append + decode step (its no-allocation
entry point, for callers under graph capture) recorded into one HIP graph:
every replay, with other GPU work and synchronizations between replays, must
give the eager calls' bits (output, both page pools and the staging rows)."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_tiles_amd import _lib as L
from kv_cache_quantization_tiles_amd import inputs
from tests.test_gpu_parity import _gpu_prefill, _paged_workload

pytestmark = pytest.mark.gpu

CASES = [
    # (recipe, lens, hkv, hq, tile, bits_k, bits_v, iters): sequences ending mid-tile and on a tile
    # boundary, a tail of fewer than 16 tokens (the float64 short-tile pass)
    (2, (600, 130, 64, 9), 2, 8, 64, 4, 4, 3),
    (5, (300, 97, 33), 2, 16, 32, 4, 2, 5),
]


@pytest.mark.parametrize("case", CASES)
def test_prefill_and_fused_step_replay_in_a_graph(case):
    wl = _paged_workload(*case, decode_steps=1)
    k, v, _, _, cache = _gpu_prefill(wl)
    kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    cu = torch.from_numpy(wl.cu_seqlens()).cuda()
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device="cuda")
    kn = torch.from_numpy(inputs.gen_decode_kv(wl, "K", 0)).cuda()
    vn = torch.from_numpy(inputs.gen_decode_kv(wl, "V", 0)).cuda()
    q = torch.from_numpy(inputs.gen_q(wl)).cuda()
    out = torch.empty((wl.num_seqs, wl.hq, 128), dtype=torch.float32, device="cuda")
    state = (out, cache.pool_k, cache.pool_v, cache.staging_k, cache.staging_v)

    def step():
        # the prefill rewrites every page of the sequences; the append then
        # re-quantizes each sequence's last tile with the new token
        cache.quantize_prefill(kt, vt, cu)
        L.kvq_append_and_decode_noalloc(cache.cfg, kn, vn, lens, wl.num_seqs, wl.hkv, cache.staging_k,
                                        cache.staging_v, cache.block_table, cache.max_blocks, cache.pool_k,
                                        cache.pool_v, q, wl.hq, max(wl.seq_lens) + 1, 1.0 / np.sqrt(128.0), out)

    def scramble():
        out.fill_(float("nan"))
        for t in state[1:]:
            t.zero_()

    scramble()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in state]
    assert not torch.isnan(ref[0]).any()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # a warm-up on the capture's side stream, as torch advises
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    noise = torch.randn(1 << 20, device="cuda")
    for r in range(4):
        scramble()
        (noise * 2.0).sum().item()   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("output", "pool_k", "pool_v", "staging_k", "staging_v"), state, ref):
            assert torch.equal(got, want), f"{case} replay {r}: {name} differs from the eager call"
    print(f"[graph] {case}: 4 replays equal the eager calls bit for bit", flush=True)
