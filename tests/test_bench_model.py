"""The bench's byte model against the page layout the oracle defines: a
token-head's share of a slot (bench.slot_bytes_per_token) is 1/16 of the
oracle's slot bytes for every code width, tile size and slot format, and the
quantize / decode byte counts of the 4 x 16K layer follow from those shares
(the figures the bench line's roofline divides by the kernel times)."""
import math

import pytest

import bench
import oracle as orc
from kv_cache_quantization_tiles_amd import inputs


@pytest.mark.parametrize("tile", [32, 64, 128])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_slot_share_per_token_is_a_sixteenth_of_the_oracle_slot(tile, bits):
    assert bench.slot_bytes_per_token(bits, tile) * 16 == orc.slot_bytes(bits, tile)
    if bits != 8:
        assert bench.slot_bytes_per_token(bits, tile, meta16=True) * 16 == orc.slot_bytes(bits, tile, meta16=True)
        assert bench.slot_bytes_per_token(bits, tile, kchan=True) * 16 == orc.slot_bytes(bits, tile, kchan=True)


def test_byte_counts_of_the_4x16k_layer():
    wl = inputs.workload(2)
    n = wl.total_tokens * wl.hkv                       # token-heads of K (and of V)
    slot = orc.slot_bytes(wl.bits_k, wl.tile_tokens)   # 4-bit, tile 64: 1280 B per 16 tokens
    assert slot == 1280
    # quantize: fp16 read + the slot share written, K and V
    q = bench.quantize_bytes(n, wl.bits_k, wl.tile_tokens) + bench.quantize_bytes(n, wl.bits_v, wl.tile_tokens)
    assert q == 2 * n * (2 * 128 + slot / 16) == 352321536
    # decode after one appended token: every page of whole tiles, K and V
    lens = [l + 1 for l in wl.seq_lens]
    pages = sum(math.ceil(l / wl.tile_tokens) * wl.tile_tokens // 16 for l in lens)
    assert bench.decode_bytes(wl, lens) == pages * wl.hkv * 2 * slot
