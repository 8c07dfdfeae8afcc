"""CPU oracle for the variance-normalized KV-cache tile quantizer and its paged
decode-attention read path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  The product path (the HIP library
and its Python binding) never imports it, and it imports nothing from the
product path: the two share no code.  The only shared module is the seeded
input generator, which holds no arithmetic of the method.

Everything here is plain NumPy in float64 (the pages fix no precision), one
tile at a time, in the order the pages give the steps.  It is slow on purpose.

Sources (the pages, cited by title and section):

* [axbrief §diff]  "Huawei's KVarN boosts vLLM KV-cache capacity by 5x without
  accuracy loss" (axbrief.com), section "기존 방식과 달라진 지점" (what differs
  from earlier methods).  Its four-step paragraph is the only description of
  the method: the cache is quantized per fixed-size token tile; each tile,
  still raw fp16, is rotated along the channel dimension with a Hadamard
  transform to spread channel-concentrated outliers; a Sinkhorn-like
  iterative variance normalization then evens out the per-channel variance;
  finally asymmetric round-to-nearest produces the low-bit cache.
* [axbrief §flag]  same page, section "별도의 캘리브레이션이나 모델 변경 없이
  플래그 하나로 적용": restates rotation + iterative variance normalization,
  and that nothing is calibrated (every statistic comes from the tile itself).
* [ttj §quant]  "화웨이가 공개한 KVarN — LLM 추론의 '메모리 먹는 하마' KV 캐시를
  양자화로 길들이기" (ttj.kr), section "양자화로 캐시를 다이어트시킨다": K and V
  are compressed and restored inside the inference pipeline, with the cache
  managed in pages.
* [aitrends §TL;DR], [aitrends §용어 해설]  aitrends.kr article 74976: the
  attention backend reads compressed KV pages directly instead of
  re-materializing fp16.

Readings where the pages are silent (each is a documented parameter or choice):

* Hadamard: Sylvester order, orthonormal (divided by sqrt(d)), applied to every
  token row of K and of V; no random signs unless a sign mask is passed in (the
  randomized variant H diag(s), restored by diag(s) H).
* "Variance": population standard deviation (divide by n), mean-centered; the
  data themselves are only scaled, never shifted (the per-token zero-point of
  the rounding step absorbs offsets).
* One iteration = a channel step (each channel divided by its spread over the
  tile's tokens) followed by a token step (each token divided by its spread
  over the channels).  The factors multiply into alpha (per channel) and beta
  (per token), so that R = diag(beta) . Y . diag(alpha) holds exactly.
* Guard: a channel (token) whose spread is at most GUARD times its RMS is left
  unscaled (factor 1).  This covers one-token tiles, repeated rows, all-zero
  rows and nearly constant columns, where dividing by the spread would blow
  up values instead of evening them out.
* Rounding granularity: per token row over the 128 channels of the tile; the
  zero-point is the row minimum (a float, not an integer); the step is
  (max - min) / (2^bits - 1); ties round to even; a row with zero range gets
  codes 0 and step 0.
* Stored metadata, fp32: alpha[128] per tile, and per token the scale
  S = beta * step and offset O = beta * min, so that the restored rotated row
  is alpha * (S * code + O) and the restored token is that row rotated back.
* Tiles are aligned to the start of each sequence; the last one may be
  partial, and its statistics use only its valid rows.
* Per-channel rounding for K (kchan): the pages do not say over which axis
  the asymmetric rounding runs.  The variant rounds each channel of a K tile
  over the tile's valid tokens: zero-point = the channel's minimum of Y,
  step = (max - min) / (2^bits - 1), ties to even.  The token factors beta
  then stay per token and the channel factors merge with the rounding, so a
  K slot stores beta per token and, per channel of the tile, the scale
  A = alpha * step and the zero offset in code units M = min / step; the
  restored rotated row is beta * A * (code + M).  A channel of zero range
  stores A = alpha * min and M = 1 (its codes are 0).  V keeps per-token
  rounding.
* Metadata precision: fp32 by default; the fp16 slot variant (meta16) moves
  one power of two per tile from the scales and offsets into the channel
  factors (see meta_fp16) and rounds all three to fp16 (nearest even).  Codes
  are decided before the metadata are rounded, so they are the same in both
  variants.

"parity unpinned" applies to nothing here: every function is pinned by the
tests in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

HEAD_DIM = 128
PAGE_TOKENS = 16
GUARD = 1e-2


# ----------------------------------------------------------------------------
# Step 2 of the tile quantizer: Hadamard rotation along channels [axbrief §diff]
# ----------------------------------------------------------------------------

def hadamard(d: int = HEAD_DIM) -> np.ndarray:
    """Orthonormal Sylvester Hadamard matrix of order d (a power of two)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / math.sqrt(d)


def fwht(x: np.ndarray) -> np.ndarray:
    """Orthonormal fast Walsh-Hadamard transform along the last axis.

    For each bit of the channel index, entries that differ only in that bit
    are replaced by their sum (bit 0) and difference (bit 1).  Equal to
    x @ hadamard(d) for every row."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < d:
        y = y.reshape(lead + (d // (2 * h), 2, h))
        lo = y[..., 0, :].copy()
        hi = y[..., 1, :].copy()
        y[..., 0, :] = lo + hi
        y[..., 1, :] = lo - hi
        y = y.reshape(lead + (d,))
        h *= 2
    return y / math.sqrt(d)


def signs_from_mask(mask) -> np.ndarray:
    """The randomized rotation's diagonal: a 128-bit mask (4 x uint32, bit c
    mod 32 of word c // 32 set = channel c negated) as a +-1 vector; None or
    all zero is the plain transform.  The rotation is then H diag(s) and the
    restore diag(s) H (H symmetric and orthonormal, s^2 = 1)."""
    if mask is None:
        return np.ones(HEAD_DIM)
    words = [int(w) & 0xFFFFFFFF for w in np.asarray(mask).reshape(-1)]
    if len(words) != HEAD_DIM // 32:
        raise ValueError("mask must hold 4 32-bit words")
    bits = np.array([(words[c // 32] >> (c % 32)) & 1 for c in range(HEAD_DIM)], np.float64)
    return 1.0 - 2.0 * bits


# ----------------------------------------------------------------------------
# Step 3: Sinkhorn-like iterative variance normalization [axbrief §diff, §flag]
# ----------------------------------------------------------------------------

def _spread_and_rms(v: np.ndarray, axis: int):
    mean = v.mean(axis=axis, keepdims=True)
    std = np.sqrt(((v - mean) ** 2).mean(axis=axis, keepdims=True))
    rms = np.sqrt((v ** 2).mean(axis=axis, keepdims=True))
    return std, rms


def _factor(v: np.ndarray, axis: int) -> np.ndarray:
    std, rms = _spread_and_rms(v, axis)
    return np.where(std > GUARD * rms, std, 1.0)


def sinkhorn(r: np.ndarray, iters: int):
    """Alternate channel and token variance normalization of a rotated tile.

    r: [n, d] rotated tile (rows are tokens).  Returns (y, alpha[d], beta[n])
    with r == beta[:, None] * y * alpha[None, :]."""
    y = np.array(r, dtype=np.float64, copy=True)
    n, d = y.shape
    alpha = np.ones(d)
    beta = np.ones(n)
    for _ in range(int(iters)):
        g = _factor(y, axis=0)          # channel step: spread over tokens
        y = y / g
        alpha = alpha * g[0]
        g = _factor(y, axis=1)          # token step: spread over channels
        y = y / g
        beta = beta * g[:, 0]
    return y, alpha, beta


# ----------------------------------------------------------------------------
# Step 4: asymmetric round-to-nearest to low-bit codes [axbrief §diff]
# ----------------------------------------------------------------------------

def rtn(y: np.ndarray, bits: int):
    """Per-row asymmetric round-to-nearest.

    Returns (codes uint8 [n, d], step[n], zero[n], pre[n, d]) where pre is the
    value before rounding, (y - zero) / step."""
    levels = (1 << bits) - 1
    zero = y.min(axis=1)
    step = (y.max(axis=1) - zero) / levels
    safe = np.where(step > 0, step, 1.0)
    pre = np.where(step[:, None] > 0, (y - zero[:, None]) / safe[:, None], 0.0)
    codes = np.clip(np.rint(pre), 0, levels).astype(np.uint8)
    return codes, step, zero, pre


def rtn_channel(y: np.ndarray, bits: int):
    """Per-channel asymmetric round-to-nearest over the tile's tokens: the
    row rule above applied to each column.  Returns (codes uint8 [n, d],
    step[d], zero[d], pre[n, d])."""
    codes, step, zero, pre = rtn(np.asarray(y, np.float64).T, bits)
    return codes.T.copy(), step, zero, pre.T.copy()


@dataclasses.dataclass
class TileQuant:
    codes: np.ndarray     # uint8 [n, d], one code per element
    alpha: np.ndarray     # float32 [d]
    scale: np.ndarray     # float32 [n]  (beta * step)
    offset: np.ndarray    # float32 [n]  (beta * zero)
    pre: np.ndarray       # float64 [n, d], value before rounding
    rotated: np.ndarray   # float64 [n, d]
    normalized: np.ndarray  # float64 [n, d]
    beta: np.ndarray      # float64 [n]
    alpha64: np.ndarray = None   # float64 [d]: the channel factors before rounding
    scale64: np.ndarray = None   # float64 [n]
    offset64: np.ndarray = None  # float64 [n]
    # per-channel rounding (kchan): alpha holds A = alpha * step per channel,
    # scale (and offset) beta per token, zp the zero offset M in code units
    kchan: bool = False
    zp: np.ndarray = None        # float32 [d]
    zp64: np.ndarray = None      # float64 [d]


def quantize_tile(x: np.ndarray, bits: int, iters: int, signs=None, kchan: bool = False) -> TileQuant:
    """The four steps on one tile of 1..T tokens: x fp16 [n, d] (signs: the
    optional sign mask of the randomized rotation, see signs_from_mask;
    kchan: round per channel instead of per token, see the module notes)."""
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[0] < 1:
        raise ValueError("tile must be [n>=1, d]")
    r = fwht(x.astype(np.float64) * signs_from_mask(signs)[None, :])
    y, alpha, beta = sinkhorn(r, iters)
    if kchan:
        codes, step, zero, pre = rtn_channel(y, bits)
        flat = step == 0
        a64 = np.where(flat, alpha * zero, alpha * step)
        m64 = np.where(flat, 1.0, zero / np.where(flat, 1.0, step))
        return TileQuant(codes=codes, alpha=a64.astype(np.float32), scale=beta.astype(np.float32),
                         offset=beta.astype(np.float32), alpha64=a64, scale64=beta, offset64=beta,
                         pre=pre, rotated=r, normalized=y, beta=beta, kchan=True,
                         zp=m64.astype(np.float32), zp64=m64)
    codes, step, zero, pre = rtn(y, bits)
    return TileQuant(codes=codes, alpha=alpha.astype(np.float32),
                     scale=(beta * step).astype(np.float32),
                     offset=(beta * zero).astype(np.float32),
                     alpha64=alpha, scale64=beta * step, offset64=beta * zero,
                     pre=pre, rotated=r, normalized=y, beta=beta)


def dequantize_tile_kchan(codes, chan_scale, zp, beta, signs=None) -> np.ndarray:
    """Restore a per-channel-rounded K tile: rotated row beta * A * (code + M),
    rotated back as in dequantize_tile.  float64 [n, d]."""
    codes = np.asarray(codes, dtype=np.float64)
    rot = np.asarray(beta, np.float64)[:, None] * np.asarray(chan_scale, np.float64)[None, :] * (
        codes + np.asarray(zp, np.float64)[None, :])
    return fwht(rot) * signs_from_mask(signs)[None, :]


def dequantize_tile(codes, alpha, scale, offset, signs=None) -> np.ndarray:
    """Restore a tile [ttj §quant]: rotated row alpha * (S * code + O), rotated
    back with the same (self-inverse) Hadamard, then the signs.  float64 [n, d]."""
    codes = np.asarray(codes, dtype=np.float64)
    rot = np.asarray(alpha, np.float64)[None, :] * (
        np.asarray(scale, np.float64)[:, None] * codes + np.asarray(offset, np.float64)[:, None])
    return fwht(rot) * signs_from_mask(signs)[None, :]


# ----------------------------------------------------------------------------
# Code packing (natural order: channel c at bit (c mod (8/bits)) * bits of
# byte c * bits / 8, low bits first)
# ----------------------------------------------------------------------------

def pack_natural(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    per = 8 // bits
    d = codes.shape[-1]
    out = np.zeros(codes.shape[:-1] + (d // per,), dtype=np.uint8)
    for c in range(d):
        out[..., c // per] |= (codes[..., c] & ((1 << bits) - 1)) << ((c % per) * bits)
    return out


def unpack_natural(packed: np.ndarray, bits: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    per = 8 // bits
    d = packed.shape[-1] * per
    out = np.zeros(packed.shape[:-1] + (d,), dtype=np.uint8)
    for c in range(d):
        out[..., c] = (packed[..., c // per] >> ((c % per) * bits)) & ((1 << bits) - 1)
    return out


# Unit order of a token's 128 codes (the stored order of dense codes and of K
# slots): 16 units of 8 fields, a unit being 8*bits bits (a 32-bit word at 4
# bits, a 16-bit half at 2 bits) taken low bits first; field m of unit u holds
# channel u + 16 m.  Equivalently: natural packing of the channels permuted by
# CODE_ORDER (position 8 u + m <- channel u + 16 m).
CODE_ORDER = np.array([(p // 8) + 16 * (p % 8) for p in range(HEAD_DIM)])


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes uint8 [..., 128] -> bytes [..., 16 * bits] in unit order."""
    return pack_natural(np.asarray(codes, np.uint8)[..., CODE_ORDER], bits)


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    q = unpack_natural(packed, bits)
    out = np.zeros_like(q)
    out[..., CODE_ORDER] = q
    return out


# ----------------------------------------------------------------------------
# Dense (logical) layout: one token run whose tile 0 starts at token 0
# ----------------------------------------------------------------------------

def quantize_dense(x: np.ndarray, tile_tokens: int, bits: int, iters: int, signs=None):
    """x fp16 [n, H, d] -> dict(codes packed [n, H, d*bits/8], alpha [ntiles, H, d],
    scale [n, H], offset [n, H], pre [n, H, d], codes_raw [n, H, d])."""
    n, heads, d = x.shape
    ntiles = (n + tile_tokens - 1) // tile_tokens
    codes = np.zeros((n, heads, d), np.uint8)
    pre = np.zeros((n, heads, d))
    alpha = np.zeros((ntiles, heads, d), np.float32)
    scale = np.zeros((n, heads), np.float32)
    offset = np.zeros((n, heads), np.float32)
    for h in range(heads):
        for j in range(ntiles):
            a, b = j * tile_tokens, min(n, (j + 1) * tile_tokens)
            tq = quantize_tile(x[a:b, h, :], bits, iters, signs)
            codes[a:b, h] = tq.codes
            pre[a:b, h] = tq.pre
            alpha[j, h] = tq.alpha
            scale[a:b, h] = tq.scale
            offset[a:b, h] = tq.offset
    return dict(codes=pack_codes(codes, bits), codes_raw=codes, alpha=alpha, scale=scale,
                offset=offset, pre=pre)


def dequantize_dense(codes_packed, alpha, scale, offset, tile_tokens: int, bits: int, signs=None) -> np.ndarray:
    """Inverse of quantize_dense from the stored codes and fp32 metadata: float64 [n, H, d]."""
    q = unpack_codes(codes_packed, bits)
    n, heads, d = q.shape
    out = np.zeros((n, heads, d))
    for h in range(heads):
        for a in range(0, n, tile_tokens):
            b = min(n, a + tile_tokens)
            out[a:b, h] = dequantize_tile(q[a:b, h], alpha[a // tile_tokens, h], scale[a:b, h],
                                          offset[a:b, h], signs)
    return out


# ----------------------------------------------------------------------------
# Paged layout.  A page holds PAGE_TOKENS consecutive tokens of one sequence;
# the pool is [num_pages][kv_heads][slot bytes].  A slot is
#   codes (16 * d * bits / 8 bytes) | scale fp32[16] | offset fp32[16] | alpha slice fp32[16 d / T]
# The page with index j inside its tile stores alpha[j * 16d/T : (j+1) * 16d/T].
# Code layouts of a slot (d = 128):
#   K slots: each token's codes in unit order (see CODE_ORDER), cut into four
#     blocks of 4 units (4*bits bytes); block k holds, token after token, units
#     4k..4k+3 of each of the 16 tokens.
#   V slots: 64 runs of 4*bits bytes, run l (at byte 4*bits*l) holding the
#     channels l (h = 0) and 64 + l (h = 1) of all 16 tokens, read as
#     little-endian 32-bit words of F = 32/bits fields.  Token t = 4g + r
#     (quad g, r < 4) of channel half h is pair p = 2g + h; word p // (F/4) of
#     the run, field 2m + (r >> 1) + (F/2)(r & 1) with m = p % (F/4), a field
#     being bits [bits*f, bits*(f+1)) of the word.
# Rows of a page past the sequence's end hold code 0, scale 0 and offset 0.
# ----------------------------------------------------------------------------

def slot_layout(bits: int, tile_tokens: int, meta16: bool = False, d: int = HEAD_DIM, page: int = PAGE_TOKENS,
                kchan: bool = False):
    """Byte layout of a slot; meta16: scale, offset and channel factors stored
    as fp16 (2 bytes each) instead of fp32.  kchan (K slots rounded per
    channel): codes | beta fp32[16] | A slice fp32[16 d / T] | M slice fp32[16 d / T],
    the page with index j in its tile holding channels j * 16d/T .. (j+1) * 16d/T - 1."""
    me = 2 if meta16 else 4
    codes = page * d * bits // 8
    alpha_len = page * d // tile_tokens
    if kchan:
        if meta16:
            raise ValueError("per-channel K slots keep fp32 metadata")
        return dict(codes=codes, scale=codes, alpha=codes + 4 * page, zp=codes + 4 * page + 4 * alpha_len,
                    alpha_len=alpha_len, total=codes + 4 * page + 8 * alpha_len, meta_dtype="<f4")
    return dict(codes=codes, scale=codes, offset=codes + me * page, alpha=codes + 2 * me * page,
                alpha_len=alpha_len, total=codes + 2 * me * page + me * alpha_len, meta_dtype="<f2" if meta16 else "<f4")


def slot_bytes(bits: int, tile_tokens: int, meta16: bool = False, kchan: bool = False) -> int:
    return slot_layout(bits, tile_tokens, meta16, kchan=kchan)["total"]


FP16_MAX = 65504.0


def meta_fp16(tq: TileQuant):
    """The tile's metadata as fp16 slots store it.  A power of two moves from
    the per-token scale and offset into the channel factors (exactly: the
    restore alpha * (S * code + O) only sees their product): with M the largest
    |S_t|, |O_t| of the tile, e = floor(log2 M) - 10 (0 if M = 0) and the
    stored values are alpha * 2^e, S * 2^-e, O * 2^-e, each rounded to fp16
    (nearest even; magnitudes beyond the fp16 range saturate at 65504).  This
    keeps S and O within [2^10, 2^11) at the top, far from fp16 overflow, even
    for tiles whose token factors grow large.  Returns (e, alpha16, scale16,
    offset16, alpha, scale, offset) with the last three the scaled float64
    values before rounding."""
    m = float(max(np.abs(tq.scale64).max(), np.abs(tq.offset64).max())) if tq.scale64.size else 0.0
    e = (math.frexp(m)[1] - 1) - 10 if m > 0 else 0
    a, sc, of = tq.alpha64 * 2.0 ** e, tq.scale64 * 2.0 ** -e, tq.offset64 * 2.0 ** -e

    def r16(x):
        return np.clip(x, -FP16_MAX, FP16_MAX).astype(np.float16)
    return e, r16(a), r16(sc), r16(of), a, sc, of


def k_codes_to_bytes(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes uint8 [16, 128] -> K-slot code bytes."""
    per_blk = 4 * bits                                  # bytes of 4 units
    tok = pack_codes(codes, bits)                       # [16, 16 * bits]
    out = np.zeros(PAGE_TOKENS * HEAD_DIM * bits // 8, np.uint8)
    for k in range(4):
        out[k * 16 * per_blk:(k + 1) * 16 * per_blk] = tok[:, k * per_blk:(k + 1) * per_blk].reshape(-1)
    return out


def bytes_to_k_codes(raw: np.ndarray, bits: int) -> np.ndarray:
    per_blk = 4 * bits
    tok = np.zeros((PAGE_TOKENS, 16 * bits), np.uint8)
    for k in range(4):
        tok[:, k * per_blk:(k + 1) * per_blk] = raw[k * 16 * per_blk:(k + 1) * 16 * per_blk].reshape(16, per_blk)
    return unpack_codes(tok, bits)


def _v_field(bits: int, c: int, t: int):
    """(byte offset of the 32-bit word in the V code area, field index) of
    channel c, token t of a page."""
    f_per_word = 32 // bits
    pairs_per_word = f_per_word // 4
    run, h = c % 64, c // 64
    g, r = divmod(t, 4)
    p = 2 * g + h
    word, m = divmod(p, pairs_per_word)
    field = 2 * m + (r >> 1) + (f_per_word // 2) * (r & 1)
    return 4 * bits * run + 4 * word, field


_V_MAPS = {}


def _v_map(bits: int):
    """For every (token, channel) of a page: index of its 32-bit word in the
    V-slot code area and the bit shift of its field (from _v_field)."""
    if bits not in _V_MAPS:
        word = np.zeros((PAGE_TOKENS, HEAD_DIM), np.int64)
        shift = np.zeros((PAGE_TOKENS, HEAD_DIM), np.int64)
        for t in range(PAGE_TOKENS):
            for c in range(HEAD_DIM):
                off, field = _v_field(bits, c, t)
                word[t, c] = off // 4
                shift[t, c] = bits * field
        _V_MAPS[bits] = (word, shift)
    return _V_MAPS[bits]


def v_codes_to_bytes(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes uint8 [16, 128] -> V-slot code bytes."""
    word, shift = _v_map(bits)
    words = np.zeros(PAGE_TOKENS * HEAD_DIM * bits // 32, np.uint64)
    vals = (np.asarray(codes, np.uint64) & np.uint64((1 << bits) - 1)) << shift.astype(np.uint64)
    np.bitwise_or.at(words, word.ravel(), vals.ravel())
    return words.astype("<u4").view(np.uint8).copy()


def bytes_to_v_codes(raw: np.ndarray, bits: int) -> np.ndarray:
    word, shift = _v_map(bits)
    words = np.ascontiguousarray(raw).view("<u4").astype(np.int64)
    return ((words[word] >> shift) & ((1 << bits) - 1)).astype(np.uint8)


def new_pool(num_pages: int, kv_heads: int, bits: int, tile_tokens: int, meta16: bool = False,
             kchan: bool = False) -> np.ndarray:
    return np.zeros((num_pages, kv_heads, slot_bytes(bits, tile_tokens, meta16, kchan)), np.uint8)


def write_slot_kchan(pool, page, head, bits, tile_tokens, codes16, beta16, a_slice, m_slice):
    lay = slot_layout(bits, tile_tokens, kchan=True)
    slot = pool[page, head]
    slot[:lay["codes"]] = k_codes_to_bytes(codes16, bits)
    slot[lay["scale"]:lay["alpha"]] = np.asarray(beta16, "<f4").view(np.uint8)
    slot[lay["alpha"]:lay["zp"]] = np.asarray(a_slice, "<f4").view(np.uint8)
    slot[lay["zp"]:lay["total"]] = np.asarray(m_slice, "<f4").view(np.uint8)


def read_slot_kchan(pool, page, head, bits, tile_tokens):
    """(codes [16, d], beta [16], A slice, M slice) of a per-channel K slot."""
    lay = slot_layout(bits, tile_tokens, kchan=True)
    slot = np.ascontiguousarray(pool[page, head])
    return (bytes_to_k_codes(slot[:lay["codes"]], bits), slot[lay["scale"]:lay["alpha"]].view("<f4").astype(np.float32),
            slot[lay["alpha"]:lay["zp"]].view("<f4").astype(np.float32),
            slot[lay["zp"]:lay["total"]].view("<f4").astype(np.float32))


def write_slot(pool, page, head, role, bits, tile_tokens, codes16, scale16, offset16, alpha_slice, meta16=False):
    lay = slot_layout(bits, tile_tokens, meta16)
    dt = lay["meta_dtype"]
    enc = k_codes_to_bytes if role == "K" else v_codes_to_bytes
    slot = pool[page, head]
    slot[:lay["codes"]] = enc(codes16, bits)
    slot[lay["scale"]:lay["offset"]] = np.asarray(scale16, dt).view(np.uint8)
    slot[lay["offset"]:lay["alpha"]] = np.asarray(offset16, dt).view(np.uint8)
    slot[lay["alpha"]:lay["total"]] = np.asarray(alpha_slice, dt).view(np.uint8)


def read_slot(pool, page, head, role, bits, tile_tokens, meta16=False):
    lay = slot_layout(bits, tile_tokens, meta16)
    dt = lay["meta_dtype"]
    slot = np.ascontiguousarray(pool[page, head])
    dec = bytes_to_k_codes if role == "K" else bytes_to_v_codes
    codes = dec(slot[:lay["codes"]], bits)
    scale = slot[lay["scale"]:lay["offset"]].view(dt).astype(np.float32)
    offset = slot[lay["offset"]:lay["alpha"]].view(dt).astype(np.float32)
    alpha = slot[lay["alpha"]:lay["total"]].view(dt).astype(np.float32)
    return codes, scale, offset, alpha


def _store_tile(pool, table_row, head, role, bits, tile_tokens, tile_index, tq: TileQuant, meta16=False):
    """Write one (possibly partial) quantized tile into its pages."""
    ppt = tile_tokens // PAGE_TOKENS
    alen = PAGE_TOKENS * HEAD_DIM // tile_tokens
    n = tq.codes.shape[0]
    if tq.kchan:
        for j in range(ppt):
            page = int(table_row[tile_index * ppt + j])
            if page < 0:
                raise ValueError("block table has no page for a started tile")
            codes16 = np.zeros((PAGE_TOKENS, HEAD_DIM), np.uint8)
            beta16 = np.zeros(PAGE_TOKENS, np.float32)
            a, b = j * PAGE_TOKENS, min(n, (j + 1) * PAGE_TOKENS)
            if b > a:
                codes16[:b - a] = tq.codes[a:b]
                beta16[:b - a] = tq.scale[a:b]
            write_slot_kchan(pool, page, head, bits, tile_tokens, codes16, beta16,
                             tq.alpha[j * alen:(j + 1) * alen], tq.zp[j * alen:(j + 1) * alen])
        return
    alpha, scale, offset = tq.alpha, tq.scale, tq.offset
    if meta16:
        _, alpha, scale, offset, _, _, _ = meta_fp16(tq)
    for j in range(ppt):
        page = int(table_row[tile_index * ppt + j])
        if page < 0:
            raise ValueError("block table has no page for a started tile")
        codes16 = np.zeros((PAGE_TOKENS, HEAD_DIM), np.uint8)
        scale16 = np.zeros(PAGE_TOKENS, np.float32)
        offset16 = np.zeros(PAGE_TOKENS, np.float32)
        a, b = j * PAGE_TOKENS, min(n, (j + 1) * PAGE_TOKENS)
        if b > a:
            codes16[:b - a] = tq.codes[a:b]
            scale16[:b - a] = scale[a:b]
            offset16[:b - a] = offset[a:b]
        write_slot(pool, page, head, role, bits, tile_tokens, codes16, scale16, offset16,
                   alpha[j * alen:(j + 1) * alen], meta16)


def quantize_to_pages(k, v, cu_seqlens, table, tile_tokens, bits_k, bits_v, iters,
                      pool_k, pool_v, staging_k=None, staging_v=None, signs=None, meta16=False, kchan=False):
    """Quantize every tile of every sequence into the page pools (in place).

    k, v: fp16 [total_tokens, Hkv, d]; table: int32 [S, max_blocks].  A tail
    that does not fill its tile is also copied, as fp16 rows, to staging
    [S, T, Hkv, d] so that later appends can re-quantize the partial tile.
    Returns dict of pre-rounding values per (seq, head, role) for the tests."""
    heads = k.shape[1]
    pre = {}
    for s in range(len(cu_seqlens) - 1):
        a0, a1 = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        n = a1 - a0
        for role, x, pool, bits, stg in (("K", k, pool_k, bits_k, staging_k),
                                         ("V", v, pool_v, bits_v, staging_v)):
            for h in range(heads):
                pre_rows = np.zeros((n, HEAD_DIM))
                for j in range((n + tile_tokens - 1) // tile_tokens):
                    a, b = j * tile_tokens, min(n, (j + 1) * tile_tokens)
                    tq = quantize_tile(x[a0 + a:a0 + b, h, :], bits, iters, signs, kchan and role == "K")
                    pre_rows[a:b] = tq.pre
                    _store_tile(pool, table[s], h, role, bits, tile_tokens, j, tq, meta16)
                pre[(s, h, role)] = pre_rows
            tail = n % tile_tokens
            if stg is not None and tail:
                stg[s, :tail] = x[a1 - tail:a1]
    return pre


def append_and_requant(k_new, v_new, lens_before, table, tile_tokens, bits_k, bits_v, iters,
                       pool_k, pool_v, staging_k, staging_v, signs=None, meta16=False, kchan=False):
    """Append one token per sequence and re-quantize its (partial) tile from the
    fp16 staging rows.  k_new, v_new fp16 [S, Hkv, d].  Returns pre-rounding
    values per (seq, head, role) of the re-quantized tile rows."""
    heads = k_new.shape[1]
    pre = {}
    for s in range(k_new.shape[0]):
        pos = int(lens_before[s])
        j, r = divmod(pos, tile_tokens)
        staging_k[s, r] = k_new[s]
        staging_v[s, r] = v_new[s]
        for role, stg, pool, bits in (("K", staging_k, pool_k, bits_k), ("V", staging_v, pool_v, bits_v)):
            for h in range(heads):
                tq = quantize_tile(stg[s, :r + 1, h, :], bits, iters, signs, kchan and role == "K")
                _store_tile(pool, table[s], h, role, bits, tile_tokens, j, tq, meta16)
                pre[(s, h, role)] = tq.pre
    return pre


def read_sequence(pool, table_row, seq_len, head, role, bits, tile_tokens, signs=None, meta16=False, kchan=False):
    """Decode one (sequence, kv head) from the pages with this module's own
    reader: returns (restored tokens float64 [L, d], codes [L, d], alpha per
    tile [ntiles, d], scale [L], offset [L]).  With kchan (K slots rounded
    per channel): (restored, codes, A per tile [ntiles, d], beta [L], M per
    tile [ntiles, d])."""
    ppt = tile_tokens // PAGE_TOKENS
    ntiles = (seq_len + tile_tokens - 1) // tile_tokens
    if kchan and role == "K":
        alen = PAGE_TOKENS * HEAD_DIM // tile_tokens
        codes = np.zeros((ntiles * tile_tokens, HEAD_DIM), np.uint8)
        beta = np.zeros(ntiles * tile_tokens, np.float32)
        cs = np.zeros((ntiles, HEAD_DIM), np.float32)
        zp = np.zeros((ntiles, HEAD_DIM), np.float32)
        for j in range(ntiles):
            for p in range(ppt):
                c16, b16, a_sl, m_sl = read_slot_kchan(pool, int(table_row[j * ppt + p]), head, bits, tile_tokens)
                t0 = j * tile_tokens + p * PAGE_TOKENS
                codes[t0:t0 + PAGE_TOKENS] = c16
                beta[t0:t0 + PAGE_TOKENS] = b16
                cs[j, p * alen:(p + 1) * alen] = a_sl
                zp[j, p * alen:(p + 1) * alen] = m_sl
        out = np.zeros((seq_len, HEAD_DIM))
        for j in range(ntiles):
            a, b = j * tile_tokens, min(seq_len, (j + 1) * tile_tokens)
            out[a:b] = dequantize_tile_kchan(codes[a:b], cs[j], zp[j], beta[a:b], signs)
        return out, codes[:seq_len], cs, beta[:seq_len], zp
    codes = np.zeros((ntiles * tile_tokens, HEAD_DIM), np.uint8)
    scale = np.zeros(ntiles * tile_tokens, np.float32)
    offset = np.zeros(ntiles * tile_tokens, np.float32)
    alpha = np.zeros((ntiles, HEAD_DIM), np.float32)
    alen = PAGE_TOKENS * HEAD_DIM // tile_tokens
    for j in range(ntiles):
        for p in range(ppt):
            page = int(table_row[j * ppt + p])
            c16, s16, o16, a = read_slot(pool, page, head, role, bits, tile_tokens, meta16)
            t0 = j * tile_tokens + p * PAGE_TOKENS
            codes[t0:t0 + PAGE_TOKENS] = c16
            scale[t0:t0 + PAGE_TOKENS] = s16
            offset[t0:t0 + PAGE_TOKENS] = o16
            alpha[j, p * alen:(p + 1) * alen] = a
    out = np.zeros((seq_len, HEAD_DIM))
    for j in range(ntiles):
        a, b = j * tile_tokens, min(seq_len, (j + 1) * tile_tokens)
        out[a:b] = dequantize_tile(codes[a:b], alpha[j], scale[a:b], offset[a:b], signs)
    return out, codes[:seq_len], alpha, scale[:seq_len], offset[:seq_len]


# ----------------------------------------------------------------------------
# Decode attention [aitrends §TL;DR]: one new query per sequence and head over
# every cached token, reading the quantized pages (here: restoring them in
# float64 with the reader above; the GPU path never restores fp16).
# ----------------------------------------------------------------------------

def attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray, sm_scale: float) -> np.ndarray:
    """Plain single-query softmax attention in float64."""
    s = sm_scale * (keys.astype(np.float64) @ np.asarray(q, np.float64))
    s = s - s.max()
    p = np.exp(s)
    p = p / p.sum()
    return p @ values.astype(np.float64)


def attention_abs_scale(q: np.ndarray, keys: np.ndarray, values: np.ndarray, sm_scale: float,
                        key_terms=None) -> float:
    """The size of the terms an attention output is made of (its rounding
    scale in fp32): max over channels c of sum_t p_t |v_t,c| (what the output
    channel sums), plus, with key_terms, max over c of
    sum_t p_t |v_t,c - o_c| sm_scale key_terms_t: the output moves by
    p_t (v_t,c - o_c) per unit of score t, and a score evaluated in fp32
    carries a rounding proportional to the terms it is summed from
    (key_score_terms below), not to its own value."""
    s = sm_scale * (keys.astype(np.float64) @ np.asarray(q, np.float64))
    p = np.exp(s - s.max())
    p = p / p.sum()
    vals = values.astype(np.float64)
    out = float((p @ np.abs(vals)).max())
    if key_terms is not None:
        o = p @ vals
        out += float(((p * sm_scale * np.asarray(key_terms, np.float64)) @ np.abs(vals - o[None])).max())
    return out


def key_score_parts(q, codes, alpha, scale, offset, tile_tokens, signs=None):
    """The two terms each cached token's score q . k is the sum of.  The
    restored key is D H (alpha * (S code + O)) [ttj §quant], so with
    qt = alpha * H D q (rotated query times the channel factors) the score is
    S sum_c qt_c code_c + O sum_c qt_c.  Returns the two terms per token
    (float64 [L] each); alpha per tile [ntiles, d] (read_sequence's layout)."""
    hq = fwht(np.asarray(q, np.float64) * signs_from_mask(signs))
    n = len(scale)
    qt = hq[None] * np.asarray(alpha, np.float64)[np.arange(n) // tile_tokens]
    return (np.asarray(scale, np.float64) * (qt * np.asarray(codes, np.float64)).sum(1),
            np.asarray(offset, np.float64) * qt.sum(1))


def key_score_parts_kchan(q, codes, chan_scale, beta, zp, tile_tokens, signs=None):
    """key_score_parts for per-channel K tiles: the restored key is
    D H (beta * A * (code + M)), so with qt = A * H D q the score is
    beta sum_c qt_c code_c + beta sum_c qt_c M_c (A, M per tile [ntiles, d])."""
    hq = fwht(np.asarray(q, np.float64) * signs_from_mask(signs))
    n = len(beta)
    tix = np.arange(n) // tile_tokens
    qt = hq[None] * np.asarray(chan_scale, np.float64)[tix]
    b = np.asarray(beta, np.float64)
    return b * (qt * np.asarray(codes, np.float64)).sum(1), b * (qt * np.asarray(zp, np.float64)[tix]).sum(1)


def key_score_terms(q, codes, alpha, scale, offset, tile_tokens, signs=None, kchan=False) -> np.ndarray:
    """|first| + |second| of key_score_parts per token: in tiles whose per-token
    factors are large (S and O of 1e4 and more in tiles of a few tokens) the
    two terms nearly cancel, and a score evaluated in fp32 carries a rounding
    proportional to them, not to its own value."""
    parts = key_score_parts_kchan if kchan else key_score_parts
    a, b = parts(q, codes, alpha, scale, offset, tile_tokens, signs)
    return np.abs(a) + np.abs(b)


def paged_decode_attn(q, table, seq_lens, pool_k, pool_v, tile_tokens, bits_k, bits_v,
                      sm_scale=None, return_scale=False, signs=None, meta16=False, kchan=False):
    """q fp16 [S, Hq, d]; seq_lens count every cached token (the newest included).
    Query head h reads kv head h // (Hq / Hkv).  Returns float64 [S, Hq, d]
    (and, with return_scale, attention_abs_scale per [S, Hq], score terms
    included)."""
    s_n, hq, d = q.shape
    hkv = pool_k.shape[1]
    g = hq // hkv
    sm = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    out = np.zeros((s_n, hq, d))
    scale = np.zeros((s_n, hq))
    for s in range(s_n):
        for kh in range(hkv):
            kx, kc, ka, ks, ko = read_sequence(pool_k, table[s], int(seq_lens[s]), kh, "K", bits_k, tile_tokens,
                                               signs, meta16, kchan)
            vx = read_sequence(pool_v, table[s], int(seq_lens[s]), kh, "V", bits_v, tile_tokens, signs, meta16)[0]
            for h in range(kh * g, (kh + 1) * g):
                out[s, h] = attention(q[s, h].astype(np.float64), kx, vx, sm)
                if return_scale:
                    terms = key_score_terms(q[s, h], kc, ka, ks, ko, tile_tokens, signs, kchan)
                    scale[s, h] = attention_abs_scale(q[s, h], kx, vx, sm, terms)
    return (out, scale) if return_scale else out


def paged_multi_query_attn(q, table, seq_lens, pool_k, pool_v, tile_tokens, bits_k, bits_v,
                           sm_scale=None, return_scale=False, signs=None, meta16=False, kchan=False):
    """Several queries per sequence over the same compressed pages (the read
    path of [aitrends §TL;DR], with a causal mask): q fp16 [S, n_q, Hq, d]
    holds the n_q newest tokens of each sequence, already in the cache, so
    seq_lens counts them; query i sits at position seq_lens[s] - n_q + i and
    attends to the cached tokens 0 .. that position.  n_q = 1 is the decode
    step.  A query at a negative position (a sequence shorter than n_q) sees
    no token: its output row is zero, as the library defines it.  Returns
    float64 [S, n_q, Hq, d] (and, with return_scale, attention_abs_scale per
    [S, n_q, Hq], score terms included)."""
    s_n, n_q, hq, d = q.shape
    hkv = pool_k.shape[1]
    g = hq // hkv
    sm = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    out = np.zeros((s_n, n_q, hq, d))
    scale = np.zeros((s_n, n_q, hq))
    for s in range(s_n):
        n = int(seq_lens[s])
        for kh in range(hkv):
            kx, kc, ka, ks, ko = read_sequence(pool_k, table[s], n, kh, "K", bits_k, tile_tokens, signs, meta16, kchan)
            vx = read_sequence(pool_v, table[s], n, kh, "V", bits_v, tile_tokens, signs, meta16)[0]
            for i in range(n_q):
                visible = n - n_q + i + 1
                if visible <= 0:
                    continue
                for h in range(kh * g, (kh + 1) * g):
                    qv = q[s, i, h].astype(np.float64)
                    out[s, i, h] = attention(qv, kx[:visible], vx[:visible], sm)
                    if return_scale:
                        terms = key_score_terms(qv, kc[:visible], ka, ks[:visible], ko if kchan else ko[:visible],
                                                tile_tokens, signs, kchan)
                        scale[s, i, h] = attention_abs_scale(qv, kx[:visible], vx[:visible], sm, terms)
    return (out, scale) if return_scale else out


# ----------------------------------------------------------------------------
# Baselines for the long-context comparison: the same paged decode attention on
# fp16 pages and on fp8 (OCP E4M3) pages with one scale per tensor, the two
# modes the aitrends.kr page (article 74976, TL;DR) runs beside its compressed
# cache.  Layouts (per page, per kv head): K page [16 tokens][128 channels],
# V page [128 channels][16 tokens] (channel-major, as paged attention usually
# keeps V).  Rows past the sequence's end are 0.
# ----------------------------------------------------------------------------

def fp8_encode(x: np.ndarray, scale: float) -> np.ndarray:
    """x / scale rounded to OCP E4M3 (nearest, ties to even) by torch's CPU
    float8_e4m3fn conversion; returns the code bytes."""
    import torch
    t = torch.from_numpy(np.asarray(x, np.float32) / np.float32(scale))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def fp8_decode(b: np.ndarray, scale: float) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.double().numpy() * float(scale)


def fp8_scale(x: np.ndarray) -> float:
    """Per-tensor scale amax / 448 (448 = largest finite E4M3 value)."""
    amax = float(np.max(np.abs(np.asarray(x, np.float32))))
    return amax / 448.0 if amax > 0 else 1.0


def new_baseline_pool(num_pages: int, kv_heads: int, fp8: bool) -> np.ndarray:
    return np.zeros((num_pages, kv_heads, PAGE_TOKENS * HEAD_DIM), np.uint8 if fp8 else np.float16)


def fill_pages_baseline(k, v, cu_seqlens, table, pool_k, pool_v, fp8=False, k_scale=1.0, v_scale=1.0):
    """Write a prefill into fp16 or fp8 page pools (in place)."""
    heads = k.shape[1]
    for s in range(len(cu_seqlens) - 1):
        a0, a1 = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        n = a1 - a0
        for j in range((n + PAGE_TOKENS - 1) // PAGE_TOKENS):
            page = int(table[s][j])
            rows = slice(a0 + j * PAGE_TOKENS, min(a1, a0 + (j + 1) * PAGE_TOKENS))
            for h in range(heads):
                kp = np.zeros((PAGE_TOKENS, HEAD_DIM), np.float16)
                vp = np.zeros((PAGE_TOKENS, HEAD_DIM), np.float16)
                m = rows.stop - rows.start
                kp[:m] = k[rows, h]
                vp[:m] = v[rows, h]
                vt = np.ascontiguousarray(vp.T)           # [channel][token]
                if fp8:
                    kb = fp8_encode(kp, k_scale)
                    vb = fp8_encode(vt, v_scale)
                    kb[m:] = 0
                    vb[:, m:] = 0
                    pool_k[page, h] = kb.reshape(-1)
                    pool_v[page, h] = vb.reshape(-1)
                else:
                    pool_k[page, h] = kp.reshape(-1)
                    pool_v[page, h] = vt.reshape(-1)


def append_pages_baseline(k_new, v_new, lens_before, table, pool_k, pool_v, fp8=False, k_scale=1.0, v_scale=1.0):
    """One decode token per sequence written at position lens_before[s] of
    fp16 or fp8 pools (in place), encoded as fill_pages_baseline encodes: K
    row p % 16 of the page holding p, V column p % 16 of it."""
    for s in range(k_new.shape[0]):
        p = int(lens_before[s])
        page, r = int(table[s][p // PAGE_TOKENS]), p % PAGE_TOKENS
        for h in range(k_new.shape[1]):
            kp = pool_k[page, h].reshape(PAGE_TOKENS, HEAD_DIM)
            vp = pool_v[page, h].reshape(HEAD_DIM, PAGE_TOKENS)
            if fp8:
                kp[r] = fp8_encode(k_new[s, h], k_scale)
                vp[:, r] = fp8_encode(v_new[s, h], v_scale)
            else:
                kp[r] = k_new[s, h]
                vp[:, r] = v_new[s, h]


def read_baseline_sequence(pool, table_row, seq_len, head, role, fp8=False, scale=1.0):
    """Restored tokens float64 [L, 128] of one (sequence, kv head)."""
    out = np.zeros((seq_len, HEAD_DIM))
    for j in range((seq_len + PAGE_TOKENS - 1) // PAGE_TOKENS):
        raw = pool[int(table_row[j]), head]
        raw = raw.reshape(PAGE_TOKENS, HEAD_DIM) if role == "K" else raw.reshape(HEAD_DIM, PAGE_TOKENS).T
        vals = fp8_decode(raw, scale) if fp8 else raw.astype(np.float64)
        m = min(PAGE_TOKENS, seq_len - j * PAGE_TOKENS)
        out[j * PAGE_TOKENS:j * PAGE_TOKENS + m] = vals[:m]
    return out


def rematerialize_pages(pool_k, pool_v, table, seq_lens, tile_tokens, bits_k, bits_v, base_k, base_v,
                        signs=None, meta16=False, kchan=False):
    """The re-materializing read path's first half: every cached token restored
    from the quantized pages (read_sequence, float64) and written, rounded to
    fp16, into fp16 baseline pools with the same block table (in place).  Pages
    past a sequence's last token are left alone; rows of its last page past the
    end are 0 (as fill_pages_baseline writes them)."""
    heads = pool_k.shape[1]
    for s in range(len(seq_lens)):
        n = int(seq_lens[s])
        if n == 0:
            continue
        kx = np.stack([read_sequence(pool_k, table[s], n, h, "K", bits_k, tile_tokens, signs, meta16, kchan)[0]
                       for h in range(heads)], 1)
        vx = np.stack([read_sequence(pool_v, table[s], n, h, "V", bits_v, tile_tokens, signs, meta16)[0]
                       for h in range(heads)], 1)
        fill_pages_baseline(kx.astype(np.float16), vx.astype(np.float16), np.array([0, n]), table[s:s + 1],
                            base_k, base_v)


def paged_decode_attn_baseline(q, table, seq_lens, pool_k, pool_v, fp8=False, k_scale=1.0, v_scale=1.0,
                               sm_scale=None):
    s_n, hq, d = q.shape
    hkv = pool_k.shape[1]
    g = hq // hkv
    sm = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    out = np.zeros((s_n, hq, d))
    for s in range(s_n):
        for kh in range(hkv):
            kx = read_baseline_sequence(pool_k, table[s], int(seq_lens[s]), kh, "K", fp8, k_scale)
            vx = read_baseline_sequence(pool_v, table[s], int(seq_lens[s]), kh, "V", fp8, v_scale)
            for h in range(kh * g, (kh + 1) * g):
                out[s, h] = attention(q[s, h].astype(np.float64), kx, vx, sm)
    return out
