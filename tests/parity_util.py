"""Comparison rules of the GPU parity tests (GPU output vs the CPU oracle).

* Codes: bit-exact, except elements whose oracle pre-rounding value lies
  within WINDOW of a rounding boundary k + 1/2 (the oracle decides in float64;
  the kernel decides in fp32 on tiles of 16 or more tokens and in float64 on
  shorter ones).  Every mismatch must be in that window; the number of
  elements in the window and the number of mismatches are reported.
* Channel factors, token scales and offsets: relative error <= META_RTOL on
  every tile.  On tiles of 16 or more tokens the kernel works in fp32 (eps
  6e-8); a spread computed over values whose mean-square is m times their
  variance carries ~eps*m relative error, and the guard admits m up to 1e4
  (spread down to 1% of RMS), so near-degenerate channels reach ~1e-4.
  Shorter tiles are quantized in float64 by the kernel, so their metadata
  agree to fp32 rounding.  The metadata are also checked through their
  effect: the oracle's codes restored with the GPU metadata must match the
  same codes restored with the oracle's metadata within DEQ_RTOL.  The codes
  check above is the binding one: it fails if a metadata error moves any code
  outside the window.
* Restored values: |gpu - ref| <= DEQ_RTOL * max(|ref|, rms of the token row).
* Attention outputs: absolute error <= ATTN_ATOL (fp32 accumulation), plus
  ATTN_ULPS units of 2^-24 times the output's own rounding scale, where the
  oracle supplies it (oracle.attention_abs_scale): max_c sum_t p_t |v_t,c|
  over the restored values, plus max_c sum_t p_t |v_t,c - o_c| times the
  scaled magnitudes of the two terms each score is the sum of
  (oracle.key_score_terms: S sum qt code and O sum qt).  For outputs of unit
  size over tiles of many tokens both are negligible against ATTN_ATOL.
  They matter where the method itself restores large values: a tile of two
  tokens put through 5 normalization iterations and 2-bit rounding (a tail
  tile of the heavy-tailed workload, one token after the append) restores
  N(0, 1) values of size ~3 as values up to ~1.5e4 (the oracle's own
  restore), so attention outputs there reach ~1.3e4 in the oracle itself,
  where 2e-3 is two fp32 ulps of the output; and its keys' S and O reach
  1e4..1e5 and cancel, so its scores carry fp32 roundings of terms ~1e4 in
  logit units, which the probabilities pass on to every output of the head
  (measured: 3.2e-3 at an output of 14 whose V-side scale is 17).  The term
  admits a fixed number of fp32 roundings of those scales.
"""
import numpy as np

WINDOW = 1e-3
META_RTOL = 1e-4
DEQ_RTOL = 1e-3
ATTN_ATOL = 2e-3
ATTN_ULPS = 16


def near_boundary(pre: np.ndarray) -> np.ndarray:
    return np.abs(pre - np.floor(pre) - 0.5) < WINDOW


def compare_codes(gpu_codes: np.ndarray, ref_codes: np.ndarray, pre: np.ndarray, what: str = ""):
    """Returns (n_elements, n_in_window, n_mismatch); asserts mismatches are in the window."""
    gpu_codes = np.asarray(gpu_codes)
    ref_codes = np.asarray(ref_codes)
    assert gpu_codes.shape == ref_codes.shape == pre.shape, (gpu_codes.shape, ref_codes.shape, pre.shape)
    window = near_boundary(pre)
    mism = gpu_codes != ref_codes
    bad = mism & ~window
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(i), int(gpu_codes[tuple(i)]), int(ref_codes[tuple(i)]), float(pre[tuple(i)]))
                  for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} code mismatches outside the window, e.g. {detail}")
    return int(mism.size), int(window.sum()), int(mism.sum())


def assert_rel(gpu, ref, rtol, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref) / np.maximum(np.abs(ref), 1e-30)
    ok = (err <= rtol) | (np.abs(gpu - ref) <= 1e-30)
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: rel err {err[tuple(i)]:.3e} at {tuple(i)} "
                             f"(gpu {gpu[tuple(i)]!r}, ref {ref[tuple(i)]!r}); max {err.max():.3e}")
    return float(err.max()) if err.size else 0.0


def assert_dequant(gpu, ref, what="", rtol=DEQ_RTOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
    tol = rtol * np.maximum(np.abs(ref), rms)
    bad = np.abs(gpu - ref) > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} restored values off, e.g. {tuple(i)} "
                             f"gpu {gpu[tuple(i)]} ref {ref[tuple(i)]}")
    den = np.broadcast_to(np.maximum(np.abs(ref), rms), ref.shape)
    ratio = np.divide(np.abs(gpu - ref), den, out=np.zeros(ref.shape), where=den > 0)   # all-zero rows: exact
    return float(ratio.max()) if ratio.size else 0.0


def attn_tol(scale=None):
    """Per-row attention tolerance; scale [...] as from the oracle's
    attention_abs_scale (None: the absolute bar alone)."""
    if scale is None:
        return ATTN_ATOL
    return ATTN_ATOL + ATTN_ULPS * 2.0 ** -24 * np.asarray(scale, np.float64)[..., None]


def assert_attn(gpu, ref, what="", scale=None):
    err = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    tol = np.broadcast_to(attn_tol(scale), err.shape)
    if not (err <= tol).all():
        i = np.argwhere(err > tol)[0]
        raise AssertionError(f"{what}: attention abs err {err[tuple(i)]:.3e} > {tol[tuple(i)]:.3e} at {tuple(i)} "
                             f"(ref {np.asarray(ref)[tuple(i)]:.6g}); max err {err.max():.3e}")
    return float(err.max())


def check_tile_metadata(codes_ref, ga, gs, go, ra, rs, ro, restore, what=""):
    """Metadata of one tile (alpha [128], scale/offset [n]) per the rules above.
    `restore(codes, alpha, scale, offset)` is the oracle's restore."""
    assert_rel(ga, ra, META_RTOL, f"{what} alpha")
    assert_rel(gs, rs, META_RTOL, f"{what} scale")
    assert_rel(go, ro, META_RTOL, f"{what} offset")
    assert_dequant(restore(codes_ref, ga, gs, go), restore(codes_ref, ra, rs, ro), f"{what} metadata effect",
                   DEQ_RTOL)


def check_tile_metadata_fp16(tq, ga, gs, go, what=""):
    """fp16 metadata of one tile (as stored: alpha*2^e, S*2^-e, O*2^-e in fp16)
    against the oracle's tile `tq`.  Each value equals the oracle's rounding,
    or is its fp16 neighbour where the oracle's unrounded value lies within
    META_RTOL of the rounding boundary between the two (the kernel rounds a
    fp32 value that agrees with the oracle's to META_RTOL).  The tile's power
    of two may differ by one where its largest |S|, |O| lies within META_RTOL
    of a power of two (then every stored value moves by that factor)."""
    import oracle as orc
    e, a16, s16, o16, a, s, o = orc.meta_fp16(tq)
    ga, gs, go = (np.asarray(x, np.float64) for x in (ga, gs, go))
    i = int(np.argmax(np.abs(a16.astype(np.float64))))
    k = int(np.round(np.log2(ga[i] / float(a16[i])))) if a16[i] != 0 and ga[i] != 0 else 0
    if k != 0:
        m = float(max(np.abs(tq.scale64).max(), np.abs(tq.offset64).max()))
        p2 = 2.0 ** np.round(np.log2(m))
        assert abs(k) == 1 and abs(m - p2) <= META_RTOL * p2, f"{what}: tile exponent off by {k} (M = {m!r})"
        a, s, o = a * 2.0 ** k, s * 2.0 ** -k, o * 2.0 ** -k
        a16, s16, o16 = (np.clip(x, -orc.FP16_MAX, orc.FP16_MAX).astype(np.float16) for x in (a, s, o))
    for g, r16, u, name in ((ga, a16, a, "alpha"), (gs, s16, s, "scale"), (go, o16, o, "offset")):
        r = r16.astype(np.float64)
        same = g == r
        up = np.nextafter(r16, np.float16(np.inf)).astype(np.float64)
        dn = np.nextafter(r16, np.float16(-np.inf)).astype(np.float64)
        nb = (g == up) | (g == dn)
        near = np.abs(u - (g + r) / 2) <= META_RTOL * np.abs(u)
        bad = ~same & ~(nb & near)
        if bad.any():
            j = int(np.argwhere(bad)[0][0])
            raise AssertionError(f"{what} {name}[{j}]: gpu {g[j]!r} oracle fp16 {r[j]!r} (unrounded {u[j]!r})")
    return int((ga != a16.astype(np.float64)).sum() + (gs != s16.astype(np.float64)).sum() +
               (go != o16.astype(np.float64)).sum())


def check_tile_metadata_kchan(tq, ga, gb, gm, what=""):
    """Per-channel K tile (oracle tile `tq`): the token factors beta within
    META_RTOL; the channel scales A and zero offsets M through their effect:
    the oracle's codes restored with the GPU's beta, A, M against the same
    codes restored with the oracle's, within DEQ_RTOL.  (A = alpha step and
    M = min / step are each ill-conditioned in a channel whose range is tiny
    next to its minimum, while their product in the restore is not.)"""
    import oracle as orc
    assert_rel(gb, tq.scale64, META_RTOL, f"{what} beta")
    assert_dequant(orc.dequantize_tile_kchan(tq.codes, ga, gm, gb),
                   orc.dequantize_tile_kchan(tq.codes, tq.alpha64, tq.zp64, tq.scale64),
                   f"{what} channel scale / zero offset effect")
