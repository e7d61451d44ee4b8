"""Pins for the oracle's quantizers (CPU only).

Each test checks the oracle against something other than itself: values on
an exactly representable grid, the round-trip bound |x - deq(q(x))| <= s/2,
exact rational arithmetic, brute-force nearest-centroid search, and a full
sort for the outlier selection.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant

F32 = np.float32


def _groups(rng, n, G, scale=1.0, dtype=np.float16):
    return (rng.standard_normal((n, G)) * scale).astype(dtype).astype(F32)


# ---------------------------------------------------------------- A1 min/max
def test_asym_minmax_on_grid_gives_exact_codes():
    # z = -1.5, s = 0.5 are exact in fp16; x = z + k*s must give code k and
    # dequantize exactly.
    k = np.array([0, 15, 3, 7, 8, 1, 14, 2] * 4)
    x = (F32(-1.5) + k.astype(F32) * F32(0.5))[None, :]
    codes, s, z = quant.asym_minmax(x, 4)
    assert float(s[0]) == 0.5 and float(z[0]) == -1.5
    assert np.array_equal(codes[0], k)
    deq = codes.astype(np.float64) * float(s[0]) + float(z[0])
    assert np.array_equal(deq, x.astype(np.float64))


def test_asym_minmax_3bit_on_grid():
    k = np.arange(64) % 8
    x = (F32(2.0) + k.astype(F32) * F32(0.25))[None, :]
    codes, s, z = quant.asym_minmax(x, 3)
    assert float(s[0]) == 0.25 and float(z[0]) == 2.0
    assert np.array_equal(codes[0], k)


def test_round_half_even():
    # lo = 0, hi = 15 -> s = 1 exactly; 2.5 -> 2, 3.5 -> 4, 0.5 -> 0
    x = np.array([[0, 15, 2.5, 3.5, 0.5, 14.5, 6, 7]], dtype=F32)
    codes, s, z = quant.asym_minmax(x, 4)
    assert float(s[0]) == 1.0
    assert codes[0].tolist() == [0, 15, 2, 4, 0, 14, 6, 7]


def test_degenerate_group():
    x = np.full((2, 32), 0.3, dtype=np.float16).astype(F32)
    codes, s, z = quant.asym_minmax(x, 4)
    assert np.all(codes == 0) and np.all(s == 0)
    assert np.all(z == np.float16(0.3))
    c8, s8 = quant.sym_q8_0(np.zeros((1, 32), dtype=F32))
    assert np.all(c8 == 0) and np.all(s8 == 0)


@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_round_trip_bound(bits, seed):
    rng = np.random.default_rng(seed)
    x = _groups(rng, 2000, 64, scale=3.0)
    x[::7, 5] *= 20  # outlier entries
    x = x.astype(np.float16).astype(F32)
    codes, s, z = quant.asym_minmax(x, bits)
    s64 = s.astype(np.float64)[:, None]
    z64 = z.astype(np.float64)[:, None]
    deq = codes * s64 + z64
    lo = x.min(axis=1).astype(np.float64)[:, None]
    err = np.abs(deq - x)
    # half a step, plus the fp16 rounding of the zero point (values below z
    # clamp to code 0), plus float32 rounding of the quotient
    bound = 0.5 * s64 + np.abs(z64 - lo) + 1e-6 * (np.abs(x) + np.abs(z64))
    assert np.all(err <= bound)
    assert codes.min() >= 0 and codes.max() <= 2 ** bits - 1


def test_scale_rounding_matters_codes_follow_rounded_scale():
    # hi - lo = 1 -> s = f16(1/15) = 0.06665039..., not 1/15.  With the rounded
    # scale the top value maps to 15.0037 -> 15, and x = 0.8 maps to
    # rint(0.8 / 0.06665039) = rint(12.003) = 12.
    x = np.array([[0.0, 1.0, 0.5, 0.2]], dtype=F32)
    codes, s, _ = quant.asym_minmax(x, 4)
    assert float(s[0]) == float(np.float16(F32(1) / F32(15)))
    assert float(s[0]) == 0.06665039062500


# ---------------------------------------------------------- exact arithmetic
def _f32(fr: Fraction) -> np.float32:
    # float(Fraction) rounds correctly to binary64; for these operands the
    # binary64 value cannot sit on a binary32 tie, so one more rounding to
    # float32 is the correctly rounded float32.
    return F32(float(fr))


def _f16_of_f32(v: np.float32) -> Fraction:
    return Fraction(float(np.float16(v)))


def _exact_asym(xs, bits, absmax_offset=False):
    fr = [Fraction(float(v)) for v in xs]
    lo, hi = min(fr), max(fr)
    if absmax_offset:
        amax = max(abs(v) for v in fr)
        s = _f16_of_f32(_f32(Fraction(float(_f32(amax))) / (2 ** (bits - 1) - 1)))
    else:
        diff = Fraction(float(_f32(hi - lo)))
        s = _f16_of_f32(_f32(diff / (2 ** bits - 1)))
    z = _f16_of_f32(F32(float(lo)))
    out = []
    for v in fr:
        if s == 0:
            out.append(0)
            continue
        num = Fraction(float(_f32(v - z)))
        qv = Fraction(float(_f32(num / s)))
        c = round(qv)                       # Python round on Fraction: half-even
        out.append(min(max(c, 0), 2 ** bits - 1))
    return out, s, z


@pytest.mark.parametrize("quantizer,bits", [("asym_minmax", 4), ("asym_minmax", 3),
                                            ("asym_absmax_offset", 3), ("asym_absmax_offset", 4)])
def test_asym_matches_exact_rational_arithmetic(quantizer, bits):
    rng = np.random.default_rng(7 + bits)
    x = _groups(rng, 300, 32, scale=2.0)
    fn = quant.asym_minmax if quantizer == "asym_minmax" else quant.asym_absmax_offset
    codes, s, z = fn(x, bits)
    for gi in range(x.shape[0]):
        ref, rs, rz = _exact_asym(x[gi], bits, absmax_offset=(quantizer != "asym_minmax"))
        assert Fraction(float(s[gi])) == rs and Fraction(float(z[gi])) == rz
        assert codes[gi].tolist() == ref


def test_q8_0_matches_exact_rational_arithmetic():
    rng = np.random.default_rng(11)
    x = np.clip(_groups(rng, 300, 32, scale=1.5), -6, 6)
    codes, s = quant.sym_q8_0(x)
    for gi in range(x.shape[0]):
        fr = [Fraction(float(v)) for v in x[gi]]
        amax = max(abs(v) for v in fr)
        rs = _f16_of_f32(_f32(amax / 127))
        assert Fraction(float(s[gi])) == rs
        ref = [min(max(round(Fraction(float(_f32(v / rs)))), -128), 127) for v in fr]
        assert codes[gi].tolist() == ref


# ---------------------------------------------------------------- A2 / q8_0
def test_absmax_offset_codes_never_exceed_6_for_3bit():
    rng = np.random.default_rng(3)
    x = _groups(rng, 5000, 64)
    codes, s, z = quant.asym_absmax_offset(x, 3)
    assert codes.max() <= 6
    # (x - min) <= 2 * absmax = 6 * scale before rounding
    assert codes.min() >= 0


def test_absmax_offset_on_grid():
    k = np.array([0, 6, 1, 2, 3, 4, 5, 6])
    x = (F32(-1.5) + k.astype(F32) * F32(0.5))[None, :]
    codes, s, z = quant.asym_absmax_offset(x, 3)
    assert float(s[0]) == 0.5 and float(z[0]) == -1.5   # absmax 1.5 / 3
    assert np.array_equal(codes[0], k)


def test_q8_0_on_grid_and_symmetry():
    s = F32(2.0 ** -4)
    k = np.array([127, -127, 0, 5, -64, 100, -1, 1] * 4)
    x = (k.astype(F32) * s)[None, :]
    codes, sc = quant.sym_q8_0(x)
    assert float(sc[0]) == float(s)
    assert np.array_equal(codes[0], k)
    cn, _ = quant.sym_q8_0(-x)
    assert np.array_equal(cn[0], -k)
    rng = np.random.default_rng(5)
    xr = np.clip(_groups(rng, 1000, 32, 1.5), -6, 6)
    cr, _ = quant.sym_q8_0(xr)
    assert cr.min() >= -127 and cr.max() <= 127          # -128 never produced


# ---------------------------------------------------------------- codebook
def _codebook(rng, H, d):
    c = np.sort(rng.standard_normal((H, d, 16)), axis=-1).astype(np.float16)
    return np.sort(c, axis=-1)


def test_codebook_centroid_maps_to_its_index():
    rng = np.random.default_rng(0)
    cb = _codebook(rng, 2, 128)
    uniq = np.all(np.diff(cb.astype(F32), axis=-1) > 0, axis=-1)
    for i in range(16):
        x = cb[..., i].astype(F32)[None]                # [1, H, d]
        codes = quant.codebook_codes(x, cb)[0]
        assert np.all(codes[uniq] == i)


def test_codebook_midpoint_goes_to_lower_index():
    cb = np.tile(np.arange(16, dtype=np.float16) * np.float16(0.5), (1, 1, 1))  # [1,1,16]
    # midpoints 0.25, 0.75, ... are exact; x exactly on a midpoint -> lower index
    x = np.array([[[0.25]], [[0.75]], [[7.25]], [[0.2500001]]], dtype=F32)
    codes = quant.codebook_codes(x, cb)
    assert codes.reshape(-1).tolist() == [0, 1, 14, 1]


def test_codebook_equals_brute_force_nearest_centroid():
    rng = np.random.default_rng(1)
    H, d = 2, 128
    cb = _codebook(rng, H, d)
    c32 = cb.astype(F32)
    # precondition: the float32 midpoints are exact for these codebooks
    assert np.all((c32[..., :-1].astype(np.float64) + c32[..., 1:]) / 2
                  == quant.codebook_midpoints(cb).astype(np.float64))
    x = (rng.standard_normal((64, H, d)) * 1.3).astype(np.float16).astype(F32)
    # also exact midpoints and neighbours of them
    mids = quant.codebook_midpoints(cb)
    x[:8] = mids[..., 3][None]
    x[8:16] = np.nextafter(mids[..., 7], np.float32(10))[None]
    codes = quant.codebook_codes(x, cb)
    dist = np.abs(x[..., None].astype(np.float64) - c32.astype(np.float64)[None])
    ref = np.argmin(dist, axis=-1)                       # argmin takes the first (lower) index on ties
    assert np.array_equal(codes, ref)


# ---------------------------------------------------------------- outliers
def test_outlier_count_for_one_percent_of_4096():
    assert quant.outlier_count(0.01, 4096) == 41
    assert quant.outlier_count(0.0, 4096) == 0
    assert quant.outlier_count(0.25, 128) == 32


def test_outliers_planted():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((3, 4096)) * 0.5).astype(F32)
    x = np.clip(x, -2.9, 2.9)
    planted = [np.sort(rng.choice(4096, 41, replace=False)) for _ in range(3)]
    for r in range(3):
        mags = 3.0 + np.arange(41) * 0.25
        signs = np.where(rng.random(41) < 0.5, -1, 1)
        x[r, planted[r]] = rng.permutation(mags) * signs
    cols, vals = quant.select_outliers(x, 41)
    for r in range(3):
        assert cols[r].tolist() == planted[r].tolist()
        assert np.array_equal(vals[r], x[r, planted[r]])


def test_outliers_tie_break_lower_index_and_brute_force():
    rng = np.random.default_rng(4)
    # few distinct magnitudes -> many ties
    x = rng.integers(-4, 5, size=(20, 256)).astype(F32) * F32(0.5)
    k = 11
    cols, vals = quant.select_outliers(x, k)
    for r in range(x.shape[0]):
        ranked = sorted(range(256), key=lambda i: (-abs(float(x[r, i])), i))
        assert cols[r].tolist() == sorted(ranked[:k])
        assert vals[r].tolist() == [float(x[r, i]) for i in sorted(ranked[:k])]


def test_codebook_tensor_replacement_semantics():
    rng = np.random.default_rng(6)
    B, T, H, d = 1, 5, 2, 128
    cb = _codebook(rng, H, d)
    x = rng.standard_normal((B, T, H, d)).astype(np.float16).astype(F32)
    enc = quant.encode_tensor(x, {"quantizer": "codebook", "bits": 4, "outlier_frac": 0.01}, cb)
    k = quant.outlier_count(0.01, H * d)
    assert enc["cols"].shape == (B, T, k)
    deq = enc["deq"]                                    # [B, H, T, d]
    for t in range(T):
        cols = enc["cols"][0, t]
        for j, c in enumerate(cols):
            h, ch = divmod(int(c), d)
            assert deq[0, h, t, ch] == x[0, t, h, ch]    # outliers are exact
        mask = np.ones(H * d, bool)
        mask[cols] = False
        flat_deq = deq[0, :, t, :].reshape(-1)
        codes = enc["codes"][0, :, t, :].reshape(-1)
        cbv = cb.astype(np.float64).reshape(H * d, 16)
        assert np.array_equal(flat_deq[mask], cbv[np.arange(H * d), codes][mask])


def test_per_channel_groups_and_tail():
    rng = np.random.default_rng(8)
    B, T, H, d, G = 1, 150, 1, 128, 64
    x = rng.standard_normal((B, T, H, d)).astype(np.float16).astype(F32)
    enc = quant.encode_tensor(x, {"quantizer": "asym_minmax", "bits": 4, "group_size": G,
                                   "layout": "per_channel"})
    assert enc["codes"].shape == (B, H, 128, d)
    assert enc["scale"].shape == (B, H, 2, d)
    assert enc["tail"].shape == (B, H, 22, d)
    # group 1, channel 9 equals the per-token quantizer applied along tokens
    c, s, z = quant.asym_minmax(x[0, 64:128, 0, 9][None], 4)
    assert np.array_equal(enc["codes"][0, 0, 64:128, 9], c[0])
    assert enc["scale"][0, 0, 1, 9] == s[0] and enc["zero"][0, 0, 1, 9] == z[0]
    assert np.array_equal(enc["deq"][0, 0, 128:, :], x[0, 128:, 0, :].astype(np.float64))


def test_outlier_mask_is_the_selected_set():
    # tie-heavy rows (few distinct magnitudes) and plain normal rows
    rng = np.random.default_rng(99)
    ties = rng.integers(-4, 5, size=(300, 512)).astype(np.float32)
    normal = rng.standard_normal((300, 512)).astype(np.float16).astype(np.float32)
    for x in (ties, normal):
        for k in (1, 6, 41):
            cols, _ = quant.select_outliers(x, k)
            want = np.zeros(x.shape, dtype=bool)
            np.put_along_axis(want, cols, True, axis=1)
            assert np.array_equal(quant.outlier_mask(x, k), want)
