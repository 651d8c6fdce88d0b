"""Pins for the oracle's number codecs (bf16 rounding, E4M3FN, E8M0, fp8 records).

Each codec is checked against an implementation it shares nothing with:
torch's float8_e4m3fn / float8_e8m0fnu / bfloat16 dtypes (library routines of
the OCP formats and of IEEE-style round-to-nearest-even), plus closed-form
facts of the formats (largest finite 448, NaN encodings, subnormal step).
The record layout follows the CSA CPU oracle page's `CacheFormat`:
(Dk - rope)/64 blocks of [1 E8M0 byte, 64 E4M3FN bytes], then rope dims as
little-endian BF16.
"""
import numpy as np
import pytest
import torch

import oracle


def torch_e4m3(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_e4m3fn_all_codes_match_library():
    codes = np.arange(256, dtype=np.uint8)
    ours = np.array([oracle.e4m3fn_value(int(c)) for c in codes])
    ref = torch_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # closed-form facts of the format
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert ours[0x80] == 0.0 and np.signbit(ours[0x80])


def test_e8m0_matches_library():
    for e in range(256):
        ours = oracle.e8m0_value(e)
        ref = torch.tensor([e], dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).item()
        if e == 255:
            assert np.isnan(ours)
        else:
            assert ours == 2.0 ** (e - 127) == ref


def test_bf16_rounding_matches_library():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        np.array([0.0, -0.0, 1.0, 3.3895314e38, -3.3895314e38, 1e-40, -1e-45, np.inf, -np.inf],
                 np.float32),
        # exact ties: low half 0x8000 with even and odd upper halves
        np.array([0x3F808000, 0x3F818000, 0x7F7F8000], np.uint32).view(np.float32),
    ])
    ours = oracle.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nan = oracle.bf16_bits(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def _blocks(seed, n=200):
    rng = np.random.default_rng(seed)
    blocks = rng.standard_normal((n, 64)).astype(np.float32)
    blocks[1] *= np.float32(1e-30)     # tiny magnitudes
    blocks[2] *= np.float32(1e30)      # huge magnitudes
    blocks[3, :] = 0.0                 # all-zero block
    blocks[4, :] = 0.0
    blocks[4, 7] = -3.0                # single nonzero
    blocks[5] = np.float32(2.0) ** np.arange(-16, 48, dtype=np.float32)  # wide dynamic range
    return blocks


def test_quantizer_scale_rule_and_codes_match_library_rounding():
    for x in _blocks(11):
        scale, codes = oracle.fp8_quantize_block64(x)
        amax = float(np.max(np.abs(x)))
        if amax == 0.0:
            assert scale == 127 and not codes.any()
            continue
        k = int(np.floor(np.log2(np.float64(amax))))
        assert scale == min(max(k - 8 + 127, 0), 254)
        # the codes are E4M3FN round-to-nearest-even of x * 2^(127 - scale),
        # saturated to +-448: compare against torch's cast of the clamped value
        scaled = np.clip(x.astype(np.float64) * 2.0 ** (127 - scale), -448.0, 448.0)
        ref = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes, ref), (x, codes, ref)


def test_quantizer_error_bound_and_saturation():
    for x in _blocks(12):
        scale, codes = oracle.fp8_quantize_block64(x)
        deq = torch_e4m3(codes) * 2.0 ** (scale - 127)
        xs = x.astype(np.float64)
        # the scaled block maximum lands in [256, 512): no saturation beyond 448
        # and every normal code is within half an ulp (2^-4 relative)
        normal = np.abs(xs * 2.0 ** (127 - scale)) >= 2.0 ** -6
        sat = np.abs(xs * 2.0 ** (127 - scale)) > 448.0
        ok = normal & ~sat
        assert np.all(np.abs(deq[ok] - xs[ok]) <= 2.0 ** -4 * np.abs(xs[ok]))
        sub = ~normal
        assert np.all(np.abs(deq[sub] - xs[sub]) <= 2.0 ** -10 * 2.0 ** (scale - 127))
        assert np.all(np.abs(deq[sat]) == 448.0 * 2.0 ** (scale - 127))


def test_quantizer_rejects_non_finite():
    x = np.zeros(64, np.float32)
    x[3] = np.inf
    with pytest.raises(ValueError):
        oracle.fp8_quantize_block64(x)
    x[3] = np.nan
    with pytest.raises(ValueError):
        oracle.fp8_quantize_block64(x)


def test_record_layout_and_round_trip():
    rng = np.random.default_rng(13)
    dk, rope = 576, 64
    assert oracle.fp8_record_bytes(dk, rope) == 8 * 65 + 128 == 648
    assert oracle.fp8_record_bytes(512, 64) == 7 * 65 + 128 == 583
    assert oracle.fp8_record_bytes(500, 64) == -1
    rows32 = rng.standard_normal((64, dk)).astype(np.float32)
    rows = (torch.from_numpy(rows32).to(torch.bfloat16).to(torch.float32)).numpy()
    rec = oracle.fp8_pack_rows(rows, rope)
    assert rec.shape == (64, 648)
    # layout: block j scale byte at 65j, codes after it, bf16 tail little-endian
    for r in range(4):
        for j in range(8):
            s, c = oracle.fp8_quantize_block64(rows[r, 64 * j:64 * j + 64])
            assert rec[r, 65 * j] == s and np.array_equal(rec[r, 65 * j + 1:65 * j + 65], c)
        tail = rec[r, 520:].view(np.uint16)
        ref_tail = torch.from_numpy(rows[r, 512:]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(tail, ref_tail)
    dec = oracle.fp8_decode_rows(rec, dk, rope)
    # decode == library E4M3FN value * 2^(e-127); tail exact
    for r in range(4):
        for j in range(8):
            ref = torch_e4m3(rec[r, 65 * j + 1:65 * j + 65]) * 2.0 ** (int(rec[r, 65 * j]) - 127)
            assert np.array_equal(dec[r, 64 * j:64 * j + 64].astype(np.float64), ref)
    assert np.array_equal(dec[:, 512:], rows[:, 512:])
    # byte-idempotent: quantizing the decoded row reproduces the record
    assert np.array_equal(oracle.fp8_pack_rows(dec, rope), rec)
    # the decoded values are exactly representable in bf16 for these scales
    assert np.array_equal(oracle.bf16_round_f32(dec), dec)


def test_f16_widening_every_bit_pattern():
    """The f16 inputs' widening against numpy's IEEE binary16 type for all
    65,536 bit patterns: subnormals (2^-24 step), normals, +-0, +-inf, NaN."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # signed zeros too
    # closed-form anchors of the format
    assert ours[0x0001] == 2.0 ** -24 and ours[0x03FF] == 1023 * 2.0 ** -24
    assert ours[0x0400] == 2.0 ** -14 and ours[0x3C00] == 1.0 and ours[0x7BFF] == 65504.0
    assert ours[0xC000] == -2.0 and np.signbit(ours[0x8000]) and ours[0x8000] == 0.0


# E4M3FN codes written out from the format: (E << 3) | M, value (1 + M/8) 2^(E-7)
# for E >= 1 and M 2^-9 for E = 0. Each entry is an exact midpoint between two
# neighbouring codes (or a value that must round to a signed zero) and the code
# that round-to-nearest-even gives it.
E4M3_MIDPOINTS = [
    (1.0625, 0x38),          # between 1.0 (0x38, M=0) and 1.125 (0x39): even M=0
    (1.1875, 0x3A),          # between 1.125 (0x39) and 1.25 (0x3A, M=2): even M=2
    (-1.3125, 0xBA),         # between -1.25 (0xBA) and -1.375 (0xBB): even
    (232.0, 0x76),           # between 224 (0x76, E=14 M=6) and 240 (0x77): even M=6
    (248.0, 0x78),           # between 240 (0x77) and 256 (0x78, next binade): even M=0
    (3.0 * 2.0 ** -10, 0x02),  # subnormal: between 1 (0x01) and 2 (0x02) x 2^-9
    (5.0 * 2.0 ** -10, 0x02),  # between 2 (0x02) and 3 (0x03) x 2^-9
    (15.0 * 2.0 ** -10, 0x08),  # between 7 x 2^-9 (0x07) and 2^-6 (0x08, smallest normal)
    (2.0 ** -10, 0x00),      # between 0 and 2^-9: even code 0
    (-(2.0 ** -10), 0x80),   # the same, negative: -0
    (-(2.0 ** -11), 0x80),   # rounds to zero: keeps its sign
    (-(2.0 ** -30), 0x80),
]


def test_quantizer_exact_midpoints_and_negative_zero():
    """Round-to-nearest-even at exact E4M3FN midpoints and the sign of values
    that round to zero. The block's maximum 300 fixes the scale byte at 127
    (floor(log2 300) = 8), so the planted values are encoded unscaled. About
    one bf16 value in 16 lands on such a midpoint, so the quantize-on-append
    bytes depend on this rule."""
    x = np.zeros(64, np.float32)
    x[0] = 300.0
    vals = [v for v, _ in E4M3_MIDPOINTS]
    x[1:1 + len(vals)] = np.array(vals, np.float32)
    assert np.array_equal(x[1:1 + len(vals)].astype(np.float64), np.array(vals))  # planted exactly
    scale, codes = oracle.fp8_quantize_block64(x)
    assert scale == 127
    want = np.array([c for _, c in E4M3_MIDPOINTS], np.uint8)
    assert np.array_equal(codes[1:1 + len(vals)], want), (codes[1:1 + len(vals)], want)
    # the library's nearest-even cast agrees on every planted value
    ref = torch.from_numpy(x.astype(np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # the same midpoints under a non-trivial scale: maximum 300 * 2^-20 gives
    # scale byte 107 and the block is divided exactly by 2^-20
    y = (x.astype(np.float64) * 2.0 ** -20).astype(np.float32)
    scale2, codes2 = oracle.fp8_quantize_block64(y)
    assert scale2 == 107 and np.array_equal(codes2, codes)


def test_quantizer_midpoints_of_every_binade_match_library():
    """Every midpoint between neighbouring finite E4M3FN magnitudes (both signs)
    rounds as the library's nearest-even cast does."""
    mags = np.array(sorted({abs(oracle.e4m3fn_value(c)) for c in range(0x7F)}))
    mids = (mags[:-1] + mags[1:]) / 2.0          # 126 exact midpoints, 0 .. 416
    vals = np.concatenate([mids, -mids])
    for start in range(0, len(vals), 63):
        x = np.zeros(64, np.float32)
        x[0] = 448.0                              # scale byte 127
        chunk = vals[start:start + 63]
        x[1:1 + len(chunk)] = chunk.astype(np.float32)
        assert np.array_equal(x[1:1 + len(chunk)].astype(np.float64), chunk)
        scale, codes = oracle.fp8_quantize_block64(x)
        assert scale == 127
        ref = torch.from_numpy(x.astype(np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes, ref)
        # and the chosen code's mantissa is even (a tie never picks the odd neighbour)
        sel = codes[1:1 + len(chunk)]
        assert np.all((sel & 1) == 0), sel
