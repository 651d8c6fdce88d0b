"""Pins for the oracle's CSA selection producer (the ratio-4 indexer).

The compressed-sparse-attention pages (onnx-runtime-ep-cpu,
src/kernels/compressed_sparse_attention.rs: `select_ratio4_topk`,
`finalize_index_query`, `apply_compressed_rope`, `hadamard_bf16`,
`fp4_roundtrip`; onnx-runtime-ep-cuda, same file, `csa_ratio4_index_select`)
score every causally complete record by a relu-weighted sum over index heads
and keep the top k in (-score, +record) order, -1 padded.

Each pin is fixed independently of the oracle:
  (i)   the E2M1 code table of the OCP microscaling spec; the block quantizer's
        scale rule, ties to the even code, saturation, zero block, idempotence;
  (ii)  the Walsh-Hadamard butterflies == scipy.linalg.hadamard(n) @ x;
  (iii) the compressed RoPE: identity at position 0, a rotation (pair norms
        kept), composition of positions, and the rotation angle of chosen
        pairs == complex multiplication by e^(i position freq);
  (iv)  scores == a float64 brute force over keys decoded with the spec table;
  (v)   the selection == numpy lexsort on (-score, record) of those scores,
        causal domain and record capacity respected, -1 padding;
  (vi)  ties, non-finite scores and total < S are flagged.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle

# OCP MX E2M1: sign | 2 exponent bits (bias 1) | 1 mantissa bit
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table():
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert abs(v) == E2M1[c & 7]
        assert (np.signbit(v) == bool(c & 8))


def test_fp4_scale_rule_and_grid():
    x = np.zeros(32, np.float32)
    x[0] = 1.0  # amax 1 -> floor(log2) 0 -> byte 125, scale 1/4, 1 -> 4
    sc, packed, out = oracle.fp4_quantize_block32(x)
    assert sc == 125 and (packed[0] & 15) == 6 and out[0] == 1.0
    for k in (-3, 0, 5):
        s = 2.0 ** k
        vals = np.array([e * s for e in E2M1] * 4, np.float32)
        vals[1::2] *= -1
        sc, packed, out = oracle.fp4_quantize_block32(vals)
        assert sc == 127 + k  # amax 6 s: floor(log2 6 s) - 2 = k
        np.testing.assert_array_equal(out, vals)


def test_fp4_ties_to_even_and_saturation():
    s = 2.0 ** -2
    base = np.zeros(32, np.float32)
    base[0] = 6 * s  # fixes the scale at s
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    x = base.copy()
    x[1:8] = np.array(mids) * s
    x[8:15] = -np.array(mids) * s
    x[15] = 7.9 * s  # amax still in [4 s, 8 s): saturates to 6 s
    sc, packed, out = oracle.fp4_quantize_block32(x)
    assert sc == 125
    np.testing.assert_array_equal(out[1:8], np.array(want, np.float32) * s)
    np.testing.assert_array_equal(out[8:15], -np.array(want, np.float32) * s)
    assert out[15] == 6 * s


def test_fp4_zero_block_idempotence_and_error():
    sc, packed, out = oracle.fp4_quantize_block32(np.zeros(32, np.float32))
    assert sc == 127 and not packed.any() and not out.any()
    rng = np.random.default_rng(0)
    for _ in range(50):
        x = (rng.standard_normal(32) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        sc, packed, out = oracle.fp4_quantize_block32(x)
        sc2, packed2, out2 = oracle.fp4_quantize_block32(out)
        assert sc2 == sc and np.array_equal(packed2, packed) and np.array_equal(out2, out)
        s = 2.0 ** (sc - 127)
        # the grid gap is at most 2 s below 6 s, and amax < 8 s saturates to 6 s
        assert np.all(np.abs(out.astype(np.float64) - x) <= 2.0 * s)
    with pytest.raises(ValueError):
        bad = np.zeros(32, np.float32)
        bad[3] = np.inf
        oracle.fp4_quantize_block32(bad)


def test_fp4_key_decode_matches_spec_table():
    rng = np.random.default_rng(1)
    keys = rng.integers(0, 256, (5, 68), dtype=np.uint8)
    keys[:, 0::17] = rng.integers(118, 134, (5, 4))
    dec = oracle.fp4_decode_keys(keys, 128)
    for i in range(5):
        for b in range(4):
            s = 2.0 ** (int(keys[i, 17 * b]) - 127)
            for j in range(32):
                byte = keys[i, 17 * b + 1 + j // 2]
                c = (byte >> (4 * (j & 1))) & 15
                v = E2M1[c & 7] * (-1.0 if c & 8 else 1.0) * s
                assert dec[i, 32 * b + j] == np.float32(v)


@pytest.mark.parametrize("n", [32, 128])
def test_hadamard_equals_scipy(n):
    rng = np.random.default_rng(2)
    x = rng.integers(-50, 50, n).astype(np.float32)  # integers: every sum is exact
    np.testing.assert_array_equal(oracle.hadamard_f32(x), scipy.linalg.hadamard(n) @ x.astype(np.float64))


def bf16(x):
    return oracle.bf16_round_f32(np.asarray(x, np.float32))


def test_rope_identity_rotation_composition():
    rng = np.random.default_rng(3)
    t = bf16(rng.standard_normal(64))
    np.testing.assert_array_equal(oracle.compressed_rope(t, 0), t)
    for pos in (1, 17, 1000, 65535):
        r = oracle.compressed_rope(t, pos).astype(np.float64)
        n0 = np.hypot(t[0::2], t[1::2])
        n1 = np.hypot(r[0::2], r[1::2])
        np.testing.assert_allclose(n1, n0, rtol=2 ** -7, atol=1e-6)
    a = oracle.compressed_rope(oracle.compressed_rope(t, 30), 12)
    b = oracle.compressed_rope(t, 42)
    np.testing.assert_allclose(a, b, rtol=2 ** -6, atol=2 ** -6)


@pytest.mark.parametrize("pair,freq", [
    (0, 1.0),                                                     # base^0, no blend
    (20, 0.5 * 160000.0 ** (-40 / 64) + 0.5 * 160000.0 ** (-40 / 64) / 16),  # half way
    (31, 160000.0 ** (-62 / 64) / 16),                            # fully divided by 16
])
def test_rope_angle_is_complex_multiplication(pair, freq):
    t = np.zeros(64, np.float32)
    t[2 * pair], t[2 * pair + 1] = 0.75, -0.5
    pos = 123
    r = oracle.compressed_rope(t, pos)
    z = (0.75 - 0.5j) * np.exp(1j * pos * freq)
    np.testing.assert_allclose([r[2 * pair], r[2 * pair + 1]], [z.real, z.imag], atol=2 ** -8)
    others = np.delete(np.arange(64), [2 * pair, 2 * pair + 1])
    assert not r[others].any()


def test_finalized_query_sits_on_the_fp4_grid():
    rng = np.random.default_rng(4)
    q = oracle.finalize_index_query(rng.standard_normal(128).astype(np.float32), 64, 777)
    for b in range(4):
        blk = q[32 * b:32 * b + 32].astype(np.float64)
        amax = np.abs(blk).max()
        s = 2.0 ** (np.floor(np.log2(amax)) - 2) if amax > 0 else 1.0
        assert set(np.abs(blk / s)) <= set(E2M1)


def make(B=2, S=3, H=16, D=128, R=60, total=220, seed=5):
    rng = np.random.default_rng(seed)
    iq = rng.standard_normal((B, S, H, D)).astype(np.float32)
    iw = rng.standard_normal((B, S, H)).astype(np.float32)
    keys = oracle.fp4_pack_keys(rng.standard_normal((B, R, D)).astype(np.float32))
    return iq, iw, keys, total


def test_scores_brute_force_and_selection_order():
    iq, iw, keys, total = make()
    B, S, H, D = iq.shape
    R = keys.shape[1]
    K = 24
    sel, flags, sc = oracle.csa_index_select(iq, iw, keys, total, K, with_scores=True)
    assert flags == 0
    dec = oracle.fp4_decode_keys(keys, D).astype(np.float64)
    for b in range(B):
        for s in range(S):
            pos = total - S + s
            n = min((pos + 1) // 4, R)
            q = np.stack([oracle.finalize_index_query(iq[b, s, h], 64, pos) for h in range(H)]).astype(np.float64)
            dots = dec[b, :n] @ q.T                                      # [n, H]
            ref = (np.maximum(dots, 0) * iw[b, s].astype(np.float64)).sum(1) / np.sqrt(D) / np.sqrt(H)
            np.testing.assert_allclose(sc[b, s, :n], ref, rtol=1e-5, atol=1e-6)
            assert np.isnan(sc[b, s, n:]).all()
            order = np.lexsort((np.arange(n), -sc[b, s, :n].astype(np.float64)))
            want = np.full(K, -1, np.int32)
            want[:min(K, n)] = order[:K]
            np.testing.assert_array_equal(sel[b, s], want)


def test_padding_causal_domain_and_capacity():
    iq, iw, keys, _ = make(B=1, S=4, R=10, total=24)
    sel, flags = oracle.csa_index_select(iq, iw, keys, 24, 8)
    # positions 20..23: (pos + 1) // 4 = 5, 5, 5, 6 complete records
    assert flags == 0
    for s, n in enumerate([5, 5, 5, 6]):
        row = sel[0, s]
        assert sorted(row[:n]) == list(range(n)) and (row[n:] == -1).all()
    # capacity 3 caps the domain
    sel, _ = oracle.csa_index_select(iq, iw, keys[:, :3], 24, 8)
    assert all(sorted(sel[0, s, :3]) == [0, 1, 2] and (sel[0, s, 3:] == -1).all() for s in range(4))


def test_ties_nonfinite_and_geometry_flagged():
    iq, iw, keys, total = make(B=1, S=1, R=20, total=80)
    keys2 = keys.copy()
    keys2[0, 7] = keys2[0, 3]  # identical keys: identical scores
    _, flags = oracle.csa_index_select(iq, iw, keys2, total, 5)
    assert flags & oracle.SEL_TIE
    iw2 = iw.copy()
    iw2[0, 0, 2] = np.inf
    _, flags = oracle.csa_index_select(iq, iw2, keys, total, 5)
    assert flags & oracle.SEL_NONFINITE
    _, flags = oracle.csa_index_select(iq, iw, keys, 0, 5)
    assert flags == oracle.SEL_GEOMETRY


def test_index_query_bf16_rounding_after_the_hadamard_scale_decides_a_code():
    """A hand-worked query where the bf16 rounding that follows the 1/sqrt(128)
    scale (the CPU page's `hadamard_bf16`) changes the FP4 block scale.

    src = 0.7109375 e_0 + 0.703125 e_1 (both exact in bf16), position 0 (the
    RoPE is the identity there). The Walsh-Hadamard output in natural
    (Sylvester) order is h_i = x_0 + (-1)^i x_1: 1.4140625 at even i, 0.0078125
    at odd i, exact in fp32. Times fl32(1/sqrt(128)) = 0.088388346 these are
    0.12498665 and 6.905e-4. bf16 spacing below 0.125 is 2^-11, and
    0.125 - 0.12498665 < 2^-12, so the even entries round up to exactly 0.125.
    FP4 per 32 values: amax 0.125 = 2^-3 gives scale 2^(-3-2) = 2^-5 and code
    0.125 / 2^-5 = 4 (value 0.125); the odd entries are 0.0221 of the scale
    and become 0. Without that rounding the maximum 0.12498665 < 2^-3 would
    give scale 2^-6, 7.9991 saturating to code 6, value 0.09375."""
    src = np.zeros(128, np.float32)
    src[0], src[1] = 0.7109375, 0.703125
    q = oracle.finalize_index_query(src, 64, 0)
    assert np.all(q[0::2] == 0.125), q[0::2]
    assert np.all(q[1::2] == 0.0), q[1::2]


# Ramp of the compressed RoPE's frequency blend, worked out by hand: 0 up to
# pair 15, rising by a tenth per pair, 1 from pair 25 on (the CPU page's
# `apply_compressed_rope`: low 15, high 25, factor 16).
ROPE_RAMP = {14: 0.0, 15: 0.0, 16: 0.1, 17: 0.2, 18: 0.3, 19: 0.4, 20: 0.5, 21: 0.6, 22: 0.7,
             23: 0.8, 24: 0.9, 25: 1.0, 26: 1.0}


@pytest.mark.parametrize("pos", [65535, 40961])
def test_rope_ramp_over_pairs_15_to_25_at_large_positions(pos):
    """Every pair of the blend region rotated at a large position, against
    complex multiplication in float64 by e^(i pos freq_p) with
    freq_p = b_p (1 - ramp_p) + b_p / 16 ramp_p and b_p = 160000^(-2p/64).
    At these positions a ramp that is off by one pair or a wrong denominator
    moves the angle by a radian or more; the oracle's fp32 angle and bf16
    output stay within 2^-8 of the float64 value."""
    t = np.zeros(64, np.float32)
    t[0::2], t[1::2] = 0.75, -0.5
    r = oracle.compressed_rope(t, pos).astype(np.float64)
    for p, ramp in ROPE_RAMP.items():
        b = 160000.0 ** (-2.0 * p / 64.0)
        freq = b * (1.0 - ramp) + b / 16.0 * ramp
        z = (0.75 - 0.5j) * np.exp(1j * pos * freq)
        assert abs(r[2 * p] - z.real) <= 2 ** -8 and abs(r[2 * p + 1] - z.imag) <= 2 ** -8, (p, r[2 * p:2 * p + 2], z)


def test_tied_scores_are_ordered_by_ascending_record():
    """Equal scores rank by ascending record (the CUDA page's (-score, +record)
    order): identical keys at records 3, 7 and 12 score alike, and a full
    selection lists them adjacent in record order."""
    iq, iw, keys, total = make(B=1, S=1, R=20, total=80)
    keys2 = keys.copy()
    keys2[0, 7] = keys2[0, 3]
    keys2[0, 12] = keys2[0, 3]
    sel, flags, sc = oracle.csa_index_select(iq, iw, keys2, total, 20, with_scores=True)
    assert flags & oracle.SEL_TIE
    s = sc[0, 0, :20]
    assert s[3] == s[7] == s[12]
    row = list(sel[0, 0])
    i3 = row.index(3)
    assert row[i3:i3 + 3] == [3, 7, 12], row
    order = np.lexsort((np.arange(20), -s.astype(np.float64)))
    assert row == list(order)
