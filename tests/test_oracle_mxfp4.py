"""Pins of the oracle's MXFP4 quantiser (OCP Microscaling MXFP4: 32-element blocks with a shared
power-of-two scale stored as an 8-bit exponent, 4-bit E2M1 elements), against what the format's
definition fixes: every representable block value survives a round trip exactly; the block exponent
is floor(log2 of the block's largest magnitude) - 2; midpoints between neighbouring E2M1 magnitudes
go to the even code; magnitudes beyond 6 saturate; the error of every element stays within half a
step of the E2M1 grid at its magnitude (or the saturation distance); element 2j sits in the low
nibble of byte j; an all-zero block is stored as zeros with scale 1.  CPU only."""
import numpy as np

from oracle import dflash_oracle as O

MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # the E2M1 magnitudes by code


def _block(vals, s):
    """One row of 32: the given element values (times 2^s) then 4 * 2^s (fixes the scale), zero-padded."""
    row = np.zeros(32)
    row[: len(vals)] = np.asarray(vals, dtype=float) * 2.0 ** s
    row[31] = 4.0 * 2.0 ** s
    return row[None, :]


def test_codes_decode_to_the_e2m1_table():
    codes = np.arange(16)
    assert np.array_equal(O.e2m1_value(codes), np.array(MAGS + [-m for m in MAGS]))


def test_representable_values_round_trip_exactly():
    for s in (-9, -3, 0, 2):
        vals = MAGS + [-m for m in MAGS[1:]]
        row = _block(vals, s)
        c, sc = O.quantize_mxfp4_rows(row)
        assert sc[0, 0] == s + 127
        assert np.array_equal(O.dequantize_mxfp4_rows(c, sc), row)


def test_block_exponent_is_floor_log2_minus_two():
    for k in range(-20, 5):
        a = 2.0 ** k
        _, sc = O.quantize_mxfp4_rows(np.full((1, 32), a))
        assert int(sc[0, 0]) - 127 == k - 2
        _, sc = O.quantize_mxfp4_rows(np.full((1, 32), a * (1 - 2.0 ** -20)))
        assert int(sc[0, 0]) - 127 == k - 3
        _, sc = O.quantize_mxfp4_rows(np.full((1, 32), -a * 1.999))
        assert int(sc[0, 0]) - 127 == k - 2


def test_midpoints_go_to_the_even_code():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]     # the neighbour with mantissa bit 0
    row = _block(mids + [-m for m in mids], 0)
    c, sc = O.quantize_mxfp4_rows(row)
    got = O.dequantize_mxfp4_rows(c, sc)[0, : 2 * len(mids)]
    assert np.array_equal(got, np.array(want + [-w for w in want]))
    # just off a midpoint the nearer neighbour wins
    eps = 2.0 ** -30
    row = _block([0.25 + eps, 0.75 - eps, 5.0 + eps], 0)
    got = O.dequantize_mxfp4_rows(*O.quantize_mxfp4_rows(row))[0, :3]
    assert np.array_equal(got, np.array([0.5, 0.5, 6.0]))


def test_magnitudes_above_six_saturate():
    row = np.zeros((1, 32))
    row[0, :4] = [7.99, 6.01, -7.5, 6.0]            # largest 7.99 -> exponent 0, grid step up to 2
    c, sc = O.quantize_mxfp4_rows(row)
    assert sc[0, 0] == 127
    assert np.array_equal(O.dequantize_mxfp4_rows(c, sc)[0, :4], np.array([6.0, 6.0, -6.0, 6.0]))


def test_error_within_half_a_grid_step():
    rng = np.random.default_rng(3)
    W = rng.normal(0, 0.02, (64, 256)) * np.exp(rng.normal(0, 2, (64, 1)))
    c, sc = O.quantize_mxfp4_rows(W)
    D = O.dequantize_mxfp4_rows(c, sc)
    s = np.repeat(sc.astype(np.int64) - 127, 32, axis=1)
    x = np.abs(W) / 2.0 ** s                            # in [0, 8)
    half_step = np.where(x < 2, 0.25, np.where(x < 4, 0.5, 1.0))
    bound = np.where(x > 6, x - 6, half_step) * 2.0 ** s
    assert np.all(np.abs(D - W) <= bound * (1 + 1e-12))
    assert np.all(np.signbit(D[D != 0]) == np.signbit(W[D != 0]))


def test_packing_low_nibble_first_and_zero_blocks():
    row = _block([0.5, 1.0, -0.5, 6.0], 0)
    c, sc = O.quantize_mxfp4_rows(row)
    assert c.shape == (1, 16) and sc.shape == (1, 1)
    assert c[0, 0] == (1 | (2 << 4))          # elements 0 (0.5, code 1) and 1 (1.0, code 2)
    assert c[0, 1] == (9 | (7 << 4))          # elements 2 (-0.5, code 9) and 3 (6.0, code 7)
    z = np.zeros((2, 64))
    z[1, 33] = -0.0
    c, sc = O.quantize_mxfp4_rows(z)
    assert np.all(sc == 127) and np.all((c & 0x77) == 0)
