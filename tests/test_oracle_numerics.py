"""Pins of the oracle's storage-format helpers against library casts and the format definitions."""
import numpy as np
import pytest
import torch

from oracle import numerics as nu


def test_bf16_decode_all_codes_match_torch():
    codes = np.arange(1 << 16, dtype=np.uint16)
    ours = nu.bf16_decode(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_encode_roundtrip_all_finite_codes():
    codes = np.arange(1 << 16, dtype=np.uint16)
    vals = nu.bf16_decode(codes)
    fin = np.isfinite(vals) & ~((vals == 0) & np.signbit(vals))
    assert (nu.bf16_encode(vals[fin]) == codes[fin]).all()


@pytest.mark.parametrize("scale", [1e-3, 1.0, 1e4, 1e-38])
def test_bf16_round_matches_torch_rne_on_float32(scale):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200_000) * scale).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert (nu.bf16_round(x.astype(np.float64)) == ref).all()


def test_bf16_ties_go_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: the even neighbour is 1.
    assert nu.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    assert nu.bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    # Just above a midpoint rounds up.
    assert nu.bf16_round(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ours = nu.e4m3_decode(codes)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    assert np.nanmax(ours) == 448.0 and np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert ours[1] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_round_matches_torch_in_range():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(200_000) * 60).astype(np.float32)
    x = x[np.abs(x) < 464]              # torch's cast does not saturate; compare in range only
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    assert (nu.e4m3_round(x.astype(np.float64)) == ref).all()
    small = (rng.standard_normal(50_000) * 2e-3).astype(np.float32)
    ref = torch.from_numpy(small).to(torch.float8_e4m3fn).double().numpy()
    assert (nu.e4m3_round(small.astype(np.float64)) == ref).all()


def test_e4m3_worked_values_and_saturation():
    # 0.1 = 1.6 * 2^-4; the 3-bit neighbours are 1.5 and 1.625 -> 1.625 * 2^-4.
    assert nu.e4m3_round(np.array([0.1]))[0] == 0.1015625
    # 464 is halfway between 448 (mantissa 110, even) and the NaN slot 480: ties to 448.
    assert nu.e4m3_round(np.array([464.0, 470.0, 1e6, -1e6])).tolist() == [448, 448, 448, -448]
    # Half the smallest subnormal ties to zero; 1.5 of it rounds to 2 quanta.
    q = 2.0 ** -9
    assert nu.e4m3_round(np.array([0.5 * q, 1.5 * q])).tolist() == [0.0, 2 * q]


def test_e4m3_encode_roundtrip():
    codes = np.arange(256, dtype=np.uint8)
    vals = nu.e4m3_decode(codes)
    ok = np.isfinite(vals) & (codes != 0x80)     # -0 encodes as +0
    assert (nu.e4m3_encode(vals[ok]) == codes[ok]).all()


# ---- MXFP4 (OCP Microscaling specification): E2M1 elements, E8M0 block scales ---------------

def test_e2m1_values_are_the_specification_table():
    # The specification lists the E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); bit 3 is
    # the sign.
    from oracle.numerics import E2M1_VALUES
    assert E2M1_VALUES[:8].tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert (E2M1_VALUES[8:] == -E2M1_VALUES[:8]).all()


def test_e8m0_decode_matches_torch():
    from oracle.numerics import e8m0_decode
    codes = np.arange(255, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(e8m0_decode(codes), want)
    assert np.isnan(e8m0_decode(np.array([255], np.uint8)))[0]


def test_mxfp4_decode_worked_example():
    # Byte 0x21: element 0 = code 1 (0.5), element 1 = code 2 (1.0). Byte 0xF7: element 0 = code 7
    # (6), element 1 = code 15 (-6). Scale 128 doubles the first block; scale 126 halves the second.
    from oracle.numerics import mxfp4_decode
    packed = np.zeros((1, 32), np.uint8)
    packed[0, 0] = 0x21
    packed[0, 16] = 0xF7
    v = mxfp4_decode(packed, np.array([[128, 126]], np.uint8))
    assert v[0, :2].tolist() == [1.0, 2.0] and (v[0, 2:32] == 0).all()
    assert v[0, 32:34].tolist() == [3.0, -3.0] and (v[0, 34:] == 0).all()


def test_mxfp4_storage_cast():
    # The inputs' MXFP4 cast: scale 2^(floor(log2 amax) - 2), nearest E2M1 with ties to the even
    # fraction bit, saturation at 6. Block: 6 (amax, scale 1), 1.25 (tie 1 | 1.5 -> 1), 1.75 (tie
    # 1.5 | 2 -> 2), 2.5 (tie 2 | 3 -> 2), 0.2 (-> 0), -5 (tie 4 | 6 -> 4).
    from long_context_compressed_07_amd.inputs import to_mxfp4
    from oracle.numerics import mxfp4_decode
    x = np.zeros((1, 32), np.float32)
    x[0, :6] = [6.0, 1.25, 1.75, 2.5, 0.2, -5.0]
    p, sc = to_mxfp4(x)
    assert sc.tolist() == [[127]]
    assert mxfp4_decode(p, sc)[0, :6].tolist() == [6.0, 1.0, 2.0, 2.0, 0.0, -4.0]
    # amax 7: scale 2^0 again, 7 saturates to 6
    x[0, 0] = 7.0
    p, sc = to_mxfp4(x)
    assert mxfp4_decode(p, sc)[0, 0] == 6.0
    # random rows: every element within half a step of its value below the block's saturation
    rng = np.random.default_rng(3)
    z = rng.standard_normal((50, 64)).astype(np.float32) * 0.1
    p, sc = to_mxfp4(z)
    y = mxfp4_decode(p, sc)
    scale = np.repeat(2.0 ** (sc.astype(np.float64) - 127), 32, axis=1)
    mag = np.abs(z) / scale
    half_step = np.where(mag < 2, 0.25, np.where(mag < 4, 0.5, 1.0)) * scale
    ok = (mag <= 6) & (np.abs(y - z) <= half_step + 1e-12)
    assert (ok | (mag > 6)).all() and (np.abs(y[mag > 6]) == 6 * scale[mag > 6]).all()
