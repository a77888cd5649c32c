"""Pins for the oracle's element decoding and E4M3FN codec (CPU only)."""

import numpy as np
import torch

import oracle


def test_e4m3_closed_form_values():
    t = oracle.e4m3_value_table()
    assert t[0x00] == 0.0 and np.signbit(t[0x80]) and t[0x80] == 0.0
    assert t[0x01] == 2.0 ** -9            # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert t[0x08] == 2.0 ** -6            # smallest normal
    assert t[0x38] == 1.0
    assert t[0x3C] == 1.5
    assert t[0x7E] == 448.0                # largest finite
    assert t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isnan(t).sum() == 2
    finite = t[:0x7F]
    assert np.all(np.diff(finite) > 0)     # codes 0x00..0x7E increase strictly
    np.testing.assert_array_equal(t[0x80:0xFF], -finite)


def test_e4m3_table_matches_torch_decode():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = oracle.e4m3_value_table()
    both_nan = np.isnan(ref) & np.isnan(t)
    assert np.array_equal(np.where(both_nan, 0, ref), np.where(both_nan, 0, t))


def test_e4m3_roundtrip_every_code():
    t = oracle.e4m3_value_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    back = oracle.e4m3_encode(t[codes].astype(np.float32))
    assert np.array_equal(back, codes)


def test_e4m3_ties_go_to_even_code():
    t = oracle.e4m3_value_table()
    for c in range(0, 0x7E):
        mid = np.float32((t[c] + t[c + 1]) / 2)
        assert float(mid) == (t[c] + t[c + 1]) / 2        # midpoint exact in float32
        got = int(oracle.e4m3_encode(np.array([mid]))[0])
        assert got == (c if c % 2 == 0 else c + 1)
        # just above / below the midpoint
        above = np.nextafter(mid, np.float32(np.inf))
        below = np.nextafter(mid, np.float32(-np.inf))
        assert int(oracle.e4m3_encode(np.array([above]))[0]) == c + 1
        assert int(oracle.e4m3_encode(np.array([below]))[0]) == c


def test_e4m3_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 50,
        rng.uniform(-448, 448, 100000).astype(np.float32),
        (rng.standard_normal(50000) * 1e-3).astype(np.float32),
        np.array([0.0, -0.0, 448.0, -448.0, 2 ** -10, -2 ** -10, 463.99997], np.float32),
    ])
    x = x[np.abs(x) < 464]      # torch's cast does not saturate; compare where it is defined
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)


def test_e4m3_saturation_and_nan_convention():
    # Convention (not fixed by the pages): overflow and infinities saturate, NaN keeps sign.
    x = np.array([464.0, 1e6, np.inf, -500.0, -np.inf, np.nan, -np.nan], np.float32)
    got = oracle.e4m3_encode(x)
    assert list(got[:5]) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert got[5] & 0x7F == 0x7F and got[6] & 0x7F == 0x7F


def test_decode_elements_exact():
    x = np.array([1.0, -2.5, 3.140625, 65504.0, 2 ** -24], np.float32)
    f16 = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.decode_elements(f16, "f16"), x.astype(np.float16))
    bf = torch.from_numpy(x).to(torch.bfloat16)
    bits = bf.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.decode_elements(bits, "bf16"),
                                  bf.to(torch.float64).numpy())
    np.testing.assert_array_equal(oracle.decode_elements(x.view(np.uint32), "f32"), x)
