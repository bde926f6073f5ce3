"""Pins for the oracle's storage formats (bf16 widening and rounding, OCP FP8
E4M3FN codec) against PyTorch's own conversions and hand-known codes."""
import numpy as np
import pytest
import torch

from oracle.numerics import bf16_round, bf16_to_f64, e4m3_decode, e4m3_encode


def test_bf16_widen_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(200000) * 10 ** rng.uniform(-6, 6, 200000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38])])
    ours = bf16_round(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # exactly two NaN codes (S.1111.111), no infinities
    assert np.isnan(ours).sum() == 2 and not np.isinf(ours).any()


@pytest.mark.parametrize("value,code", [(0.0, 0x00), (1.0, 0x38), (-1.0, 0xB8), (448.0, 0x7E),
                                        (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (0.875 * 2.0 ** -6, 0x07),
                                        (1.125, 0x39), (-448.0, 0xFE)])
def test_e4m3_known_codes(value, code):
    # OCP 8-bit FP spec, E4M3: bias 7, 3 mantissa bits, max normal 448
    assert int(e4m3_encode(np.array([value]))[0]) == code
    assert e4m3_decode(np.array([code], dtype=np.uint8))[0] == value


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(300000) * 10 ** rng.uniform(-4, 2.6, 300000)
    x = np.clip(x, -448, 448)
    # include exact midpoints between neighbouring codes (ties to even)
    vals = e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, mids, -mids])
    ours = e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates():
    x = np.array([449.0, 464.0, 480.0, 1e6, -500.0, -1e30])
    assert e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
