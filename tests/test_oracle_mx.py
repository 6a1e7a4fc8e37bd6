"""Pins of the oracle's MXFP8 decoding (OCP Microscaling Formats: E8M0 block
scales over E4M3 elements, blocks of 32 along the head dim) and of the input
module's MX quantiser."""
import numpy as np
import pytest

import gdpa_inputs as gi
import oracle


def test_e8m0_matches_torch_for_every_code():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float32).numpy().astype(np.float64)
    got = oracle.decode_e8m0(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got[255])
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_e8m0_hand_values():
    # 2^(code - 127): the bias, its neighbours and both ends of the range
    got = oracle.decode_e8m0(np.array([127, 128, 126, 0, 254, 255], np.uint8))
    assert got[0] == 1.0 and got[1] == 2.0 and got[2] == 0.5
    assert got[3] == 2.0 ** -127 and got[4] == 2.0 ** 127 and np.isnan(got[5])


def test_mxfp8_each_element_takes_its_own_blocks_scale():
    # two rows of 64 elements: row r block b gets scale 127 + 2 r - b; element
    # codes 0x38 (1.0) and 0xC4 (-3.0 = -1.5 * 2) alternate
    codes = np.tile(np.array([0x38, 0xC4], np.uint8), (2, 32))
    scales = np.array([[127, 126], [129, 128]], np.uint8)
    got = oracle.decode_mxfp8(codes, scales)
    base = np.tile([1.0, -3.0], 32)
    assert np.array_equal(got[0, :32], base[:32]) and np.array_equal(got[0, 32:], 0.5 * base[32:])
    assert np.array_equal(got[1, :32], 4.0 * base[:32]) and np.array_equal(got[1, 32:], 2.0 * base[32:])


def test_mxfp8_matches_e4m3_times_scale_on_random_codes():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(3, 5, 128), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x40   # no NaN codes
    scales = rng.integers(100, 150, size=(3, 5, 4), dtype=np.uint8)
    got = oracle.decode_mxfp8(codes, scales)
    for d in range(128):
        want = oracle.decode_e4m3(codes[..., d]) * 2.0 ** (scales[..., d // 32].astype(np.float64) - 127)
        assert np.array_equal(got[..., d], want)


def test_quantiser_round_trip_and_scale_rule():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((7, 3, 128)).astype(np.float32)
    x[0, 0, :32] = 0.0                       # an all-zero block
    x[1, 2, 32:64] *= 1e-30                  # a tiny block
    codes, scales = gi.quantize_mxfp8(x)
    assert codes.shape == x.shape and scales.shape == (7, 3, 4)
    back = oracle.decode_mxfp8(codes, scales)
    blocks = x.reshape(7, 3, 4, 32).astype(np.float64)
    amax = np.abs(blocks).max(-1)
    # shared exponent floor(log2 amax) - 8: the block's largest element lands in [256, 512)
    nz = amax > 0
    e = scales.astype(np.int64) - 127
    assert np.all(np.floor(np.log2(amax[nz])) - 8 == e[nz]) and np.all(e[~nz] == 0)
    # every element within E4M3's half-ulp (2^-4 relative, 2^-10 absolute in
    # the subnormal range, in units of 2^e) of x, after saturation at 448 * 2^e
    # (a block maximum in (448, 512) * 2^e is clipped, as the spec's conversion
    # to E4M3 saturates)
    lim = 448.0 * np.exp2(e.astype(np.float64))[..., None]
    target = np.clip(blocks, -lim, lim)
    err = np.abs(back.reshape(blocks.shape) - target)
    tol = np.maximum(np.abs(target) * 2.0 ** -4, np.exp2(e - 10.0)[..., None])
    assert np.all(err <= tol)
    assert np.any(np.abs(blocks) > lim)      # the draw exercises saturation
    assert np.all(back[0, 0, :32] == 0.0)
