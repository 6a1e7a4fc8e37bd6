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


# ------------------------------------------------------------------ MXFP4
def _golden_e2m1():
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.json")) as f:
        return json.load(f)


def test_e2m1_every_code_matches_the_hand_table():
    fx = _golden_e2m1()
    got = oracle.decode_e2m1(np.array(fx["codes"], np.uint8))
    want = np.array(fx["values"])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))   # code 8 is -0


def test_fp4_nibble_order_hand_bytes():
    # byte 0x21: element 0 = low nibble 1 (0.5), element 1 = high nibble 2 (1.0);
    # byte 0xF7: element 2 = 7 (6.0), element 3 = 0xF (-6.0)
    codes = oracle.unpack_fp4(np.array([[0x21, 0xF7]], np.uint8))
    assert codes.tolist() == [[1, 2, 7, 15]]
    got = oracle.decode_mxfp4(np.tile(np.array([0x21, 0xF7], np.uint8), 8)[None], np.array([[128]], np.uint8))
    assert np.array_equal(got[0, :4], [1.0, 2.0, 12.0, -12.0])


def test_mxfp4_each_element_takes_its_own_blocks_scale():
    # a row of 64 elements, all code 2 (1.0): block 0 scale 2^-1, block 1 scale 2^3
    packed = np.full((1, 32), 0x22, np.uint8)
    got = oracle.decode_mxfp4(packed, np.array([[126, 130]], np.uint8))
    assert np.array_equal(got[0, :32], np.full(32, 0.5)) and np.array_equal(got[0, 32:], np.full(32, 8.0))


def test_mxfp4_quantiser_scale_rule_and_rounding():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((5, 3, 128)).astype(np.float32)
    x[0, 0, :32] = 0.0
    packed, scales = gi.quantize_mxfp4(x)
    assert packed.shape == (5, 3, 64) and scales.shape == (5, 3, 4)
    back = oracle.decode_mxfp4(packed, scales)
    blocks = x.reshape(5, 3, 4, 32).astype(np.float64)
    amax = np.abs(blocks).max(-1)
    e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1))) - 2, 0)
    assert np.array_equal(scales.astype(np.int64) - 127, e.astype(np.int64))
    assert np.all(back[0, 0, :32] == 0.0)
    # every element is a nearest grid point of x / 2^e (within half the local
    # spacing, at most 1 unit at magnitudes 4..6), or the saturated +-6
    y = blocks / np.exp2(e)[..., None]
    b = back.reshape(5, 3, 4, 32) / np.exp2(e)[..., None]
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    near = np.abs(np.abs(y)[..., None] - grid).min(-1)
    sat = np.abs(y) > 6.0
    assert np.all(np.where(sat, np.abs(b) == 6.0, np.isclose(np.abs(np.abs(b) - np.abs(y)), near)))
    assert np.all((np.sign(b) == np.sign(y)) | (b == 0))
    # ties go to the even code: 0.25 -> 0, 0.75 -> 1.0, 2.5 -> 2.0, 5.0 -> 4.0 (block max 5 -> e = 0)
    t = np.zeros((1, 32), np.float32)
    t[0, :5] = [0.25, 0.75, 2.5, 5.0, 1.25]
    p2, s2 = gi.quantize_mxfp4(t)
    assert s2[0, 0] == 127
    assert oracle.decode_mxfp4(p2, s2)[0, :5].tolist() == [0.0, 1.0, 2.0, 4.0, 1.0]
