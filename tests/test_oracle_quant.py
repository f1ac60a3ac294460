"""Pins of the fp8 quantize-on-write oracle (E4M3 encoder and the per-row
quantizer).

The encoder is a brute-force nearest-code search; it is pinned against the
OCP E4M3 code table (every finite code encodes to itself), hand-picked
midpoints (ties to the even mantissa), saturation, and torch's own
float8_e4m3fn conversion on random in-range values.
"""
import numpy as np
import torch

from oracle import numerics as on


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(on.encode_e4m3(on.decode_e4m3(codes)), codes)


def test_midpoints_tie_to_even_and_saturation():
    # 1.0625 lies halfway between 1.0 (0x38, mantissa 0) and 1.125 (0x39): -> 1.0
    assert on.encode_e4m3(np.array([1.0625]))[0] == 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even): -> 1.25
    assert on.encode_e4m3(np.array([1.1875]))[0] == 0x3A
    # the largest subnormal step: 2^-9 * 0.5 -> 0 (even), 2^-9 * 1.5 -> 2 * 2^-9 (even)
    assert on.encode_e4m3(np.array([2.0 ** -10]))[0] == 0x00
    assert on.encode_e4m3(np.array([1.5 * 2.0 ** -9]))[0] == 0x02
    # past the largest finite value: saturate to 448, keep the sign
    assert list(on.encode_e4m3(np.array([460.0, 464.0, 1e6, -1e6]))) == [0x7E, 0x7E, 0x7E, 0xFE]
    assert on.encode_e4m3(np.array([-0.0]))[0] == 0x80


def test_matches_torch_float8_e4m3fn_in_range():
    g = np.random.default_rng(0)
    x = np.concatenate([g.normal(size=4000) * 30, g.normal(size=2000) * 0.01, g.uniform(-448, 448, 2000)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(on.encode_e4m3(x), ref)


def test_row_quantizer_bounds():
    g = np.random.default_rng(1)
    y = (g.normal(size=(50, 128)) * np.exp(g.normal(size=(50, 1)))).astype(np.float32)
    y[3] = 0.0
    codes, scale = on.quant_fp8_rows_f32(y)
    assert scale[3] == 1.0 and np.all(codes[3] == 0)
    back = on.dequant_fp8_rows(codes, scale)
    # each row's largest magnitude maps to 448 (up to the fp32 division), and
    # every element is within half an E4M3 step of its value
    assert np.all(np.abs(on.decode_e4m3(codes)).max(axis=1)[np.arange(50) != 3] == 448.0)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(y / scale[:, None]), 2.0 ** -6))) - 3)
    assert np.all(np.abs(back - y) <= 0.5 * step * scale[:, None] * (1 + 1e-6) + 1e-30)


def test_dequant_fp8_rows_hand_decoded():
    """x = E4M3(code) * scale of the code's row.  Codes decoded by hand from the
    OCP E4M3 bit fields: 0x38 = 2^0 = 1, 0x40 = 2^1 = 2, 0xB8 = -1, 0x7E =
    1.75 * 2^8 = 448, 0x01 = 1/8 * 2^-6 = 2^-9 (subnormal), 0x30 = 2^-1,
    0x4C = 1.5 * 2^2 = 6, 0x00 = 0, 0xC4 = -(1.5 * 2^1) = -3.  A square block
    with three distinct row scales: a scale broadcast along the wrong axis, a
    divide in place of the multiply or a dropped scale each give other values."""
    codes = np.array([[0x38, 0x40, 0xB8],
                      [0x7E, 0x01, 0x30],
                      [0x4C, 0x00, 0xC4]], dtype=np.uint8)
    scale = np.array([0.5, 3.0, 0.25], dtype=np.float32)
    want = np.array([[0.5, 1.0, -0.5],
                     [1344.0, 3.0 * 2.0 ** -9, 1.5],
                     [1.5, 0.0, -0.75]])
    got = on.dequant_fp8_rows(codes, scale)
    assert got.dtype == np.float64 and got.shape == (3, 3)
    assert np.array_equal(got, want)
    # batch axes in front: [2, 3, 3] codes with [2, 3] scales, one scale per row
    codes2 = np.stack([codes, codes[::-1]])
    scale2 = np.stack([scale, scale * 2])
    got2 = on.dequant_fp8_rows(codes2, scale2)
    assert np.array_equal(got2[0], want)
    assert np.array_equal(got2[1], (want[::-1] / scale[::-1, None]) * (2 * scale)[:, None])


def test_dequant_fp8_rows_round_trip():
    """Per-row quantize-on-write followed by dequant_fp8_rows gives every row back
    within half an E4M3 step at the row's scale, and each row's largest
    magnitude exactly (it maps to 448 = amax / scale)."""
    g = np.random.default_rng(5)
    y = (g.normal(size=(16, 128)) * np.exp(3 * g.normal(size=(16, 1)))).astype(np.float32)
    codes, scale = on.quant_fp8_rows_f32(y)
    back = on.dequant_fp8_rows(codes, scale)
    amax = np.abs(y).max(axis=1)
    assert np.allclose(np.abs(back).max(axis=1), amax, rtol=1e-6, atol=0)
    v = np.abs(y / scale[:, None])
    step = np.exp2(np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3)
    assert np.all(np.abs(back - y) <= 0.5 * step * scale[:, None] * (1 + 1e-6) + 1e-30)


def test_e2m1_midpoints_ties_and_clamp():
    # 0.25 -> 0 (even), 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2, 3.5 -> 4, 5 -> 4, 7 -> 6
    got = on.encode_e2m1(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.1, -5.5]))
    assert list(got) == [0, 2, 2, 4, 4, 6, 6, 7, 0, 0xF]
    codes = np.arange(16, dtype=np.uint8)
    back = on.encode_e2m1(on.decode_e2m1(codes))
    assert np.array_equal(back, np.where(codes == 8, 0, codes))     # -0 is written +0


def test_mxfp4_rows_round_trip_and_bound():
    g = np.random.default_rng(2)
    y = (g.normal(size=(40, 128)) * np.exp(2 * g.normal(size=(40, 4)).repeat(32, axis=1))).astype(np.float32)
    y[5, 32:64] = 0.0
    packed, scales = on.quant_mxfp4_rows_f32(y)
    back = on.dequant_mxfp4(packed, scales)
    blocks = y.reshape(40, 4, 32).astype(np.float64)
    amax = np.abs(blocks).max(axis=-1)
    s = on.decode_e8m0(scales)
    # the largest element of a block lands on 4 or 6 (amax / 2^E in [4, 8))
    big = np.abs(on.dequant_mxfp4(packed, scales).reshape(40, 4, 32)).max(axis=-1)
    nz = amax > 0
    assert np.all(np.isin(np.round(big[nz] / s[nz], 6), [4.0, 6.0]))
    assert scales[5, 1] == 0 and np.all(back.reshape(40, 4, 32)[5, 1] == 0)
    # every element within half an E2M1 step (1 above 4, 0.25 below 1, ...) of its value, or clamped at 6
    v = blocks / s[..., None]
    a = np.abs(v)
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    err = np.abs(back.reshape(40, 4, 32) / s[..., None] - v)
    assert np.all((err <= 0.5 * step + 1e-12) | (a > 6))
    # a hand-checked block: amax 3 -> E = floor(log2 3) - 2 = -1, elements doubled
    blk = np.zeros((1, 32), np.float32)
    blk[0, :4] = [3.0, -0.6, 0.2, 1.1]
    p1, s1 = on.quant_mxfp4_rows_f32(blk)
    assert s1[0, 0] == 126
    # 6.0 -> 7, -1.2 -> 1.0 (code 2, negative: 0xA), 0.4 -> 0.5 (code 1), 2.2 -> 2.0 (code 4)
    assert p1[0, 0] == (7 | (0xA << 4)) and p1[0, 1] == (1 | (4 << 4))


def test_mxfp4_shared_exponent_at_powers_of_two():
    """E = floor(log2 amax) - 2: a block whose amax is 2^e gets E = e - 2 and
    its largest element lands on 4; the float just below 2^e gets e - 3 and
    lands on 6 (7.99.. rounds and clamps to 6).  E8M0 decodes to 2^E."""
    for e in range(-30, 31, 3):
        blk = np.zeros((2, 32), np.float32)
        blk[0, 7] = 2.0 ** e
        blk[1, 7] = -np.nextafter(np.float32(2.0 ** e), np.float32(0))
        blk[:, 0] = np.float32(2.0 ** (e - 4))          # 1/16 of 2^e: E2M1 0.25 -> rounds to 0
        packed, scales = on.quant_mxfp4_rows_f32(blk)
        assert list(scales[:, 0]) == [e - 2 + 127, e - 3 + 127]
        assert list(on.decode_e8m0(scales[:, 0])) == [2.0 ** (e - 2), 2.0 ** (e - 3)]
        back = on.dequant_mxfp4(packed, scales)
        assert back[0, 7] == 2.0 ** e and back[1, 7] == -6 * 2.0 ** (e - 3)
        assert back[0, 0] == 0.0 and back[1, 0] == 0.5 * 2.0 ** (e - 3)   # 2^(e-4) / 2^(e-3) = 0.5, exact


def test_mxfp4_exponent_clamps_at_e8m0_zero():
    """A block of float32 subnormals: floor(log2 amax) - 2 falls below -127,
    so E clamps to -127 (E8M0 byte 0) and the elements, scaled by 2^127, are
    still tiny; at amax = 2^-125, E = -127 exactly."""
    blk = np.zeros((2, 32), np.float32)
    blk[0, 3] = np.float32(2.0 ** -140)
    blk[0, 4] = np.float32(-3 * 2.0 ** -128)            # 3 * 2^-128 / 2^-127 = 1.5: code 3
    blk[1, 0] = np.float32(2.0 ** -125)
    packed, scales = on.quant_mxfp4_rows_f32(blk)
    assert list(scales[:, 0]) == [0, 0]
    back = on.dequant_mxfp4(packed, scales)
    assert back[0, 3] == 0.0 and back[0, 4] == np.float32(-3 * 2.0 ** -128) and back[1, 0] == 2.0 ** -125
