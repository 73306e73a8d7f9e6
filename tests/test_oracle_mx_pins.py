"""Pins of the oracle's MXFP8 (OCP microscaling, E4M3 values with one E8M0
scale per 32 along K) quantization, against the format's definition: the
E4M3 and E8M0 encodings written out by hand, brute-force nearest-value
search over all 256 codes, hand-worked blocks, and the error bound the
scale choice guarantees."""

import math

import numpy as np
import pytest

import oracle as O


def test_e4m3_hand_codes():
    # S.EEEE.MMM, bias 7; exponent 0 subnormal (m 2^-9); S.1111.111 NaN
    cases = {0x00: 0.0, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x30: 0.5, 0x7E: 448.0,
             0x77: 240.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in cases.items():
        assert O.e4m3_value(c) == v, hex(c)
    assert math.isnan(O.e4m3_value(0x7F)) and math.isnan(O.e4m3_value(0xFF))
    assert math.copysign(1.0, O.e4m3_value(0x80)) == -1.0
    vals = [O.e4m3_value(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:]))  # positive codes increase with the value


def test_e8m0_hand_values():
    assert O.e8m0_value(127) == 1.0 and O.e8m0_value(120) == 2.0 ** -7
    assert O.e8m0_value(0) == 2.0 ** -127 and O.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(O.e8m0_value(255))


def _nearest_even_by_search(y):
    """Nearest finite E4M3 value to y by search over all codes, ties to the
    even code (the one whose last mantissa bit is 0), clamped to +-448."""
    sgn = 0x80 if math.copysign(1.0, y) < 0 else 0
    a = min(abs(y), 448.0)
    best = None
    for c in range(0x7F):
        d = abs(O.e4m3_value(c) - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return sgn | best[1]


def test_e4m3_encode_is_nearest_even_by_brute_force():
    rng = np.random.default_rng(0)
    ys = list(rng.standard_normal(400) * 30) + list(rng.standard_normal(200) * 0.01) + \
        list(np.exp2(rng.uniform(-12, 9.5, 300)) * rng.choice([-1, 1], 300))
    # exact ties: midpoints between neighbouring codes (normal and subnormal), and the clamp
    ys += [(O.e4m3_value(c) + O.e4m3_value(c + 1)) / 2 for c in range(0x7E)]
    ys += [448.0, 449.0, 463.9, 464.0, 1e6, -1e6, 0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10]
    for y in ys:
        assert O.e4m3_encode(float(y)) == _nearest_even_by_search(float(y)), y


def test_e4m3_encode_round_trips_every_code_and_ties_go_even():
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        assert O.e4m3_encode(O.e4m3_value(c)) == c, hex(c)
    assert O.e4m3_encode(1.0625) == 0x38      # between 1.0 (mantissa 000) and 1.125 (001): even
    assert O.e4m3_encode(1.1875) == 0x3A      # between 1.125 (001) and 1.25 (010): even
    assert O.e4m3_encode(0.5 * 2.0 ** -9) == 0x00 and O.e4m3_encode(1.5 * 2.0 ** -9) == 0x02
    assert O.e4m3_encode(1.0625 + 1e-12) == 0x39


def test_e4m3_encode_array_equals_the_scalar_definition():
    rng = np.random.default_rng(1)
    # every bf16 value of magnitude below 512 with random signs, plus random doubles
    bits = np.arange(0, 0x4400, dtype=np.uint32) << 16
    ys = bits.view(np.float32).astype(np.float64)
    ys = np.concatenate([ys, -ys, rng.standard_normal(3000) * 50, np.exp2(rng.uniform(-14, 10, 3000))])
    got = O.e4m3_encode_array(ys)
    want = np.array([O.e4m3_encode(float(y)) for y in ys], np.uint8)
    assert np.array_equal(got, want)


def test_quantize_mx8_hand_blocks():
    v = np.zeros((4, 64))
    v[0, :2] = [1.0, 3.0]          # max 3 = 1.5 2^1 -> scale 2^(1-8) = 2^-7: codes of 128 and 384
    v[0, 32] = 1.9                 # max 1.9 = 1.9 2^0 > 1.75 2^0 -> scale 2^-7 (2^-8 would clamp it)
    v[1, 32:] = 0.0                # an all-zero block
    v[1, 5] = -2.0 ** -140         # below the smallest scale 2^-127: rounds to -0 (code 0x80)
    v[2, 3] = np.nan
    v[3, 40] = np.inf
    v[3, 0] = 448.0                # exactly 448: scale 2^0, code 0x7E
    codes, scales = O.quantize_mx8(v)
    assert scales[0, 0] == 127 - 7 and codes[0, 0] == 0x70 and codes[0, 1] == 0x7C
    assert scales[0, 1] == 127 - 7
    # 1.9 / 2^-7 = 243.2 -> nearest E4M3 240 (1.875 2^7, code 0x77)
    assert codes[0, 32] == 0x77 and O.dequantize_mx8(codes, scales)[0, 32] == 1.875
    assert scales[1, 1] == 0 and not codes[1, 32:].any()
    assert scales[1, 0] == 0 and codes[1, 5] == 0x80
    assert scales[2, 0] == 255 and scales[3, 1] == 255 and scales[2, 1] == 0 and scales[3, 0] == 127
    assert codes[3, 0] == 0x7E and O.dequantize_mx8(codes, scales)[3, 0] == 448.0
    d = O.dequantize_mx8(codes, scales)
    assert d[0, 0] == 1.0 and d[0, 1] == 3.0 and np.isnan(d[2, :32]).all() and np.isnan(d[3, 32:]).all()


def test_quantize_mx8_scale_is_minimal_and_error_bounded():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((50, 256)) * np.exp2(rng.integers(-20, 20, (50, 1)))
    codes, scales = O.quantize_mx8(v)
    d = O.dequantize_mx8(codes, scales)
    blk = np.abs(v).reshape(50, 8, 32).max(axis=2)
    X = np.exp2(scales.astype(np.float64) - 127)
    assert (blk <= 448 * X).all() and (blk > 224 * X).all()       # 2^s is the smallest fitting power of two
    err = np.abs(d - v).reshape(50, 8, 32).max(axis=2)
    # within a block, values in the top binade (224, 448] step by 32 X: half a step is 16 X < blk / 14
    assert (err <= 16 * X).all() and (err / blk).max() < 1 / 14
    # the block layout: the scale of row r, columns [32b, 32b + 32) is scales[r, b]
    one = v.copy()
    one[7, 64:96] *= 2.0
    _, s2 = O.quantize_mx8(one)
    assert s2[7, 2] == scales[7, 2] + 1 and (np.delete(s2.reshape(-1), 7 * 8 + 2) ==
                                            np.delete(scales.reshape(-1), 7 * 8 + 2)).all()


def test_linear_mx8_is_exact_on_representable_operands():
    # operands that are already MXFP8 values quantize to themselves, so the
    # product equals the plain fp64 product of the same numbers
    rng = np.random.default_rng(3)
    codes_x = rng.integers(0, 0x7F, (5, 64)) | (rng.integers(0, 2, (5, 64)) << 7)
    codes_w = rng.integers(0, 0x7F, (7, 64)) | (rng.integers(0, 2, (7, 64)) << 7)
    x = O.dequantize_mx8(codes_x.astype(np.uint8), np.full((5, 2), 120, np.uint8))
    w = O.dequantize_mx8(codes_w.astype(np.uint8), np.full((7, 2), 125, np.uint8))
    # force each block's max to 448 units so the block's scale is the one used above
    x[:, 0] = 448 * 2.0 ** -7
    x[:, 32] = 448 * 2.0 ** -7
    w[:, 0] = 448 * 2.0 ** -2
    w[:, 32] = -448 * 2.0 ** -2
    b = rng.standard_normal(7)
    assert np.array_equal(O.linear_mx8(x, w, b), x @ w.T + b)
    # and a random product moves by no more than the operands' quantization allows
    xr, wr = rng.standard_normal((9, 128)), rng.standard_normal((11, 128)) * 0.02
    got, ref = O.linear_mx8(xr, wr, np.zeros(11)), xr @ wr.T
    bound = (np.abs(xr).sum(axis=1)[:, None] * np.abs(wr).max() + np.abs(xr).max() * np.abs(wr).sum(axis=1)[None]) / 14
    assert (np.abs(got - ref) <= bound).all() and np.abs(got - ref).max() > 0


@pytest.mark.parametrize("mode", ["bf16", "mxfp8", "mxfp4"])
def test_zero_gate_block_identity_holds_in_mxfp8_mode(mode):
    import synthetic as S
    from synthetic.configs import scaled
    cfg = scaled(S.get_config("c1"), stream="bf16")
    w = S.block_weights(cfg, 0)
    lay = O.pack_layout(cfg)
    cos, sin = O.rope_cache(cfg)
    mod = np.random.default_rng(8).standard_normal((1, 6, cfg.hidden))
    mod[:, 2] = 0.0
    mod[:, 5] = 0.0
    x = O.round_f32(S.inputs(cfg)["x"].astype(np.float64))
    assert np.array_equal(O.block_forward(cfg, x, mod, w, 0, lay, cos, sin, mode), x)
    mod[:, 2] = 1.0
    a = O.block_forward(cfg, x, mod, w, 0, lay, cos, sin, "bf16")
    b = O.block_forward(cfg, x, mod, w, 0, lay, cos, sin, "mxfp8")
    rel = np.abs(a - b).max() / np.sqrt(np.mean(a * a))
    assert 1e-3 < rel < 0.2   # the fp8 operands move the block, by the size of their rounding


def test_mx_step_control_accumulation():
    """The MXFP8 mode's control arm: exact on small-integer products, within
    half a grid step (2^-17 of the step's magnitude sum) per 64-product step
    plus the fp32 accumulation, and different from the exact product."""
    rng = np.random.default_rng(9)
    xi = rng.integers(-3, 4, (6, 256)).astype(np.float64)
    wi = rng.integers(-3, 4, (5, 256)).astype(np.float64)
    assert np.array_equal(O.linear(xi, wi, np.zeros(5), accum="mx_step"), xi @ wi.T)
    x = rng.standard_normal((6, 256))
    w = rng.standard_normal((5, 256))
    got = O.linear(x, w, np.zeros(5), accum="mx_step")
    exact = x @ w.T
    mag = sum(np.abs(x[:, k:k + 64]) @ np.abs(w[:, k:k + 64]).T for k in range(0, 256, 64))
    assert np.all(np.abs(got - exact) <= 2.0 ** -17 * mag + 4 * 2.0 ** -24 * mag)
    assert np.abs(got - exact).max() > 0


# ---------------------------------------------------------------- MXFP4 (E2M1 values, E8M0 scales per 32)

def test_e2m1_hand_codes():
    # S.EE.M, bias 1; exponent 0 subnormal (m / 2); the OCP FP4 value table
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert O.e2m1_value(c) == table[c]
        assert O.e2m1_value(c | 8) == -table[c]
    assert math.copysign(1.0, O.e2m1_value(8)) == -1.0
    assert O.e2m1_value(0x17) == 6.0          # only the low nibble is a code


def _e2m1_by_search(y):
    """Nearest E2M1 value to y by search over the 8 magnitudes, ties to the
    code whose mantissa bit is 0, clamped to +-6."""
    sgn = 8 if math.copysign(1.0, y) < 0 else 0
    a = min(abs(y), 6.0)
    best = None
    for c in range(8):
        d = abs(O.e2m1_value(c) - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return sgn | best[1]


def test_e2m1_encode_is_nearest_even_by_brute_force():
    rng = np.random.default_rng(10)
    ys = list(rng.standard_normal(500) * 3) + list(rng.uniform(-7, 7, 500))
    ys += [(O.e2m1_value(c) + O.e2m1_value(c + 1)) / 2 for c in range(7)]   # every tie
    ys += [0.0, -0.0, 6.0, 6.5, 100.0, -100.0, 0.25, 0.7499999, 0.7500001]
    for y in ys:
        assert O.e2m1_encode(float(y)) == _e2m1_by_search(float(y)), y
    # the ties by hand: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4
    for y, v in [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0), (3.5, 4.0), (5.0, 4.0)]:
        assert O.e2m1_value(O.e2m1_encode(y)) == v
    ys = np.array(ys, np.float64)
    assert np.array_equal(O.e2m1_encode_array(ys), np.array([O.e2m1_encode(float(y)) for y in ys], np.uint8))


def test_quantize_mx4_hand_blocks():
    v = np.zeros((4, 64))
    v[0, :3] = [1.0, 3.0, 0.3]     # max 3 = 1.5 2^1 -> scale 2^(1-2) = 2^-1: 2 -> code 4, 6 -> code 7, 0.6 -> 0.5 (code 1)
    v[0, 32] = 1.6                 # max 1.6 = 1.6 2^0 > 1.5 2^0 -> scale 2^-1 (2^-2 would clamp it): 3.2 -> 3 (code 5)
    v[1, 5] = -2.0 ** -140         # below the smallest scale: rounds to -0 (code 8)
    v[2, 3] = np.nan
    v[3, 40] = np.inf
    v[3, 0] = 6.0                  # exactly 6: scale 2^0, code 7
    codes, scales = O.quantize_mx4(v)
    assert scales[0, 0] == 126 and list(codes[0, :3]) == [4, 7, 1]
    assert scales[0, 1] == 126 and codes[0, 32] == 5
    d = O.dequantize_mx4(codes, scales)
    assert d[0, 0] == 1.0 and d[0, 1] == 3.0 and d[0, 2] == 0.25 and d[0, 32] == 1.5
    assert scales[1, 0] == 0 and codes[1, 5] == 8 and scales[1, 1] == 0 and not codes[1, 32:].any()
    assert scales[2, 0] == 255 and scales[3, 1] == 255 and not codes[2, :32].any() and not codes[3, 32:].any()
    assert scales[3, 0] == 127 and codes[3, 0] == 7 and d[3, 0] == 6.0
    assert np.isnan(d[2, :32]).all() and np.isnan(d[3, 32:]).all()
    # packing: the code at even K in the low nibble
    p = O.pack_e2m1(codes)
    assert p.shape == (4, 32) and p[0, 0] == 4 | (7 << 4) and p[0, 1] == 1 and p[3, 0] == 7


def test_quantize_mx4_scale_is_minimal_and_error_bounded():
    rng = np.random.default_rng(11)
    v = rng.standard_normal((50, 256)) * np.exp2(rng.integers(-20, 20, (50, 1)))
    codes, scales = O.quantize_mx4(v)
    d = O.dequantize_mx4(codes, scales)
    blk = np.abs(v).reshape(50, 8, 32).max(axis=2)
    X = np.exp2(scales.astype(np.float64) - 127)
    assert (blk <= 6 * X).all() and (blk > 3 * X).all()            # 2^s is the smallest fitting power of two
    # in units of X, the grid steps 0.5 below 2, 1 in [2, 4) and 2 in [4, 6]: half a step per binade
    y = np.abs(v) / np.repeat(X, 32, axis=1)
    half_step = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    assert (np.abs(d - v) <= half_step * np.repeat(X, 32, axis=1) * (1 + 1e-12)).all()
    # relative to the block max the worst case is a max near 5 X, half way between 4 and 6: error 1 X in 5 X
    r = (np.abs(d - v).reshape(50, 8, 32).max(axis=2) / blk).max()
    assert 0.15 < r <= 1 / 5 + 1e-12


def test_linear_mx4_is_exact_on_representable_operands():
    # weights already on the MXFP4 grid and activations on the MXFP8 grid quantize
    # to themselves: the product is the plain fp64 product of the same numbers
    rng = np.random.default_rng(12)
    codes_x = rng.integers(0, 0x7F, (5, 64)) | (rng.integers(0, 2, (5, 64)) << 7)
    x = O.dequantize_mx8(codes_x.astype(np.uint8), np.full((5, 2), 120, np.uint8))
    x[:, 0] = 448 * 2.0 ** -7
    x[:, 32] = 448 * 2.0 ** -7
    w = O.dequantize_mx4(rng.integers(0, 16, (7, 64)).astype(np.uint8), np.full((7, 2), 124, np.uint8))
    w[:, 0] = 6 * 2.0 ** -3
    w[:, 32] = -6 * 2.0 ** -3
    b = rng.standard_normal(7)
    assert np.array_equal(O.linear_mx4(x, w, b), x @ w.T + b)
    # and MXFP4 weights move a random product more than MXFP8 weights do
    xr, wr = rng.standard_normal((9, 128)), rng.standard_normal((11, 128)) * 0.02
    e4 = np.abs(O.linear_mx4(xr, wr, np.zeros(11)) - xr @ wr.T).max()
    e8 = np.abs(O.linear_mx8(xr, wr, np.zeros(11)) - xr @ wr.T).max()
    assert e4 > 2 * e8 > 0
