"""Pins of the oracle's number formats and quantiser (CPU only).

The bf16 and e4m3 codecs are checked against torch's own casts (a library
routine independent of the oracle's C code) and against values the OCP 8-bit
floating point format fixes; the quantiser against its defining properties.
"""
import numpy as np
import pytest
import torch

import oracle


def test_bf16_decode_all_patterns():
    bits = np.arange(0, 1 << 16, 97, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_e4m3_decode_all_256_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_e4m3_format_landmarks():
    # values the e4m3fn layout fixes: max normal, min normal, subnormal extremes, NaN
    assert oracle.e4m3_decode(0x7E)[0] == 448.0
    assert oracle.e4m3_decode(0x08)[0] == 2.0 ** -6
    assert oracle.e4m3_decode(0x07)[0] == 7 * 2.0 ** -9
    assert oracle.e4m3_decode(0x01)[0] == 2.0 ** -9
    assert oracle.e4m3_decode(0x38)[0] == 1.0
    assert oracle.e4m3_decode(0xB8)[0] == -1.0
    assert np.isnan(oracle.e4m3_decode(0x7F)[0]) and np.isnan(oracle.e4m3_decode(0xFF)[0])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 3,
        rng.standard_normal(5000) * 1e-2,
        (2.0 ** rng.uniform(-12, 8.8, 5000)) * rng.choice([-1, 1], 5000),
    ]).astype(np.float32)
    got = oracle.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_encode_midpoints_round_to_even():
    # every midpoint between neighbouring codes, and one fp32 ulp either side
    grid = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))   # +0 .. 448
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    got = oracle.e4m3_encode(vals)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    # above the largest finite value the format has no infinity: this codec
    # saturates to +-448 (torch would give NaN far beyond 448)
    v = np.array([448.0, 449.0, 463.9, 470.0, 1e6, np.inf, -500.0, -np.inf], np.float32)
    got = oracle.e4m3_encode(v)
    assert list(got) == [0x7E] * 6 + [0xFE] * 2


def test_e4m3_round_trip_of_representables():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    back = oracle.e4m3_encode(vals)
    # -0 and +0 both decode to a zero; compare the values
    assert np.array_equal(oracle.e4m3_decode(back), oracle.e4m3_decode(codes))


def test_quantiser_scale_and_bounds():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(4096) * 5).astype(np.float32)
    q, s = oracle.quantise_group(v)
    assert s == np.float32(np.abs(v).max()) / np.float32(448.0)
    deq = oracle.e4m3_decode(q) * float(s)
    assert np.all(np.abs(oracle.e4m3_decode(q)) <= 448.0)
    # relative spacing of e4m3 normals is 2^-3: |v - q*s| <= 2^-4 |v| (+ subnormal floor)
    err = np.abs(deq - v.astype(np.float64))
    assert np.all(err <= np.abs(v) * 2.0 ** -4 + 2.0 ** -10 * float(s) + 1e-12)
    # the largest element maps to the largest code
    assert oracle.e4m3_decode(q[np.argmax(np.abs(v))])[0] in (448.0, -448.0)


def test_quantiser_identity_when_amax_is_448():
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    v = oracle.e4m3_decode(codes).astype(np.float32)  # includes 448
    q, s = oracle.quantise_group(v)
    assert s == np.float32(1.0)
    assert np.array_equal(oracle.e4m3_decode(q), v.astype(np.float64))


def test_quantiser_all_zero_group():
    q, s = oracle.quantise_group(np.zeros(128, np.float32))
    assert s == np.float32(1.0) and np.all(q == 0)


@pytest.mark.parametrize("quant", ["fp8_per_tensor", "fp8_block128"])
def test_activation_quantisation_matches_definition(quant):
    from workloads import random_activations, bf16_bits_to_f32
    a = random_activations(5, 256, 4, seed=11)
    codes, scales = oracle.quantise_activations(a["x"], quant)
    xf = bf16_bits_to_f32(a["x"])
    if quant == "fp8_per_tensor":
        s = np.float32(np.abs(xf).max()) / np.float32(448)
        assert scales == s
        ref = torch.from_numpy((xf / s).astype(np.float32)).to(torch.float8_e4m3fn)
        assert np.array_equal(codes, ref.view(torch.uint8).numpy())
    else:
        blk = xf.reshape(5, 2, 128)
        s = (np.abs(blk).max(axis=2).astype(np.float32) / np.float32(448)).astype(np.float32)
        assert np.array_equal(scales, s)
        ref = torch.from_numpy((blk / s[:, :, None]).astype(np.float32)).to(torch.float8_e4m3fn)
        assert np.array_equal(codes, ref.view(torch.uint8).numpy().reshape(5, 256))


# ---------------------------------------------------------------------- MX --
def test_mx_scale_rule_landmarks():
    """E8M0 byte = floor(log2 amax) - 8 + 127 (8 = e4m3's largest exponent): amax 448 and 256
    keep scale 1, just under 256 halves it, 1.0 gives 2^-8; an all-zero group takes byte 0 and
    tiny magnitudes clamp at byte 0."""
    assert oracle.mx_scale_byte(448.0) == 127
    assert oracle.mx_scale_byte(256.0) == 127
    assert oracle.mx_scale_byte(511.9) == 127
    assert oracle.mx_scale_byte(255.9) == 126
    assert oracle.mx_scale_byte(1.0) == 119
    assert oracle.mx_scale_byte(0.75) == 118
    assert oracle.mx_scale_byte(0.0) == 0
    assert oracle.mx_scale_byte(2.0 ** -130) == 0
    assert oracle.mx_scale_byte(3.0e38) == 246   # floor(log2) = 127: fp32 never reaches the upper clamp


def test_mx_group_codes_and_range():
    """Every nonzero group's largest |v| / scale lies in [256, 512) (so its code is >= 256 or
    saturates at 448); the codes are torch's e4m3 cast of v / scale, saturated."""
    rng = np.random.default_rng(11)
    for trial in range(200):
        v = (rng.standard_normal(32) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32)
        q, b = oracle.quantise_group_mx(v)
        scale = 2.0 ** (b - 127)
        r = np.max(np.abs(v)) / scale
        assert 256.0 <= r < 512.0, (trial, r)
        ref = torch.clamp(torch.from_numpy(v.astype(np.float64) / scale).float(), -448.0, 448.0)
        assert np.array_equal(q, ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    q, b = oracle.quantise_group_mx(np.zeros(32, np.float32))
    assert b == 0 and not q.any()
