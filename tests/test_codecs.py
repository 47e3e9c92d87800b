"""Pins for the oracle's decoders and the input encoders (CPU only).

The decoders are checked against the format definitions (OCP FP8, OCP MX v1.0),
against an independent bit-field decoder (oracle.brute) and against torch's
own float8 / e8m0 / bfloat16 dtypes.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, codecs
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codecs.e4m3(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert nan.sum() == 2          # 0x7F and 0xFF only (E4M3FN has no infinities)


def test_e4m3_closed_form_points():
    t = codecs.E4M3_TABLE
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0xB8] == -1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x01] == 2.0 ** -9                              # smallest subnormal
    assert t[0x08] == 2.0 ** -6                              # smallest normal
    assert t[0x07] == 7 * 2.0 ** -9                          # largest subnormal
    assert math.copysign(1.0, t[0x80]) == -1.0 and t[0x80] == 0.0


def test_e4m3_brute_decoder_agrees():
    for c in range(256):
        a, b = codecs.E4M3_TABLE[c], brute.e4m3_scalar(c)
        assert (math.isnan(a) and math.isnan(b)) or a == b, c


def test_e2m1_table_is_ocp_fp4():
    expect = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(codecs.E2M1_TABLE[:8]) == expect
    assert list(codecs.E2M1_TABLE[8:]) == [-x for x in expect]
    for c in range(16):
        assert codecs.E2M1_TABLE[c] == brute.e2m1_scalar(c)


def test_e2m1_nibble_order():
    # element 2i is the low nibble: 0x21 -> [0.5, 1.0]; 0xF7 -> [6, -6]
    out = codecs.e2m1_unpack(np.array([[0x21, 0xF7]], dtype=np.uint8))
    assert out.tolist() == [[0.5, 1.0, 6.0, -6.0]]


def test_e8m0_matches_torch():
    e = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = e.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = codecs.e8m0(e.numpy())
    assert np.array_equal(ref[:255], ours[:255])
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_bf16_decode_matches_torch():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(4096, generator=g) * 100
    b = x.to(torch.bfloat16)
    ours = codecs.bf16(b.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(ours, b.to(torch.float64).numpy())
    assert brute.bf16_scalar(int(b.view(torch.int16)[3]) & 0xFFFF) == float(b[3])


def test_global_row_decode_matches_brute():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(3, 32), dtype=np.uint8)    # D = 64
    e8 = rng.integers(120, 134, size=(3, 2), dtype=np.uint8)
    rho = np.array([0.5, 1.25, 3.0], dtype=np.float32)
    ours = codecs.global_rows(codes, e8, rho)
    for r in range(3):
        assert ours[r].tolist() == brute.global_row(codes[r], e8[r], rho[r])


# ---------------------------------------------------------------- encoders

def test_encode_e4m3_saturates_and_rounds_even():
    x = torch.tensor([1000.0, -1000.0, 1.0, 1.0625, 1.1875, 0.0], dtype=torch.float32)
    c = synth.encode_e4m3(x).numpy()
    v = codecs.e4m3(c)
    # 1.0625 is halfway between 1.0 and 1.125 -> even mantissa (1.0);
    # 1.1875 is halfway between 1.125 and 1.25 -> even mantissa (1.25)
    assert v.tolist() == [448.0, -448.0, 1.0, 1.0, 1.25, 0.0]


def test_encode_mx_roundtrip_and_error_bound():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(64, 1664, generator=g)
    for rs in (False, True):
        codes, e8, rho = synth.encode_mx_e2m1(x, rs)
        assert codes.shape == (64, 832) and e8.shape == (64, 52)
        v = codecs.global_rows(codes.numpy(), e8.numpy(), None if rho is None else rho.numpy())
        xs = x.double().numpy()
        # OCP MX: shared exponent floor(log2(block amax)) - 2, so a block's top
        # elements may saturate at 6 * scale; after that clip, each element is
        # within half the widest E2M1 spacing (2 * scale) of its input.
        scale = np.repeat(codecs.e8m0(e8.numpy()), 32, axis=1)
        if rho is not None:
            scale = scale * rho.double().numpy()[:, None]
        clipped = np.clip(xs, -6 * scale, 6 * scale)
        assert np.all(np.abs(v - clipped) <= scale * 1.0 + 1e-6 * np.abs(xs))
        assert np.all(np.abs(xs) < 8 * scale * (1 + 1e-6))       # amax < 2^(floor(log2 amax)+1)
        # block maxima land on representable magnitudes without saturation error beyond 1 spacing
        assert np.all(np.abs(v) <= 6 * scale + 1e-12)


def test_encode_mx_exact_values_roundtrip():
    # values already on the E2M1 grid times a power of two survive exactly
    grid = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    row = torch.cat([grid, -grid, grid * 0.25, -grid * 0.25]) * 2.0 ** -3     # 32 values
    x = row.repeat(1, 4)                                                       # D = 128
    codes, e8, _ = synth.encode_mx_e2m1(x, False)
    v = codecs.global_rows(codes.numpy(), e8.numpy(), None)
    # the block max is 6 * 2^-3 -> E - 127 = -3; an element survives exactly iff |x| / 2^-3 is on the grid
    y = np.abs(x.double().numpy()) / 2.0 ** -3
    exact = np.isin(y, grid.double().numpy())
    assert exact.sum() > 64
    assert np.array_equal(v[exact], x.double().numpy()[exact])
    # 0.75 (a tie between 0.5 and 1.0) rounds to the even code, 1.0
    tie = y == 0.75
    assert tie.any() and np.all(np.abs(v[tie]) == 1.0 * 2.0 ** -3)


def test_row_bytes_match_pages():
    pc = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    D = 1664
    fp4_row = D // 2 + D // 32 + 4           # codes + E8M0 per 32 + fp32 row scale
    assert fp4_row == 888
    assert abs(fp4_row - pc["global_kv_bytes_per_token"]["value"]) / 890 < 0.01
    fp8_row = D + 4                          # one byte per element + fp32 scale
    smaller = 1 - fp4_row / fp8_row
    assert abs(smaller - pc["fp4_kv_smaller_than_fp8"]["value"]) < 0.03
    assert synth.WORKLOADS["decode_8k"]["W"] == pc["window_positions"]["value"]
    H, nq = synth.WORKLOADS["replay_h100k"]["replay"]
    assert nq == pc["replay_clip_offset"]["value"]


def test_e4m3_encoder_matches_torch_cast():
    """The oracle's round-to-nearest-even E4M3 encoder against torch's float8_e4m3fn cast
    (after clamping to +-448, which torch does not saturate), sign of zero included."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100_000) * s for s in (1e-3, 1.0, 30.0, 300.0)])
    x = np.concatenate([x, [0.0, -0.0, 448.0, 460.0, 1e9, -1e9, 2.0 ** -10, -(2.0 ** -10),
                            2.0 ** -9 * 1.5, 2.0 ** -11]]).astype(np.float32)
    mine = codecs.e4m3_encode(x)
    ref = torch.tensor(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)
    # a tie between two codes goes to the even one: 1.0625 lies halfway between 1.0 (0x38)
    # and 1.125 (0x39), 1.1875 between 1.125 and 1.25 (0x3A)
    assert codecs.e4m3_encode(np.array([1.0625, 1.1875])).tolist() == [0x38, 0x3A]


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(100_000) * 10.0 ** rng.integers(-5, 5, 100_000)
    x32 = x.astype(np.float32)
    mine = codecs.bf16_round(x32)
    ref = torch.tensor(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    # one rounding from float64, not two: 1 + 2^-8 + 2^-30 lies just above the midpoint
    # between 1 (0x3F80) and 1 + 2^-7 (0x3F81), so it rounds up; going through float32 first
    # would land exactly on the midpoint and round to the even 0x3F80.  The midpoint itself
    # goes to the even pattern; subnormals round on the 2^-133 grid.
    assert codecs.bf16_round(np.array([1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -8,
                                       1 + 3 * 2.0 ** -8, 1.5 * 2.0 ** -133, -0.0])).tolist() == \
        [0x3F81, 0x3F80, 0x3F82, 0x0002, 0x8000]
