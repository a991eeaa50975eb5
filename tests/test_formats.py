"""Storage formats: the generator's encoders and the oracle's decoders are each
checked against the format definitions and against torch's own dtypes."""
import numpy as np
import pytest

import oracle as O
import synth

torch = pytest.importorskip("torch")


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = O.decode_e4m3(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2  # 0x7F and 0xFF
    np.testing.assert_array_equal(mine[~nan], theirs[~nan])
    # spot values from the OCP definition
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0
    assert mine[0x38] == 1.0 and mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9
    assert mine[0x07] == 7 * 2.0 ** -9


def test_bf16_roundtrip_and_rounding_vs_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        rng.standard_normal(1000).astype(np.float32) * 1e-30,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.0e38], np.float32)])
    # exact ties: 1 + 2^-8 (tie, round to even -> 1) and 1 + 3*2^-8 (tie -> up)
    bits = synth.f32_to_bf16_bits(x)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, t)
    np.testing.assert_array_equal(O.decode_bf16(bits),
                                  torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
                                  .to(torch.float64).numpy())


def test_e4m3_encode_vs_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-460, 460, 200000), rng.uniform(-0.03, 0.03, 50000),
                        O.E4M3_VALUES[np.isfinite(O.E4M3_VALUES)],
                        # midpoints between neighbouring codes: exact ties
                        0.5 * (O.E4M3_VALUES[0:0x7E] + O.E4M3_VALUES[1:0x7F])]).astype(np.float32)
    codes = synth.f32_to_e4m3(x)
    clamped = torch.from_numpy(np.clip(x, -448, 448))
    t = clamped.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # zero: torch keeps the sign of -0.0; so do we
    np.testing.assert_array_equal(codes, t)


def test_block_quantisation_scales():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 3, 16)).astype(np.float32)
    x[128:256, 1] = 0.0
    codes, scales = synth.quantize_blocks_e4m3(x, 128)
    assert scales.shape == (3, 3)
    assert scales[1, 1] == 1.0
    for b in range(3):
        blk = x[b * 128:(b + 1) * 128]
        amax = np.abs(blk).max(axis=(0, 2))
        for h in range(3):
            if amax[h] > 0:
                assert scales[b, h] == np.float32(amax[h] / np.float32(448.0))
                dq = O.decode_e4m3(codes[b * 128:(b + 1) * 128, h]) * scales[b, h]
                # RNE to 3 mantissa bits: relative error <= 2^-4 above the subnormal range
                big = np.abs(blk[:, h]) >= scales[b, h] * 2.0 ** -6
                err = np.abs(dq - blk[:, h])
                assert np.all(err[big] <= np.abs(blk[:, h][big]) * 2.0 ** -4 + 1e-12)
                assert np.abs(dq).max() <= 448.0 * scales[b, h] * (1 + 1e-7)
