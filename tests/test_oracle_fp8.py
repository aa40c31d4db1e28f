"""Pins of the oracle's FP8 e4m3 -> fp32 -> int4 converter front-end.

The e4m3 decode is checked against PyTorch's float8_e4m3fn (an independent
implementation of the same format) on all 256 codes and against hand-worked
values of the format's definition (bias 7, subnormals m * 2^-9, no
infinities); the 128 x 128 block-scale placement against a numpy expansion of
the scale grid; the pack against pack_int4 of independently dequantised
weights.
"""
import numpy as np
import pytest
import torch


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def test_e4m3_all_codes_match_torch(ref):
    codes = np.arange(256, dtype=np.uint8)
    want = _torch_decode(codes)
    got = np.array([ref.e4m3_to_f32(int(c)) for c in codes], np.float32)
    nan = np.isnan(want)
    assert nan.sum() == 2 and set(codes[nan]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert np.all(got[nan] == 0.0)  # NaN codes convert to 0


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0)])
def test_e4m3_hand_values(ref, code, value):
    assert ref.e4m3_to_f32(code) == np.float32(value)


def test_block_scales_cover_128x128_tiles(ref):
    rng = np.random.RandomState(5)
    rows, cols = 200, 320  # ragged: 2 x 3 blocks, partial last ones
    q8 = rng.randint(0, 256, size=(rows, cols)).astype(np.uint8)
    q8[q8 == 0x7F] = 0x7E
    q8[q8 == 0xFF] = 0xFE
    bs = (2.0 ** rng.randint(-8, 8, size=(2, 3)) * rng.uniform(0.5, 1.0, size=(2, 3))).astype(np.float32)
    grid = np.repeat(np.repeat(bs, 128, axis=0), 128, axis=1)[:rows, :cols]
    want = (_torch_decode(q8) * grid).astype(np.float32)  # fp32 product, one rounding
    np.testing.assert_array_equal(ref.fp8_to_f32(q8, bs), want)


def test_pack_fp8_is_pack_of_dequantised(ref):
    rng = np.random.RandomState(6)
    rows, cols = 130, 256
    q8 = rng.randint(0, 256, size=(rows, cols)).astype(np.uint8)
    q8[q8 == 0x7F] = 0
    q8[q8 == 0xFF] = 0
    q8[7] = 0  # an all-zero row packs to zero codes and scale 0
    bs = rng.uniform(1e-3, 1e-2, size=(2, 2)).astype(np.float32)
    grid = np.repeat(np.repeat(bs, 128, axis=0), 128, axis=1)[:rows, :cols]
    w = (_torch_decode(q8) * grid).astype(np.float32)
    q_want, s_want = ref.pack_int4(w)
    q, s = ref.pack_fp8_int4(q8, bs)
    np.testing.assert_array_equal(q, q_want)
    np.testing.assert_array_equal(s, s_want)
    assert s[7] == 0 and np.all(q[7] == 0)
