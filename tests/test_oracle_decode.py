"""Pins for oracle.decode: the fp8 / bf16 decoders against PyTorch's casts."""
import numpy as np
import pytest
import torch

from oracle.decode import decode_bf16, decode_fp8_e4m3, fp8_e4m3_table
from psattn_inputs import f32_to_bf16_bits, f32_to_fp8_bits


def test_fp8_table_matches_torch_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = fp8_e4m3_table()
    nan = np.isnan(ref)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], ref[~nan])
    assert tab[0x7E] == 448.0 and tab[0x01] == 2.0 ** -9


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_generator_encoders_round_to_nearest_even():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(50000).astype(np.float32) * 3
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # ties to even
    b = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)
    f8 = f32_to_fp8_bits(x)
    assert np.array_equal(decode_fp8_e4m3(f8), torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy())
