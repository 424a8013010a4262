"""Storage encoders (synth) and the oracle's own decoders, checked against
torch's CPU casts -- an independent implementation of both formats."""
import numpy as np
import pytest
import torch

from synth.codecs import f32_to_bf16_bits, f32_to_fp8_rowwise, FP8_E4M3_MAX
from oracle import bf16_bits_to_f64, fp8_e4m3fn_to_f64, round_to_storage


def _edge_f32():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3.4e38], dtype=np.float32),
    ])
    # values exactly half-way between two bf16 numbers (both tie directions)
    halves = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32) * np.float32(1.0)
    return np.concatenate([x, halves.astype(np.float32)])


def test_bf16_encoder_matches_torch_cast():
    x = _edge_f32()
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_decoder_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_fp8_decoder_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8_e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.nanmax(ours) == FP8_E4M3_MAX
    assert ours[1] == 2.0 ** -9          # smallest subnormal


def test_fp8_encoder_matches_torch_cast():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((64, 300)) * 0.02).astype(np.float32)
    w[3, 7] = 0.0
    w[5, :] = 0.0                         # an all-zero row keeps scale 1
    codes, scale = f32_to_fp8_rowwise(w)
    x = w.astype(np.float64) / scale.astype(np.float64)[:, None]
    assert np.abs(x).max() <= FP8_E4M3_MAX * (1 + 1e-6)
    # torch rounds binary32 inputs; feed it the exactly representable quotient
    # rounded to binary32 only where that is exact enough not to move a tie.
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    deq = fp8_e4m3fn_to_f64(codes) * scale[:, None]
    rel = np.abs(deq - w) / np.maximum(np.abs(w).max(axis=1, keepdims=True), 1e-30)
    assert rel.max() <= 2.0 ** -4 + 1e-12   # half a step of the 3-bit mantissa


def test_round_to_storage():
    x = np.array([1.0 + 2 ** -9, 1.0 + 3 * 2 ** -9, -2.0 ** -130, 1e-3], dtype=np.float64)
    b = round_to_storage(x, "bf16")
    ref = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(b, ref)
    f = round_to_storage(x, "fp32")
    assert np.array_equal(f, x.astype(np.float32).astype(np.float64))
