"""Pins for the bit-pattern codecs (oracle side) and the input generator."""
import numpy as np
import pytest
import torch

import fa_inputs as fi
from oracle import decode_bf16, decode_e4m3fn, decode_f16, dequant_fp8_rows


# ---------------------------------------------------------------------------
# decoders, exhaustively, against library interpretations of the same bits
# ---------------------------------------------------------------------------

@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_bf16_decode_all_codes():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = decode_bf16(codes)
    lib = (codes.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], lib[~nan])


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_f16_decode_all_codes():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = decode_f16(codes)
    lib = codes.view(np.float16).astype(np.float64)
    nan = np.isnan(lib)
    assert nan.sum() == 2 * 1023
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], lib[~nan])
    assert ours[0x3C00] == 1.0 and ours[0x7BFF] == 65504.0 and ours[0x0001] == 2.0 ** -24
    assert ours[0x0400] == 2.0 ** -14 and ours[0xC000] == -2.0 and ours[0x7C00] == np.inf


@pytest.mark.filterwarnings("ignore:overflow encountered in cast:RuntimeWarning")
def test_f16_encode_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.float32([0.0, -0.0, 65504.0, 65520.0, 1e-8, 2.0 ** -25, 3 * 2.0 ** -25,
                                    1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11])])
    ours = fi.f32_to_f16_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # ties to even: 1 + 2^-11 lies halfway between 1 and 1 + 2^-10
    assert ours[-2] == 0x3C00 and ours[-1] == 0x3C02 and ours[-6] == 0x7C00


def test_e4m3fn_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_e4m3fn(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], lib[~nan])
    assert ours[0x7E] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9
    assert ours[0x38] == 1.0 and ours[0xFE] == -448.0 and ours[0xBE] == -1.75


def test_dequant_rows():
    codes = np.full((2, 130, 3), 0x38, dtype=np.uint8)   # all 1.0
    scales = np.array([[1.0, 2.0, 4.0], [0.5, 0.25, 8.0]], dtype=np.float32)
    x = dequant_fp8_rows(codes, scales)
    assert x.shape == (2, 130, 3)
    assert np.all(x[0, :64] == 1.0) and np.all(x[0, 64:128] == 2.0) and np.all(x[0, 128:] == 4.0)
    assert np.all(x[1, 127] == 0.25) and np.all(x[1, 129] == 8.0)


# ---------------------------------------------------------------------------
# encoders in the input generator
# ---------------------------------------------------------------------------

def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-38).astype(np.float32),   # subnormals
        np.array([0.0, -0.0, 1.0, -2.5, 3.0e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                  np.inf, -np.inf], dtype=np.float32),
    ])
    ours = fi.f32_to_bf16_bits(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, lib)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert fi.f32_to_bf16_bits(np.array([1.0 + 2 ** -8], np.float32))[0] == 0x3F80
    assert fi.f32_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8], np.float32))[0] == 0x3F82


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    y = np.concatenate([
        rng.standard_normal(100000) * 50,
        rng.standard_normal(10000) * 1e-2,
        decode_e4m3fn(np.arange(256, dtype=np.uint8)[np.r_[0:0x7F, 0x80:0xFF]]),
    ])
    y = np.clip(y, -448, 448).astype(np.float32).astype(np.float64)
    ours = fi.f64_to_e4m3fn_codes(y)
    lib = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of a value that rounds to zero; compare magnitudes there
    zero = decode_e4m3fn(lib) == 0
    np.testing.assert_array_equal(ours[~zero], lib[~zero])
    assert np.all(decode_e4m3fn(ours[zero]) == 0)


def test_e4m3_encode_ties_and_saturation():
    enc = fi.f64_to_e4m3fn_codes
    assert enc(np.array([1.0 + 2 ** -4]))[0] == 0x38          # tie -> even mantissa 0
    assert enc(np.array([1.0 + 3 * 2 ** -4]))[0] == 0x3A      # tie -> even mantissa 2
    assert enc(np.array([2.0 ** -10]))[0] == 0x00             # half the smallest subnormal
    assert enc(np.array([3 * 2.0 ** -10]))[0] == 0x02         # tie between 1 and 2 quanta
    assert enc(np.array([448.0, 460.0, 470.0, 1e9]))[0] == 0x7E
    assert np.all(enc(np.array([448.0, 460.0, 470.0, 1e9])) == 0x7E)
    assert np.all(enc(np.array([-470.0, -1e9])) == 0xFE)
    assert enc(np.array([7.5 * 2 ** -9]))[0] == 0x08          # rounds up to the first normal


def test_block_quantiser():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((200, 16)).astype(np.float32)
    x[70:128] = 0.0
    x[64:70] *= 1e-3
    codes, scales = fi.quantize_e4m3_rows(x)
    assert codes.shape == (200, 16) and scales.shape == (4,)
    xh = dequant_fp8_rows(codes, scales)
    for bi in range(4):
        blk = x[bi * 64:(bi + 1) * 64].astype(np.float64)
        amax = np.abs(blk).max()
        assert scales[bi] == np.float32(amax / np.float32(448.0))
        # the block maximum maps to the code 448, so it is reproduced to float32 precision
        assert np.abs(xh[bi * 64:(bi + 1) * 64]).max() == pytest.approx(amax, rel=2 ** -23)
        # every element within half an e4m3 quantum of its dequantised value
        rel = np.abs(xh[bi * 64:(bi + 1) * 64] - blk)
        assert np.all(rel <= np.maximum(np.abs(blk) * 2 ** -4, 2 ** -10 * scales[bi]) * (1 + 1e-6))
    zero = np.zeros((64, 4), np.float32)
    c0, s0 = fi.quantize_e4m3_rows(zero)
    assert s0[0] == 1.0 and np.all(c0 == 0)


# ---------------------------------------------------------------------------
# the generator: per-(b,h) reproducibility, shapes, outlier rate
# ---------------------------------------------------------------------------

def test_streams_reproducible_and_distinct():
    a = fi.normals(1, fi.Q_ID, 0, 0, 4, 8)
    b = fi.normals(1, fi.Q_ID, 0, 0, 4, 8)
    c = fi.normals(1, fi.K_ID, 0, 0, 4, 8)
    d = fi.normals(1, fi.Q_ID, 0, 1, 4, 8)
    assert np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)
    full = fi.bf16_tensor(2, fi.V_ID, 2, 3, 16, 8)
    np.testing.assert_array_equal(full[1, 2], fi.bf16_slice(2, fi.V_ID, 1, 2, 16, 8))


def test_fp8_outliers_and_slices():
    codes, scales = fi.fp8_tensor(5, fi.K_ID, 1, 2, 512, 128)
    assert codes.shape == (1, 2, 512, 128) and scales.shape == (1, 2, 8)
    c1, s1 = fi.fp8_slice(5, fi.K_ID, 0, 1, 512, 128)
    np.testing.assert_array_equal(codes[0, 1], c1)
    np.testing.assert_array_equal(scales[0, 1], s1)
    m = fi.stream(5, fi.OUTLIER_MASK_ID[fi.K_ID], 0, 0).random(size=(512, 128)) < 1e-3
    assert 20 < m.sum() < 120     # about 65 expected
    # outlier blocks have larger scales than the N(0,1) bulk
    assert scales.max() > 4.0 / 448


def test_workload_table():
    w = fi.WORKLOADS
    assert (w[3].B, w[3].H, w[3].N, w[3].d, w[3].causal) == (1, 16, 16384, 128, (True,))
    assert (w[4].B, w[4].H, w[4].Lkv, w[4].num_splits) == (8, 32, 65536, 64)
    assert w[1].out_dtype == "fp32" and w[2].causal == (False, True)
    assert w[5].kind == "fwd_fp8"
    assert w[2].scale == pytest.approx(128 ** -0.5)
