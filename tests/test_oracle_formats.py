"""Pins of the oracle's format decoders against published definitions."""
import os

import numpy as np
import pytest
import torch

from oracle import formats, mx
from synth import f32_to_bf16_bits


def _golden_e2m1(golden_dir):
    table = {}
    with open(os.path.join(golden_dir, "ocp_mx_e2m1.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            table[int(code, 16)] = float(val)
    return table


def test_e2m1_matches_ocp_table(golden_dir):
    table = _golden_e2m1(golden_dir)
    assert sorted(table) == list(range(16))
    got = formats.e2m1_to_f64(np.arange(16))
    for c in range(16):
        assert got[c] == table[c], c
        # the sign bit is kept: codes 0x8.. are the negatives (and -0.0)
        assert np.signbit(got[c]) == (c >= 8), c


def test_e8m0_scale():
    b = np.arange(256)
    v = formats.e8m0_to_f64(b)
    assert v[127] == 1.0 and v[128] == 2.0 and v[119] == 2.0 ** -8 and v[123] == 2.0 ** -4
    assert v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127
    assert np.isnan(v[255])


def test_mxfp4_grid_all_codes_and_workload_scales(golden_dir):
    """16 codes x 5 scales land on {0,.5,1,1.5,2,3,4,6} x 2^e, exactly in bf16."""
    table = _golden_e2m1(golden_dir)
    for S in range(119, 124):
        codes = np.zeros((1, 16), np.uint8)
        # elements 0..31: element 2i = low nibble, 2i+1 = high nibble of byte i
        elems = np.array([c % 16 for c in range(32)], dtype=np.uint8)
        codes[0] = elems[0::2] | (elems[1::2] << 4)
        scales = np.full((1, 1), S, np.uint8)
        v = formats.mxfp4_to_f64(codes, scales)[0]
        for i in range(32):
            assert v[i] == table[i % 16] * 2.0 ** (S - 127)
        # every such value is exactly a bfloat16 (<= 2 significant bits)
        bits = f32_to_bf16_bits(v.astype(np.float32))
        assert np.array_equal(formats.bf16_to_f64(bits), v)


def test_mxfp4_nibble_order_and_block_axis():
    # byte 0x71: element 0 = code 1 (0.5), element 1 = code 7 (6.0)
    codes = np.zeros((2, 32), np.uint8)
    codes[0, 0] = 0x71
    codes[1, 16] = 0x2F   # row 1, elements 32 (code 0xF = -6) and 33 (code 2 = 1.0)
    scales = np.full((2, 2), 127, np.uint8)
    scales[1, 1] = 129    # second block of row 1 scaled by 4
    v = formats.mxfp4_to_f64(codes, scales)
    assert v.shape == (2, 64)
    assert v[0, 0] == 0.5 and v[0, 1] == 6.0 and np.count_nonzero(v[0]) == 2
    assert v[1, 32] == -24.0 and v[1, 33] == 4.0 and np.count_nonzero(v[1]) == 2


def test_mxfp4_rejects_mismatched_scales():
    with pytest.raises(ValueError):
        formats.mxfp4_to_f64(np.zeros((2, 16), np.uint8), np.zeros((2, 2), np.uint8))


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(10000) * np.exp(rng.uniform(-20, 20, 10000))).astype(np.float32)
    bits = f32_to_bf16_bits(v)
    ours = formats.bf16_to_f64(bits)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    # and the bit patterns equal torch's own rounding
    tb = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, tb)


def test_bf16_round_half_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1.0078125 -> even (1.0)
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], np.float32)
    got = formats.bf16_to_f64(f32_to_bf16_bits(v))
    assert list(got) == [1.0, 1.0 + 2.0 ** -6, -1.0]


# ---------------------------------------------------------------- NVFP4

def _nvfp4_fixture(golden_dir):
    d = {}
    with open(os.path.join(golden_dir, "nvfp4_worked.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            d[key] = vals
    codes = np.array([int(v, 16) for v in d["codes"]], np.uint8)[None, :]
    scales = np.array([int(v, 16) for v in d["scales"]], np.uint8)[None, :]
    return codes, scales, float(d["tensor_scale"][0]), np.array([float(v) for v in d["values"]])


def test_nvfp4_worked_example(golden_dir):
    codes, scales, ts, want = _nvfp4_fixture(golden_dir)
    got = formats.nvfp4_to_f64(codes, scales, ts)[0]
    assert got.shape == want.shape
    assert np.array_equal(got, want)
    assert np.signbit(got[7]) and not np.signbit(got[15])  # code 8 is -0, code 0 is +0


def test_nvfp4_block_axis_is_16_and_nibble_order():
    """A single nonzero code at element j picks up the scale of block j // 16 only."""
    K = 64
    scales = np.array([[0x38, 0x40, 0x30, 0x3C]], np.uint8)      # E4M3: 1, 2, 0.5, 1.5
    per_block = [1.0, 2.0, 0.5, 1.5]
    for j in range(K):
        elems = np.zeros(K, np.uint8)
        elems[j] = 0x7                                            # E2M1 6.0
        codes = (elems[0::2] | (elems[1::2] << 4))[None, :]
        v = formats.nvfp4_to_f64(codes, scales, 1.0)[0]
        assert np.count_nonzero(v) == 1 and v[j] == 6.0 * per_block[j // 16]


def test_nvfp4_unit_scales_reduce_to_e2m1():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 256, size=(3, 16), dtype=np.uint8)
    v = formats.nvfp4_to_f64(codes, np.full((3, 2), 0x38, np.uint8), 1.0)
    nib = np.empty((3, 32), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = codes & 15, codes >> 4
    assert np.array_equal(v, formats.e2m1_to_f64(nib))


def test_nvfp4_matches_torch_composition(golden_dir):
    """Block scales through torch's float8_e4m3fn, E2M1 from the OCP table, the tensor scale as fp32."""
    table = _golden_e2m1(golden_dir)
    rng = np.random.default_rng(12)
    rows, K = 5, 96
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(rows, K // 16), dtype=np.uint8)   # every finite positive E4M3
    ts = np.float32(0.0173)
    got = formats.nvfp4_to_f64(codes, scales, ts)
    sc = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64)
    nib = torch.empty((rows, K), dtype=torch.int64)
    nib[:, 0::2] = torch.from_numpy(codes & 15).to(torch.int64)
    nib[:, 1::2] = torch.from_numpy(codes >> 4).to(torch.int64)
    e2m1 = torch.tensor([table[c] for c in range(16)], dtype=torch.float64)[nib]
    want = e2m1 * sc.repeat_interleave(16, dim=1) * float(torch.tensor(0.0173, dtype=torch.float32))
    assert np.array_equal(got, want.numpy())


def test_nvfp4_values_are_exact_in_bf16_before_the_tensor_scale():
    """E2M1 x E4M3 has at most 6 significant bits: exact in bf16 (the GPU's decode relies on it)."""
    vals = formats.e2m1_to_f64(np.arange(16))[:, None] * mx.e4m3_to_f64(np.arange(0x7F))[None, :]
    v = vals.ravel()
    bits = f32_to_bf16_bits(v.astype(np.float32))
    assert np.array_equal(formats.bf16_to_f64(bits), v)


def test_nvfp4_rejects_mismatched_scales():
    with pytest.raises(ValueError):
        formats.nvfp4_to_f64(np.zeros((2, 16), np.uint8), np.zeros((2, 1), np.uint8), 1.0)
