"""Pins of the MXFP8 activation quantizer (native MXFP4 mode) against the OCP
MX v1.0 definitions, an independent library conversion and a hand-worked
fixture."""
import os

import numpy as np
import pytest
import torch

from oracle import formats, moe, mx


def _golden_blocks(golden_dir):
    blocks = []
    with open(os.path.join(golden_dir, "mxfp8_worked.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            a, b = line.split()
            if a == "block":
                blocks.append((int(b), [], []))
                continue
            v = float.fromhex(a) if a.lstrip("-").startswith("0x") else float(a)
            blocks[-1][1].append(v)
            blocks[-1][2].append(int(b, 16))
    return blocks


def test_e4m3_special_values():
    # OCP MX v1.0 E4M3: max normal S.1111.110 = 448, min normal S.0001.000 = 2^-6,
    # max subnormal S.0000.111 = 0.875 * 2^-6, min subnormal S.0000.001 = 2^-9,
    # NaN S.1111.111, no infinities
    d = mx.e4m3_to_f64
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6 and d(0x07) == 0.875 * 2.0 ** -6 and d(0x01) == 2.0 ** -9
    assert d(0x38) == 1.0 and d(0x3C) == 1.5 and d(0x40) == 2.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x00) == 0.0 and d(0x80) == 0.0 and np.signbit(d(0x80))


def test_e4m3_decode_matches_torch_for_all_codes():
    c = np.arange(256)
    ours = mx.e4m3_to_f64(c)
    ref = torch.tensor(c, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_rounding_matches_torch_on_every_bf16_in_range():
    # every bf16 bit pattern whose magnitude is at most 448 (torch does not saturate,
    # so the comparison stops there); float32 -> float8_e4m3fn is round to nearest even
    bits = np.arange(65536, dtype=np.uint32)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # drop Inf / NaN patterns
    v = formats.bf16_to_f64(bits.astype(np.uint16))
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    v = v[keep]
    ours = mx.round_to_e4m3(v)
    ref = torch.tensor(v, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_above_448():
    v = np.array([448.0, 449.0, 463.9, 464.0, 479.0, 480.0, 1e6, -470.0, -1e30])
    got = mx.round_to_e4m3(v)
    assert got.tolist() == [0x7E] * 7 + [0xFE, 0xFE]


def test_hand_worked_blocks(golden_dir):
    for want_scale, vals, codes in _golden_blocks(golden_dir):
        row = np.zeros((1, 32))
        row[0, :len(vals)] = vals
        q, s = mx.mxfp8_quantize(row)
        assert s.tolist() == [[want_scale]]
        assert q[0, :len(vals)].tolist() == codes, (vals, q[0, :len(vals)], codes)
        assert not q[0, len(vals):].any()


@pytest.mark.parametrize("p", [-20, -8, -1, 0, 3, 15])
def test_block_scale_closed_form(p):
    # amax in [2^p, 2^(p+1)) -> X = 2^(p-8), byte p - 8 + 127
    rng = np.random.default_rng(p + 100)
    for amax in (2.0 ** p, 1.999 * 2.0 ** p, 1.5 * 2.0 ** p):
        row = rng.uniform(-1, 1, size=(1, 32)) * amax
        row[0, 7] = -amax
        assert mx.block_scale_bytes(row).tolist() == [[p - 8 + 127]]


def test_block_maximum_lands_in_top_binade():
    # X = 2^(floor(log2 amax) - 8) puts the block's largest magnitude in [256, 512),
    # i.e. codes 0x78..0x7E (saturated at 448); a scale off by one binade would not
    rng = np.random.default_rng(5)
    v = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, size=(64, 1)))
    q, s = mx.mxfp8_quantize(v)
    qb = (q & 0x7F).reshape(64, 8, 32)
    vb = np.abs(v).reshape(64, 8, 32)
    top = np.take_along_axis(qb, vb.argmax(axis=2)[..., None], axis=2)[..., 0]
    assert ((top >= 0x78) & (top <= 0x7E)).all()


def test_quantization_error_bound():
    # within the normal range of the scaled values the error is at most half an
    # E4M3 ulp (2^-4 relative); below 2^-6 X it is at most half a subnormal step
    # (2^-10 X); saturated values (v / X > 448) lose at most 64 X
    rng = np.random.default_rng(6)
    v = rng.standard_normal((128, 128)) * np.exp2(rng.integers(-12, 12, size=(128, 128)))
    q, s = mx.mxfp8_quantize(v)
    X = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    err = np.abs(mx.mxfp8_to_f64(q, s) - v)
    a = np.abs(v) / X
    normal = (a >= 2.0 ** -6) & (a <= 448)
    assert (err[normal] <= 2.0 ** -4 * np.abs(v[normal])).all()
    assert (err[a < 2.0 ** -6] <= 2.0 ** -10 * X[a < 2.0 ** -6]).all()
    assert (err[a > 448] <= 64 * X[a > 448]).all()
    assert np.array_equal(np.signbit(mx.e4m3_to_f64(q)), np.signbit(v))


def test_zero_block_and_clamped_scale():
    q, s = mx.mxfp8_quantize(np.zeros((2, 64)))
    assert not q.any() and not s.any()
    # exponents below -127 clamp to byte 0 and the codes still follow v / 2^-127
    tiny = np.full((1, 32), 2.0 ** -131)
    tiny[0, 1] = 2.0 ** -140            # 2^-13 after scaling: below half a subnormal step
    q, s = mx.mxfp8_quantize(tiny)
    assert s.tolist() == [[0]]
    assert q[0, 0] == 0x18 and q[0, 1] == 0x00   # 2^-4 -> exponent field 3
    assert mx.mxfp8_to_f64(q, s)[0, 0] == 2.0 ** -131


def test_round_to_bf16_matches_torch():
    # float32 inputs: torch's float -> bfloat16 is round to nearest even with no
    # double rounding, so it is the definition
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(200000) * np.exp2(rng.integers(-40, 40, 200000))).astype(np.float32)
    ours = mx.round_to_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_swiglu_expert_mx_composition():
    # the native-mode expert built from torch's own conversions: codes from
    # torch's E4M3 rounding of v / X, torch's bf16 rounding of the hidden vector
    rng = np.random.default_rng(8)
    n, H, I = 5, 64, 96
    X = formats.bf16_to_f64(rng.integers(0, 65536, size=(n, H)).astype(np.uint16) & 0xBFFF)
    X = np.clip(X, -8, 8)
    Wg, Wu = rng.standard_normal((I, H)) * 0.1, rng.standard_normal((I, H)) * 0.1
    Wd = rng.standard_normal((H, I)) * 0.1

    def torch_mx(v):
        s = mx.block_scale_bytes(v)
        Xs = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
        c = torch.tensor(np.clip(v / Xs, -448, 448), dtype=torch.float32).to(torch.float8_e4m3fn)
        return c.to(torch.float64).numpy() * Xs

    Xq = torch_mx(X)
    G, U = Xq @ Wg.T, Xq @ Wu.T
    h = G / (1.0 + np.exp(-G)) * U
    hb = torch.tensor(h, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    want = torch_mx(hb) @ Wd.T
    got, got_h = moe.swiglu_expert_mx(X, Wg, Wu, Wd, return_hidden=True)
    # (torch rounds float64 -> float32 -> bf16; no value here sits where that differs)
    assert np.array_equal(got_h, hb)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_native_layer_stays_near_the_exact_layer():
    # MXFP8 activations change the layer by a few percent, not more (a quantizer
    # that dropped a scale or a block would not)
    rng = np.random.default_rng(9)
    T, H, I, E, k = 6, 128, 64, 4, 2
    x = formats.bf16_to_f64((rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    W = [(rng.standard_normal((I, H)) * 0.05, rng.standard_normal((I, H)) * 0.05,
          rng.standard_normal((H, I)) * 0.05) for _ in range(E)]
    logits = rng.standard_normal((T, E)).astype(np.float32)
    kw = dict(k=k, E=E, gating="softmax", renormalize=True, experts=lambda e: W[e], logits=logits)
    exact = moe.moe_layer(x, **kw)["out"]
    native = moe.moe_layer(x, native_mx=True, **kw)["out"]
    rel = np.linalg.norm(native - exact) / np.linalg.norm(exact)
    assert 1e-3 < rel < 6e-2
