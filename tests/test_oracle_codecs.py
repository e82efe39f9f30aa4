"""Pins for the oracle's number formats and activation-quantisation rule.

The oracle's codecs are pinned to torch's CPU float8/bfloat16 casts (library
routines), to the closed-form definitions of the OCP formats, and to
invariants any correct quantiser must satisfy.
"""
import numpy as np
import pytest
import torch

import oracle


def _fp32_patterns():
    """fp32 values whose low mantissa bits sit on and around every rounding
    boundary of 3- and 7-bit mantissas, for every exponent and sign."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF,
                     0x0FFFFF & 0xFFFF, 0x0800, 0x1000], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    # also vary the bits that decide 3-bit-mantissa ties (bits 19..20)
    extra = (hi[:, None] | np.array([0x80000 - 1, 0x80000, 0x80001, 0x100000 - 1],
                                    dtype=np.uint32)[None, :]).ravel()
    v = np.concatenate([bits, extra]).view(np.float32)
    return v[np.isfinite(v)]


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_e4m3_closed_form_special_values():
    d = oracle.e4m3_decode
    assert d(0x7E) == 448.0                 # largest finite
    assert d(0x01) == 2.0 ** -9             # smallest subnormal
    assert d(0x08) == 2.0 ** -6             # smallest normal
    assert d(0x38) == 1.0                   # exponent field 7 = bias
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))


def test_e4m3_encode_matches_torch_rne():
    v = _fp32_patterns()
    v = np.clip(v, -448.0, 448.0).astype(np.float32)
    # keep the test quick: every 3rd pattern plus all tiny/huge ones
    sel = (np.arange(v.size) % 3 == 0) | (np.abs(v) < 2 ** -5) | (np.abs(v) > 256)
    v = v[sel]
    ours = oracle.e4m3_encode(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (v[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_e4m3_encode_saturates():
    for a in (448.0, 448.5, 463.9, 464.0, 500.0, 1e30):
        assert oracle.e4m3_encode(np.array([a]))[0] == 0x7E
        assert oracle.e4m3_encode(np.array([-a]))[0] == 0xFE


def test_bf16_round_matches_torch():
    v = _fp32_patterns()
    v = v[np.abs(v) < 3e38]
    v = v[::5]
    ours = oracle.bf16_round(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (v[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint16)
    ours = oracle.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e8m0_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_e2m1_closed_form():
    # (-1)^s * 2^(E-1) * (1 + M/2) for E > 0; (-1)^s * M/2 for E == 0
    for c in range(16):
        s, E, M = c >> 3, (c >> 1) & 3, c & 1
        ref = (M / 2.0) if E == 0 else 2.0 ** (E - 1) * (1 + M / 2.0)
        ref = -ref if s else ref
        assert oracle.e2m1_decode(np.array([c]))[0] == ref


# ------------------------------------------------------------------ quantisation
def _torch_quant_token(v32):
    """Per-group FP8 quantisation written with torch ops: fp32 scale
    amax/448, fp32 division, clamp, torch's RNE cast."""
    t = torch.from_numpy(v32.astype(np.float32))
    amax = t.abs().amax(dim=1, keepdim=True)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = torch.clamp(t / s, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.numpy(), s.to(torch.float64).numpy()[:, 0]


@pytest.mark.parametrize("fmt,g", [(oracle.A_FP8_TOKEN, 512), (oracle.A_FP8_G128, 128)])
def test_fp8_group_quant_matches_torch(fmt, g):
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((6, 512)) * 0.02).astype(np.float32)
    v[2] = 0.0                                  # an all-zero row
    v[3, :5] = [1e-8, -1e-8, 3.0, -3.0, 0.0]   # wide dynamic range
    q, s = oracle.quant_rows(v.astype(np.float64), fmt)
    qr, sr = _torch_quant_token(v.reshape(-1, g))
    np.testing.assert_array_equal(q.reshape(-1, g), qr)
    np.testing.assert_array_equal(s.reshape(-1), sr)


def test_fp8_quant_invariants():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal((4, 256)) * 0.05).astype(np.float32).astype(np.float64)
    q, s = oracle.quant_rows(v, oracle.A_FP8_TOKEN)
    deq = oracle.e4m3_decode(q) * s
    # the largest magnitude lands on the top code
    for r in range(4):
        i = np.argmax(np.abs(v[r]))
        assert (q[r, i] & 0x7F) == 0x7E
    # half-ulp relative error for normals (3 mantissa bits), absolute 2^-10*s below
    err = np.abs(deq - v)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * s)
    assert np.all(err <= bound * (1 + 1e-12))
    zq, zs = oracle.quant_rows(np.zeros((1, 128)), oracle.A_FP8_TOKEN)
    assert zs[0, 0] == 1.0 and not zq.any()


def test_mxfp8_quant_rule():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((3, 64)) * 0.03).astype(np.float32).astype(np.float64)
    v[1, 32:] = 0.0
    q, X = oracle.quant_rows(v, oracle.A_MXFP8_G32)
    assert X.shape == (3, 2)
    for r in range(3):
        for b in range(2):
            blk = v[r, 32 * b:32 * b + 32]
            a = np.abs(blk).max()
            if a == 0:
                assert X[r, b] == 2.0 ** -127
                assert not q[r, 32 * b:32 * b + 32].any()
                continue
            # X is a power of two with amax / X in [256, 512)
            m, e = np.frexp(X[r, b])
            assert m == 0.5
            assert 256 <= a / X[r, b] < 512
            scaled = blk / X[r, b]
            ref = torch.from_numpy(np.clip(scaled, -448, 448).astype(np.float32)).to(
                torch.float8_e4m3fn).view(torch.uint8).numpy()
            np.testing.assert_array_equal(q[r, 32 * b:32 * b + 32], ref)
