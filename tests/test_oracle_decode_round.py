"""Pins for the oracle's E4M3 decode and its fp64 -> bf16/fp16/fp32 rounding.

The decode is checked against torch's float8_e4m3fn (a library definition of
OCP E4M3) on every code and against values the OCP format fixes; the rounding
is checked against numpy's direct double->half and double->float casts and,
for bf16, against torch's bf16 value set (every representable value, every
midpoint between neighbours, and points just either side of each midpoint).
"""
import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_decode_matches_torch_all_codes():
    t = oracle.e4m3_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan], ref[~nan])
    # signed zeros too
    assert np.array_equal(np.signbit(t[~nan]), np.signbit(ref[~nan]))


def test_decode_format_landmarks():
    v = oracle.e4m3_value
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0           # largest finite
    assert v(0x08) == 2.0 ** -6                             # smallest normal
    assert v(0x01) == 2.0 ** -9                             # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9                         # largest subnormal
    assert v(0x38) == 1.0 and v(0xB8) == -1.0
    assert v(0x00) == 0.0 and not math.copysign(1, v(0x00)) < 0
    assert v(0x80) == 0.0 and math.copysign(1, v(0x80)) < 0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))      # only NaNs, no infinities
    t = oracle.e4m3_table()
    assert np.isnan(t).sum() == 2 and not np.isinf(t).any()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                         # monotone in the code


def _rand_doubles(rng, n, lo_exp, hi_exp):
    mant = rng.random(n) + 0.5
    e = rng.integers(lo_exp, hi_exp, n)
    s = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    return s * np.ldexp(mant, e)


def test_round_fp32_matches_numpy():
    rng = np.random.default_rng(11)
    x = np.concatenate([_rand_doubles(rng, 200000, -160, 130),
                        [0.0, -0.0, np.inf, -np.inf, 3.4028235677973366e38, 3.40282357e38,
                         2.0 ** -149, 2.0 ** -150, 3 * 2.0 ** -151]])
    got = oracle.round_bits(x, "fp32")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, ref)


def test_round_fp16_matches_numpy():
    rng = np.random.default_rng(12)
    # random values over the whole fp16 range plus constructed ties
    x = _rand_doubles(rng, 200000, -27, 18)
    ties = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -25, 3 * 2.0 ** -25,
                     65504.0, 65519.99, 65520.0, 65536.0, -65520.0, 2.0 ** -14 * (1 - 2.0 ** -11)])
    x = np.concatenate([x, ties, -ties, [0.0, -0.0, np.inf, -np.inf]])
    got = oracle.round_bits(x, "fp16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def _bf16_values():
    bits = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16)  # +0 .. max finite
    return bits.view(torch.bfloat16).double().numpy(), np.arange(0, 0x7F80, dtype=np.uint16)


def test_round_bf16_against_value_set():
    vals, bits = _bf16_values()
    # representable values round to themselves (both signs)
    assert np.array_equal(oracle.round_bits(vals, "bf16"), bits)
    assert np.array_equal(oracle.round_bits(-vals[1:], "bf16"), bits[1:] | 0x8000)
    # midpoints round to the neighbour with an even code; off-midpoints to the nearer
    lo, hi = vals[:-1], vals[1:]
    mid = (lo + hi) / 2                               # exact in fp64
    even = np.where(bits[:-1] % 2 == 0, bits[:-1], bits[1:])
    assert np.array_equal(oracle.round_bits(mid, "bf16"), even)
    eps = (hi - lo) * 2.0 ** -20
    assert np.array_equal(oracle.round_bits(mid - eps, "bf16"), bits[:-1])
    assert np.array_equal(oracle.round_bits(mid + eps, "bf16"), bits[1:])
    # overflow: the first value past max + half an ulp goes to +inf
    mx = vals[-1]
    half = (mx - vals[-2]) / 2
    assert oracle.round_bits(np.array([mx + half]), "bf16")[0] == 0x7F80
    assert oracle.round_bits(np.array([mx + half * (1 - 2.0 ** -20)]), "bf16")[0] == 0x7F7F
    assert oracle.round_bits(np.array([-np.inf]), "bf16")[0] == 0xFF80
    assert oracle.round_bits(np.array([np.nan]), "bf16")[0] & 0x7FFF > 0x7F80


def test_round_bf16_is_one_step_from_fp64():
    # 1 + 2^-8 is a tie (-> 1.0); 1 + 2^-8 + 2^-40 is not, and must go up.
    # A two-step fp64->fp32->bf16 cast would lose the 2^-40 and round down.
    x = np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 1 + 3 * 2.0 ** -8])
    got = oracle.bits_to_f64(oracle.round_bits(x, "bf16"), "bf16")
    assert list(got) == [1.0, 1 + 2.0 ** -7, 1 + 2.0 ** -6]


def test_ulp_landmarks():
    assert oracle.ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -7
    assert oracle.ulp(np.array([1.0]), "fp16")[0] == 2.0 ** -10
    assert oracle.ulp(np.array([1.0]), "fp32")[0] == 2.0 ** -23
    assert oracle.ulp(np.array([0.0]), "fp16")[0] == 2.0 ** -24
    assert oracle.ulp(np.array([1.9999999]), "bf16")[0] == 2.0 ** -7
    assert oracle.ulp(np.array([2.0]), "bf16")[0] == 2.0 ** -6
