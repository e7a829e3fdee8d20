"""Pins of the oracle's quantisers (the E4M3 encoder, per-token 1x128 row
quantisation of activations and 128x128 block quantisation of weights)
against what the format and the definition fix:

- the encoder inverts the decoder on every finite code (incl. -0);
- midpoints between neighbouring codes go to the even code, points just off
  a midpoint to the nearer code;
- it agrees with torch's float8_e4m3fn cast (an independent library routine,
  round to nearest even, no saturation) on every bf16 value in [-448, 448]
  and on random fp32 values;
- closed forms of the row quantiser: a constant group maps to +-448 with
  a_s = |v|/448, an all-zero group to +-0 with the 1e-12 floor;
- dequantisation stays within half an E4M3 step of the input;
- weight blocks: a constant block maps to +-448, a block's scale depends on
  its own 128x128 elements only (ragged last block row included), and the
  torch-op recipe and the input generator give the same codes and scales.

Quantisation recipe: FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8
matmul for Hopper", section "Description" (per-token FP8 E4M3 activations
with de-quant scales); the amax/448 scale is the reading of that recipe.
"""
import numpy as np
import pytest
import torch

import oracle


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def torch_e4m3_codes(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def finite_codes():
    return [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_encode_inverts_decode_on_every_finite_code():
    for c in finite_codes():
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c, hex(c)


def test_midpoints_round_to_even_code():
    pos = [c for c in finite_codes() if c < 0x7F]
    for c in pos[:-1]:
        lo, hi = oracle.e4m3_value(c), oracle.e4m3_value(c + 1)
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even, hex(c)
        assert oracle.e4m3_encode(-mid) == 0x80 | even, hex(c)
        eps = (hi - lo) * 1e-6
        assert oracle.e4m3_encode(mid - eps) == c
        assert oracle.e4m3_encode(mid + eps) == c + 1


def test_saturation_at_448():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(464.0) == 0x7E      # torch's cast gives 448 here too
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE


def test_encode_matches_torch_on_every_bf16_in_range():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bf16_to_f32(bits)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    vals = vals[keep]
    want = torch_e4m3_codes(vals)
    got = np.array([oracle.e4m3_encode(float(v)) for v in vals], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_encode_matches_torch_on_random_fp32():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1e-2, 20000),
                        np.ldexp(rng.uniform(-1, 1, 20000), rng.integers(-12, -5, 20000))]).astype(np.float32)
    want = torch_e4m3_codes(v)
    got = np.array([oracle.e4m3_encode(float(x)) for x in v], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_quantize_constant_group_maps_to_448():
    for v in (1.0, -3.5, 0.0078125, 300.0, -1e-20):
        x = np.full((2, 256), v, dtype=np.float32)
        q, a_s = oracle.quantize_rows(bf16_bits(x))
        vb = float(bf16_to_f32(bf16_bits(np.array([v], np.float32)))[0])
        want_s = np.float32(max(abs(vb), np.float32(1e-12))) / np.float32(448.0)
        assert np.all(a_s == want_s)
        code = 0x7E if vb > 0 else 0xFE
        if abs(vb) < 1e-12:     # below the floor: x/a_s is small, not 448
            return
        assert np.all(q == code), (v, np.unique(q))


def test_quantize_zero_groups_keep_sign_and_floor():
    x = np.zeros((3, 128), dtype=np.float32)
    x[1] = -0.0
    q, a_s = oracle.quantize_rows(bf16_bits(x))
    assert np.all(a_s == np.float32(1e-12) / np.float32(448.0))
    assert np.all(q[0] == 0) and np.all(q[1] == 0x80)


def test_quantize_groups_and_scales_are_per_row_and_per_128():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(5, 384)).astype(np.float32)
    x[2, 128:256] *= 1000.0
    q, a_s = oracle.quantize_rows(bf16_bits(x))
    xb = bf16_to_f32(bf16_bits(x)).reshape(5, 3, 128)
    amax = np.abs(xb).max(axis=2)
    assert np.array_equal(a_s, np.maximum(amax, np.float32(1e-12)).astype(np.float32) / np.float32(448.0))
    # every group holds its +-448 code at the position of its amax
    flat = q.reshape(5, 3, 128)
    for m in range(5):
        for g in range(3):
            k = int(np.argmax(np.abs(xb[m, g])))
            assert flat[m, g, k] & 0x7F == 0x7E


def test_dequantised_within_half_a_step():
    rng = np.random.default_rng(11)
    x = (rng.normal(size=(64, 512)) * np.exp(rng.normal(size=(64, 1)) * 3)).astype(np.float32)
    bits = bf16_bits(x)
    q, a_s = oracle.quantize_rows(bits)
    table = oracle.e4m3_table()
    xb = bf16_to_f32(bits).astype(np.float64)
    s = np.repeat(a_s.astype(np.float64), 128, axis=1)
    deq = table[q] * s
    y = xb / s                                   # in units of the scale
    step = np.where(np.abs(y) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 1e-300))) - 3))
    # half a step of the quotient plus the fp32 rounding of x / a_s itself
    assert np.all(np.abs(deq - xb) <= (0.5 * step + np.abs(y) * 2.0 ** -23) * s * (1 + 1e-12))


@pytest.mark.parametrize("shape", [(1, 128), (7, 256), (3, 1024)])
def test_quantize_matches_torch_recipe(shape):
    """The recipe written with torch ops (fp32 division, clamp, RNE cast)
    gives the same codes and scales: torch's cast is the library routine the
    encoder reduces to once the quotient is clamped."""
    rng = np.random.default_rng(shape[0] * shape[1])
    x = rng.normal(size=shape).astype(np.float32)
    bits = bf16_bits(x)
    q, a_s = oracle.quantize_rows(bits)
    xt = torch.from_numpy(bf16_to_f32(bits)).view(shape[0], -1, 128)
    amax = xt.abs().amax(dim=2)
    s = torch.clamp(amax, min=float(np.float32(1e-12))) / 448.0
    qt = torch.clamp(xt / s[..., None], -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(a_s, s.numpy())
    assert np.array_equal(q, qt.reshape(shape).numpy())


# ---------------------------------------------------------------------------
# 128 x 128 weight blocks (section "Description": [block_n, block_k] = [128, 128]
# weight de-quant scales).
# ---------------------------------------------------------------------------
def test_blocks_constant_block_maps_to_448():
    w = np.full((128, 256), -0.02, dtype=np.float32)
    w[:, 128:] = 3.0
    q, b_s = oracle.quantize_blocks(bf16_bits(w))
    v0 = float(bf16_to_f32(bf16_bits(np.array([-0.02], np.float32)))[0])
    assert b_s.shape == (1, 2)
    assert b_s[0, 0] == np.float32(abs(v0)) / np.float32(448.0)
    assert b_s[0, 1] == np.float32(3.0) / np.float32(448.0)
    assert np.all(q[:, :128] == 0xFE) and np.all(q[:, 128:] == 0x7E)


def test_blocks_scale_is_local_to_its_block():
    rng = np.random.default_rng(4)
    w = (rng.normal(size=(300, 384)) * 0.02).astype(np.float32)
    q0, s0 = oracle.quantize_blocks(bf16_bits(w))
    w2 = w.copy()
    w2[130, 300] = 5.0                       # block (1, 2) only
    q1, s1 = oracle.quantize_blocks(bf16_bits(w2))
    changed = np.argwhere(s0 != s1)
    assert changed.tolist() == [[1, 2]]
    diff_rows, diff_cols = np.nonzero(q0 != q1)
    assert diff_rows.min() >= 128 and diff_rows.max() < 256
    assert diff_cols.min() >= 256 and diff_cols.max() < 384


def test_blocks_ragged_last_block_row():
    """N = 300: the third block row holds rows 256..299 only; its amax ignores
    nothing and includes nothing else."""
    rng = np.random.default_rng(5)
    w = (rng.normal(size=(300, 128)) * 0.02).astype(np.float32)
    w[299, 7] = -2.5
    q, b_s = oracle.quantize_blocks(bf16_bits(w))
    assert b_s.shape == (3, 1)
    assert b_s[2, 0] == np.float32(2.5) / np.float32(448.0)
    assert q[299, 7] == 0xFE


def test_blocks_match_torch_recipe_and_generator():
    """The recipe written with torch ops (block amax, fp32 division, clamp,
    RNE cast), and the input generator's own weight quantiser, give the same
    codes and scales."""
    import workloads
    rng = np.random.default_rng(6)
    w = (rng.normal(size=(256, 512)) * 0.02).astype(np.float32)
    bits = bf16_bits(w)
    q, b_s = oracle.quantize_blocks(bits)
    wt = torch.from_numpy(bf16_to_f32(bits)).view(2, 128, 4, 128)
    s = torch.clamp(wt.abs().amax(dim=(1, 3)), min=float(np.float32(1e-12))) / 448.0
    qt = torch.clamp(wt / s[:, None, :, None], -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(b_s, s.numpy())
    assert np.array_equal(q, qt.reshape(256, 512).numpy())
    qg, sg = workloads.quantize_blocks(bf16_to_f32(bits))
    assert np.array_equal(qg, q) and np.array_equal(sg, b_s)


def test_blocks_dequantised_within_half_a_step():
    rng = np.random.default_rng(12)
    w = (rng.normal(size=(260, 640)) * np.exp(rng.normal(size=(260, 1)))).astype(np.float32)
    bits = bf16_bits(w)
    q, b_s = oracle.quantize_blocks(bits)
    table = oracle.e4m3_table()
    wb = bf16_to_f32(bits).astype(np.float64)
    s = np.repeat(np.repeat(b_s.astype(np.float64), 128, axis=0)[:260], 128, axis=1)
    y = wb / s
    step = np.where(np.abs(y) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 1e-300))) - 3))
    assert np.all(np.abs(table[q] * s - wb) <= (0.5 * step + np.abs(y) * 2.0 ** -23) * s * (1 + 1e-12))
