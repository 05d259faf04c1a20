"""Pins of the oracle's number formats against hand tables and library routines.

NVFP4 = E2M1 codes (OCP MX v1.0) with one E4M3 scale (OCP OFP8) per 16
elements along the input dimension; Module glm5next_mlp names the routed
experts NVFP4 W4A16.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from golden_io import e2m1_table, e4m3_samples, pyval, rows


def same_bits(a, b):
    return np.asarray(a, np.float64).view(np.uint64).tolist() == np.asarray(b, np.float64).view(np.uint64).tolist()


def test_e2m1_all_codes_match_hand_table():
    table = e2m1_table()
    got = O.decode_e2m1(np.arange(16))
    want = np.array([table[c] for c in range(16)])
    assert same_bits(got, want)          # includes -0.0 for code 8


def test_e4m3_samples_match_hand_table():
    for b, v in e4m3_samples().items():
        got = float(O.decode_e4m3(np.array([b]))[0])
        if math.isnan(v):
            assert math.isnan(got), hex(b)
        else:
            assert same_bits([got], [v]), (hex(b), got, v)


def test_e4m3_structure_over_all_bytes():
    """Monotone, evenly spaced within a binade, continuous at the subnormal edge, odd in sign."""
    pos = O.decode_e4m3(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)
    assert pos[0x7E] == 448.0 and np.isnan(O.decode_e4m3(np.array([0x7F, 0xFF]))).all()
    steps = np.diff(pos)
    # subnormals 0x00..0x08 step 2^-9; then each binade of 8 codes has one spacing that doubles.
    assert np.all(steps[:8] == 2.0 ** -9)
    for e in range(1, 15):
        blk = steps[8 * e: 8 * e + 8]
        assert np.all(blk == 2.0 ** (e - 10)), e
    neg = O.decode_e4m3(np.arange(0x80, 0xFF))
    assert same_bits(neg, -pos)


def test_nvfp4_worked_products():
    for r in rows("nvfp4_products.txt"):
        code, scale, val = int(r[0], 16), int(r[1], 16), float(r[2])
        q = np.zeros((1, 8), np.uint8)
        q[0, 0] = code                       # column 0 = low nibble of byte 0
        s = np.full((1, 1), scale, np.uint8)
        w = O.dequant_nvfp4(q, s)
        assert same_bits([w[0, 0]], [val]), (hex(code), hex(scale), w[0, 0], val)


def test_dequant_grid_equals_table_products():
    """All 16 codes x sample scales: dequant equals the hand-table product (exact)."""
    t2 = e2m1_table()
    t8 = {b: v for b, v in e4m3_samples().items() if not math.isnan(v)}
    scales = sorted(t8)
    rows_ = len(scales)
    codes = np.tile(np.arange(16, dtype=np.uint8), (rows_, 1))          # [rows, 16]
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    s = np.array(scales, np.uint8)[:, None]
    got = O.dequant_nvfp4(q, s)
    want = np.array([[t2[c] * t8[b] for c in range(16)] for b in scales])
    assert same_bits(got, want)


def test_nibble_order_and_block_index():
    """Low nibble = even column; scale index = column // 16 of the same row."""
    q = np.zeros((2, 16), np.uint8)          # 2 rows x 32 columns, 2 blocks per row
    q[0, 0] = 0x21                           # col0 code 1 (0.5), col1 code 2 (1.0)
    q[0, 8] = 0x70                           # col16 code 0, col17 code 7 (6.0)
    q[1, 15] = 0xE0                          # col31 code 14 (-4.0)
    s = np.array([[0x38, 0x30], [0x40, 0x48]], np.uint8)   # 1.0, 0.5 / 2.0, 4.0
    W = O.dequant_nvfp4(q, s)
    assert W[0, 0] == 0.5 and W[0, 1] == 1.0
    assert W[0, 16] == 0.0 and W[0, 17] == 6.0 * 0.5
    assert W[1, 31] == -4.0 * 4.0
    assert np.count_nonzero(W) == 4


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(0).integers(0, 1 << 16, size=20000).astype(np.uint16)
    bits = bits[~np.isnan(O.decode_bf16(bits))]
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert same_bits(O.decode_bf16(bits), t)


def test_round_bf16_hand_cases():
    for r in rows("bf16_rne.txt"):
        x, want = pyval(r[0]), pyval(r[1])
        got = float(O.round_bf16(np.array([x]))[0])
        assert same_bits([got], [want]), (r, got, want)


def test_round_bf16_matches_torch_on_fp32_inputs():
    """For fp32-representable inputs, fp64->bf16 RNE equals torch's fp32->bf16 (RNE)."""
    g = np.random.default_rng(1)
    v = np.concatenate([g.standard_normal(50000) * 10.0 ** g.integers(-30, 30, 50000),
                        g.standard_normal(1000) * 1e-39]).astype(np.float32)
    t = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert same_bits(O.round_bf16(v.astype(np.float64)), t)


def test_e4m3_encoder_round_trips():
    """synth's encoder is the inverse of the decoder on every finite non-negative byte,
    and rounds to nearest even between neighbours."""
    b = np.arange(0x7F, dtype=np.uint8)
    v = O.decode_e4m3(b)
    assert np.array_equal(synth.encode_e4m3(v), b)
    mid = 0.5 * (v[:-1] + v[1:])
    enc = synth.encode_e4m3(mid)
    lower = np.arange(0x7E)
    want = np.where(lower % 2 == 0, lower, lower + 1)
    assert np.array_equal(enc, want.astype(np.uint8))


@pytest.mark.parametrize("bits", [0x0000, 0x3F80, 0xBF80, 0x7F7F, 0x0001])
def test_bf16_encoder_round_trips(bits):
    v = O.decode_bf16(np.array([bits], np.uint16))
    assert int(synth.encode_bf16(v)[0]) == bits
