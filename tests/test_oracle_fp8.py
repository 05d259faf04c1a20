"""Pins of the oracle's FP8 block-scaled experts (E4M3 weights, one fp32 scale
per 128 x 128 block; the reading of the FP8 checkpoint named on the
TensorRT-LLM page "Add GLM-5.3-Flash (glm5_next) support", Description).

* worked E4M3 x scale products from the bit fields (tests/golden);
* the block index: a non-symmetric grid of block scales over unit codes;
* the library routine: torch's own float8_e4m3fn decoder and matmul;
* a closed-form expert: gate rows first, the asymmetric clamp, bf16 h;
* the layer against a dense routing-matrix formulation over all experts.
"""
import math

import numpy as np
import torch

import oracle as O
import synth
from golden_io import rows


def same_bits(a, b):
    return np.asarray(a, np.float64).view(np.uint64).tolist() == np.asarray(b, np.float64).view(np.uint64).tolist()


def test_fp8_worked_products():
    for r in rows("fp8_block_products.txt"):
        byte, val, scale, prod = int(r[0], 16), float(r[2]), float(r[3]), float(r[4])
        assert same_bits(O.decode_e4m3(np.array([byte])), [val]), hex(byte)
        q = np.full((128, 128), byte, np.uint8)
        w = O.dequant_fp8_block(q, np.full((1, 1), scale))
        assert same_bits([w[5, 77]], [prod]), (hex(byte), w[5, 77], prod)


def test_fp8_block_index():
    """Unit codes (0x38 = 1.0) over a 2 x 3 grid of distinct block scales: every weight
    equals the scale of the 128 x 128 block holding it (row block r // 128, column block
    c // 128)."""
    s = np.array([[1.0, 2.0, 4.0], [8.0, 16.0, 32.0]])
    w = O.dequant_fp8_block(np.full((256, 384), 0x38, np.uint8), s)
    for (r, c), v in {(0, 0): 1.0, (0, 127): 1.0, (0, 128): 2.0, (127, 383): 4.0, (128, 0): 8.0,
                      (255, 255): 16.0, (200, 300): 32.0, (129, 130): 16.0}.items():
        assert w[r, c] == v, (r, c, w[r, c], v)
    assert np.array_equal(np.unique(w[128:, 256:]), [32.0])


def test_fp8_linear_matches_torch_float8_decode():
    """Library routine: torch's float8_e4m3fn decoder and an fp64 matmul, row-major [out, in]
    weights, with unit scales and then with per-block scales applied by torch."""
    rng = np.random.default_rng(7)
    q = rng.integers(0, 256, size=(256, 384), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38                          # no NaN bytes
    x = rng.standard_normal((5, 384))
    Wt = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64)
    ref = (torch.from_numpy(x) @ Wt.T).numpy()
    np.testing.assert_allclose(O.fp8_linear(x, q, np.ones((2, 3))), ref, rtol=1e-12, atol=1e-9)
    s = rng.uniform(0.01, 2.0, size=(2, 3))
    S = torch.from_numpy(s).repeat_interleave(128, 0).repeat_interleave(128, 1)
    ref = (torch.from_numpy(x) @ (Wt * S).T).numpy()
    np.testing.assert_allclose(O.fp8_linear(x, q, s), ref, rtol=1e-12, atol=1e-9)


def test_fp8_expert_closed_form():
    """H = I = 128.  Gate rows: byte 0x38 (1.0), block scale 10/128; up rows: 0x30 (0.5),
    scale 1/32; down: 0x38, scale 1; x = 1.  Then g = 10 (clamped to L = 7), u = 2,
    h = silu(7) * 2, y[r] = 128 * h (contract mode: h rounded to bf16 first).  With the
    gate and up rows swapped h would be silu(2) * 7."""
    q13 = np.concatenate([np.full((128, 128), 0x38, np.uint8), np.full((128, 128), 0x30, np.uint8)])
    s13 = np.array([[10.0 / 128.0], [1.0 / 32.0]])
    q2 = np.full((128, 128), 0x38, np.uint8)
    s2 = np.ones((1, 1))
    x = np.ones((1, 128))
    h = 7.0 / (1.0 + math.exp(-7.0)) * 2.0
    y = O.routed_expert_fp8(x, q13, s13, q2, s2, 7.0, mode="exact")
    np.testing.assert_allclose(y, np.full((1, 128), 128.0 * h), rtol=1e-14)
    assert abs(h - 2.0 / (1.0 + math.exp(-2.0)) * 7.0) > 1.0
    yc = O.routed_expert_fp8(x, q13, s13, q2, s2, 7.0, mode="contract")
    assert np.all(yc == 128.0 * 14.0)                    # bf16(13.98...) = 14.0 (spacing 1/16 in [8, 16))


def test_fp8_layer_equals_dense_routing_matrix_formulation():
    w = synth.workload("tiny_decode_fp8", T=6, E=6, K=2)
    xb = synth.x_rows(w)
    x = O.decode_bf16(xb)
    experts = {e: synth.expert_w13(w, e) + synth.expert_w2(w, e) for e in range(w.E)}
    wts = O.RoutedWeights(synth.router_weight(w), synth.router_bias(w), synth.w13_globals(w),
                          synth.w2_globals(w), lambda e: experts[e], synth.shared_w13(w), synth.shared_w2(w),
                          fmt="fp8")
    out, ids, wk = O.moe_layer(xb, wts, w.K, w.rsf, w.swiglu_limit, mode="exact")
    R = np.zeros((w.T, w.E))
    for t in range(w.T):
        for k in range(w.K):
            R[t, ids[t, k]] = wk[t, k]
    Y = np.stack([O.routed_expert_fp8(x, *experts[e], w.swiglu_limit, mode="exact") for e in range(w.E)], axis=1)
    shared = O.bf16_mlp(x, wts.shared_w13, wts.shared_w2, w.swiglu_limit, mode="exact")
    np.testing.assert_allclose(out, shared + np.einsum("te,teh->th", R, Y), rtol=1e-13, atol=1e-13)
    # the same layer read as NVFP4 would not even accept these weights
    try:
        O.moe_layer(xb, O.RoutedWeights(wts.router_w, wts.router_bias, wts.w13_g, wts.w2_g, wts.expert,
                                        wts.shared_w13, wts.shared_w2), w.K, w.rsf, w.swiglu_limit)
        raise AssertionError("FP8 weights read as NVFP4 went through")
    except ValueError:
        pass


def test_fp8_generator_recipe():
    """The synthetic FP8 experts: no NaN bytes, block scales of the stated range, RMS weight
    within 10% of an NVFP4 expert's."""
    w = synth.workload("tiny_decode_fp8")
    lo, hi = 0.5 * synth.SHARED_SIGMA / synth.FP8_CODE_SIGMA, 1.5 * synth.SHARED_SIGMA / synth.FP8_CODE_SIGMA
    sq = []
    for e in range(w.E):                    # 16 experts x 6 blocks of 128 x 128
        for q, s in (synth.expert_w13(w, e), synth.expert_w2(w, e)):
            assert not np.any((q & 0x7F) == 0x7F)
            assert np.all(s >= lo * (1 - 1e-6)) and np.all(s <= hi * (1 + 1e-6))
            sq.append(np.mean(O.dequant_fp8_block(q, s) ** 2) * q.size)
    rms = float(np.sqrt(np.sum(sq) / (w.E * 3 * w.I * w.H)))
    assert abs(rms / synth.SHARED_SIGMA - 1.0) < 0.1, rms
