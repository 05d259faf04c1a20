"""Pins of the oracle's SwiGLU, expert projections and whole routed/dense layer.

Module glm5next_mlp: "The stack this layer runs" (routed NVFP4 experts,
BF16 shared expert, moe_combine; DENSE gate/up -> clamped SwiGLU -> down) and
"Traps this module exists to hold" (asymmetric clamp; shared expert not
scaled by routed_scaling_factor).
"""
import numpy as np
import pytest

import oracle as O
import synth
from golden_io import e2m1_table, rows

# --------------------------------------------------------------------------
# Clamped SwiGLU.
# --------------------------------------------------------------------------


def _split(field):
    expr, _, val = field.partition("=")
    return None if expr == "-" else float(val)


def test_swiglu_tail_table():
    for r in rows("swiglu_tails.txt"):
        g, u = float(r[0]), float(r[1])
        h, wrong = _split(r[2]), [_split(f) for f in r[3:6]]
        got = float(O.swiglu_clamped(np.array([g]), np.array([u]), 7.0)[0])
        assert got == pytest.approx(h, rel=1e-14, abs=1e-300)
        for wv in wrong:
            if wv is not None:                 # the plausible wrong readings are told apart
                assert abs(got - wv) > 1e-3 * abs(wv)


def test_swiglu_huge_limit_is_plain_swiglu():
    g = np.random.default_rng(8).standard_normal(1000) * 20
    u = np.random.default_rng(9).standard_normal(1000) * 20
    import scipy.special
    np.testing.assert_allclose(O.swiglu_clamped(g, u, 1e30), g * scipy.special.expit(g) * u,
                               rtol=1e-13, atol=1e-300)


# --------------------------------------------------------------------------
# Projections.
# --------------------------------------------------------------------------


def _pack(codes):
    codes = np.asarray(codes, np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def test_unit_scales_reduce_to_matmul_of_code_table():
    """All scales 0x38 (1.0), global 1: W is the E2M1 table itself."""
    g = np.random.default_rng(10)
    rows_, cols = 24, 64
    codes = g.integers(0, 16, (rows_, cols))
    table = e2m1_table()
    W = np.vectorize(table.get)(codes).astype(np.float64)
    x = g.standard_normal((5, cols))
    got = O.nvfp4_linear(x, _pack(codes), np.full((rows_, cols // 16), 0x38, np.uint8), 1.0)
    np.testing.assert_allclose(got, np.matmul(x, W.T), rtol=1e-14, atol=1e-13)


def test_global_scale_multiplies_after_dot():
    g = np.random.default_rng(11)
    q = g.integers(0, 256, (8, 16), dtype=np.uint8)
    s = synth.encode_e4m3(np.abs(g.standard_normal((8, 2))) * 0.05)
    x = g.standard_normal((3, 32))
    base = O.nvfp4_linear(x, q, s, 1.0)
    for gs in (0.75, 2.0 ** -3):
        np.testing.assert_allclose(O.nvfp4_linear(x, q, s, gs), gs * base, rtol=1e-15, atol=0)


# --------------------------------------------------------------------------
# Hand-built tiny layers.
# --------------------------------------------------------------------------

H, I, E = 32, 16, 4


def _tiny_weights(seed=12, shared=True, w2_zero=False, g13=None, g2=None, unit_scales=False):
    g = np.random.default_rng(seed)
    exp = {}
    for e in range(E):
        q13 = g.integers(0, 256, (2 * I, H // 2), dtype=np.uint8)
        s13 = synth.encode_e4m3(np.abs(g.standard_normal((2 * I, H // 16))) * 0.05)
        q2 = g.integers(0, 256, (H, I // 2), dtype=np.uint8)
        s2 = synth.encode_e4m3(np.abs(g.standard_normal((H, I // 16))) * 0.05)
        if unit_scales:
            s13[:] = 0x38
            s2[:] = 0x38
        if w2_zero:
            q2[:] = 0
        exp[e] = (q13, s13, q2, s2)
    sw13 = synth.encode_bf16(g.standard_normal((2 * I, H)) * 0.15) if shared else None
    sw2 = synth.encode_bf16(g.standard_normal((H, I)) * 0.15) if shared else None
    return O.RoutedWeights(
        router_w=(g.standard_normal((E, H)) * 0.3).astype(np.float32),
        router_bias=g.uniform(-0.1, 0.1, E).astype(np.float32),
        w13_g=np.ones((E, 2), np.float32) if g13 is None else np.asarray(g13, np.float32),
        w2_g=np.ones(E, np.float32) if g2 is None else np.asarray(g2, np.float32),
        expert=lambda e: exp[e], shared_w13=sw13, shared_w2=sw2)


def _tiny_x(seed=13, T=6, scale=3.0):
    return synth.encode_bf16(np.random.default_rng(seed).standard_normal((T, H)) * scale)


def test_clamp_tails_through_an_expert():
    """x = 2.5 on column 0 against a single code-6 (4.0) weight at scale 1.0
    gives pre-activations of exactly +-10; the expert's h follows the tail table."""
    L = 7.0
    cases = [(10, 10), (10, -10), (-10, -10), (-10, 10)]
    x = np.zeros((1, H))
    x[0, 0] = 2.5
    codes13 = np.zeros((2 * I, H), np.uint8)
    for j, (gv, uv) in enumerate(cases):
        codes13[j, 0] = 6 if gv > 0 else 14              # +-4.0
        codes13[I + j, 0] = 6 if uv > 0 else 14
    q13 = _pack(codes13)
    s13 = np.full((2 * I, H // 16), 0x38, np.uint8)
    # down projection = identity on the first 4 hidden units: W2[r, r] = 1.0 (code 2)
    codes2 = np.zeros((H, I), np.uint8)
    for j in range(len(cases)):
        codes2[j, j] = 2
    y = O.routed_expert(x, q13, s13, [1.0, 1.0], _pack(codes2), np.full((H, I // 16), 0x38, np.uint8),
                        1.0, L, mode="exact")
    want = {(r[0], r[1]): float(r[2].partition("=")[2]) for r in rows("swiglu_tails.txt")}
    for j, (gv, uv) in enumerate(cases):
        assert y[0, j] == pytest.approx(want[(str(gv), str(uv))], rel=1e-14)
    assert np.all(y[0, len(cases):] == 0)


def test_gate_rows_come_first():
    """Rows [0, I) are the gate, [I, 2I) the up projection: g=10, u=-10 gives
    silu(7)*-7; swapped halves would give silu(-10)*7."""
    x = np.zeros((1, H))
    x[0, 0] = 2.5
    codes13 = np.zeros((2 * I, H), np.uint8)
    codes13[0, 0] = 6
    codes13[I, 0] = 14
    codes2 = np.zeros((H, I), np.uint8)
    codes2[0, 0] = 2
    y = O.routed_expert(x, _pack(codes13), np.full((2 * I, H // 16), 0x38, np.uint8), [1, 1],
                        _pack(codes2), np.full((H, I // 16), 0x38, np.uint8), 1.0, 7.0, mode="exact")
    assert y[0, 0] == pytest.approx(-48.95535849147437, rel=1e-14)


def test_expert_global_scales_act_on_gate_and_up():
    """g13 multiplies the gate and up dot products: global c on both equals x scaled by c."""
    wts = _tiny_weights()
    x = O.decode_bf16(_tiny_x())
    q13, s13, q2, s2 = wts.expert(1)
    a = O.routed_expert(x, q13, s13, [0.125, 0.125], q2, s2, 1.0, 7.0, mode="exact")
    b = O.routed_expert(x * 0.125, q13, s13, [1.0, 1.0], q2, s2, 1.0, 7.0, mode="exact")
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-14)
    c = O.routed_expert(x, q13, s13, [1.0, 1.0], q2, s2, 0.75, 7.0, mode="exact")
    d = O.routed_expert(x, q13, s13, [1.0, 1.0], q2, s2, 1.0, 7.0, mode="exact")
    np.testing.assert_allclose(c, 0.75 * d, rtol=1e-15, atol=0)


def test_layer_equals_dense_routing_matrix_formulation():
    """out = shared(x) + R @ Y, with R[t, e] = w at the chosen experts, 0 elsewhere,
    and Y[t, e] = expert e applied to x[t] for EVERY expert."""
    wts = _tiny_weights()
    xb = _tiny_x()
    x = O.decode_bf16(xb)
    K = 2
    out, ids, w = O.moe_layer(xb, wts, K, 2.5, 7.0, mode="exact")
    R = np.zeros((x.shape[0], E))
    for t in range(x.shape[0]):
        for k in range(K):
            R[t, ids[t, k]] = w[t, k]
    Y = np.stack([O.routed_expert(x, *wts.expert(e)[:2], wts.w13_g[e], *wts.expert(e)[2:], wts.w2_g[e],
                                  7.0, mode="exact") for e in range(E)], axis=1)        # [T, E, H]
    shared = O.bf16_mlp(x, wts.shared_w13, wts.shared_w2, 7.0, mode="exact")
    want = shared + np.einsum("te,teh->th", R, Y)
    np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-13)


def test_unit_scale_layer_against_plain_matmuls():
    """Unit scales and globals: the routed path is plain matmuls of the code table."""
    wts = _tiny_weights(unit_scales=True, shared=False)
    xb = _tiny_x()
    x = O.decode_bf16(xb)
    table = e2m1_table()
    lut = np.array([table[c] for c in range(16)])
    out, ids, w = O.moe_layer(xb, wts, 2, 2.5, 7.0, mode="exact")
    for t in range(x.shape[0]):
        acc = np.zeros(H)
        for k in range(2):
            q13, _, q2, _ = wts.expert(int(ids[t, k]))
            W13 = lut[O.unpack_codes(q13)]
            W2 = lut[O.unpack_codes(q2)]
            a = np.matmul(W13, x[t])
            gg, uu = np.minimum(a[:I], 7.0), np.clip(a[I:], -7.0, 7.0)
            acc += w[t, k] * np.matmul(W2, gg / (1 + np.exp(-gg)) * uu)
        np.testing.assert_allclose(out[t], acc, rtol=1e-13, atol=1e-12)


def _plain_shared(x, w13_bits, w2_bits):
    """Shared expert by plain matmuls of the decoded bf16 weights (exact mode)."""
    a = np.matmul(x, O.decode_bf16(w13_bits).T)
    n = a.shape[1] // 2
    gg, uu = np.minimum(a[:, :n], 7.0), np.clip(a[:, n:], -7.0, 7.0)
    return np.matmul(gg / (1 + np.exp(-gg)) * uu, O.decode_bf16(w2_bits).T)


def test_shared_expert_only_when_routed_down_is_zero():
    wts = _tiny_weights(w2_zero=True)
    xb = _tiny_x()
    out, _, _ = O.moe_layer(xb, wts, 2, 2.5, 7.0, mode="exact")
    np.testing.assert_allclose(out, _plain_shared(O.decode_bf16(xb), wts.shared_w13, wts.shared_w2),
                               rtol=1e-13, atol=1e-12)
    outc, _, _ = O.moe_layer(xb, wts, 2, 2.5, 7.0, mode="contract")
    shared = O.bf16_mlp(O.decode_bf16(xb), wts.shared_w13, wts.shared_w2, 7.0, mode="contract")
    assert np.array_equal(outc, O.round_bf16(shared))


def test_routed_part_is_linear_in_rsf_and_shared_is_unscaled():
    wts = _tiny_weights()
    xb = _tiny_x()
    shared = _plain_shared(O.decode_bf16(xb), wts.shared_w13, wts.shared_w2)
    oa, ida, _ = O.moe_layer(xb, wts, 2, 2.5, 7.0, mode="exact")
    ob, idb, _ = O.moe_layer(xb, wts, 2, 1.0, 7.0, mode="exact")
    assert np.array_equal(ida, idb)
    np.testing.assert_allclose(oa - shared, 2.5 * (ob - shared), rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(oa - 2.5 * ob)) > 1e-3           # scaling the shared part too would differ


def test_contract_mode_rounds_h_and_output_only():
    wts = _tiny_weights()
    xb = _tiny_x()
    oc, _, _ = O.moe_layer(xb, wts, 2, 2.5, 7.0, mode="contract")
    oe, _, _ = O.moe_layer(xb, wts, 2, 2.5, 7.0, mode="exact")
    assert np.array_equal(oc, O.round_bf16(oc))           # output is bf16-representable
    rel = np.linalg.norm(oc - oe) / np.linalg.norm(oe)
    assert 0 < rel < 1e-2


def test_subset_of_tokens_matches_full_run():
    wts = _tiny_weights()
    xb = _tiny_x(T=9)
    full, ids, w = O.moe_layer(xb, wts, 3, 2.5, 7.0)
    sub, ids_s, w_s = O.moe_layer(xb, wts, 3, 2.5, 7.0, tokens=[7, 2])
    assert np.array_equal(sub, full[[7, 2]]) and np.array_equal(ids_s, ids[[7, 2]])


def test_dense_ffn_matches_plain_matmuls():
    g = np.random.default_rng(14)
    w13 = synth.encode_bf16(g.standard_normal((2 * 24, H)) * 0.15)
    w2 = synth.encode_bf16(g.standard_normal((H, 24)) * 0.15)
    xb = _tiny_x()
    x = O.decode_bf16(xb)
    a = np.matmul(x, O.decode_bf16(w13).T)
    gg, uu = np.minimum(a[:, :24], 7.0), np.clip(a[:, 24:], -7.0, 7.0)
    want = np.matmul(gg / (1 + np.exp(-gg)) * uu, O.decode_bf16(w2).T)
    np.testing.assert_allclose(O.dense_ffn(xb, w13, w2, 7.0, mode="exact"), want, rtol=1e-13, atol=1e-12)
    assert np.array_equal(O.dense_ffn(xb, w13, w2, 7.0), O.round_bf16(O.dense_ffn(xb, w13, w2, 7.0)))
