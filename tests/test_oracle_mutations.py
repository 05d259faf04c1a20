"""The oracle's pins have teeth: each plausible mistake planted in the oracle
(on the CPU, via monkeypatch) makes at least one pin fail."""
import numpy as np
import pytest

import oracle
import oracle.moe_oracle as M
import test_oracle_formats as TF
import test_oracle_fp8 as TF8
import test_oracle_layer as TL
import test_oracle_router as TR


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(M, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _unpack_swapped(q):
    q = np.asarray(q, np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = q >> 4
    out[..., 1::2] = q & 0x0F
    return out


def _e4m3_bias8(b):
    b = np.asarray(b).astype(np.int64)
    e, m = (b >> 3) & 15, b & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -7), np.ldexp(1.0 + m / 8.0, e - 8))
    return np.where((b >> 7) & 1, -mag, mag)


def _dequant_scale_per_row_block(q, s):
    codes = M.unpack_codes(q)
    vals = M.decode_e2m1(np.arange(16))[codes]
    scl = M.decode_e4m3(np.asarray(s))
    return vals * np.repeat(scl.reshape(-1)[: codes.shape[0]][:, None], codes.shape[1], axis=1)


def _swiglu_symmetric_gate(g, u, L):
    return M.silu(np.clip(g, -L, L)) * np.clip(u, -L, L)


def _swiglu_up_upper_only(g, u, L):
    return M.silu(np.minimum(g, L)) * np.minimum(u, L)


def _route_biased_weights(x, Wr, b, k, rsf):
    l = M.router_logits(x, Wr)
    sel = M.sigmoid(l) + np.asarray(b, np.float64)[None, :]
    ids = M.select_topk(sel, k)
    c = np.take_along_axis(sel, ids, -1)
    return ids, c / c.sum(-1, keepdims=True) * rsf, l, sel


def _route_no_renorm(x, Wr, b, k, rsf):
    l = M.router_logits(x, Wr)
    s = M.sigmoid(l)
    sel = s + np.asarray(b, np.float64)[None, :]
    ids = M.select_topk(sel, k)
    return ids, np.take_along_axis(s, ids, -1) * rsf, l, sel


def _select_ascending(sel, k):
    return np.argsort(np.asarray(sel), axis=-1, kind="stable")[..., :k]


def _round_bf16_via_fp32(a):
    import torch
    t = torch.from_numpy(np.asarray(a, np.float64).astype(np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


_orig_routed_expert = M.routed_expert
_orig_bf16_mlp = M.bf16_mlp


def _routed_expert_swapped(x, q13, s13, g13, q2, s2, g2, limit, mode="contract"):
    q13 = np.asarray(q13)
    s13 = np.asarray(s13)
    I = q13.shape[0] // 2
    q13 = np.concatenate([q13[I:], q13[:I]])
    s13 = np.concatenate([s13[I:], s13[:I]])
    return _orig_routed_expert(x, q13, s13, g13, q2, s2, g2, limit, mode)


def _bf16_mlp_scaled(x, w13, w2, limit, mode="contract"):
    return 2.5 * _orig_bf16_mlp(x, w13, w2, limit, mode)


def _no_global_after_dot(x, q, s, g):
    return np.asarray(x, np.float64) @ M.dequant_nvfp4(q, s).T


def _fp8_scale_transposed(q, s, block=128):
    return _orig_dequant_fp8(q, np.asarray(s).T, block)


def _fp8_scale_per_row_block(q, s, block=128):
    s = np.asarray(s, np.float64)
    return _orig_dequant_fp8(q, np.repeat(s[:, :1], s.shape[1], axis=1), block)


_orig_dequant_fp8 = M.dequant_fp8_block
_orig_routed_expert_fp8 = M.routed_expert_fp8


def _routed_expert_fp8_swapped(x, q13, s13, q2, s2, limit, mode="contract"):
    q13, s13 = np.asarray(q13), np.asarray(s13)
    I, Ib = q13.shape[0] // 2, s13.shape[0] // 2
    return _orig_routed_expert_fp8(x, np.concatenate([q13[I:], q13[:I]]), np.concatenate([s13[Ib:], s13[:Ib]]),
                                   q2, s2, limit, mode)


def _expert_rows_ignores_format(job):
    expert, e, xr, g13, g2, limit, mode, fmt = job
    q13, s13, q2, s2 = expert(e)
    return M.routed_expert(xr, q13, s13, g13, q2, s2, g2, limit, mode)


MUTATIONS = [
    ("dequant_fp8_block", _fp8_scale_transposed, [TF8.test_fp8_block_index]),
    ("dequant_fp8_block", _fp8_scale_per_row_block, [TF8.test_fp8_block_index]),
    ("routed_expert_fp8", _routed_expert_fp8_swapped, [TF8.test_fp8_expert_closed_form]),
    ("expert_rows", _expert_rows_ignores_format, [TF8.test_fp8_layer_equals_dense_routing_matrix_formulation]),
    ("unpack_codes", _unpack_swapped, [TF.test_nibble_order_and_block_index]),
    ("decode_e4m3", _e4m3_bias8, [TF.test_e4m3_samples_match_hand_table]),
    ("dequant_nvfp4", _dequant_scale_per_row_block, [TF.test_nibble_order_and_block_index]),
    ("swiglu_clamped", _swiglu_symmetric_gate, [TL.test_swiglu_tail_table]),
    ("swiglu_clamped", _swiglu_up_upper_only, [TL.test_swiglu_tail_table]),
    ("route", _route_biased_weights, [TR.test_bias_steers_selection_only]),
    ("route", _route_no_renorm, [TR.test_weights_sum_to_rsf_and_follow_score_ratios]),
    ("select_topk", _select_ascending, [TR.test_topk_tie_goes_to_lower_index]),
    ("round_bf16", _round_bf16_via_fp32, [TF.test_round_bf16_hand_cases]),
    ("routed_expert", _routed_expert_swapped, [TL.test_gate_rows_come_first]),
    ("bf16_mlp", _bf16_mlp_scaled, [TL.test_routed_part_is_linear_in_rsf_and_shared_is_unscaled,
                                    TL.test_shared_expert_only_when_routed_down_is_zero]),
    ("nvfp4_linear", _no_global_after_dot, [TL.test_global_scale_multiplies_after_dot]),
]


@pytest.mark.parametrize("name,fn,pins", MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn, pins):
    _patch(monkeypatch, name, fn)
    caught = False
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught = True
    assert caught, f"no pin caught the planted mistake in {name}"
