"""Calibrate the synthetic input recipe with the oracle (offline script).

Run:  python -m oracle.calibrate

It prints the two recipe constants that synth/ freezes:

* x_scale per hidden size: the scale of x at which ~1.0% of the chosen
  experts' gate/up pre-activations fire the clamp, counting gate values
  above L and up values outside [-L, L] over all gate and up values
  (L = swiglu_limit = 7).
* bias_amp for E=288, K=8: the amplitude of the U(-amp, amp) correction
  bias at which the bias changes the chosen expert set on ~30% of tokens.

Pre-activations are linear in x_scale, so the script computes them once on
unit-scale rows and bisects on the scale (the bf16 rounding of x is left out
of the calibration; the CPU test on generated inputs includes it).  Inputs
come from synth (raw draws only); all arithmetic is the oracle's.
"""

from __future__ import annotations

import numpy as np

import synth
from oracle import moe_oracle as O

CLAMP_TARGET = 0.010
CHANGE_TARGET = 0.30


def clamp_rate(g, u, limit):
    fired = np.count_nonzero(g > limit) + np.count_nonzero(np.abs(u) > limit)
    return fired / (g.size + u.size)


def calibrate_x_scale(w: synth.Workload, n_tokens: int, cal_seed: int) -> float:
    x1 = synth.unit_normal_rows(cal_seed, n_tokens, w.H)
    Wr = synth.router_weight(w)
    b = synth.router_bias(w)
    l1 = O.router_logits(x1, Wr)
    a1 = {}
    for e in range(w.E):
        q13, s13 = synth.expert_w13(w, e)
        a1[e] = x1 @ O.dequant_nvfp4(q13, s13).T          # [n, 2I] at x_scale 1

    def rate(xs):
        sel = O.sigmoid(xs * l1) + b[None, :]
        ids = O.select_topk(sel, w.K)
        gs, us = [], []
        for t in range(n_tokens):
            for e in ids[t]:
                gs.append(xs * a1[int(e)][t, :w.I])
                us.append(xs * a1[int(e)][t, w.I:])
        return clamp_rate(np.concatenate(gs), np.concatenate(us), w.swiglu_limit)

    lo, hi = 0.01, 20.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if rate(mid) < CLAMP_TARGET:
            lo = mid
        else:
            hi = mid
    xs = 0.5 * (lo + hi)
    print(f"  {w.name}: x_scale={xs:.5g} clamp rate={rate(xs):.4%}")
    return xs


def selection_change_rate(l, b_unit, amp, k):
    s = O.sigmoid(l)
    plain = np.sort(O.select_topk(s, k), axis=-1)
    biased = np.sort(O.select_topk(s + amp * b_unit[None, :], k), axis=-1)
    return float(np.mean(np.any(plain != biased, axis=-1)))


def calibrate_bias_amp(w: synth.Workload, x_scale: float, n_tokens: int, cal_seed: int) -> float:
    x1 = synth.unit_normal_rows(cal_seed, n_tokens, w.H)
    l = O.router_logits(x1 * x_scale, synth.router_weight(w))
    b_unit = synth.router_bias(w.with_(bias_amp=1.0, hot_experts=0)).astype(np.float64)
    lo, hi = 0.0, 0.1
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if selection_change_rate(l, b_unit, mid, w.K) < CHANGE_TARGET:
            lo = mid
        else:
            hi = mid
    amp = 0.5 * (lo + hi)
    print(f"  {w.name}: bias_amp={amp:.5g} change rate="
          f"{selection_change_rate(l, b_unit, amp, w.K):.2%}")
    return amp


def main():
    print("x_scale (1% clamp firing):")
    xs256 = calibrate_x_scale(synth.workload("tiny_decode"), 2048, 9000)
    xs4096 = calibrate_x_scale(synth.workload("flash_decode_t1"), 48, 9001)
    print("bias_amp (30% selection change, E=288, K=8):")
    amp = calibrate_bias_amp(synth.workload("flash_decode_t1"), xs4096, 4096, 9001)
    print(f"X_SCALE_H256 = {xs256:.5g}\nX_SCALE_H4096 = {xs4096:.5g}\nBIAS_AMP_E288_K8 = {amp:.4g}")


if __name__ == "__main__":
    main()
