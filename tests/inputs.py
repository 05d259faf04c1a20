"""Test inputs: synth's raw draws plus near-tie rejection by the oracle's router.

Expert ids must match bit-exactly between the GPU (fp32 router) and the
oracle (fp64), so a token whose biased scores have a near-tie among its top
K+1 values (adjacent gap below DELTA) is redrawn from its own stream (attempt
counter).  DELTA = 1e-5 leaves a ~30x margin over the fp32 error of a score.
"""
import functools

import numpy as np

import oracle as O
import synth

DELTA = 1e-5


def near_tie_tokens(sel, k, delta=DELTA):
    s = -np.sort(-sel, axis=-1)
    m = min(k + 1, sel.shape[-1])
    gaps = s[:, : m - 1] - s[:, 1:m]
    return np.nonzero(np.any(gaps < delta, axis=-1))[0]


class RoutedInputs:
    """One routed workload's inputs (host arrays) and the oracle's view of them."""

    def __init__(self, w: synth.Workload, T=None, reject_near_ties=True, max_rounds=50):
        self.w = w
        self.T = w.T if T is None else T
        self.router_w = synth.router_weight(w)
        self.router_bias = synth.router_bias(w)
        self.w13_g = synth.w13_globals(w)
        self.w2_g = synth.w2_globals(w)
        self.attempts = np.zeros(self.T, np.int64)
        self.x = synth.x_rows(w, self.T)
        if reject_near_ties:
            for _ in range(max_rounds):
                _, _, _, sel = O.route(O.decode_bf16(self.x), self.router_w, self.router_bias, w.K, w.rsf)
                bad = near_tie_tokens(sel, w.K)
                if bad.size == 0:
                    break
                for t in bad:
                    self.attempts[t] += 1
                    self.x[t] = synth.x_row(w, int(t), int(self.attempts[t]))
            else:
                raise RuntimeError("near-tie rejection did not converge")
        self.shared_w13 = synth.shared_w13(w) if w.Is else None
        self.shared_w2 = synth.shared_w2(w) if w.Is else None

    @functools.lru_cache(maxsize=64)
    def expert(self, e):
        return synth.expert_w13(self.w, e) + synth.expert_w2(self.w, e)

    def oracle_weights(self):
        return O.RoutedWeights(self.router_w, self.router_bias, self.w13_g, self.w2_g, self.expert,
                               self.shared_w13, self.shared_w2, fmt=self.w.fmt)

    def oracle(self, tokens=None, mode="contract", parallel=False):
        """The oracle's layer output on these inputs.  parallel=True runs the
        per-expert work in the oracle_pool worker processes (same result)."""
        if not parallel:
            return O.moe_layer(self.x, self.oracle_weights(), self.w.K, self.w.rsf, self.w.swiglu_limit,
                               mode=mode, tokens=tokens)
        from oracle_pool import SynthExpert, pool_map
        wts = O.RoutedWeights(self.router_w, self.router_bias, self.w13_g, self.w2_g, SynthExpert(self.w),
                              self.shared_w13, self.shared_w2, fmt=self.w.fmt)
        return O.moe_layer(self.x, wts, self.w.K, self.w.rsf, self.w.swiglu_limit, mode=mode, tokens=tokens,
                           map_fn=pool_map)
