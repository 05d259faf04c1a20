"""Device-side test inputs: a workload's bytes uploaded to the GPU, plus the
parity metrics.  Every input comes from synth (through tests/inputs.py); no
expected value comes from the HIP path."""
import collections
import sys

import numpy as np
import torch

import synth
from inputs import RoutedInputs
from routed_expert_mlp_amd import capi

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def config_of(w: synth.Workload) -> capi.Config:
    if w.kind == "dense":
        return capi.Config(kind=capi.KIND_DENSE, hidden=w.H, moe_intermediate=0, num_experts=0, top_k=0,
                           n_shared_experts=0, shared_intermediate=0, dense_intermediate=w.Id,
                           routed_scaling_factor=w.rsf, swiglu_limit=w.swiglu_limit)
    kind = capi.KIND_ROUTED_FP8 if w.fmt == "fp8" else capi.KIND_ROUTED
    return capi.Config(kind=kind, hidden=w.H, moe_intermediate=w.I, num_experts=w.E, top_k=w.K,
                       n_shared_experts=1 if w.Is else 0, shared_intermediate=w.Is, dense_intermediate=0,
                       routed_scaling_factor=w.rsf, swiglu_limit=w.swiglu_limit)


class DeviceRouted:
    """A routed workload resident on the GPU (weights for all E experts)."""

    def __init__(self, inp: RoutedInputs, w13_g=None, w2_g=None):
        w = inp.w
        self.inp, self.w, self.cfg = inp, w, config_of(w)
        E, H, I = w.E, w.H, w.I
        wt = capi.Weights(
            router_w=torch.from_numpy(inp.router_w).to(DEV),
            router_bias=torch.from_numpy(inp.router_bias).to(DEV))
        if w.fmt == "fp8":
            B = capi.FP8_BLOCK
            wt.w13_f8 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device=DEV)
            wt.w13_f8_scale = torch.empty((E, 2 * I // B, H // B), dtype=torch.float32, device=DEV)
            wt.w2_f8 = torch.empty((E, H, I), dtype=torch.uint8, device=DEV)
            wt.w2_f8_scale = torch.empty((E, H // B, I // B), dtype=torch.float32, device=DEV)
            dst = (wt.w13_f8, wt.w13_f8_scale, wt.w2_f8, wt.w2_f8_scale)
        else:
            wt.w13_q = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=DEV)
            wt.w13_s = torch.empty((E, 2 * I, H // 16), dtype=torch.uint8, device=DEV)
            wt.w13_g = torch.from_numpy(inp.w13_g if w13_g is None else np.asarray(w13_g, np.float32)).to(DEV)
            wt.w2_q = torch.empty((E, H, I // 2), dtype=torch.uint8, device=DEV)
            wt.w2_s = torch.empty((E, H, I // 16), dtype=torch.uint8, device=DEV)
            wt.w2_g = torch.from_numpy(inp.w2_g if w2_g is None else np.asarray(w2_g, np.float32)).to(DEV)
            dst = (wt.w13_q, wt.w13_s, wt.w2_q, wt.w2_s)
        if w13_g is not None:
            inp.w13_g = np.asarray(w13_g, np.float32)
        if w2_g is not None:
            inp.w2_g = np.asarray(w2_g, np.float32)

        def put(e, q13, s13, q2, s2):
            for d, v in zip(dst, (q13, s13, q2, s2)):
                d[e].copy_(torch.from_numpy(v))

        synth.for_each_expert(w, put)
        if w.Is:
            wt.shared_w13 = bf16_dev(inp.shared_w13)
            wt.shared_w2 = bf16_dev(inp.shared_w2)
        self.weights = wt
        self.x = bf16_dev(inp.x)
        torch.cuda.synchronize()

    def run(self, prefill: bool, x=None, stream=None):
        x = self.x if x is None else x
        T = x.shape[0]
        out = torch.empty((T, self.w.H), dtype=torch.bfloat16, device=DEV)
        ids = torch.empty((T, self.w.K), dtype=torch.int32, device=DEV)
        wts = torch.empty((T, self.w.K), dtype=torch.float32, device=DEV)
        fn = capi.moe_mlp_prefill if prefill else capi.moe_mlp_decode
        fn(self.cfg, self.weights, x, out, ids, wts, stream=stream)
        return out, ids, wts


_CACHE = collections.OrderedDict()


def device_workload(name: str, keep: int = 2, **overrides) -> DeviceRouted:
    key = (name, tuple(sorted(overrides.items())))
    if key in _CACHE:
        _CACHE.move_to_end(key)
        return _CACHE[key]
    while len(_CACHE) >= keep:
        _CACHE.popitem(last=False)
        torch.cuda.empty_cache()
    w = synth.workload(name, **overrides)
    say(f"[inputs] generating {w.name} T={w.T} H={w.H} I={w.I} E={w.E} K={w.K}")
    d = DeviceRouted(RoutedInputs(w))
    _CACHE[key] = d
    return d


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def assert_output_close(got_bits: np.ndarray, ref: np.ndarray, what: str):
    """Output parity: rel-L2 <= 5e-3 and max-abs <= 1e-2 * max|ref| (bf16 GPU vs fp64 oracle)."""
    from oracle import decode_bf16
    got = decode_bf16(got_bits)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref)))
    lim = 1e-2 * float(np.max(np.abs(ref)))
    say(f"[parity] {what}: rel_l2={r:.3e} max_abs={m:.3e} (limit {lim:.3e})")
    assert r <= 5e-3, f"{what}: rel L2 {r}"
    assert m <= lim, f"{what}: max abs {m} > {lim}"


def assert_router_close(ids_gpu, w_gpu, ids_ref, w_ref, what: str):
    ids_gpu = np.asarray(ids_gpu)
    assert np.array_equal(ids_gpu, np.asarray(ids_ref)), f"{what}: ids differ"
    rel = np.max(np.abs(np.asarray(w_gpu, np.float64) - w_ref) / np.abs(w_ref))
    say(f"[parity] {what}: ids equal, max rel weight err {rel:.2e}")
    assert rel <= 1e-6, f"{what}: weight rel err {rel}"
