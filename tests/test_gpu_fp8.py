"""GPU parity of the FP8 block-scaled expert layer (MOE_MLP_KIND_ROUTED_FP8:
E4M3 weights with one fp32 scale per 128 x 128 block, the reading of the FP8
checkpoint on the TensorRT-LLM page "Add GLM-5.3-Flash (glm5_next) support")
through the C ABI against the fp64 oracle (routed_expert_fp8), every token:
ids bit-exact, weights within 1e-6 relative, output rel-L2 <= 5e-3 and
max-abs <= 1e-2 * max|ref|.

Paths: 1..4 tokens run the three fused decode launches (decode_fp8.hpp; the
GLM-Flash shape with its geometry compiled in, other shapes generic); more
tokens, and prefill, run the FP8 grouped GEMM (gemm_fp8.hpp)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_util import DeviceRouted, assert_output_close, assert_router_close, bf16_host_bits, device_workload, say
from inputs import RoutedInputs
from routed_expert_mlp_amd import capi

pytestmark = pytest.mark.gpu


def _check(d, prefill, what, x=None, toks=None):
    w = d.w
    T = w.T if x is None else x.shape[0]
    say(f"[case] fp8 {what}: {'prefill' if prefill else 'decode'} T={T} H={w.H} I={w.I} E={w.E} K={w.K}")
    out, ids, wts = d.run(prefill, x=x)
    torch.cuda.synchronize()
    toks = np.arange(T) if toks is None else toks
    xs = d.inp.x[toks]
    ids_ref, w_ref, _, _ = O.route(O.decode_bf16(xs), d.inp.router_w, d.inp.router_bias, w.K, w.rsf)
    assert_router_close(ids.cpu().numpy(), wts.cpu().numpy(), ids_ref, w_ref, f"fp8 {what}")
    ref, _, _ = d.inp.oracle(tokens=toks, parallel=w.H * w.I * len(toks) * w.K > 2 ** 26)
    assert_output_close(bf16_host_bits(out), ref, f"fp8 {what} ({T} tokens)")
    return out


def _fresh(name, prefill, **overrides):
    w = synth.workload(name, **overrides)
    return _check(DeviceRouted(RoutedInputs(w)), prefill, f"{name} {overrides or ''}")


FP8_LAYERS = [("tiny_decode_fp8", False), ("flash_decode_t1_fp8", False), ("flash_decode_t16_fp8", False),
              ("ragged_decode_fp8", False), ("ragged_prefill_fp8", True), ("prefill_t4096_fp8", True)]


@pytest.mark.parametrize("name,prefill", FP8_LAYERS, ids=[f"{n}_{'prefill' if p else 'decode'}" for n, p in FP8_LAYERS])
def test_fp8_layer_parity(name, prefill):
    _check(device_workload(name), prefill, name)


@pytest.mark.parametrize("T", [2, 3, 4])
def test_fp8_few_token_full_size(T):
    """2..4 tokens (MTP verify shapes) on the fused FP8 decode launches at the GLM-Flash shape."""
    d = device_workload("flash_decode_t16_fp8")
    _check(d, False, f"few-token T={T}", x=d.x[:T].contiguous(), toks=np.arange(T))


FP8_EDGES = [dict(T=8, K=16), dict(T=5, E=1, K=1), dict(T=3, Is=0), dict(T=1, K=16), dict(T=4, E=1, K=1)]


@pytest.mark.parametrize("overrides", FP8_EDGES, ids=[str(o) for o in FP8_EDGES])
@pytest.mark.parametrize("prefill", [False, True])
def test_fp8_edge_cases(overrides, prefill):
    """K = E = 16, a single expert, no shared expert; one-token and grouped-GEMM forms."""
    _fresh("tiny_decode_fp8", prefill, **overrides)


def test_fp8_decode_and_prefill_agree():
    """The fused few-token FP8 kernels and the FP8 grouped GEMM on the same 4 tokens."""
    d = device_workload("flash_decode_t16_fp8")
    x = d.x[:4].contiguous()
    a, ida, _ = d.run(False, x=x)
    b, idb, _ = d.run(True, x=x)
    torch.cuda.synchronize()
    assert torch.equal(ida, idb)
    ra = a.float().cpu().numpy()
    rb = b.float().cpu().numpy()
    r = float(np.linalg.norm(ra - rb) / np.linalg.norm(rb))
    say(f"[parity] fp8 decode vs prefill (4 tokens): rel_l2={r:.3e}")
    assert r < 5e-3


def test_fp8_noalloc_equals_decode():
    d = device_workload("flash_decode_t1_fp8")
    ref, ref_ids, ref_w = d.run(False)
    out = torch.empty_like(ref)
    ids = torch.empty_like(ref_ids)
    wts = torch.empty_like(ref_w)
    capi.moe_mlp_decode_noalloc(d.cfg, d.weights, d.x, out, ids, wts)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(ids, ref_ids) and torch.equal(wts, ref_w)
