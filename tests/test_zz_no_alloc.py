"""moe_mlp_decode_noalloc (the library's per-device scratch array as the
workspace) against moe_mlp_decode (caller workspace) through the C ABI: the
same kernels, so the outputs, ids and weights must be equal bitwise, and
within the oracle's tolerance.  Consecutive calls of decreasing size share
the one scratch array (64 tokens -> grouped-GEMM form, 16 -> expert GEMVs,
1 -> one-token kernels)."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, assert_output_close, assert_router_close, bf16_host_bits, device_workload, say
from routed_expert_mlp_amd import capi

pytestmark = pytest.mark.gpu


def _noalloc(d, x):
    T = x.shape[0]
    out = torch.empty((T, d.w.H), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((T, d.w.K), dtype=torch.int32, device=DEV)
    wts = torch.empty((T, d.w.K), dtype=torch.float32, device=DEV)
    capi.moe_mlp_decode_noalloc(d.cfg, d.weights, x, out, ids, wts)
    return out, ids, wts


def test_noalloc_equals_decode_on_consecutive_calls():
    d = device_workload("flash_decode_t64")
    xs = [d.x, d.x[:16].contiguous(), d.x[16:17].contiguous()]
    got = [_noalloc(d, x) for x in xs]            # back to back on one stream, one scratch array
    torch.cuda.synchronize()
    for x, (out, ids, wts) in zip(xs, got):
        T = x.shape[0]
        say(f"[case] noalloc decode T={T}")
        ref_out, ref_ids, ref_w = d.run(False, x=x)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"T={T}: output differs"
        assert torch.equal(ids, ref_ids), f"T={T}: ids differ"
        assert torch.equal(wts, ref_w), f"T={T}: weights differ"
    # the last (smallest) call against the oracle as well
    out, ids, wts = got[-1]
    from oracle import decode_bf16, route
    ids_ref, w_ref, _, _ = route(decode_bf16(d.inp.x[16:17]), d.inp.router_w, d.inp.router_bias, d.w.K, d.w.rsf)
    assert_router_close(ids.cpu().numpy(), wts.cpu().numpy(), ids_ref, w_ref, "noalloc T=1")
    ref, _, _ = d.inp.oracle(tokens=np.arange(16, 17))
    assert_output_close(bf16_host_bits(out), ref, "noalloc T=1")


def test_noalloc_rejects_calls_beyond_the_scratch_array():
    d = device_workload("flash_decode_t64")
    need = capi.moe_mlp_workspace_size(d.cfg, capi.DECODE_MAX_T, False)
    assert need > capi.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((capi.DECODE_MAX_T, d.w.H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(x)
    with pytest.raises(capi.MoeMlpError) as e:
        capi.moe_mlp_decode_noalloc(d.cfg, d.weights, x, out)
    assert e.value.status == capi.ERR_SCRATCH_LIMIT
