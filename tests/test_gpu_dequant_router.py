"""GPU parity, levels 1-3: NVFP4 dequant bit-exact; router ids bit-exact and
weights within 1e-6 relative of the fp64 oracle (moe_nvfp4_dequant,
moe_router_topk through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_util import DEV, assert_router_close, say
from inputs import RoutedInputs
from routed_expert_mlp_amd import capi

pytestmark = pytest.mark.gpu


def _bits64(a):
    return np.asarray(a, np.float64).view(np.uint64)


def _dequant_both(q, s, g):
    qd, sd = torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV)
    rows, cols = q.shape[0], q.shape[1] * 2
    f = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
    b = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    capi.moe_nvfp4_dequant(qd, sd, g, out_f32=f, out_bf16=b)
    torch.cuda.synchronize()
    return f.cpu().numpy(), b.view(torch.int16).cpu().numpy().view(np.uint16)


def _check_exact(q, s, g, what):
    f, b = _dequant_both(q, s, g)
    ref = O.dequant_nvfp4(q, s) * g
    assert np.array_equal(_bits64(f.astype(np.float64)), _bits64(ref)), f"{what}: fp32 dequant not bit-exact"
    refb = O.round_bf16(ref)
    assert np.array_equal(_bits64(O.decode_bf16(b)), _bits64(refb)), f"{what}: bf16 dequant not bit-exact"
    say(f"[parity] dequant {what}: {q.shape[0]}x{2 * q.shape[1]} bit-exact (fp32 and bf16)")


def test_dequant_all_codes_times_sample_scales():
    scales = np.array([0x00, 0x01, 0x07, 0x08, 0x15, 0x30, 0x38, 0x3B, 0x7E, 0x80, 0xB8, 0xFE], np.uint8)
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)                    # 32 columns = 2 blocks
    q = np.tile((codes[0::2] | (codes[1::2] << 4)).astype(np.uint8), (len(scales), 1))
    s = np.repeat(scales[:, None], 2, axis=1)
    _check_exact(q, s, 1.0, "code x scale table")


@pytest.mark.parametrize("rows,cols,g", [(37, 4128, 1.0), (3, 32, 1.0), (64, 1536, 0.75), (5, 256, 2.0 ** -3)])
def test_dequant_random(rows, cols, g):
    rng = np.random.default_rng(rows * cols)
    q = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    s = synth.encode_e4m3(np.abs(rng.standard_normal((rows, cols // 16))) * 0.05)
    s[0, : min(4, s.shape[1])] = [0x7E, 0x01, 0x00, 0x08][: min(4, s.shape[1])]
    _check_exact(q, s, g, f"random g={g}")


ROUTER_CASES = ["tiny_decode", "flash_decode_t1", "flash_decode_t64", "skewed_decode_t64_k16", "ragged_prefill",
                "prefill_t4096", "flash_decode_t64_literal_bias", "prefill_t4096_literal_bias"]


@pytest.mark.parametrize("name", ROUTER_CASES)
def test_router_topk_parity(name):
    w = synth.workload(name)
    inp = RoutedInputs(w)
    from gpu_util import bf16_dev, config_of
    cfg = config_of(w)
    say(f"[case] router {name} T={w.T} E={w.E} K={w.K}")
    ids = torch.empty((w.T, w.K), dtype=torch.int32, device=DEV)
    wts = torch.empty((w.T, w.K), dtype=torch.float32, device=DEV)
    capi.moe_router_topk(cfg, torch.from_numpy(inp.router_w).to(DEV), torch.from_numpy(inp.router_bias).to(DEV),
                         bf16_dev(inp.x), ids, wts)
    torch.cuda.synchronize()
    ids_ref, w_ref, _, _ = O.route(O.decode_bf16(inp.x), inp.router_w, inp.router_bias, w.K, w.rsf)
    assert_router_close(ids.cpu().numpy(), wts.cpu().numpy(), ids_ref, w_ref, f"router {name}")
