"""C ABI checks that need no GPU: the library loads, exports every entry point
include/moe_mlp.h declares, and validates its arguments (every error path
returns before anything is enqueued, so fake device addresses are safe)."""
import ctypes
import math
import os
import re

import pytest

import routed_expert_mlp_amd as R
from routed_expert_mlp_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000          # 16-byte aligned fake device address (never dereferenced)


def header_functions():
    text = open(os.path.join(ROOT, "include", "moe_mlp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(moe_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(capi.EXPORTED)
    L = R.lib()
    for n in names:
        assert getattr(L, n) is not None


def test_status_strings():
    for code, name in [(0, "MOE_MLP_OK"), (-1, "NULL_ARG"), (-2, "BAD_SHAPE"), (-3, "BAD_TOPK"),
                       (-4, "BAD_VALUE"), (-5, "MISALIGNED"), (-6, "WORKSPACE_TOO_SMALL"),
                       (-7, "KIND_MISMATCH"), (-8, "ERR_HIP"), (-99, "UNKNOWN")]:
        assert name in R.moe_mlp_status_string(code)


def cfg(**kw):
    base = dict(kind=0, hidden=256, moe_intermediate=128, num_experts=16, top_k=4, n_shared_experts=1,
                shared_intermediate=128, dense_intermediate=0, routed_scaling_factor=2.5, swiglu_limit=7.0)
    base.update(kw)
    return capi.moe_mlp_config(**base)


def full_weights(**override):
    names = [f[0] for f in capi.moe_mlp_weights._fields_]
    vals = {n: FAKE + 0x100000 * i for i, n in enumerate(names)}
    vals.update(override)
    return capi.moe_mlp_weights(**vals)


def ws_size(c, T, prefill):
    n = ctypes.c_size_t(0)
    st = R.lib().moe_mlp_workspace_size(ctypes.byref(c), T, prefill, ctypes.byref(n))
    return st, n.value


def call(entry, c, w, T=1, x=FAKE, out=FAKE + 0x10000, ids=None, wo=None, ws=FAKE + 0x20000, wsb=None):
    if wsb is None:
        st, wsb = ws_size(c, max(T, 0), entry == "moe_mlp_prefill") if c is not None else (1, 0)
        if st:
            wsb = 1 << 40
    fn = getattr(R.lib(), entry)
    return fn(ctypes.byref(c) if c is not None else None, ctypes.byref(w) if w is not None else None,
              x, T, out, ids, wo, ws, wsb, None)


ENTRIES = ["moe_mlp_decode", "moe_mlp_prefill"]


@pytest.mark.parametrize("entry", ENTRIES)
def test_null_and_kind(entry):
    assert call(entry, None, full_weights()) == capi.ERR_NULL_ARG
    assert call(entry, cfg(), None) == capi.ERR_NULL_ARG
    assert call(entry, cfg(kind=7), full_weights()) == capi.ERR_BAD_VALUE
    assert call(entry, cfg(), full_weights(), x=None) == capi.ERR_NULL_ARG
    assert call(entry, cfg(), full_weights(), out=None) == capi.ERR_NULL_ARG
    assert call(entry, cfg(), full_weights(), ws=None) == capi.ERR_NULL_ARG


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("kw,code", [
    (dict(hidden=100), capi.ERR_BAD_SHAPE), (dict(hidden=0), capi.ERR_BAD_SHAPE),
    (dict(hidden=-32), capi.ERR_BAD_SHAPE), (dict(hidden=1 << 17), capi.ERR_BAD_SHAPE),
    (dict(moe_intermediate=48), capi.ERR_BAD_SHAPE), (dict(shared_intermediate=40), capi.ERR_BAD_SHAPE),
    (dict(n_shared_experts=2), capi.ERR_BAD_VALUE),
    (dict(num_experts=0), capi.ERR_BAD_VALUE), (dict(num_experts=1025, top_k=4), capi.ERR_BAD_VALUE),
    (dict(top_k=0), capi.ERR_BAD_TOPK), (dict(top_k=17, num_experts=64), capi.ERR_BAD_TOPK),
    (dict(top_k=5, num_experts=4), capi.ERR_BAD_TOPK),
    (dict(swiglu_limit=0.0), capi.ERR_BAD_VALUE), (dict(swiglu_limit=-1.0), capi.ERR_BAD_VALUE),
    (dict(swiglu_limit=math.nan), capi.ERR_BAD_VALUE), (dict(swiglu_limit=math.inf), capi.ERR_BAD_VALUE),
    (dict(routed_scaling_factor=0.0), capi.ERR_BAD_VALUE),
    (dict(routed_scaling_factor=math.nan), capi.ERR_BAD_VALUE),
    (dict(kind=1, dense_intermediate=0), capi.ERR_BAD_SHAPE),
    (dict(kind=1, dense_intermediate=33), capi.ERR_BAD_SHAPE),
])
def test_config_validation(entry, kw, code):
    assert call(entry, cfg(**kw), full_weights()) == code
    assert ws_size(cfg(**kw), 1, entry == "moe_mlp_prefill")[0] == code


def test_token_count_limits():
    assert call("moe_mlp_decode", cfg(), full_weights(), T=-1) == capi.ERR_BAD_SHAPE
    assert call("moe_mlp_decode", cfg(), full_weights(), T=capi.DECODE_MAX_T + 1) == capi.ERR_BAD_SHAPE
    assert ws_size(cfg(), capi.DECODE_MAX_T + 1, 1)[0] == capi.OK
    assert ws_size(cfg(top_k=16), 1 << 27, 1)[0] == capi.ERR_BAD_SHAPE     # T*K >= 2^31


@pytest.mark.parametrize("entry", ENTRIES)
def test_zero_tokens_is_a_noop(entry):
    assert call(entry, cfg(), full_weights(), T=0, x=None, out=None, ws=None, wsb=0) == capi.OK


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("missing", ["router_w", "router_bias", "w13_q", "w13_s", "w13_g", "w2_q", "w2_s",
                                     "w2_g", "shared_w13", "shared_w2"])
def test_missing_weights(entry, missing):
    # without tile-layout codes the row-major codes are required
    off = {missing: None, "w13_q_tiled": None, "w13_s_tiled": None, "w2_q_tiled": None, "w2_s_tiled": None}
    assert call(entry, cfg(), full_weights(**off)) == capi.ERR_KIND_MISMATCH


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("proj", ["w13", "w2"])
def test_tiled_only_codes_rules(entry, proj):
    """Row-major codes may be left out when the projection's tile-layout codes
    AND scales are given, for reductions (H for gate/up, I for down) that are
    a multiple of 256 and at least 512; otherwise the call is refused before
    anything runs."""
    # tiled codes without tiled scales: the codes count as missing
    assert call(entry, cfg(hidden=512, moe_intermediate=512),
                full_weights(**{f"{proj}_q": None, f"{proj}_s_tiled": None})) == capi.ERR_KIND_MISMATCH
    # reduction below 512 or not a multiple of 256: no tile kernel for it
    small = dict(hidden=256, moe_intermediate=256)
    assert call(entry, cfg(**small), full_weights(**{f"{proj}_q": None})) == capi.ERR_BAD_SHAPE
    odd = dict(hidden=768 + 32, moe_intermediate=768 + 32)
    assert call(entry, cfg(**odd), full_weights(**{f"{proj}_q": None})) == capi.ERR_BAD_SHAPE


@pytest.mark.parametrize("entry", ENTRIES)
def test_weights_per_kind(entry):
    # no shared expert: its tensors are not needed
    assert call(entry, cfg(n_shared_experts=0), full_weights(shared_w13=None, shared_w2=None),
                wsb=0) == capi.ERR_WORKSPACE_TOO_SMALL
    dense = cfg(kind=1, dense_intermediate=512)
    assert call(entry, dense, full_weights(dense_w2=None)) == capi.ERR_KIND_MISMATCH
    assert call(entry, dense, full_weights(router_w=None, w13_q=None), wsb=0) == capi.ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("entry", ENTRIES)
def test_alignment(entry):
    assert call(entry, cfg(), full_weights(), x=FAKE + 8) == capi.ERR_MISALIGNED
    assert call(entry, cfg(), full_weights(), out=FAKE + 2) == capi.ERR_MISALIGNED
    assert call(entry, cfg(), full_weights(w13_q=FAKE + 4)) == capi.ERR_MISALIGNED
    assert call(entry, cfg(), full_weights(), ids=FAKE + 4) == capi.ERR_MISALIGNED


@pytest.mark.parametrize("entry", ENTRIES)
def test_workspace_too_small(entry):
    st, need = ws_size(cfg(), 5, entry == "moe_mlp_prefill")
    assert st == 0 and need > 0
    assert call(entry, cfg(), full_weights(), T=5, wsb=need - 1) == capi.ERR_WORKSPACE_TOO_SMALL


def test_workspace_grows_with_tokens():
    for pf in (0, 1):
        sizes = [ws_size(cfg(), T, pf)[1] for T in (1, 2, 16, 64, 256)]
        assert sizes == sorted(sizes) and sizes[0] > 0
    assert ws_size(cfg(), 1, 0)[0] == capi.OK
    n = ctypes.c_size_t(0)
    assert R.lib().moe_mlp_workspace_size(ctypes.byref(cfg()), 1, 0, None) == capi.ERR_NULL_ARG


def test_router_topk_validation():
    L = R.lib()
    c = cfg()
    assert L.moe_router_topk(ctypes.byref(c), None, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 1 << 30, None) == capi.ERR_NULL_ARG
    assert L.moe_router_topk(ctypes.byref(cfg(top_k=20)), FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 1 << 30,
                             None) == capi.ERR_BAD_TOPK
    assert L.moe_router_topk(ctypes.byref(cfg(kind=1, dense_intermediate=64)), FAKE, FAKE, FAKE, 4, FAKE, FAKE,
                             FAKE, 1 << 30, None) == capi.ERR_KIND_MISMATCH
    assert L.moe_router_topk(ctypes.byref(c), FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, 16, None) == \
        capi.ERR_WORKSPACE_TOO_SMALL
    assert L.moe_router_topk(ctypes.byref(c), FAKE, FAKE, FAKE, 0, None, None, None, 0, None) == capi.OK


def test_dequant_validation():
    L = R.lib()
    assert L.moe_nvfp4_dequant(None, FAKE, 1.0, 4, 64, FAKE, None, None) == capi.ERR_NULL_ARG
    assert L.moe_nvfp4_dequant(FAKE, FAKE, 1.0, 4, 64, None, None, None) == capi.ERR_NULL_ARG
    assert L.moe_nvfp4_dequant(FAKE, FAKE, 1.0, 4, 48, FAKE, None, None) == capi.ERR_BAD_SHAPE
    assert L.moe_nvfp4_dequant(FAKE, FAKE, 1.0, -1, 64, FAKE, None, None) == capi.ERR_BAD_SHAPE
    assert L.moe_nvfp4_dequant(FAKE, FAKE, math.inf, 4, 64, FAKE, None, None) == capi.ERR_BAD_VALUE
    assert L.moe_nvfp4_dequant(FAKE + 4, FAKE, 1.0, 4, 64, FAKE, None, None) == capi.ERR_MISALIGNED
    assert L.moe_nvfp4_dequant(FAKE, FAKE + 1, 1.0, 4, 64, FAKE, None, None) == capi.ERR_MISALIGNED
    assert L.moe_nvfp4_dequant(FAKE, FAKE, 1.0, 0, 64, FAKE, None, None) == capi.OK


def test_tile_pack_validation():
    L = R.lib()
    assert L.moe_nvfp4_tile_pack(None, FAKE, 2, 64, 512, FAKE, FAKE, None) == capi.ERR_NULL_ARG
    assert L.moe_nvfp4_tile_pack(FAKE, FAKE, 2, 64, 512, FAKE, None, None) == capi.ERR_NULL_ARG
    assert L.moe_nvfp4_tile_pack(FAKE, FAKE, 2, 48, 512, FAKE, FAKE, None) == capi.ERR_BAD_SHAPE
    assert L.moe_nvfp4_tile_pack(FAKE, FAKE, 2, 64, 384, FAKE, FAKE, None) == capi.ERR_BAD_SHAPE
    assert L.moe_nvfp4_tile_pack(FAKE, FAKE, -1, 64, 512, FAKE, FAKE, None) == capi.ERR_BAD_SHAPE
    assert L.moe_nvfp4_tile_pack(FAKE, FAKE, 2, 0, 512, FAKE, FAKE, None) == capi.ERR_BAD_SHAPE
    assert L.moe_nvfp4_tile_pack(FAKE + 8, FAKE, 2, 64, 512, FAKE, FAKE, None) == capi.ERR_MISALIGNED
    assert L.moe_nvfp4_tile_pack(FAKE, FAKE, 2, 64, 512, FAKE, FAKE + 4, None) == capi.ERR_MISALIGNED
    assert L.moe_nvfp4_tile_pack(FAKE, FAKE, 0, 64, 512, FAKE, FAKE, None) == capi.OK


def test_misaligned_tiled_weights_rejected():
    for field in ["w13_q_tiled", "w13_s_tiled", "w2_q_tiled", "w2_s_tiled"]:
        assert call("moe_mlp_prefill", cfg(), full_weights(**{field: FAKE + 8})) == capi.ERR_MISALIGNED


def test_profiled_entry_validation():
    L = R.lib()
    c = cfg()
    w = full_weights()
    n = 3                               # one-token decode stages of this config
    names = [L.moe_mlp_stage_name(ctypes.byref(c), 1, 0, i) for i in range(n + 1)]
    assert [x.decode() for x in names[:n]] == ["logits_shared_gateup", "routed_gateup",
                                                   "shared_routed_down_combine"]
    assert names[n] is None
    assert [L.moe_mlp_stage_name(ctypes.byref(c), 8, 0, i).decode() for i in range(7)][3] == "routed_gateup"
    assert L.moe_mlp_stage_name(ctypes.byref(c), 4, 0, 2).decode() == "shared_routed_down_combine"
    assert L.moe_mlp_stage_name(ctypes.byref(c), 64, 0, 2).decode() == "permute"
    assert L.moe_mlp_stage_name(ctypes.byref(c), 2, 1, 8) is None
    assert L.moe_mlp_stage_name(None, 1, 0, 0) is None
    ev_t = ctypes.c_void_p * 6
    evs = ev_t(*[FAKE + 64 * i for i in range(6)])
    st, need = ws_size(c, 1, 0)
    f = L.moe_mlp_forward_profiled
    assert f(ctypes.byref(c), ctypes.byref(w), FAKE, 1, FAKE, None, None, FAKE, need, None, 0, None, 6) == \
        capi.ERR_NULL_ARG
    assert f(ctypes.byref(c), ctypes.byref(w), FAKE, 1, FAKE, None, None, FAKE, need, None, 0, evs, 5) == \
        capi.ERR_BAD_VALUE
    evs[3] = None
    assert f(ctypes.byref(c), ctypes.byref(w), FAKE, 1, FAKE, None, None, FAKE, need, None, 0, evs, 6) == \
        capi.ERR_NULL_ARG
    evs[3] = FAKE
    assert f(ctypes.byref(c), ctypes.byref(w), FAKE, 1, FAKE, None, None, FAKE, need - 1, None, 0, evs, 6) == \
        capi.ERR_WORKSPACE_TOO_SMALL


def test_noalloc_decode_validation():
    """moe_mlp_decode_noalloc validates like moe_mlp_decode, and rejects a call whose workspace
    exceeds its scratch array, before touching the device."""
    L = R.lib()
    flash = cfg(hidden=4096, moe_intermediate=1536, num_experts=288, top_k=8, shared_intermediate=1536)
    w = full_weights()

    def noalloc(c, T, x=FAKE, out=FAKE + 0x10000):
        return L.moe_mlp_decode_noalloc(ctypes.byref(c) if c is not None else None, ctypes.byref(w), x, T, out,
                                        None, None, None)
    assert noalloc(None, 1) == capi.ERR_NULL_ARG
    assert noalloc(cfg(top_k=17), 1) == capi.ERR_BAD_TOPK
    assert noalloc(flash, capi.DECODE_MAX_T + 1) == capi.ERR_BAD_SHAPE
    assert noalloc(flash, 0, x=None, out=None) == capi.OK
    assert ws_size(flash, capi.DECODE_MAX_T, 0)[1] > capi.NOALLOC_SCRATCH_BYTES
    assert noalloc(flash, capi.DECODE_MAX_T) == capi.ERR_SCRATCH_LIMIT
    assert "SCRATCH_LIMIT" in R.moe_mlp_status_string(capi.ERR_SCRATCH_LIMIT)


def test_fp8_kind_validation():
    """MOE_MLP_KIND_ROUTED_FP8: H and I multiples of 128, the FP8 weight fields required
    (the NVFP4 ones are not)."""
    fp8 = dict(kind=capi.KIND_ROUTED_FP8)
    assert ws_size(cfg(**fp8), 1, 0)[0] == capi.OK
    assert ws_size(cfg(hidden=416, **fp8), 1, 0)[0] == capi.ERR_BAD_SHAPE
    assert ws_size(cfg(moe_intermediate=160, **fp8), 1, 1)[0] == capi.ERR_BAD_SHAPE
    for missing in ("w13_f8", "w13_f8_scale", "w2_f8", "w2_f8_scale", "router_w", "shared_w2"):
        for entry in ENTRIES:
            assert call(entry, cfg(**fp8), full_weights(**{missing: None})) == capi.ERR_KIND_MISMATCH, missing
    no_nvfp4 = full_weights(w13_q=None, w13_s=None, w13_g=None, w2_q=None, w2_s=None, w2_g=None)
    for entry in ENTRIES:
        assert call(entry, cfg(**fp8), no_nvfp4, wsb=0) == capi.ERR_WORKSPACE_TOO_SMALL
    # the stage names follow the routed forms
    L = R.lib()
    assert L.moe_mlp_stage_name(ctypes.byref(cfg(**fp8)), 1, 0, 2).decode() == "shared_routed_down_combine"
    assert L.moe_mlp_stage_name(ctypes.byref(cfg(**fp8)), 16, 0, 3).decode() == "routed_gateup"
