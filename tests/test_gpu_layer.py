"""GPU parity, level 4 (plus ids/weights from the layer calls): moe_mlp_decode
and moe_mlp_prefill through the C ABI against the fp64 oracle in contract
mode, on the same seeded inputs.

Tolerance: rel-L2 <= 5e-3 and max-abs <= 1e-2 * max|ref| for the bf16 output;
ids bit-exact; weights within 1e-6 relative.  Every workload compares every
token's ids, weights and output, the GLM-Flash-sized ones included (the
oracle's per-expert work runs in worker processes, tests/oracle_pool.py).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_util import (DEV, DeviceRouted, assert_output_close, assert_router_close, bf16_dev, bf16_host_bits,
                      config_of, device_workload, rel_l2, say)
from inputs import RoutedInputs
from routed_expert_mlp_amd import capi

pytestmark = pytest.mark.gpu


def _sample(T, n, seed=0):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    s = np.sort(rng.choice(T, size=n, replace=False))
    s[0], s[-1] = 0, T - 1                  # always the first and the last token
    return np.unique(s)


def _check_layer(d: DeviceRouted, prefill: bool, n_sample: int, what: str):
    w = d.w
    say(f"[case] {what}: {'prefill' if prefill else 'decode'} T={w.T} H={w.H} I={w.I} E={w.E} K={w.K}")
    out, ids, wts = d.run(prefill)
    torch.cuda.synchronize()
    ids_ref, w_ref, _, _ = O.route(O.decode_bf16(d.inp.x), d.inp.router_w, d.inp.router_bias, w.K, w.rsf)
    assert_router_close(ids.cpu().numpy(), wts.cpu().numpy(), ids_ref, w_ref, what)
    toks = _sample(w.T, n_sample)
    ref, _, _ = d.inp.oracle(tokens=toks, parallel=w.H * w.I * len(toks) * w.K > 2 ** 26)
    assert_output_close(bf16_host_bits(out)[toks], ref, f"{what} ({len(toks)} of {w.T} tokens)")
    return out


ALL = 1 << 30      # compare every token

DECODE = [("tiny_decode", ALL), ("ragged_decode", ALL), ("flash_decode_t1", ALL),
          ("flash_decode_t1_literal_bias", ALL), ("flash_decode_t16", ALL), ("flash_decode_t64", ALL),
          ("skewed_decode_t64_k16", ALL), ("flash_decode_t16_literal_bias", ALL),
          ("flash_decode_t64_literal_bias", ALL)]


@pytest.mark.parametrize("name,n_sample", DECODE, ids=[d[0] for d in DECODE])
def test_decode_parity(name, n_sample):
    _check_layer(device_workload(name), False, n_sample, name)


# Decode batches whose routed down projection runs k_skinny_f4_down
# (reduction I a multiple of 512 up to 2048, output rows a multiple of 64):
# groups within one LDS pass (12 rows) and groups of several passes, the
# expert-GEMV form (below 64 tokens) and the grouped-GEMM form (64..256
# tokens), each unit count the kernel is built for.
SKINNY = [dict(T=16, H=512, I=512, E=4, K=4, Is=128),       # 16 rows per expert: 2 passes
          dict(T=7, H=1024, I=1024, E=16, K=4, Is=0),
          dict(T=24, H=2048, I=1536, E=16, K=4, Is=128),
          dict(T=24, H=256, I=1536, E=16, K=4, Is=128),
          dict(T=40, H=512, I=512, E=16, K=4, Is=128),
          dict(T=48, H=192, I=2048, E=6, K=2, Is=96),       # 16 rows per expert
          dict(T=100, H=1024, I=1536, E=8, K=4, Is=128),    # ~50 rows per expert: 5 passes
          dict(T=256, H=512, I=512, E=16, K=2, Is=128)]


@pytest.mark.parametrize("o", SKINNY, ids=[f"T{o['T']}_H{o['H']}_I{o['I']}_E{o['E']}" for o in SKINNY])
def test_decode_parity_skinny(o):
    _check_layer(device_workload("ragged_decode", **o), False, ALL, f"ragged_decode {o}")


# Batches of 33..64 tokens with more than 512 slots (top-k above 8) in the
# grouped-GEMM form (decode at 64 tokens, the prefill entry below): the routed
# gate/up splits the tiles of more than 32 rows into one workgroup per 32-row
# pass (every expert full at E = K; a mix of long and short tiles otherwise).
SPLIT = [dict(T=64, H=512, I=512, E=16, K=16, Is=128),
         dict(T=64, H=1024, I=1024, E=24, K=12, Is=128),
         dict(T=48, H=512, I=512, E=40, K=16, Is=0),
         dict(T=33, H=768, I=512, E=20, K=16, Is=64)]


@pytest.mark.parametrize("o", SPLIT, ids=[f"T{o['T']}_E{o['E']}_K{o['K']}" for o in SPLIT])
def test_parity_split_passes(o):
    _check_layer(device_workload("ragged_decode", **o), o["T"] < 64, ALL, f"ragged_decode {o}")


PREFILL = [("ragged_prefill", ALL), ("prefill_t4096", ALL), ("prefill_t4096_literal_bias", ALL)]


@pytest.mark.parametrize("name,n_sample", PREFILL, ids=[p[0] for p in PREFILL])
def test_prefill_parity(name, n_sample):
    _check_layer(device_workload(name), True, n_sample, name)


def test_decode_and_prefill_agree_on_every_token():
    """Two different kernel paths (expert GEMVs below 64 tokens vs the MFMA grouped GEMM)
    on the same 48 tokens."""
    d = device_workload("flash_decode_t64")
    x = d.x[:48].contiguous()
    a, ida, wa = d.run(False, x=x)
    b, idb, wb = d.run(True, x=x)
    torch.cuda.synchronize()
    assert torch.equal(ida, idb)
    assert torch.allclose(wa, wb, rtol=1e-6, atol=0)
    r = rel_l2(a.float().cpu().numpy(), b.float().cpu().numpy())
    say(f"[parity] decode vs prefill (48 tokens): rel_l2={r:.3e}")
    assert r < 5e-3


def test_prefill_matches_decode_on_a_token_subset():
    """Tokens are independent: prefill over 4096 tokens equals decode (expert GEMVs) of a
    48-token subset (within tolerance)."""
    d = device_workload("prefill_t4096")
    out, ids, _ = d.run(True)
    sub = torch.arange(0, 4096, 85, device=DEV)[:48]
    o2, ids2, _ = d.run(False, x=d.x[sub].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(ids[sub], ids2)
    r = rel_l2(out[sub].float().cpu().numpy(), o2.float().cpu().numpy())
    say(f"[parity] prefill vs decode on 48 sampled tokens: rel_l2={r:.3e}")
    assert r < 5e-3


@pytest.mark.parametrize("prefill", [False, True])
def test_runs_are_bitwise_deterministic(prefill):
    d = device_workload("flash_decode_t64")
    a = d.run(prefill)
    b = d.run(prefill)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int8) if y.dtype == torch.bfloat16 else y)


def test_concurrent_streams_equal_solo():
    d = device_workload("flash_decode_t64")
    solo_d = d.run(False)[0]
    solo_p = d.run(True)[0]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        c_d = d.run(False, stream=s1)[0]
    with torch.cuda.stream(s2):
        c_p = d.run(True, stream=s2)[0]
    torch.cuda.synchronize()
    assert torch.equal(solo_d.view(torch.int16), c_d.view(torch.int16))
    assert torch.equal(solo_p.view(torch.int16), c_p.view(torch.int16))


# ---------------------------------------------------------------------------
# Edge cases (tiny shapes, full oracle).
# ---------------------------------------------------------------------------

def _fresh(name, prefill, n_sample=64, w13_g=None, w2_g=None, **overrides):
    w = synth.workload(name, **overrides)
    d = DeviceRouted(RoutedInputs(w), w13_g=w13_g, w2_g=w2_g)
    return _check_layer(d, prefill, n_sample, f"{name} {overrides or ''}")


# Routed NVFP4 grouped GEMM (reduction lengths that are multiples of 256, at
# least 512): experts with two and three 128-row tiles, column blocks cut by
# the matrix edge in gate/up and in down, reductions of 8, 12 and 16 stages
# (no, one and two middle blocks of the DMA schedule), and a 256-long
# reduction (the other grouped GEMM kernel); every token checked.
# H=1024 I=160 and H=256 I=512 run one projection on the tile kernel and the
# other on the fallback kernel.
FP4_TILES = [dict(T=600, H=512, I=512, E=16, K=4, Is=256),
             dict(T=300, H=768, I=512, E=8, K=2, Is=96),
             dict(T=200, H=1024, I=160, E=8, K=2, Is=96),
             dict(T=700, H=512, I=768, E=4, K=2, Is=0),
             dict(T=100, H=256, I=256, E=4, K=2, Is=64),
             dict(T=150, H=256, I=512, E=8, K=2, Is=64)]


@pytest.mark.parametrize("overrides", FP4_TILES, ids=[f"T{o['T']}_H{o['H']}_I{o['I']}_E{o['E']}" for o in FP4_TILES])
def test_grouped_gemm_nvfp4_tiles(overrides):
    _fresh("ragged_prefill", True, n_sample=100000, **overrides)


# Up to 256 tokens the gate/up tiles of at most 32 rows run on the small-tile
# NVFP4 kernel (the rest on the 128-row one, which the scheduler gives the
# tiles of more than 32 rows, listed first): expert counts around 128 (short
# second tiles), around 32 and 25 (both kernels side by side), and at most 32
# tokens (the small-tile kernel alone); reductions (H) of 768, 1280, 1536 and
# 512, and 1024 below (2 to 6 blocks of four stages: the first block doubling
# as the second to last, and both parities of the last).
SMALL_TILES = [dict(T=256, H=768, I=768, E=4, K=2, Is=0),
               dict(T=256, H=1280, I=1024, E=8, K=1, Is=64),
               dict(T=200, H=1536, I=512, E=16, K=2, Is=64),
               dict(T=32, H=512, I=1024, E=4, K=2, Is=0)]


@pytest.mark.parametrize("overrides", SMALL_TILES,
                         ids=[f"T{o['T']}_H{o['H']}_I{o['I']}_E{o['E']}_K{o['K']}" for o in SMALL_TILES])
def test_grouped_gemm_small_tiles(overrides):
    _fresh("ragged_prefill", True, n_sample=100000, **overrides)


# The decode form runs the grouped GEMM from 64 tokens.  Up to 64 tokens the
# small-tile kernel takes every gate/up tile, one of more than 32 rows in two
# passes (expert counts 40, 36, 25, 27 and 27, 37 here, reductions of 768 and
# 1280); above, the tiles of more than 32 rows go to the 128-row kernel (100
# tokens over 8 experts, K=2: 25 rows per expert on average).
DECODE_GEMM_SMALL = [dict(T=64, H=768, I=512, E=4, K=2, Is=64), dict(T=64, H=1280, I=512, E=2, K=1, Is=64),
                     dict(T=100, H=1024, I=512, E=8, K=2, Is=64)]


@pytest.mark.parametrize("overrides", DECODE_GEMM_SMALL,
                         ids=[f"T{o['T']}_H{o['H']}_E{o['E']}_K{o['K']}" for o in DECODE_GEMM_SMALL])
def test_decode_gemm_form_small_tiles(overrides):
    _fresh("ragged_decode", False, n_sample=100000, **overrides)


@pytest.mark.parametrize("prefill", [False, True])
def test_top_k_equals_e_at_the_kernel_limit(prefill):
    _fresh("tiny_decode", prefill, T=8, K=16)


@pytest.mark.parametrize("prefill", [False, True])
def test_single_expert(prefill):
    _fresh("tiny_decode", prefill, T=5, E=1, K=1)


@pytest.mark.parametrize("prefill", [False, True])
def test_no_shared_expert(prefill):
    _fresh("tiny_decode", prefill, T=7, Is=0)


@pytest.mark.parametrize("prefill", [False, True])
def test_global_scales(prefill):
    E = 16
    g13 = np.stack([np.full(E, 0.75), np.full(E, 2.0 ** -3)], axis=1).astype(np.float32)
    g2 = np.linspace(0.5, 2.0, E).astype(np.float32)
    _fresh("tiny_decode", prefill, T=9, w13_g=g13, w2_g=g2)


@pytest.mark.parametrize("prefill", [False, True])
def test_minimum_hidden_size(prefill):
    _fresh("tiny_decode", prefill, T=3, H=32, I=32, Is=32)


def test_decode_maximum_tokens():
    _fresh("ragged_decode", False, n_sample=256, T=capi.DECODE_MAX_T)


@pytest.mark.parametrize("overrides", [dict(T=63), dict(T=48, K=8, E=8), dict(T=33, K=2)],
                         ids=["T63", "T48_E8_K8", "T33_K2"])
def test_decode_gemv_path_below_the_gemm_switch(overrides):
    """Ragged shapes on the expert-GEMV decode path (fewer than 64 tokens): many token
    groups per expert, every expert touched (E=8, K=8), and K=2."""
    _fresh("ragged_decode", False, n_sample=64, **overrides)


def test_prefill_one_token():
    _fresh("tiny_decode", True, T=1)


@pytest.mark.parametrize("prefill", [False, True])
def test_zero_tokens(prefill):
    d = device_workload("tiny_decode")
    x = torch.empty((0, d.w.H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((0, d.w.H), dtype=torch.bfloat16, device=DEV)
    fn = capi.moe_mlp_prefill if prefill else capi.moe_mlp_decode
    fn(d.cfg, d.weights, x, out)


# ---------------------------------------------------------------------------
# Dense FFN variant.
# ---------------------------------------------------------------------------

def _dense(name, prefill, n_sample, **overrides):
    w = synth.workload(name, **overrides)
    say(f"[case] dense {name} {'prefill' if prefill else 'decode'} T={w.T} H={w.H} Id={w.Id}")
    x = synth.x_rows(w)
    w13, w2 = synth.dense_w13(w), synth.dense_w2(w)
    cfg = config_of(w)
    wt = capi.Weights(dense_w13=bf16_dev(w13), dense_w2=bf16_dev(w2))
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)
    (capi.moe_mlp_prefill if prefill else capi.moe_mlp_decode)(cfg, wt, bf16_dev(x), out)
    torch.cuda.synchronize()
    toks = _sample(w.T, n_sample)
    ref = O.dense_ffn(x, w13, w2, w.swiglu_limit, tokens=toks)
    assert_output_close(bf16_host_bits(out)[toks], ref, f"dense {name} T={w.T}")


@pytest.mark.parametrize("prefill", [False, True])
def test_dense_ragged(prefill):
    _dense("ragged_dense_prefill", prefill, 300, T=256 if not prefill else 300)


# BF16 tile GEMM shapes: row tails of 44, 77 and 1 rows; weight-row blocks cut at
# the matrix edge (gate/up 320 = 2.5 x 128 columns, down 640 = 2.5 x 256 rows);
# the shortest reduction (128 = one pair of 64-wide stages); a down reduction
# of 320 (not a multiple of 128) that takes the 32x32 fallback kernel.
DENSE_TILES = [dict(T=300, H=640, Id=384), dict(T=77, H=512, Id=320),
               dict(T=513, H=256, Id=1024), dict(T=40, H=128, Id=128)]


@pytest.mark.parametrize("overrides", DENSE_TILES, ids=[f"T{o['T']}_H{o['H']}_Id{o['Id']}" for o in DENSE_TILES])
def test_dense_bf16_tiles(overrides):
    _dense("ragged_dense_prefill", True, 100000, **overrides)


def test_dense_prefill_full_size():
    _dense("dense_prefill_t4096", True, ALL)


def test_dense_decode_full_width():
    _dense("dense_prefill_t4096", False, 4, T=4)


ONE_TOKEN = [dict(K=16), dict(E=1, K=1), dict(Is=0), dict(H=32, I=32, Is=32), dict(K=2),
             dict(I=96, Is=224), dict(H=4096, I=2048, Is=2048, E=12, K=8)]


@pytest.mark.parametrize("overrides", ONE_TOKEN, ids=[str(o) for o in ONE_TOKEN])
def test_one_token_path_edge_cases(overrides):
    """T=1 runs the three-launch one-token kernels: block shapes for K up to 16, no shared
    expert, the smallest hidden size, ragged row counts, and the largest H / I / Is it takes."""
    _fresh("tiny_decode", False, T=1, **overrides)


FEW_TOKEN = [dict(T=2), dict(T=3), dict(T=4, K=16), dict(T=3, E=1, K=1), dict(T=2, Is=0),
             dict(T=4, H=32, I=32, Is=32), dict(T=4, I=96, Is=224)]


@pytest.mark.parametrize("overrides", FEW_TOKEN, ids=[str(o) for o in FEW_TOKEN])
def test_few_token_path_edge_cases(overrides):
    """2..4 tokens (the MTP verify shapes) run the three fused launches with a slot per
    (token, k): up to 64 slots, no shared expert, the smallest hidden size, ragged rows."""
    _fresh("tiny_decode", False, **overrides)


@pytest.mark.parametrize("T", [2, 3, 4])
def test_few_token_path_full_size(T):
    d = device_workload("flash_decode_t16")
    x = d.x[:T].contiguous()
    say(f"[case] few-token decode flash T={T}")
    out, ids, wts = d.run(False, x=x)
    torch.cuda.synchronize()
    ids_ref, w_ref, _, _ = O.route(O.decode_bf16(d.inp.x[:T]), d.inp.router_w, d.inp.router_bias, d.w.K, d.w.rsf)
    assert_router_close(ids.cpu().numpy(), wts.cpu().numpy(), ids_ref, w_ref, f"few-token T={T}")
    ref, _, _ = d.inp.oracle(tokens=np.arange(T))
    assert_output_close(bf16_host_bits(out), ref, f"few-token flash T={T}")
    # the GEMV path on the same tokens agrees too (tokens are independent)
    big = d.run(False)[0]
    torch.cuda.synchronize()
    r = rel_l2(out.float().cpu().numpy(), big[:T].float().cpu().numpy())
    say(f"[parity] few-token vs 16-token GEMV path on {T} tokens: rel_l2={r:.3e}")
    assert r < 5e-3


def test_one_token_path_repeated_calls():
    """Many calls in a row on one workspace (which starts as garbage) give the same bits."""
    d = device_workload("flash_decode_t1")
    ws = capi.workspace(d.cfg, 1, False, DEV)
    ws.fill_(0xFF)
    ref = d.run(False)[0]
    outs = []
    for _ in range(20):
        o = torch.empty_like(ref)
        capi.moe_mlp_decode(d.cfg, d.weights, d.x, o, ws=ws)
        outs.append(o)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))


def test_single_token_general_path():
    """I > 2048 takes the general decode kernels at T=1 (not the one-token path)."""
    _fresh("tiny_decode", False, T=1, I=2080)


@pytest.mark.parametrize("name,prefill", [("flash_decode_t1", False), ("flash_decode_t16", False),
                                          ("ragged_prefill", True)])
def test_profiled_entry_matches_plain_call(name, prefill):
    import ctypes
    d = device_workload(name)
    out, ids, wts = d.run(prefill)
    names = capi.stage_names(d.cfg, d.w.T, prefill)
    hip = ctypes.CDLL("libamdhip64.so.7")
    evs = []
    for _ in range(2 * len(names)):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    out2 = torch.empty_like(out)
    capi.moe_mlp_forward_profiled(d.cfg, d.weights, d.x, out2, prefill, evs)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    times = []
    for i in range(len(names)):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(evs[2 * i]),
                                       ctypes.c_void_p(evs[2 * i + 1])) == 0
        times.append(ms.value)
        hip.hipEventDestroy(ctypes.c_void_p(evs[2 * i]))
        hip.hipEventDestroy(ctypes.c_void_p(evs[2 * i + 1]))
    say(f"[stages] {name}: " + ", ".join(f"{n}={t * 1e3:.1f}us" for n, t in zip(names, times)))
    assert all(t >= 0 for t in times) and sum(times) > 0


# ---------------------------------------------------------------------------
# HIP graph capture (hipGraph through torch.cuda.CUDAGraph): the layer's
# launches replay from a graph.  Every replay, with eager work and a new input
# copied into the captured input buffer in between, equals an eager call on
# the same input bitwise.
# ---------------------------------------------------------------------------

GRAPH_CASES = [("flash_decode_t1", 1, False), ("flash_decode_t16", 4, False), ("ragged_prefill", 300, True)]


@pytest.mark.parametrize("name,T,prefill", GRAPH_CASES, ids=[f"{c[0]}_T{c[1]}" for c in GRAPH_CASES])
def test_hip_graph_replays_equal_eager(name, T, prefill):
    d = device_workload(name)
    say(f"[case] graph {name} T={T} {'prefill' if prefill else 'decode'}")
    fn = capi.moe_mlp_prefill if prefill else capi.moe_mlp_decode
    H, K = d.w.H, d.w.K
    xs = [d.x[:T].clone(), d.x[T:2 * T].clone() if d.x.shape[0] >= 2 * T else d.x[:T].flip(0).contiguous()]
    x_in = xs[0].clone()
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    wts = torch.empty((T, K), dtype=torch.float32, device=DEV)
    ws = capi.workspace(d.cfg, T, prefill, DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(d.cfg, d.weights, x_in, out, ids, wts, ws=ws)          # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn(d.cfg, d.weights, x_in, out, ids, wts, ws=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        xr = xs[rep % 2]
        ref_out = torch.empty_like(out)
        ref_ids = torch.empty_like(ids)
        ref_w = torch.empty_like(wts)
        fn(d.cfg, d.weights, xr, ref_out, ref_ids, ref_w)       # eager, own workspace
        x_in.copy_(xr)
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {rep}: output differs"
        assert torch.equal(ids, ref_ids), f"replay {rep}: ids differ"
        assert torch.equal(wts, ref_w), f"replay {rep}: weights differ"
    say(f"[parity] graph {name}: 4 replays equal eager bitwise")


def test_bound_call_equals_plain_call():
    """capi.bind_layer (arguments marshalled once) issues the same call as moe_mlp_decode."""
    d = device_workload("flash_decode_t16")
    ref = d.run(False)[0]
    out = torch.empty_like(ref)
    call = capi.bind_layer(d.cfg, d.weights, d.x, out)
    for _ in range(3):
        out.fill_(0)
        call()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
