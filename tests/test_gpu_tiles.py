"""GPU: the tile layout of the routed NVFP4 weights (moe_nvfp4_tile_pack) and
the grouped GEMM reading it.

The layout is restated here in numpy from its definition in include/moe_mlp.h
and compared byte for byte with the library's pack.  A layer given the tiled
copies must produce bitwise the output (and ids, weights) it produces from
the row-major arrays alone: the tile kernel loads the same bytes into the same
LDS positions, so nothing after the loads differs.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, DeviceRouted, bf16_host_bits, device_workload, say
from inputs import RoutedInputs
from routed_expert_mlp_amd import capi

pytestmark = pytest.mark.gpu


def _z(i):
    return ((i >> 1) & 3) ^ ((i >> 3) & 1)


def tiled_codes(q):
    """q [mats, rows, cols/2] -> the tile layout: per (matrix, 16-row group,
    128-column unit) 64 pieces of 16 bytes, piece L = row 16r + L/4, bytes
    64u + 16((L % 4) ^ z(L / 4)) .. +15."""
    mats, rows, half = q.shape
    src = q.reshape(mats, rows // 16, 16, half // 64, 64)
    out = np.empty((mats, rows // 16, half // 64, 64, 16), np.uint8)
    for L in range(64):
        piece = (L % 4) ^ _z(L // 4)
        out[:, :, :, L, :] = src[:, :, L // 4, :, 16 * piece:16 * piece + 16]
    return out.reshape(q.shape)


def tiled_scales(s):
    """s [mats, rows, cols/16] -> per (matrix, 32-row group, 256-column unit)
    a 512-byte block, stage-major: bytes 128 t + 4 l .. +3 = scale bytes
    16v + 4t .. +3 of row 32r + l."""
    mats, rows, n = s.shape
    g = s.reshape(mats, rows // 32, 32, n // 16, 4, 4)          # m, r, l, v, t, byte
    return g.transpose(0, 1, 3, 4, 2, 5).reshape(s.shape).copy()   # m, r, v, t, l, byte


@pytest.mark.parametrize("mats,rows,cols", [(3, 96, 768), (1, 32, 256), (2, 64, 1024)])
def test_tile_pack_matches_layout(mats, rows, cols):
    say(f"[case] tile pack mats={mats} rows={rows} cols={cols}")
    g = np.random.default_rng(7)
    q = g.integers(0, 256, (mats, rows, cols // 2), dtype=np.uint8)
    s = g.integers(0, 256, (mats, rows, cols // 16), dtype=np.uint8)
    qt, st = capi.moe_nvfp4_tile_pack(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(qt.cpu().numpy(), tiled_codes(q))
    assert np.array_equal(st.cpu().numpy(), tiled_scales(s))


def _run_both(d: DeviceRouted, what: str, prefill=True, drop=False):
    out0, ids0, w0 = d.run(prefill)
    plain = d.weights
    d.weights = capi.with_tiled_weights(plain, drop_row_major_codes=drop)
    if drop:
        say(f"[case] row-major codes left out: w13_q {d.weights.w13_q is None}, w2_q {d.weights.w2_q is None}")
    try:
        out1, ids1, w1 = d.run(prefill)
    finally:
        d.weights = plain
    torch.cuda.synchronize()
    assert torch.equal(ids0, ids1) and torch.equal(w0, w1), what
    a, b = bf16_host_bits(out0), bf16_host_bits(out1)
    n_diff = int((a != b).sum())
    say(f"[parity] tiled vs row-major weights, {what}: {n_diff} of {a.size} outputs differ")
    assert n_diff == 0


# the tile-kernel shapes of the routed grouped-GEMM tests (both projections,
# one of them, neither) and the full-size prefill workload
TILE_CASES = [dict(T=600, H=512, I=512, E=16, K=4, Is=256),
              dict(T=300, H=768, I=512, E=8, K=2, Is=96),
              dict(T=200, H=1024, I=160, E=8, K=2, Is=96),
              dict(T=150, H=256, I=512, E=8, K=2, Is=64),
              dict(T=100, H=256, I=256, E=4, K=2, Is=64)]


@pytest.mark.parametrize("overrides", TILE_CASES, ids=[f"T{o['T']}_H{o['H']}_I{o['I']}" for o in TILE_CASES])
def test_tiled_weights_bitwise(overrides):
    w = synth.workload("ragged_prefill", **overrides)
    say(f"[case] tiled weights T={w.T} H={w.H} I={w.I} E={w.E} K={w.K}")
    _run_both(DeviceRouted(RoutedInputs(w)), str(overrides))


def test_tiled_weights_bitwise_full_size():
    say("[case] tiled weights prefill_t4096")
    _run_both(device_workload("prefill_t4096"), "prefill_t4096")


@pytest.mark.parametrize("T", [1, 16, 64])
def test_tiled_weights_decode_bitwise(T):
    """Decode reads the tiled copies in the down projection of the expert-GEMV
    form (below 64 tokens) and in both projections from 64 tokens on
    (grouped-GEMM form): bitwise the same either way."""
    w = synth.workload("ragged_decode", T=T, H=512, I=512, E=16, K=4, Is=128)
    say(f"[case] tiled weights, decode T={w.T} H={w.H} I={w.I} E={w.E} K={w.K}")
    _run_both(DeviceRouted(RoutedInputs(w)), f"decode T={T}", prefill=False)


@pytest.mark.parametrize("T,E,K", [(64, 16, 16), (48, 40, 16)])
def test_tiled_weights_split_passes_bitwise(T, E, K):
    """Batches whose routed gate/up splits the long tiles into one workgroup
    per 32-row pass (decode at 64 tokens, prefill below), on both weight
    layouts."""
    w = synth.workload("ragged_decode", T=T, H=512, I=512, E=E, K=K, Is=128)
    say(f"[case] tiled weights, {'prefill' if T < 64 else 'decode'} T={w.T} H={w.H} I={w.I} E={w.E} K={w.K}")
    _run_both(DeviceRouted(RoutedInputs(w)), f"T={T} E={E} K={K}", prefill=T < 64)


# One resident copy of the codes: the row-major codes left out, every kernel
# (one-token and few-token decode, GEMV decode, grouped GEMM) reads the
# tile-layout codes; the bytes and the arithmetic are the same, so the results
# are bitwise those of the row-major run.  H=512, I=256 leaves out only the
# gate/up codes (the down reduction is below 512), so the two layouts mix.
ONE_COPY = [dict(T=1, H=512, I=512), dict(T=3, H=512, I=512), dict(T=16, H=512, I=512),
            dict(T=40, H=512, I=512), dict(T=64, H=512, I=512), dict(T=16, H=512, I=256),
            dict(T=1, H=512, I=256)]


@pytest.mark.parametrize("o", ONE_COPY, ids=[f"T{o['T']}_H{o['H']}_I{o['I']}" for o in ONE_COPY])
def test_tiled_codes_only_decode_bitwise(o):
    w = synth.workload("ragged_decode", T=o["T"], H=o["H"], I=o["I"], E=16, K=4, Is=128)
    say(f"[case] tile-layout codes only, decode T={w.T} H={w.H} I={w.I} E={w.E} K={w.K}")
    _run_both(DeviceRouted(RoutedInputs(w)), f"codes tiled only, decode T={o['T']}", prefill=False, drop=True)


@pytest.mark.parametrize("name,prefill", [("flash_decode_t1", False), ("flash_decode_t16", False),
                                          ("prefill_t4096", True)])
def test_tiled_codes_only_full_size_bitwise(name, prefill):
    say(f"[case] tile-layout codes only, {name}")
    _run_both(device_workload(name), f"codes tiled only, {name}", prefill=prefill, drop=True)
