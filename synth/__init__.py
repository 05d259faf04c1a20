"""Seeded synthetic inputs for the GLM-5.3-Flash routed MoE MLP.

This module only draws raw tensors in their storage formats (NVFP4 code
bytes, e4m3 scale bytes, bf16 bit patterns, fp32 arrays).  It holds none of
the layer's arithmetic: no dequantisation, no router, no SwiGLU.  Both the
CPU oracle's tests and the GPU path's tests and benchmark take their inputs
from here, so the two sides see the same bytes.

Every tensor comes from its own PCG64 stream, keyed by (seed, tensor id,
index), so one expert, one token row or one chunk of a BF16 matrix can be
regenerated on its own without drawing the rest.

Value recipe (the workload descriptions of the GLM-5.3-Flash routed MLP this
package is built for; the format definitions are the OCP MX v1.0 FP4 E2M1 and
OCP OFP8 E4M3 specifications):

* NVFP4 expert codes: every 4-bit code uniform over 0..15 (a uniform byte
  carries two independent uniform nibbles).
* e4m3 block scales: |N(0,1)| * 0.05 rounded to e4m3 (round to nearest even;
  the largest draw is far below the e4m3 maximum 448).
* global fp32 scales: 1.0.
* x: N(0,1) * x_scale, rounded to fp32 and then to bf16 (nearest even).
* router weight: fp32 N(0, 0.02^2).
* correction bias: U(-amp, amp) fp32, or +hot_value on a seeded set of hot
  experts plus U(-hot_amp, hot_amp) on the others.
* shared and dense BF16 weights: N(0, sigma^2) rounded to bf16, with
  sigma = sqrt(E[e2m1^2] * E[scale^2]) = sqrt(8.5625 * 0.0025) = 0.14631, the
  RMS of an NVFP4 expert weight under the distribution above, so a BF16
  projection sees pre-activations of the same size as a routed one.
"""

from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload",
    "encode_e4m3", "encode_bf16", "bf16_bits_to_f32",
    "expert_w13", "expert_w2", "w13_globals", "w2_globals",
    "router_weight", "router_bias", "shared_w13", "shared_w2",
    "dense_w13", "dense_w2", "x_row", "x_rows", "unit_normal_rows",
    "for_each_expert", "SHARED_SIGMA", "FP8_CODE_SIGMA", "fp8_code_table",
]

# Stream ids: one per tensor kind.  Never renumber (it changes every input).
_TID_X = 1
_TID_ROUTER_W = 2
_TID_BIAS = 3
_TID_W13_Q = 4
_TID_W13_S = 5
_TID_W2_Q = 6
_TID_W2_S = 7
_TID_SHARED_W13 = 8
_TID_SHARED_W2 = 9
_TID_DENSE_W13 = 10
_TID_DENSE_W2 = 11
_TID_HOT = 12
_TID_X_UNIT = 13
_TID_W13_F8Q = 14
_TID_W13_F8S = 15
_TID_W2_F8Q = 16
_TID_W2_F8S = 17

_ROW_CHUNK = 256          # rows per stream for the large BF16 matrices
SCALE_STD = 0.05          # e4m3 block scale = |N(0,1)| * SCALE_STD
ROUTER_STD = 0.02
SHARED_SIGMA = math.sqrt(8.5625 * SCALE_STD * SCALE_STD)   # 0.14631...


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


# --------------------------------------------------------------------------
# Storage-format encoders (inputs only; the layer never encodes).
# --------------------------------------------------------------------------

def encode_e4m3(v) -> np.ndarray:
    """Non-negative float64 -> OCP E4M3 ("fn") byte, round to nearest even.

    E4M3: bias 7, normal = 2^(e-7) * (1 + m/8), subnormal = 2^-6 * m/8,
    largest finite 0x7E = 448; values above saturate to 0x7E.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or not np.all(np.isfinite(v)):
        raise ValueError("encode_e4m3 takes finite non-negative values")
    out = np.empty(v.shape, dtype=np.int64)
    sub = v < 2.0 ** -6
    # Subnormal grid: multiples of 2^-9.  A result of 8 is the code of 2^-6.
    out[sub] = np.rint(v[sub] * 2.0 ** 9).astype(np.int64)
    vn = v[~sub]
    frac, ex = np.frexp(vn)                 # vn = frac * 2^ex, frac in [0.5, 1)
    e_unb = ex.astype(np.int64) - 1         # vn = (2 frac) * 2^e_unb
    mant = np.rint((2.0 * frac - 1.0) * 8.0).astype(np.int64)
    carry = mant == 8
    e_unb = e_unb + carry
    mant = np.where(carry, 0, mant)
    code = ((e_unb + 7) << 3) | mant
    code = np.minimum(code, 0x7E)           # saturate (0x7F is NaN)
    out[~sub] = code
    return out.astype(np.uint8)


def encode_bf16(v) -> np.ndarray:
    """float64 -> bf16 bit pattern (uint16): round to fp32, then to bf16.

    Both roundings are to nearest even.  Non-finite values are rejected.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("encode_bf16 takes finite values")
    u = v.astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit pattern -> float32 value (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


# --------------------------------------------------------------------------
# Workloads.
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes, value parameters and seed of one synthetic workload."""
    name: str
    T: int                      # tokens
    H: int                      # hidden size
    I: int                      # routed expert (moe) intermediate size
    E: int                      # routed experts, full count
    K: int                      # experts per token
    Is: int                     # shared expert intermediate (0 = no shared expert)
    seed: int
    x_scale: float
    bias_amp: float             # bias U(-bias_amp, bias_amp) on every non-hot expert
    hot_experts: int = 0        # number of hot experts (bias +hot_value)
    hot_value: float = 1.0
    rsf: float = 2.5            # routed_scaling_factor
    swiglu_limit: float = 7.0
    kind: str = "routed"        # "routed" or "dense"
    Id: int = 0                 # dense FFN intermediate (kind == "dense")
    prefill: bool = False       # which entry point the workload exercises
    fmt: str = "nvfp4"          # routed expert weights: "nvfp4" or "fp8" (128 x 128 block scales)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def expert_bytes(self) -> int:
        """Bytes of one routed expert, both projections: NVFP4 codes + e4m3 scales, or FP8
        bytes + fp32 block scales."""
        if self.fmt == "fp8":
            return 3 * self.I * self.H + 4 * 3 * (self.I // 128) * (self.H // 128)
        return 3 * self.I * self.H // 2 + 3 * self.I * self.H // 16


# x_scale sets ~1% of gate/up clamp firings; bias_amp of the GLM-Flash-sized
# decode/prefill workloads makes the bias change the selected set on ~30% of
# tokens.  Both come from oracle/calibrate.py (bisection on a calibration
# batch); the rates they achieve are checked by a CPU test.
X_SCALE_H256 = 1.1477
X_SCALE_H4096 = 0.30141
BIAS_AMP_E288_K8 = 0.004682

_BASE_FLASH = dict(H=4096, I=1536, E=288, Is=1536, x_scale=X_SCALE_H4096)

WORKLOADS: Dict[str, Workload] = {}


def _add(w: Workload) -> None:
    WORKLOADS[w.name] = w


_add(Workload("tiny_decode", T=1, H=256, I=128, E=16, K=4, Is=128, seed=1000,
              x_scale=X_SCALE_H256, bias_amp=0.1))
_add(Workload("flash_decode_t1", T=1, K=8, seed=1001, bias_amp=BIAS_AMP_E288_K8, **_BASE_FLASH))
_add(Workload("flash_decode_t16", T=16, K=8, seed=1002, bias_amp=BIAS_AMP_E288_K8, **_BASE_FLASH))
_add(Workload("flash_decode_t64", T=64, K=8, seed=1012, bias_amp=BIAS_AMP_E288_K8, **_BASE_FLASH))
_add(Workload("skewed_decode_t64_k16", T=64, K=16, seed=1003, bias_amp=0.1, hot_experts=8,
              hot_value=1.0, **_BASE_FLASH))
_add(Workload("prefill_t4096", T=4096, K=8, seed=1004, bias_amp=BIAS_AMP_E288_K8, prefill=True,
              **_BASE_FLASH))
_add(Workload("dense_prefill_t4096", T=4096, H=4096, I=1536, E=288, K=8, Is=0, seed=1005,
              x_scale=X_SCALE_H4096, bias_amp=0.0, kind="dense", Id=12288, prefill=True))
# The literal U(-0.1, 0.1) bias on the GLM-Flash-sized workloads: selection
# changes on nearly every token and expert load is far less even.
for _n in ("flash_decode_t1", "flash_decode_t16", "flash_decode_t64", "prefill_t4096"):
    _w = WORKLOADS[_n]
    _add(_w.with_(name=_n + "_literal_bias", seed=_w.seed + 100, bias_amp=0.1))


# FP8 block-scaled experts (E4M3 weights, one fp32 scale per 128 x 128
# block): the GLM-Flash shapes, and small shapes whose H and I are multiples
# of the 128-wide scale blocks but not of the GEMM tiles.
for _n in ("flash_decode_t1", "flash_decode_t16", "prefill_t4096"):
    _w = WORKLOADS[_n]
    _add(_w.with_(name=_n + "_fp8", seed=_w.seed + 200, fmt="fp8"))
_X_SCALE_H384 = X_SCALE_H256 * math.sqrt(256 / 384)
_add(Workload("tiny_decode_fp8", T=1, H=256, I=128, E=16, K=4, Is=128, seed=1200,
              x_scale=X_SCALE_H256, bias_amp=0.1, fmt="fp8"))
_add(Workload("ragged_prefill_fp8", T=700, H=384, I=256, E=8, K=2, Is=128, seed=2201,
              x_scale=_X_SCALE_H384, bias_amp=0.05, prefill=True, fmt="fp8"))
_add(Workload("ragged_decode_fp8", T=40, H=384, I=256, E=8, K=2, Is=128, seed=2202,
              x_scale=_X_SCALE_H384, bias_amp=0.05, fmt="fp8"))


# Small parity workloads that still span several GEMM tiles and ragged tails:
# H = 416 and I = 160 are not multiples of the 128-wide k blocks and output
# tiles; T*K/E = 250 rows per expert crosses the 128-row M tiles.
_X_SCALE_H416 = X_SCALE_H256 * math.sqrt(256 / 416)
_add(Workload("ragged_prefill", T=1000, H=416, I=160, E=8, K=2, Is=96, seed=2001,
              x_scale=_X_SCALE_H416, bias_amp=0.05, prefill=True))
_add(Workload("ragged_decode", T=200, H=416, I=160, E=8, K=2, Is=96, seed=2002,
              x_scale=_X_SCALE_H416, bias_amp=0.05))
_add(Workload("ragged_dense_prefill", T=300, H=416, I=0, E=0, K=0, Is=0, seed=2003,
              x_scale=_X_SCALE_H416, bias_amp=0.0, kind="dense", Id=160, prefill=True))


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w


# --------------------------------------------------------------------------
# Routed experts (NVFP4: codes [rows, cols/2] u8, scales [rows, cols/16] e4m3).
# --------------------------------------------------------------------------

def _nvfp4_matrix(seed: int, tid_q: int, tid_s: int, e: int, rows: int, cols: int):
    q = _rng(seed, tid_q, e).integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    s = encode_e4m3(np.abs(_rng(seed, tid_s, e).standard_normal((rows, cols // 16))) * SCALE_STD)
    return q, s


# FP8 expert weights: the E4M3 byte of each weight is one of the 256
# equiprobable quantiles of N(0, FP8_CODE_SIGMA^2) (rounded to E4M3), picked
# by a uniform byte, so a 128 x 128 block spans most of the E4M3 range as a
# max-scaled block would; each block's fp32 scale is
# (SHARED_SIGMA / FP8_CODE_SIGMA) * U(0.5, 1.5), which keeps the RMS weight
# near that of an NVFP4 expert.
FP8_CODE_SIGMA = 64.0
_FP8_TABLE: Optional[np.ndarray] = None


def fp8_code_table() -> np.ndarray:
    global _FP8_TABLE
    if _FP8_TABLE is None:
        from statistics import NormalDist
        v = np.array([NormalDist().inv_cdf((i + 0.5) / 256.0) for i in range(256)]) * FP8_CODE_SIGMA
        _FP8_TABLE = (encode_e4m3(np.abs(v)) | np.where(v < 0, 0x80, 0).astype(np.uint8)).astype(np.uint8)
    return _FP8_TABLE


def _fp8_matrix(seed: int, tid_q: int, tid_s: int, e: int, rows: int, cols: int):
    if rows % 128 or cols % 128:
        raise ValueError("FP8 experts need rows and cols that are multiples of 128")
    q = fp8_code_table()[_rng(seed, tid_q, e).integers(0, 256, size=(rows, cols), dtype=np.uint8)]
    s = (SHARED_SIGMA / FP8_CODE_SIGMA) * (0.5 + _rng(seed, tid_s, e).random((rows // 128, cols // 128)))
    return q, s.astype(np.float32)


def expert_w13(w: Workload, e: int) -> Tuple[np.ndarray, np.ndarray]:
    """Gate/up of expert e: rows [0, I) gate, [I, 2I) up; cols = H.  NVFP4 (codes, e4m3
    scales) or FP8 (e4m3 bytes, fp32 128 x 128 block scales) by w.fmt."""
    if w.fmt == "fp8":
        return _fp8_matrix(w.seed, _TID_W13_F8Q, _TID_W13_F8S, e, 2 * w.I, w.H)
    return _nvfp4_matrix(w.seed, _TID_W13_Q, _TID_W13_S, e, 2 * w.I, w.H)


def expert_w2(w: Workload, e: int) -> Tuple[np.ndarray, np.ndarray]:
    """Down projection of expert e: rows = H, cols = I (format by w.fmt)."""
    if w.fmt == "fp8":
        return _fp8_matrix(w.seed, _TID_W2_F8Q, _TID_W2_F8S, e, w.H, w.I)
    return _nvfp4_matrix(w.seed, _TID_W2_Q, _TID_W2_S, e, w.H, w.I)


def w13_globals(w: Workload) -> np.ndarray:
    return np.ones((w.E, 2), dtype=np.float32)


def w2_globals(w: Workload) -> np.ndarray:
    return np.ones((w.E,), dtype=np.float32)


def for_each_expert(w: Workload, fn, experts=None, threads: Optional[int] = None) -> None:
    """Call fn(e, q13, s13, q2, s2) for each expert, generating in a thread pool.

    fn is called from the calling thread, in expert order.
    """
    experts = list(range(w.E)) if experts is None else list(experts)
    threads = threads or min(16, os.cpu_count() or 4)

    def gen(e):
        return (e,) + expert_w13(w, e) + expert_w2(w, e)

    with _cf.ThreadPoolExecutor(threads) as ex:
        window = []
        it = iter(experts)
        for e in it:
            window.append(ex.submit(gen, e))
            if len(window) >= 2 * threads:
                fn(*window.pop(0).result())
        for f in window:
            fn(*f.result())


# --------------------------------------------------------------------------
# Router.
# --------------------------------------------------------------------------

def router_weight(w: Workload) -> np.ndarray:
    """[E, H] fp32, N(0, 0.02^2)."""
    return (_rng(w.seed, _TID_ROUTER_W).standard_normal((w.E, w.H)) * ROUTER_STD).astype(np.float32)


def hot_expert_ids(w: Workload) -> np.ndarray:
    if w.hot_experts == 0:
        return np.zeros((0,), dtype=np.int64)
    return np.sort(_rng(w.seed, _TID_HOT).choice(w.E, size=w.hot_experts, replace=False))


def router_bias(w: Workload) -> np.ndarray:
    """[E] fp32 correction bias."""
    b = _rng(w.seed, _TID_BIAS).uniform(-1.0, 1.0, size=w.E) * w.bias_amp
    hot = hot_expert_ids(w)
    if hot.size:
        b[hot] = w.hot_value
    return b.astype(np.float32)


# --------------------------------------------------------------------------
# BF16 matrices (shared expert, dense FFN), generated in 256-row chunks.
# --------------------------------------------------------------------------

def _bf16_matrix(seed: int, tid: int, rows: int, cols: int) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint16)
    for c0 in range(0, rows, _ROW_CHUNK):
        c1 = min(rows, c0 + _ROW_CHUNK)
        g = _rng(seed, tid, c0 // _ROW_CHUNK)
        out[c0:c1] = encode_bf16(g.standard_normal((c1 - c0, cols)) * SHARED_SIGMA)
    return out


def shared_w13(w: Workload) -> np.ndarray:
    """[2*Is, H] bf16 bits: gate rows then up rows."""
    return _bf16_matrix(w.seed, _TID_SHARED_W13, 2 * w.Is, w.H)


def shared_w2(w: Workload) -> np.ndarray:
    """[H, Is] bf16 bits."""
    return _bf16_matrix(w.seed, _TID_SHARED_W2, w.H, w.Is)


def dense_w13(w: Workload) -> np.ndarray:
    """[2*Id, H] bf16 bits: gate rows then up rows."""
    return _bf16_matrix(w.seed, _TID_DENSE_W13, 2 * w.Id, w.H)


def dense_w2(w: Workload) -> np.ndarray:
    """[H, Id] bf16 bits."""
    return _bf16_matrix(w.seed, _TID_DENSE_W2, w.H, w.Id)


# --------------------------------------------------------------------------
# Activations.
# --------------------------------------------------------------------------

def x_row(w: Workload, t: int, attempt: int = 0) -> np.ndarray:
    """Token t's [H] bf16 bits; `attempt` selects a redraw of the same token."""
    g = _rng(w.seed, _TID_X, t, attempt)
    return encode_bf16(g.standard_normal(w.H) * w.x_scale)


def x_rows(w: Workload, T: Optional[int] = None, attempts=None) -> np.ndarray:
    """[T, H] bf16 bits (attempts: optional per-token redraw counters)."""
    T = w.T if T is None else T
    out = np.empty((T, w.H), dtype=np.uint16)
    for t in range(T):
        out[t] = x_row(w, t, 0 if attempts is None else int(attempts[t]))
    return out


def unit_normal_rows(seed: int, T: int, H: int) -> np.ndarray:
    """[T, H] float64 N(0,1) rows, unrounded (calibration batches)."""
    return _rng(seed, _TID_X_UNIT).standard_normal((T, H))
