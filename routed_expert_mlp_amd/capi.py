"""ctypes binding of the C ABI in include/moe_mlp.h (argument marshalling only).

Every function here has the name of the C entry point it calls; it checks
dtype, shape, device and contiguity of the torch tensors it is given, passes
their device pointers and torch's current HIP stream, and raises MoeMlpError
on a non-zero status.  All computation happens in the HIP library; if the
library is missing, loading fails loudly (there is no fallback).
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libmoe_mlp.so")

OK = 0
ERR_NULL_ARG = -1
ERR_BAD_SHAPE = -2
ERR_BAD_TOPK = -3
ERR_BAD_VALUE = -4
ERR_MISALIGNED = -5
ERR_WORKSPACE_TOO_SMALL = -6
ERR_KIND_MISMATCH = -7
ERR_HIP = -8
ERR_SCRATCH_LIMIT = -9

MAX_TOP_K = 16
MAX_EXPERTS = 1024
DECODE_MAX_T = 256
NOALLOC_SCRATCH_BYTES = 64 << 20
KIND_ROUTED = 0
KIND_DENSE = 1
KIND_ROUTED_FP8 = 2
FP8_BLOCK = 128

EXPORTED = ("moe_mlp_workspace_size", "moe_mlp_decode", "moe_mlp_prefill", "moe_mlp_forward_profiled",
            "moe_mlp_stage_name", "moe_router_topk", "moe_nvfp4_dequant", "moe_nvfp4_tile_pack",
            "moe_mlp_status_string", "moe_mlp_decode_noalloc")


class MoeMlpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_mlp_status_string(status)} ({status})")


class moe_mlp_config(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("hidden", ctypes.c_int32), ("moe_intermediate", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("n_shared_experts", ctypes.c_int32),
                ("shared_intermediate", ctypes.c_int32), ("dense_intermediate", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("swiglu_limit", ctypes.c_float)]


class moe_mlp_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router_w", "router_bias", "w13_q", "w13_s", "w13_g", "w2_q", "w2_s", "w2_g",
        "shared_w13", "shared_w2", "dense_w13", "dense_w2",
        "w13_q_tiled", "w13_s_tiled", "w2_q_tiled", "w2_s_tiled",
        "w13_f8", "w13_f8_scale", "w2_f8", "w2_f8_scale")]


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"HIP library not built: {LIB_PATH} (run python -m routed_expert_mlp_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        cfgp, wp = ctypes.POINTER(moe_mlp_config), ctypes.POINTER(moe_mlp_weights)
        L.moe_mlp_workspace_size.argtypes = [cfgp, i64, ctypes.c_int, ctypes.POINTER(sz)]
        for f in (L.moe_mlp_decode, L.moe_mlp_prefill):
            f.argtypes = [cfgp, wp, vp, i64, vp, vp, vp, vp, sz, vp]
        L.moe_mlp_decode_noalloc.argtypes = [cfgp, wp, vp, i64, vp, vp, vp, vp]
        L.moe_mlp_decode_noalloc.restype = ctypes.c_int
        L.moe_mlp_forward_profiled.argtypes = [cfgp, wp, vp, i64, vp, vp, vp, vp, sz, vp, ctypes.c_int,
                                               ctypes.POINTER(vp), ctypes.c_int]
        L.moe_mlp_forward_profiled.restype = ctypes.c_int
        L.moe_mlp_stage_name.argtypes = [cfgp, i64, ctypes.c_int, ctypes.c_int]
        L.moe_mlp_stage_name.restype = ctypes.c_char_p
        L.moe_router_topk.argtypes = [cfgp, vp, vp, vp, i64, vp, vp, vp, sz, vp]
        L.moe_nvfp4_dequant.argtypes = [vp, vp, ctypes.c_float, i64, i64, vp, vp, vp]
        L.moe_nvfp4_tile_pack.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp]
        L.moe_mlp_status_string.argtypes = [ctypes.c_int]
        L.moe_mlp_status_string.restype = ctypes.c_char_p
        for n in ("moe_mlp_workspace_size", "moe_mlp_decode", "moe_mlp_prefill", "moe_router_topk",
                  "moe_nvfp4_dequant"):
            getattr(L, n).restype = ctypes.c_int
        _LIB = L
    return _LIB


def moe_mlp_status_string(status: int) -> str:
    return lib().moe_mlp_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise MoeMlpError(status, where)


# --------------------------------------------------------------------------
# Config and weights.
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Config:
    """Layer geometry; every field explicit (no defaults)."""
    kind: int
    hidden: int
    moe_intermediate: int
    num_experts: int
    top_k: int
    n_shared_experts: int
    shared_intermediate: int
    dense_intermediate: int
    routed_scaling_factor: float
    swiglu_limit: float

    def c(self) -> moe_mlp_config:
        return moe_mlp_config(*[getattr(self, f.name) for f in dataclasses.fields(self)])


@dataclasses.dataclass
class Weights:
    """Device tensors of one layer's weight contract (see include/moe_mlp.h)."""
    router_w: Optional[torch.Tensor] = None      # [E, H] f32
    router_bias: Optional[torch.Tensor] = None   # [E] f32
    w13_q: Optional[torch.Tensor] = None         # [E, 2I, H/2] u8
    w13_s: Optional[torch.Tensor] = None         # [E, 2I, H/16] u8
    w13_g: Optional[torch.Tensor] = None         # [E, 2] f32
    w2_q: Optional[torch.Tensor] = None          # [E, H, I/2] u8
    w2_s: Optional[torch.Tensor] = None          # [E, H, I/16] u8
    w2_g: Optional[torch.Tensor] = None          # [E] f32
    shared_w13: Optional[torch.Tensor] = None    # [2 Is, H] bf16
    shared_w2: Optional[torch.Tensor] = None     # [H, Is] bf16
    dense_w13: Optional[torch.Tensor] = None     # [2 Id, H] bf16
    dense_w2: Optional[torch.Tensor] = None      # [H, Id] bf16
    # optional tile-layout copies of the routed codes / scales (moe_nvfp4_tile_pack)
    w13_q_tiled: Optional[torch.Tensor] = None   # [E, 2I, H/2] u8
    w13_s_tiled: Optional[torch.Tensor] = None   # [E, 2I, H/16] u8
    w2_q_tiled: Optional[torch.Tensor] = None    # [E, H, I/2] u8
    w2_s_tiled: Optional[torch.Tensor] = None    # [E, H, I/16] u8
    # FP8 block-scaled experts (KIND_ROUTED_FP8): E4M3 bytes and fp32 128 x 128 block scales
    w13_f8: Optional[torch.Tensor] = None        # [E, 2I, H] u8
    w13_f8_scale: Optional[torch.Tensor] = None  # [E, 2I/128, H/128] f32
    w2_f8: Optional[torch.Tensor] = None         # [E, H, I] u8
    w2_f8_scale: Optional[torch.Tensor] = None   # [E, H/128, I/128] f32

    def check(self, cfg: Config) -> None:
        H, I, E = cfg.hidden, cfg.moe_intermediate, cfg.num_experts
        Is, Id = cfg.shared_intermediate, cfg.dense_intermediate
        want = {}
        B = FP8_BLOCK
        if cfg.kind == KIND_DENSE:
            want["dense_w13"] = ((2 * Id, H), torch.bfloat16)
            want["dense_w2"] = ((H, Id), torch.bfloat16)
        elif cfg.kind == KIND_ROUTED_FP8:
            want.update(router_w=((E, H), torch.float32), router_bias=((E,), torch.float32),
                        w13_f8=((E, 2 * I, H), torch.uint8), w13_f8_scale=((E, 2 * I // B, H // B), torch.float32),
                        w2_f8=((E, H, I), torch.uint8), w2_f8_scale=((E, H // B, I // B), torch.float32))
            if cfg.n_shared_experts:
                want["shared_w13"] = ((2 * Is, H), torch.bfloat16)
                want["shared_w2"] = ((H, Is), torch.bfloat16)
        else:
            want.update(router_w=((E, H), torch.float32), router_bias=((E,), torch.float32),
                        w13_q=((E, 2 * I, H // 2), torch.uint8), w13_s=((E, 2 * I, H // 16), torch.uint8),
                        w13_g=((E, 2), torch.float32), w2_q=((E, H, I // 2), torch.uint8),
                        w2_s=((E, H, I // 16), torch.uint8), w2_g=((E,), torch.float32),
                        w13_q_tiled=((E, 2 * I, H // 2), torch.uint8),
                        w13_s_tiled=((E, 2 * I, H // 16), torch.uint8),
                        w2_q_tiled=((E, H, I // 2), torch.uint8), w2_s_tiled=((E, H, I // 16), torch.uint8))
            if cfg.n_shared_experts:
                want["shared_w13"] = ((2 * Is, H), torch.bfloat16)
                want["shared_w2"] = ((H, Is), torch.bfloat16)
        for name, (shape, dt) in want.items():
            t = getattr(self, name)
            if t is None:
                continue      # the library reports the missing tensor (KIND_MISMATCH)
            _check_tensor(t, name, shape, dt)

    def c(self) -> moe_mlp_weights:
        return moe_mlp_weights(*[_ptr(getattr(self, f.name)) for f in dataclasses.fields(self)])


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_tensor(t: torch.Tensor, name: str, shape, dtype) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# --------------------------------------------------------------------------
# Entry points.
# --------------------------------------------------------------------------

def moe_mlp_workspace_size(cfg: Config, T: int, prefill: bool) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_mlp_workspace_size(ctypes.byref(cfg.c()), int(T), int(bool(prefill)), ctypes.byref(n)),
           "moe_mlp_workspace_size")
    return n.value


def workspace(cfg: Config, T: int, prefill: bool, device="cuda") -> torch.Tensor:
    """A workspace tensor of the size the library asks for (allocated by torch)."""
    return torch.empty(max(1, moe_mlp_workspace_size(cfg, T, prefill)), dtype=torch.uint8, device=device)


def _layer(fn_name: str, cfg: Config, w: Weights, x: torch.Tensor, out: torch.Tensor,
           ids_out=None, w_out=None, ws: Optional[torch.Tensor] = None, stream=None, prefill=False) -> None:
    T = x.shape[0] if x.dim() == 2 else -1
    _check_tensor(x, "x", (T, cfg.hidden), torch.bfloat16)
    _check_tensor(out, "out", (T, cfg.hidden), torch.bfloat16)
    if ids_out is not None:
        _check_tensor(ids_out, "ids_out", (T, cfg.top_k), torch.int32)
    if w_out is not None:
        _check_tensor(w_out, "w_out", (T, cfg.top_k), torch.float32)
    w.check(cfg)
    if ws is None:
        ws = workspace(cfg, T, prefill, x.device)
    _check_tensor(ws, "workspace", None, torch.uint8)
    st = getattr(lib(), fn_name)(ctypes.byref(cfg.c()), ctypes.byref(w.c()), x.data_ptr(), T, out.data_ptr(),
                                 _ptr(ids_out), _ptr(w_out), ws.data_ptr(), ws.numel(), _stream(stream))
    _check(st, fn_name)


def bind_layer(cfg: Config, w: Weights, x: torch.Tensor, out: torch.Tensor, ids_out=None, w_out=None,
               ws: Optional[torch.Tensor] = None, stream=None, prefill=False):
    """Check and marshal the arguments of one moe_mlp_decode / moe_mlp_prefill call once and return
    a zero-argument callable that issues it again on the same buffers (for tight loops: the C call
    with prebuilt ctypes arguments).  The callable raises MoeMlpError on a non-zero status."""
    T = x.shape[0] if x.dim() == 2 else -1
    _check_tensor(x, "x", (T, cfg.hidden), torch.bfloat16)
    _check_tensor(out, "out", (T, cfg.hidden), torch.bfloat16)
    if ids_out is not None:
        _check_tensor(ids_out, "ids_out", (T, cfg.top_k), torch.int32)
    if w_out is not None:
        _check_tensor(w_out, "w_out", (T, cfg.top_k), torch.float32)
    w.check(cfg)
    if ws is None:
        ws = workspace(cfg, T, prefill, x.device)
    _check_tensor(ws, "workspace", None, torch.uint8)
    name = "moe_mlp_prefill" if prefill else "moe_mlp_decode"
    fn = getattr(lib(), name)
    c_cfg, c_w = cfg.c(), w.c()
    args = (ctypes.byref(c_cfg), ctypes.byref(c_w), x.data_ptr(), T, out.data_ptr(), _ptr(ids_out), _ptr(w_out),
            ws.data_ptr(), ws.numel(), _stream(stream))
    keep = (c_cfg, c_w, x, out, ids_out, w_out, ws, w)     # the buffers outlive the callable

    def call():
        st = fn(*args)
        if st:
            _check(st, name)
    call.keep = keep
    return call


def moe_mlp_decode(cfg: Config, w: Weights, x: torch.Tensor, out: torch.Tensor, ids_out=None, w_out=None,
                   ws: Optional[torch.Tensor] = None, stream=None) -> None:
    _layer("moe_mlp_decode", cfg, w, x, out, ids_out, w_out, ws, stream, prefill=False)


def moe_mlp_decode_noalloc(cfg: Config, w: Weights, x: torch.Tensor, out: torch.Tensor, ids_out=None,
                           w_out=None, stream=None) -> None:
    """moe_mlp_decode with the library's own per-device scratch array as the workspace
    (no allocation by the library or here)."""
    T = x.shape[0] if x.dim() == 2 else -1
    _check_tensor(x, "x", (T, cfg.hidden), torch.bfloat16)
    _check_tensor(out, "out", (T, cfg.hidden), torch.bfloat16)
    if ids_out is not None:
        _check_tensor(ids_out, "ids_out", (T, cfg.top_k), torch.int32)
    if w_out is not None:
        _check_tensor(w_out, "w_out", (T, cfg.top_k), torch.float32)
    w.check(cfg)
    st = lib().moe_mlp_decode_noalloc(ctypes.byref(cfg.c()), ctypes.byref(w.c()), x.data_ptr(), T,
                                      out.data_ptr(), _ptr(ids_out), _ptr(w_out), _stream(stream))
    _check(st, "moe_mlp_decode_noalloc")


def moe_mlp_prefill(cfg: Config, w: Weights, x: torch.Tensor, out: torch.Tensor, ids_out=None, w_out=None,
                    ws: Optional[torch.Tensor] = None, stream=None) -> None:
    _layer("moe_mlp_prefill", cfg, w, x, out, ids_out, w_out, ws, stream, prefill=True)


def moe_mlp_stage_name(cfg: Config, T: int, prefill: bool, stage: int) -> Optional[str]:
    r = lib().moe_mlp_stage_name(ctypes.byref(cfg.c()), int(T), int(bool(prefill)), int(stage))
    return None if r is None else r.decode()


def stage_names(cfg: Config, T: int, prefill: bool):
    names = []
    while True:
        n = moe_mlp_stage_name(cfg, T, prefill, len(names))
        if n is None:
            return names
        names.append(n)


def moe_mlp_forward_profiled(cfg: Config, w: Weights, x: torch.Tensor, out: torch.Tensor, prefill: bool,
                             events, ids_out=None, w_out=None, ws: Optional[torch.Tensor] = None,
                             stream=None) -> None:
    """As moe_mlp_decode / moe_mlp_prefill, with stage i's kernels bracketed by the raw
    hipEvent_t handles events[2i] (start) and events[2i+1] (stop)."""
    T = x.shape[0]
    _check_tensor(x, "x", (T, cfg.hidden), torch.bfloat16)
    _check_tensor(out, "out", (T, cfg.hidden), torch.bfloat16)
    w.check(cfg)
    if ws is None:
        ws = workspace(cfg, T, prefill, x.device)
    ev = (ctypes.c_void_p * len(events))(*events)
    st = lib().moe_mlp_forward_profiled(ctypes.byref(cfg.c()), ctypes.byref(w.c()), x.data_ptr(), T,
                                        out.data_ptr(), _ptr(ids_out), _ptr(w_out), ws.data_ptr(), ws.numel(),
                                        _stream(stream), int(bool(prefill)), ev, len(events))
    _check(st, "moe_mlp_forward_profiled")


def moe_router_topk(cfg: Config, router_w: torch.Tensor, router_bias: torch.Tensor, x: torch.Tensor,
                    ids: torch.Tensor, w: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None) -> None:
    T = x.shape[0]
    _check_tensor(router_w, "router_w", (cfg.num_experts, cfg.hidden), torch.float32)
    _check_tensor(router_bias, "router_bias", (cfg.num_experts,), torch.float32)
    _check_tensor(x, "x", (T, cfg.hidden), torch.bfloat16)
    _check_tensor(ids, "ids", (T, cfg.top_k), torch.int32)
    _check_tensor(w, "w", (T, cfg.top_k), torch.float32)
    if ws is None:
        ws = workspace(cfg, T, True, x.device)
    st = lib().moe_router_topk(ctypes.byref(cfg.c()), router_w.data_ptr(), router_bias.data_ptr(), x.data_ptr(),
                               T, ids.data_ptr(), w.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
    _check(st, "moe_router_topk")


def moe_nvfp4_dequant(q: torch.Tensor, s: torch.Tensor, global_scale: float, out_f32=None, out_bf16=None,
                      stream=None) -> None:
    rows, half = q.shape
    cols = 2 * half
    _check_tensor(q, "q", (rows, half), torch.uint8)
    _check_tensor(s, "s", (rows, cols // 16), torch.uint8)
    if out_f32 is not None:
        _check_tensor(out_f32, "out_f32", (rows, cols), torch.float32)
    if out_bf16 is not None:
        _check_tensor(out_bf16, "out_bf16", (rows, cols), torch.bfloat16)
    st = lib().moe_nvfp4_dequant(q.data_ptr(), s.data_ptr(), float(global_scale), rows, cols, _ptr(out_f32),
                                 _ptr(out_bf16), _stream(stream))
    _check(st, "moe_nvfp4_dequant")


def moe_nvfp4_tile_pack(q: torch.Tensor, s: torch.Tensor, q_tiled=None, s_tiled=None, stream=None):
    """Row-major NVFP4 codes q [.., rows, cols/2] and scales s [.., rows, cols/16]
    (u8, any number of leading matrix dims) -> (q_tiled, s_tiled) of the same
    shapes in the grouped GEMM's tile layout (see include/moe_mlp.h)."""
    rows, half = q.shape[-2], q.shape[-1]
    cols = 2 * half
    mats = q.numel() // max(1, rows * half)
    _check_tensor(q, "q", tuple(q.shape), torch.uint8)
    _check_tensor(s, "s", tuple(q.shape[:-1]) + (cols // 16,), torch.uint8)
    q_tiled = torch.empty_like(q) if q_tiled is None else q_tiled
    s_tiled = torch.empty_like(s) if s_tiled is None else s_tiled
    _check_tensor(q_tiled, "q_tiled", tuple(q.shape), torch.uint8)
    _check_tensor(s_tiled, "s_tiled", tuple(s.shape), torch.uint8)
    st = lib().moe_nvfp4_tile_pack(q.data_ptr(), s.data_ptr(), mats, rows, cols, q_tiled.data_ptr(),
                                   s_tiled.data_ptr(), _stream(stream))
    _check(st, "moe_nvfp4_tile_pack")
    return q_tiled, s_tiled


def _tileable(q: torch.Tensor) -> bool:
    return q.shape[-2] % 32 == 0 and (2 * q.shape[-1]) % 256 == 0


def with_tiled_weights(w: Weights, stream=None, drop_row_major_codes: bool = False) -> Weights:
    """A copy of w whose routed codes and scales also come in the tile layout,
    for each projection whose shape has one (rows a multiple of 32, columns a
    multiple of 256); allocated by torch, the row-major tensors are shared.

    drop_row_major_codes: the copy keeps no reference to the row-major codes
    of each packed projection whose reduction is at least 512 (w13_q / w2_q
    become None): every kernel then reads the tile-layout codes, and the codes
    are resident once (the row-major scales stay: the decode kernels read
    them).  The caller frees the row-major codes by dropping its own
    references."""
    q13 = s13 = q2 = s2 = None
    rq13, rq2 = w.w13_q, w.w2_q
    if _tileable(w.w13_q):
        q13, s13 = moe_nvfp4_tile_pack(w.w13_q, w.w13_s, stream=stream)
        if drop_row_major_codes and 2 * w.w13_q.shape[-1] >= 512:
            rq13 = None
    if _tileable(w.w2_q):
        q2, s2 = moe_nvfp4_tile_pack(w.w2_q, w.w2_s, stream=stream)
        if drop_row_major_codes and 2 * w.w2_q.shape[-1] >= 512:
            rq2 = None
    return dataclasses.replace(w, w13_q=rq13, w2_q=rq2, w13_q_tiled=q13, w13_s_tiled=s13, w2_q_tiled=q2,
                               w2_s_tiled=s2)
