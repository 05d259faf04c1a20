"""fp64 CPU oracle of the GLM-5.3-Flash routed MoE MLP -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path never calls it; it shares no code with
the HIP library (no kernels, headers, tables or helpers), and imports nothing
from it.

This is the plain definition of what the layer computes, written out in
float64 with NumPy, one step per function, in the order the pages give:

  Module glm5next_mlp (GLM-5.3-Flash MLP production surface), section
  "The stack this layer runs": a ROUTED layer projects the token onto fp32
  router logits, picks K experts by top-k, runs each chosen expert's NVFP4
  gate/up projection, clamped SwiGLU and NVFP4 down projection, runs the BF16
  shared expert (same shape) on every token, and sums the weighted routed
  outputs with the shared output; a DENSE layer is one BF16 gate/up, clamped
  SwiGLU, down FFN;

and the rules of the same page's section "Traps this module exists to hold",
written here as formulas (L = swiglu_limit, a required config value):
  * h = silu(min(g, L)) * clip(u, -L, L): g is clipped from above only;
  * experts are ranked by s + b (s the sigmoid score, b the correction
    bias), and the weight of a chosen expert is built from s alone;
  * w_k = rsf * s_k / sum_j s_j over the K chosen of all E experts; rsf
    enters only through w, and the shared output is added with factor 1.
  Constants, KERNEL_MAX_TOP_K: K <= 16.

Number formats (not on the pages; public specifications):
  * NVFP4 element = FP4 E2M1 of the OCP Microscaling Formats (MX) v1.0 spec:
    1 sign, 2 exponent (bias 1), 1 mantissa bit, no Inf/NaN.
  * NVFP4 block scale = E4M3 of the OCP 8-bit Floating Point (OFP8) spec,
    one per 16 consecutive elements along the input dimension; bias 7,
    subnormals, 0x7F/0xFF NaN, no Inf.
  * one fp32 global scale per (expert, projection), multiplied after the
    dot product.

Readings where the pages are silent:
  * the correction bias is added to the sigmoid score (score space);
  * no expert groups: one flat top-K over all E experts;
  * ids are in descending biased-score order, exact ties to the lower index;
  * weights: renormalise over the chosen K, then multiply by rsf, no epsilon;
  * SwiGLU = silu(min(g, L)) * min(max(u, -L), L), silu(z) = z / (1 + e^-z);
  * "contract" mode rounds h (routed and shared) to bf16 before the down
    projection and the output to bf16 once after the fp64 combine (W4A16:
    16-bit activations into every weight product); "exact" mode rounds
    neither;
  * NVFP4 layout: [out, in] row-major, low nibble = even column, unswizzled
    scales [out, in/16].
  * FP8 experts (the second checkpoint format of the TensorRT-LLM
    GLM-5.3-Flash page, "the official FP8 checkpoint", which gives no
    layout): E4M3 ("fn") bytes [out, in] row-major and one fp32 scale per
    128 x 128 block [out/128, in/128], multiplied; no global scale; bf16
    activations (W8A16).

Parity pins: every function here is pinned by a CPU test against hand
tables, closed forms, brute force or a library routine (tests/test_oracle_*).
The whole-layer output beyond those decompositions is "parity unpinned": the
pages print no worked layer output.
"""

from __future__ import annotations

import numpy as np

F64 = np.float64

# --------------------------------------------------------------------------
# Number formats.
# --------------------------------------------------------------------------


def decode_e2m1(codes) -> np.ndarray:
    """FP4 E2M1 code (0..15) -> value, from the bit fields.

    exponent field 0: subnormal, value = 0.5 * m; otherwise
    2^(e-1) * (1 + m/2).  Bit 3 is the sign (code 8 is -0.0).
    """
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(sign == 1, -mag, mag).astype(F64)


def decode_e4m3(b) -> np.ndarray:
    """OCP E4M3 ("fn") byte -> value.

    exponent field 0: 2^-6 * m/8; otherwise 2^(e-7) * (1 + m/8);
    e == 15 and m == 7 is NaN.  Bit 7 is the sign.
    """
    b = np.asarray(b).astype(np.int64)
    sign = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag).astype(F64)


def decode_bf16(bits) -> np.ndarray:
    """bf16 bit pattern -> value: the top 16 bits of an IEEE binary32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(F64)


_BF16_MAX = np.ldexp(255.0, 120)          # 0x7F7F = (2 - 2^-7) * 2^127


def round_bf16(a) -> np.ndarray:
    """Round float64 to the nearest bf16 value, ties to even (as float64).

    bf16 keeps 8 significant bits; the smallest normal is 2^-126 and the
    subnormal spacing is 2^-133.  Values past the largest finite bf16 round
    to +-inf.
    """
    a = np.asarray(a, dtype=F64)
    _, ex = np.frexp(a)                       # a = frac * 2^ex, |frac| in [0.5, 1)
    q = np.maximum(ex, -125) - 8              # exponent of the bf16 spacing at a
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)
    return np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, a), r)


def unpack_codes(q) -> np.ndarray:
    """[rows, cols/2] bytes -> [rows, cols] 4-bit codes; low nibble = even column."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = q & 0x0F
    out[..., 1::2] = q >> 4
    return out


def dequant_nvfp4(q, s) -> np.ndarray:
    """NVFP4 weight W[r, c] = E2M1(code[r, c]) * E4M3(scale[r, c // 16]), exact in fp64.

    The per-tensor global scale is not part of W: it multiplies the dot
    product (nvfp4_linear).
    """
    codes = unpack_codes(q)
    rows, cols = codes.shape
    s = np.asarray(s, dtype=np.uint8)
    if s.shape != (rows, cols // 16) or cols % 16:
        raise ValueError("scale shape must be [rows, cols/16]")
    vals = decode_e2m1(np.arange(16))[codes]
    scl = np.repeat(decode_e4m3(s), 16, axis=1)
    return vals * scl


def nvfp4_linear(x, q, s, g) -> np.ndarray:
    """y[n, r] = g * sum_c x[n, c] * W[r, c] for an NVFP4 weight (W4A16 projection)."""
    W = dequant_nvfp4(q, s)
    return float(g) * (np.asarray(x, dtype=F64) @ W.T)


FP8_BLOCK = 128


def dequant_fp8_block(q, s, block: int = FP8_BLOCK) -> np.ndarray:
    """FP8 block-scaled weight W[r, c] = E4M3(q[r, c]) * S[r // 128, c // 128], exact in fp64.

    q [rows, cols] holds OCP E4M3 ("fn") bytes; S [rows/128, cols/128] one
    fp32 scale per 128 x 128 block, multiplied (see the FP8 reading in the
    module docstring).
    """
    q = np.asarray(q, dtype=np.uint8)
    rows, cols = q.shape
    s = np.asarray(s, dtype=F64)
    nb = (-(-rows // block), -(-cols // block))
    if s.shape != nb:
        raise ValueError(f"scale shape must be {nb}")
    vals = decode_e4m3(np.arange(256))[q]
    scl = np.repeat(np.repeat(s, block, axis=0)[:rows], block, axis=1)[:, :cols]
    return vals * scl


def fp8_linear(x, q, s) -> np.ndarray:
    """y[n, r] = sum_c x[n, c] * W[r, c] for an FP8 block-scaled weight (W8A16 projection)."""
    return np.asarray(x, dtype=F64) @ dequant_fp8_block(q, s).T


def bf16_linear(x, w_bits) -> np.ndarray:
    """y[n, r] = sum_c x[n, c] * W[r, c] for a bf16 weight [rows, cols]."""
    return np.asarray(x, dtype=F64) @ decode_bf16(w_bits).T


# --------------------------------------------------------------------------
# Router (Module glm5next_mlp: "The stack this layer runs" and "Traps").
# --------------------------------------------------------------------------


def router_logits(x, router_w) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * Wr[e, h]  (gate.weight -> logits)."""
    return np.asarray(x, dtype=F64) @ np.asarray(router_w, dtype=F64).T


def sigmoid(z) -> np.ndarray:
    """1 / (1 + e^-z)."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=F64)))


def select_topk(sel, k: int) -> np.ndarray:
    """Indices of the k largest values per row, largest first; ties -> lower index."""
    sel = np.asarray(sel, dtype=F64)
    order = np.argsort(-sel, axis=-1, kind="stable")
    return order[..., :k]


def route(x, router_w, router_bias, k: int, rsf: float):
    """Sigmoid router top-k.

    s = sigmoid(logits); the correction bias is added to s for SELECTION only;
    the emitted weight of a chosen expert is its unbiased score renormalised
    over the K chosen experts, then multiplied by routed_scaling_factor.

    Returns (ids [T, K] int64, weights [T, K] fp64, logits [T, E], sel [T, E]).
    """
    l = router_logits(x, router_w)
    s = sigmoid(l)
    sel = s + np.asarray(router_bias, dtype=F64)[None, :]
    ids = select_topk(sel, k)
    s_chosen = np.take_along_axis(s, ids, axis=-1)
    w = s_chosen / s_chosen.sum(axis=-1, keepdims=True) * float(rsf)
    return ids, w, l, sel


# --------------------------------------------------------------------------
# Clamped SwiGLU (Module glm5next_mlp, "Traps": asymmetric clamp).
# --------------------------------------------------------------------------


def silu(z) -> np.ndarray:
    """z / (1 + e^-z)."""
    z = np.asarray(z, dtype=F64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_clamped(g, u, limit: float) -> np.ndarray:
    """silu(min(g, L)) * min(max(u, -L), L): gate bounded above only, up both ways."""
    L = float(limit)
    return silu(np.minimum(g, L)) * np.minimum(np.maximum(u, -L), L)


# --------------------------------------------------------------------------
# Experts.
# --------------------------------------------------------------------------


def routed_expert(x, q13, s13, g13, q2, s2, g2, limit, mode="contract") -> np.ndarray:
    """One routed NVFP4 expert on rows x [n, H] -> y [n, H].

    gate/up = rows [0, I) and [I, 2I) of W13, each with its own global scale;
    h = clamped SwiGLU (bf16 in contract mode); y = g2 * (W2 . h).
    """
    W13 = dequant_nvfp4(q13, s13)
    I = W13.shape[0] // 2
    a = np.asarray(x, dtype=F64) @ W13.T
    g = float(g13[0]) * a[:, :I]
    u = float(g13[1]) * a[:, I:]
    h = swiglu_clamped(g, u, limit)
    if mode == "contract":
        h = round_bf16(h)
    return nvfp4_linear(h, q2, s2, g2)


def routed_expert_fp8(x, q13, s13, q2, s2, limit, mode="contract") -> np.ndarray:
    """One routed FP8 block-scaled expert on rows x [n, H] -> y [n, H].

    gate/up = rows [0, I) and [I, 2I) of W13 (scales over the stacked
    [2I, H] matrix); h = clamped SwiGLU (bf16 in contract mode);
    y = W2 . h.  No per-expert global scale: the block scales carry it.
    """
    W13 = dequant_fp8_block(q13, s13)
    I = W13.shape[0] // 2
    a = np.asarray(x, dtype=F64) @ W13.T
    h = swiglu_clamped(a[:, :I], a[:, I:], limit)
    if mode == "contract":
        h = round_bf16(h)
    return fp8_linear(h, q2, s2)


def bf16_mlp(x, w13_bits, w2_bits, limit, mode="contract") -> np.ndarray:
    """BF16 gate/up -> clamped SwiGLU -> BF16 down (shared expert, dense FFN).

    Returns the fp64 down-projection output (before any output rounding).
    """
    a = bf16_linear(x, w13_bits)
    n = a.shape[1] // 2
    h = swiglu_clamped(a[:, :n], a[:, n:], limit)
    if mode == "contract":
        h = round_bf16(h)
    return bf16_linear(h, w2_bits)


# --------------------------------------------------------------------------
# Layers.
# --------------------------------------------------------------------------


class RoutedWeights:
    """The routed layer's weight contract, in storage formats.

    router_w [E, H] fp32; router_bias [E] fp32; w13_g [E, 2] fp32;
    w2_g [E] fp32; shared_w13 [2 Is, H] and shared_w2 [H, Is] bf16 bits (or
    None when there is no shared expert); expert(e) -> (q13, s13, q2, s2)
    returns expert e's weights: NVFP4 codes and E4M3 scales (fmt "nvfp4"),
    or E4M3 bytes and fp32 128 x 128 block scales (fmt "fp8", which has no
    global scales: w13_g / w2_g are not used).
    """

    def __init__(self, router_w, router_bias, w13_g, w2_g, expert, shared_w13=None, shared_w2=None,
                 fmt="nvfp4"):
        if fmt not in ("nvfp4", "fp8"):
            raise ValueError(f"unknown expert format {fmt!r}")
        self.router_w = router_w
        self.router_bias = router_bias
        self.w13_g = w13_g
        self.w2_g = w2_g
        self.expert = expert
        self.shared_w13 = shared_w13
        self.shared_w2 = shared_w2
        self.fmt = fmt


def expert_rows(job):
    """One chosen expert on the rows routed to it: job = (expert source, e,
    x rows, gate/up globals, down global, limit, mode, format) -> the
    expert's output for those rows (routed_expert or routed_expert_fp8)."""
    expert, e, xr, g13, g2, limit, mode, fmt = job
    q13, s13, q2, s2 = expert(e)
    if fmt == "fp8":
        return routed_expert_fp8(xr, q13, s13, q2, s2, limit, mode)
    return routed_expert(xr, q13, s13, g13, q2, s2, g2, limit, mode)


def moe_layer(x_bits, wts: RoutedWeights, k: int, rsf: float, limit: float, mode="contract",
              tokens=None, map_fn=map):
    """Routed MoE MLP for tokens x [T, H] (bf16 bits).

    out[t] = shared(x[t]) + sum_k w[t, k] * expert_{ids[t, k]}(x[t]), summed
    over k in order, rounded to bf16 once in contract mode.  `tokens`
    restricts the computation to a subset of rows (the router still runs on
    those rows only; tokens are independent).  `map_fn(expert_rows, jobs)`
    evaluates the per-expert jobs (the builtin map by default; any map that
    returns expert_rows(job) for each job in order, e.g. a process pool's,
    gives the same result, since the experts are independent).

    Returns (out [n, H] fp64, ids [n, K], w [n, K]).
    """
    x = decode_bf16(x_bits)
    if tokens is not None:
        x = x[np.asarray(tokens)]
    n, H = x.shape
    ids, w, _, _ = route(x, wts.router_w, wts.router_bias, k, rsf)
    y = np.zeros((n, k, H), dtype=F64)
    chosen = [int(e) for e in np.unique(ids)]
    where = [np.nonzero(ids == e) for e in chosen]
    jobs = [(wts.expert, e, x[rows], wts.w13_g[e], wts.w2_g[e], limit, mode, wts.fmt)
            for e, (rows, _) in zip(chosen, where)]
    for (rows, slots), ye in zip(where, map_fn(expert_rows, jobs)):
        y[rows, slots] = ye
    acc = np.zeros((n, H), dtype=F64)
    if wts.shared_w13 is not None:
        acc = acc + bf16_mlp(x, wts.shared_w13, wts.shared_w2, limit, mode)
    for j in range(k):
        acc = acc + w[:, j:j + 1] * y[:, j]
    out = round_bf16(acc) if mode == "contract" else acc
    return out, ids, w


def dense_ffn(x_bits, w13_bits, w2_bits, limit: float, mode="contract", tokens=None) -> np.ndarray:
    """DENSE layer: out = down(clamped SwiGLU(gate/up(x))), bf16 output in contract mode."""
    x = decode_bf16(x_bits)
    if tokens is not None:
        x = x[np.asarray(tokens)]
    y = bf16_mlp(x, w13_bits, w2_bits, limit, mode)
    return round_bf16(y) if mode == "contract" else y
