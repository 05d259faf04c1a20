// Decode projections: bandwidth-bound GEMVs over the touched experts' rows.
//
// "Module glm5next_mlp", Constants, W4A16_GEMV_MODULE: every routed-expert
// projection at decode is M=1, and a tile GEMM there ran 26x below the
// memory roofline; the decode kernel must stream the weights.  Here each
// wavefront owns a few weight rows and its 64 lanes read consecutive 16-byte
// chunks of every row (one coalesced 1 KB load per row per instruction).  An
// NVFP4 chunk is 32 codes = two E4M3 blocks: the codes are decoded to bf16
// pairs in registers and dot2-accumulated against the bf16 activations per
// 16-block, and each block sum is scaled by its E4M3 scale in fp32.  A BF16
// chunk is 8 weights (4 dot2).  The tokens routed to one expert share each
// loaded chunk (up to TC at a time).
//
// Gate/up mode computes the gate row j and the up row I+j of the same
// expert in one wavefront and applies the asymmetric clamped SwiGLU ("Traps":
// gate bounded above only, up both ways) before storing h in bf16.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int GEMV_TC = 4;   // tokens per pass over a wavefront's rows (default)

enum GemvMode { GEMV_GATEUP = 0, GEMV_DOWN_F32 = 1, GEMV_DOWN_BF16 = 2 };

struct GemvArgs {
  // weights: NVFP4 (codes + E4M3 scales, routed: expert-major) or BF16
  const uint8_t* wq;
  const uint8_t* ws;
  const uint16_t* wb;
  int64_t stride_q;      // bytes of codes per expert
  int64_t stride_s;      // bytes of scales per expert
  const float* gscale;   // routed globals: gate/up [E,2] or down [E]; null = 1
  int half_rows;         // gate/up: I (rows j and I+j); down: number of rows
  int cols;              // input length (H for gate/up, I for down)
  // token groups: routed = per-expert slot lists; null n_groups = one group of T tokens
  const int32_t* n_groups;
  const int32_t* g_expert;
  const int32_t* g_count;
  const int32_t* g_offset;
  const int32_t* g_slots;
  int T;
  int K;                 // slot -> token = slot / K for the routed gate/up input
  const uint16_t* in;    // input rows (bf16), row length `cols`
  void* out;             // gate/up: bf16 [.., half_rows]; down: fp32 or bf16 [.., half_rows]
  float limit;
  int sorted_out;        // routed gate/up: output row = the slot's position in the group lists
};

// One 16-byte chunk of an NVFP4 row against one token's 32 activations.
__device__ __forceinline__ float nvfp4_chunk_dot(uint4 c, uint32_t sc2, const uint32_t* xp, float acc) {
  const float s0 = e4m3_to_f32<0>(sc2);
  const float s1 = e4m3_to_f32<1>(sc2);
  const float b0 = e2m1x16_dot(c.x, c.y, xp);
  const float b1 = e2m1x16_dot(c.z, c.w, xp + 8);
  acc = fmaf(b0, s0, acc);
  return fmaf(b1, s1, acc);
}

__device__ __forceinline__ float bf16_chunk_dot(uint4 w, const uint32_t* xp, float acc) {
  acc = dot2_bf16(w.x, xp[0], acc);
  acc = dot2_bf16(w.y, xp[1], acc);
  acc = dot2_bf16(w.z, xp[2], acc);
  return dot2_bf16(w.w, xp[3], acc);
}

// Grid: x = row blocks of 4*RW (gate/up: gate rows), y = token groups (routed:
// the tokens of one expert; otherwise TC consecutive tokens).
// NC > 0: every row has at most 64*NC chunks; a wavefront loads all of its
// rows' chunks (NC per lane) before any arithmetic and keeps them in
// registers for every token pass, so it waits for memory once.  NC == 0:
// rows of any length, one chunk per lane per loop iteration.
// CT: routed codes in the tile layout (nvfp4_code_off), scales row-major.
// TC: tokens per pass.  Each pass holds TC tokens' activations and sums in
// registers; with one or two tokens per expert group (decode of up to 16
// tokens) TC = 1 leaves room for more wavefronts per SIMD, which hide the
// load latency better than the shared weight chunks of a wider pass.
template <bool NVFP4, int MODE, int RW, int NC = 0, int TC = GEMV_TC, bool CT = false>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  constexpr int NR = (MODE == GEMV_GATEUP) ? 2 * RW : RW;   // weight rows per wavefront
  constexpr int XW = NVFP4 ? 16 : 4;                        // activation words per chunk
  const int grp = blockIdx.y;
  int n_tok, e = 0, slot_base = 0;
  if (a.n_groups) {
    if (grp >= *a.n_groups) return;
    e = a.g_expert[grp];
    n_tok = a.g_count[grp];
    slot_base = a.g_offset[grp];
  } else {
    // one group per TC tokens (grid.y); a group's rows stay on one XCD
    // when gridDim.x is a multiple of 8, so the groups share its L2
    slot_base = grp * TC;
    n_tok = min(TC, a.T - slot_base);
    if (n_tok <= 0) return;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r0 = blockIdx.x * (4 * RW) + wv * RW;            // first (gate) row of this wavefront
  if (r0 >= a.half_rows) return;
  const int nch = NVFP4 ? (a.cols >> 5) : (a.cols >> 3);     // 16-byte chunks per row
  const int64_t row_s = a.cols >> 4;                         // scale bytes per row
  const uint8_t* wq = NVFP4 ? a.wq + e * a.stride_q : nullptr;
  const uint8_t* wsc = NVFP4 ? a.ws + e * a.stride_s : nullptr;
  int rows[NR];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    rows[r] = min(r0 + r, a.half_rows - 1);
    if (MODE == GEMV_GATEUP) rows[RW + r] = rows[r] + a.half_rows;
  }
  float g0 = 1.0f, g1 = 1.0f;
  if (a.gscale) {
    if (MODE == GEMV_GATEUP) {
      g0 = a.gscale[2 * e];
      g1 = a.gscale[2 * e + 1];
    } else {
      g0 = a.gscale[e];
    }
  }
  constexpr int NCW = NC > 0 ? NC : 1;
  uint4 wr[NR][NCW];
  uint32_t scr[NR][NCW];
  if constexpr (NC > 0) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < nch;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (NVFP4) {
          wr[r][i] = ok ? *reinterpret_cast<const uint4*>(wq + nvfp4_code_off<CT>(rows[r], c, a.cols)) : make_uint4(0, 0, 0, 0);
          scr[r][i] = ok ? *reinterpret_cast<const uint16_t*>(wsc + rows[r] * row_s + 2 * c) : 0u;
        } else {
          wr[r][i] = ok ? *reinterpret_cast<const uint4*>(a.wb + static_cast<int64_t>(rows[r]) * a.cols + 8 * c)
                        : make_uint4(0, 0, 0, 0);
          scr[r][i] = 0u;
        }
      }
    }
  }
  for (int t0 = 0; t0 < n_tok; t0 += TC) {
    const int nt = min(TC, n_tok - t0);
    int in_row[TC], out_row[TC];
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      const int p = t0 + min(t, nt - 1);
      const int slot = a.n_groups ? a.g_slots[slot_base + p] : slot_base + p;
      out_row[t] = a.sorted_out ? slot_base + p : slot;
      in_row[t] = (a.n_groups && MODE == GEMV_GATEUP) ? slot / a.K : slot;
    }
    float acc[NR][TC];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int t = 0; t < TC; ++t) acc[r][t] = 0.0f;
    auto chunk = [&](int c, const uint4 (&w)[NR], const uint32_t (&sc)[NR]) {
#pragma unroll
      for (int t = 0; t < TC; ++t) {
        if (t < nt) {
          uint32_t xp[XW];
          const uint4* xs = reinterpret_cast<const uint4*>(a.in + static_cast<int64_t>(in_row[t]) * a.cols +
                                                           (NVFP4 ? 32 : 8) * c);
#pragma unroll
          for (int q = 0; q < XW / 4; ++q) {
            const uint4 v = xs[q];
            xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
          }
#pragma unroll
          for (int r = 0; r < NR; ++r)
            acc[r][t] = NVFP4 ? nvfp4_chunk_dot(w[r], sc[r], xp, acc[r][t]) : bf16_chunk_dot(w[r], xp, acc[r][t]);
        }
      }
    };
    if constexpr (NC > 0) {
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
          uint4 w[NR];
          uint32_t sc[NR];
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            w[r] = wr[r][i];
            sc[r] = scr[r][i];
          }
          chunk(c, w, sc);
        }
      }
    } else {
      for (int c = lane; c < nch; c += 64) {
        uint4 w[NR];
        uint32_t sc[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          if (NVFP4) {
            w[r] = *reinterpret_cast<const uint4*>(wq + nvfp4_code_off<CT>(rows[r], c, a.cols));
            sc[r] = *reinterpret_cast<const uint16_t*>(wsc + rows[r] * row_s + 2 * c);
          } else {
            w[r] = *reinterpret_cast<const uint4*>(a.wb + static_cast<int64_t>(rows[r]) * a.cols + 8 * c);
            sc[r] = 0u;
          }
        }
        chunk(c, w, sc);
      }
    }
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      if (t < nt) {
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r][t] = wave_sum(acc[r][t]);
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < TC; ++t) {
        if (t >= nt) continue;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          if (r0 + r >= a.half_rows) continue;
          const int64_t o = static_cast<int64_t>(out_row[t]) * a.half_rows + r0 + r;
          if (MODE == GEMV_GATEUP) {
            const float h = swiglu_clamped(g0 * acc[r][t], g1 * acc[RW + r][t], a.limit);
            static_cast<uint16_t*>(a.out)[o] = f32_to_bf16(h);
          } else if (MODE == GEMV_DOWN_F32) {
            static_cast<float*>(a.out)[o] = g0 * acc[r][t];
          } else {
            static_cast<uint16_t*>(a.out)[o] = f32_to_bf16(g0 * acc[r][t]);
          }
        }
      }
    }
  }
}

// out[t][c] = bf16(ys[t][c] + sum_k w[t,k] * y[t*K+k][c]), k in order (fp32);
// ys the sum of ys_parts reduction parts [ys_parts][T][H] (added in order).
// KMAX >= K: the K loads of a thread are all issued before the first sum (a
// loop over a run-time K waited on each load in turn; measured slower).
template <int KMAX>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y, const float* __restrict__ ys,
                                                 const float* __restrict__ wts, int T, int K, int H,
                                                 uint16_t* __restrict__ out, int ys_parts) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // float4 index
  const int64_t nq = static_cast<int64_t>(T) * (H >> 2);
  if (q >= nq) return;
  const int64_t t = q / (H >> 2);
  const int c4 = static_cast<int>(q - t * (H >> 2));
  float w[KMAX];
  float4 v[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k < K) {
      w[k] = wts[t * K + k];
      v[k] = reinterpret_cast<const float4*>(y + (t * K + k) * H)[c4];
    }
  }
  // the shared expert's output, or the sum of its reduction parts (in order)
  float4 acc = ys ? reinterpret_cast<const float4*>(ys)[q] : make_float4(0, 0, 0, 0);
  for (int p = 1; p < ys_parts; ++p) {
    const float4 v = reinterpret_cast<const float4*>(ys + static_cast<int64_t>(p) * T * H)[q];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k < K) {
      acc.x = fmaf(w[k], v[k].x, acc.x);
      acc.y = fmaf(w[k], v[k].y, acc.y);
      acc.z = fmaf(w[k], v[k].z, acc.z);
      acc.w = fmaf(w[k], v[k].w, acc.w);
    }
  }
  uint2 o;
  o.x = pack_bf16x2(acc.x, acc.y);
  o.y = pack_bf16x2(acc.z, acc.w);
  reinterpret_cast<uint2*>(out)[q] = o;
}


// hs[t][j] = bf16(SwiGLU(sum_q gu[q][t][j], sum_q gu[q][t][Is + j])) over the
// nparts reduction parts [nparts][T][2 Is] (added in order) of the shared
// expert's gate/up, clamped as in every other gate/up path.
__global__ __launch_bounds__(256) void k_swiglu_parts(const float* __restrict__ gu, int nparts, int64_t pstride,
                                                      int T, int Is, float L, uint16_t* __restrict__ hs) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(T) * Is) return;
  const int64_t t = i / Is;
  const int j = static_cast<int>(i - t * Is);
  const float* r = gu + t * 2 * Is;
  float g = r[j], u = r[Is + j];
  for (int q = 1; q < nparts; ++q) {
    g += r[q * pstride + j];
    u += r[q * pstride + Is + j];
  }
  hs[i] = f32_to_bf16(swiglu_clamped(g, u, L));
}

}  // namespace moe
