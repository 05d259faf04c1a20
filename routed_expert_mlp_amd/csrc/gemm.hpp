// Prefill projections on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// "Module glm5next_mlp", forward_prefill_gemm / MOE_GROUPED_MODULE: routed
// prefill runs each expert's sorted rows through a grouped W4A16 GEMM.  The
// same kernel, with BF16 weights and identity rows, runs the shared expert and
// the dense FFN ("DENSE: gate_proj/up_proj -> clamped SwiGLU -> down_proj").
//
// Tiling (one workgroup = 4 wavefronts, 128 rows of A):
//   * A (activations, bf16) is staged through LDS in MFMA-fragment order, two
//     stages of 128 x 128; every wavefront reads all 128 rows from LDS.
//   * B (weights) goes straight from HBM into each wavefront's registers:
//     wavefront w owns 64 output columns (4 MFMA n-tiles).  For NVFP4 a lane
//     loads 16 bytes = 32 codes of one weight row and their two E4M3 scales,
//     and turns them into four bf16x8 MFMA operands (exact: e2m1 x e4m3 fits
//     bf16); the per-expert fp32 global scale is applied in the epilogue.
//   * The reduction order inside a 128-wide k block is permuted identically
//     for A and B (lane group g covers k0+32g..k0+32g+31 and k-step s its
//     elements 8s..8s+7), which leaves the dot products unchanged.
//   * Gate/up: a wavefront's n-tiles are gate columns j..j+31 and the up
//     columns I+j..I+j+31, so the clamped SwiGLU pairs accumulators held by
//     the same lane.
//   * Rows past the tile's valid count are zero in A, their MFMAs skipped
//     (16-row granularity) and their outputs not stored.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int GM_BM = 128;
constexpr int GM_BK = 128;

enum GemmMode {
  GEMM_GATEUP = 0,          // h[row][j] = bf16(swiglu(G0*gate, G1*up))
  GEMM_DOWN_SLOT_F32 = 1,   // y[perm(row)][n] = G2*acc (routed down, un-permuted)
  GEMM_DOWN_BF16 = 2,       // out[row][n] = bf16(acc) (dense down)
  GEMM_DOWN_F32 = 3,        // ys[row][n] = acc (shared down)
};

struct GemmArgs {
  const uint16_t* a;         // activations, row length kdim
  int kdim;                  // reduction length (multiple of 32)
  const uint8_t* bq;         // NVFP4 codes [E][rows][kdim/2]
  const uint8_t* bs;         // NVFP4 scales [E][rows][kdim/16]
  const uint16_t* bb;        // BF16 weights [rows][kdim]
  int64_t stride_q, stride_s;
  const float* gscale;       // routed globals (gate/up: [E,2]; down: [E]); null = 1
  int half_n;                // gate/up: I (gate rows, up rows = I + j); down: output columns
  // routed tiles
  const int32_t* n_tiles;
  const int32_t* tile_expert;
  const int32_t* tile_m0;
  const int32_t* count;
  const int32_t* offset;
  const int32_t* perm;
  int T;                     // dense rows
  int K;                     // slot -> token = slot / K (routed gate/up gather)
  void* out;
  int ldo;
  float limit;
};

template <bool NVFP4, int MODE, bool ROUTED>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  __shared__ uint4 lds[2][8 * 4 * 64];   // 2 stages x (8 m-tiles x 4 k-steps x 64 lanes x 16 B)
  const int tile = blockIdx.x, nblk = blockIdx.y;   // x: M tiles, y: N blocks
  int e = 0, m0, valid, p0;
  if (ROUTED) {
    if (tile >= *a.n_tiles) return;
    e = a.tile_expert[tile];
    m0 = a.tile_m0[tile];
    valid = min(GM_BM, a.count[e] - m0);
    p0 = a.offset[e] + m0;
  } else {
    m0 = tile * GM_BM;
    if (m0 >= a.T) return;
    valid = min(GM_BM, a.T - m0);
    p0 = m0;
  }
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int kdim = a.kdim;
  const int mt_valid = static_cast<int>(cdiv(valid, 16));

  // ---- A loader: thread owns row r, half h (64 columns of a 128 block)
  const int ar = tid >> 1, ah = tid & 1;
  const uint16_t* arow = nullptr;
  if (ar < valid) {
    if (ROUTED && MODE == GEMM_GATEUP) {
      const int slot = a.perm[p0 + ar];
      arow = a.a + static_cast<int64_t>(slot / a.K) * kdim;
    } else {
      arow = a.a + static_cast<int64_t>(p0 + ar) * kdim;
    }
  }

  // ---- B rows of this wavefront's 4 n-tiles
  const int g = lane >> 4, ln = lane & 15;
  int brow[4];
  bool bvalid[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    if (MODE == GEMM_GATEUP) {
      const int j = nblk * 128 + wv * 32 + (nt & 1) * 16 + ln;
      bvalid[nt] = j < a.half_n;
      const int jj = bvalid[nt] ? j : 0;
      brow[nt] = nt < 2 ? jj : a.half_n + jj;
    } else {
      const int n = nblk * 256 + wv * 64 + nt * 16 + ln;
      bvalid[nt] = n < a.half_n;
      brow[nt] = bvalid[nt] ? n : 0;
    }
  }
  const uint8_t* bq = nullptr;
  const uint8_t* bs = nullptr;
  if (NVFP4) {
    bq = a.bq + e * a.stride_q;
    bs = a.bs + e * a.stride_s;
  }

  f32x4 acc[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  uint4 av[8];
  auto load_a = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int col = k0 + 64 * ah + 8 * q;
      av[q] = (arow && col < kdim) ? *reinterpret_cast<const uint4*>(arow + col) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int gg = 2 * ah + (q >> 2), ks = q & 3;
      lds[buf][((ar >> 4) * 4 + ks) * 64 + (ar & 15) + 16 * gg] = av[q];
    }
  };

  const int nkb = static_cast<int>(cdiv(kdim, GM_BK));
  load_a(0);
  store_a(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * GM_BK;
    const int buf = kb & 1;
    const int kg = k0 + 32 * g;              // first k of this lane's group
    const bool kvalid = kg < kdim;
    // B for this k block
    uint4 bcode[4];
    uint32_t bscale[4];
    if (NVFP4) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (kvalid) {
          bcode[nt] = *reinterpret_cast<const uint4*>(bq + static_cast<int64_t>(brow[nt]) * (kdim >> 1) + (kg >> 1));
          bscale[nt] = *reinterpret_cast<const uint16_t*>(bs + static_cast<int64_t>(brow[nt]) * (kdim >> 4) + (kg >> 4));
        } else {
          bcode[nt] = make_uint4(0, 0, 0, 0);
          bscale[nt] = 0;
        }
      }
    }
    if (kb + 1 < nkb) load_a(k0 + GM_BK);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 bfrag[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        uint4 v;
        if (NVFP4) {
          const uint32_t cw = ks == 0 ? bcode[nt].x : ks == 1 ? bcode[nt].y : ks == 2 ? bcode[nt].z : bcode[nt].w;
          const float s = (ks < 2) ? e4m3_to_f32<0>(bscale[nt]) : e4m3_to_f32<1>(bscale[nt]);
          uint32_t o[4];
          e2m1x8_scaled_bf16(cw, s, o);
          v = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
          v = kvalid ? *reinterpret_cast<const uint4*>(a.bb + static_cast<int64_t>(brow[nt]) * kdim + kg + 8 * ks)
                     : make_uint4(0, 0, 0, 0);
        }
        bfrag[nt] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        if (mt < mt_valid) {
          const bf16x8 af = __builtin_bit_cast(bf16x8, lds[buf][(mt * 4 + ks) * 64 + lane]);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfrag[nt], acc[mt][nt], 0, 0, 0);
        }
      }
    }
    if (kb + 1 < nkb) store_a(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows mt*16 + 4*(lane>>4) + i, column ln of each n-tile
  float g0 = 1.0f, g1 = 1.0f;
  if (ROUTED && a.gscale) {
    if (MODE == GEMM_GATEUP) {
      g0 = a.gscale[2 * e];
      g1 = a.gscale[2 * e + 1];
    } else {
      g0 = a.gscale[e];
    }
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if (mt >= mt_valid) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mt * 16 + 4 * (lane >> 4) + i;
      if (row >= valid) continue;
      if (MODE == GEMM_GATEUP) {
        uint16_t* o = static_cast<uint16_t*>(a.out) + static_cast<int64_t>(p0 + row) * a.ldo;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          if (!bvalid[nt]) continue;
          const int j = nblk * 128 + wv * 32 + nt * 16 + ln;
          o[j] = f32_to_bf16(swiglu_clamped(g0 * acc[mt][nt][i], g1 * acc[mt][nt + 2][i], a.limit));
        }
      } else {
        int64_t orow;
        if (MODE == GEMM_DOWN_SLOT_F32) orow = a.perm[p0 + row];
        else orow = p0 + row;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (!bvalid[nt]) continue;
          const int n = nblk * 256 + wv * 64 + nt * 16 + ln;
          if (MODE == GEMM_DOWN_BF16)
            static_cast<uint16_t*>(a.out)[orow * a.ldo + n] = f32_to_bf16(acc[mt][nt][i]);
          else
            static_cast<float*>(a.out)[orow * a.ldo + n] = g0 * acc[mt][nt][i];
        }
      }
    }
  }
}

// NVFP4 -> fp32 / bf16 dequantisation, through the same device routines as
// the GEMV and GEMM: one thread per 32 columns of a row.
__global__ __launch_bounds__(256) void k_nvfp4_dequant(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                       float global, int64_t rows, int cols,
                                                       float* out_f32, uint16_t* out_bf16) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int nch = cols >> 5;
  if (idx >= rows * nch) return;
  const int64_t r = idx / nch;
  const int c = static_cast<int>(idx - r * nch);
  const uint4 cw = *reinterpret_cast<const uint4*>(q + r * (cols >> 1) + 16 * c);
  const uint32_t sc = *reinterpret_cast<const uint16_t*>(s + r * (cols >> 4) + 2 * c);
  const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float scale = (w < 2 ? e4m3_to_f32<0>(sc) : e4m3_to_f32<1>(sc)) * global;
    const int64_t o = r * cols + 32 * c + 8 * w;
    if (out_bf16) {
      uint32_t p[4];
      e2m1x8_scaled_bf16(words[w], scale, p);
      *reinterpret_cast<uint4*>(out_bf16 + o) = make_uint4(p[0], p[1], p[2], p[3]);
    }
    if (out_f32) {
      const f32x2 v0 = e2m1x2_to_f32<0>(words[w]), v1 = e2m1x2_to_f32<1>(words[w]);
      const f32x2 v2 = e2m1x2_to_f32<2>(words[w]), v3 = e2m1x2_to_f32<3>(words[w]);
      float4* of = reinterpret_cast<float4*>(out_f32 + o);
      of[0] = make_float4(v0.x * scale, v0.y * scale, v1.x * scale, v1.y * scale);
      of[1] = make_float4(v2.x * scale, v2.y * scale, v3.x * scale, v3.y * scale);
    }
  }
}

}  // namespace moe
