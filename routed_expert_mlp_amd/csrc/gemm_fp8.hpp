// Grouped GEMM for FP8 block-scaled routed experts (E4M3 "fn" bytes [out, in],
// one fp32 scale per 128 x 128 block; the FP8 checkpoint named on the
// TensorRT-LLM page "Add GLM-5.3-Flash (glm5_next) support"): the
// forward_prefill_gemm step of "Module glm5next_mlp" with W8A16 weights.
//
// The tiling of k_gemm (gemm.hpp): one workgroup of 4 wavefronts per 128
// expert-sorted rows, A (bf16 activations) staged through LDS in MFMA
// fragment order, B straight from HBM into registers, v_mfma_f32_16x16x32_bf16
// with the k order permuted identically for A and B.  B here is E4M3: a lane
// loads the 32 bytes of its k range of one weight row per 128-wide k block
// and converts them to bf16 exactly.  A k block is exactly one 128-column
// scale block and an n-tile (16 weight rows) lies in one 128-row scale block,
// so every k block accumulates into a fresh tile and is then added to the
// running sum times its scale: products stay exact, as on the GEMV path.
#pragma once

#include "common.hpp"
#include "decode_fp8.hpp"
#include "gemm.hpp"

namespace moe {

template <int MODE>
__global__ __launch_bounds__(256) void k_gemm_f8(GemmArgs a) {
  __shared__ uint4 lds[2][8 * 4 * 64];   // 2 stages x (8 m-tiles x 4 k-steps x 64 lanes x 16 B)
  const int tile = blockIdx.x, nblk = blockIdx.y;   // x: M tiles, y: N blocks
  if (tile >= *a.n_tiles) return;
  const int e = a.tile_expert[tile];
  const int m0 = a.tile_m0[tile];
  const int valid = min(GM_BM, a.count[e] - m0);
  const int p0 = a.offset[e] + m0;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int kdim = a.kdim;                  // multiple of 128
  const int mt_valid = static_cast<int>(cdiv(valid, 16));

  // ---- A loader: thread owns row r, half h (64 columns of a 128 block)
  const int ar = tid >> 1, ah = tid & 1;
  const uint16_t* arow = nullptr;
  if (ar < valid) {
    if (MODE == GEMM_GATEUP) {
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
  const int nkb = kdim / F8_BLOCK;
  const uint8_t* bq = a.bq + e * a.stride_q;
  const float* bsf = a.bsf + e * a.stride_s;
  // every n-tile's 16 rows lie in one 128-row scale block
  const float* srow[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) srow[nt] = bsf + static_cast<int64_t>(brow[nt] / F8_BLOCK) * nkb;

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
      av[q] = arow ? *reinterpret_cast<const uint4*>(arow + col) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int gg = 2 * ah + (q >> 2), ks = q & 3;
      lds[buf][((ar >> 4) * 4 + ks) * 64 + (ar & 15) + 16 * gg] = av[q];
    }
  };

  load_a(0);
  store_a(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * F8_BLOCK;
    const int buf = kb & 1;
    const int kg = k0 + 32 * g;              // first k of this lane's group
    // B for this k block: 32 E4M3 bytes per n-tile, and the block scales
    uint4 bcode[4][2];
    float bscale[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const uint4* p = reinterpret_cast<const uint4*>(bq + static_cast<int64_t>(brow[nt]) * kdim + kg);
      bcode[nt][0] = p[0];
      bcode[nt][1] = p[1];
      bscale[nt] = srow[nt][kb];
    }
    if (kb + 1 < nkb) load_a(k0 + F8_BLOCK);
    f32x4 part[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) part[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 bfrag[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint4 c = bcode[nt][ks >> 1];
        const uint32_t w0 = (ks & 1) ? c.z : c.x, w1 = (ks & 1) ? c.w : c.y;
        const bf16x2 p0 = e4m3x2_to_bf16<0>(w0), p1 = e4m3x2_to_bf16<1>(w0);
        const bf16x2 p2 = e4m3x2_to_bf16<0>(w1), p3 = e4m3x2_to_bf16<1>(w1);
        bfrag[nt] = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        if (mt < mt_valid) {
          const bf16x8 af = __builtin_bit_cast(bf16x8, lds[buf][(mt * 4 + ks) * 64 + lane]);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            part[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfrag[nt], part[mt][nt], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][nt][i] = fmaf(bscale[nt], part[mt][nt][i], acc[mt][nt][i]);
    if (kb + 1 < nkb) store_a(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows mt*16 + 4*(lane>>4) + i, column ln of each n-tile
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
          o[j] = f32_to_bf16(swiglu_clamped(acc[mt][nt][i], acc[mt][nt + 2][i], a.limit));
        }
      } else {
        const int64_t orow = a.perm[p0 + row];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (!bvalid[nt]) continue;
          const int n = nblk * 256 + wv * 64 + nt * 16 + ln;
          static_cast<float*>(a.out)[orow * a.ldo + n] = acc[mt][nt][i];
        }
      }
    }
  }
}

}  // namespace moe
