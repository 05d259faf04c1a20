// Shared-expert (and any BF16) projection for a few tokens, as fp32 parts of
// the reduction: out[q][t][n] = sum of x[t][k] W[n][k] over k in part q
// (kr columns each).  The parts are added afterwards in order (k_swiglu_parts
// for gate/up, k_combine for down), exactly as for the split BF16 GEMM.
//
// "Module glm5next_mlp", the shared expert of the routed layer: BF16 gate/up
// and down of every token.  With up to 64 tokens the weights (25 MB gate/up and
// 12.6 MB down at GLM-Flash size) are the whole cost, so the kernel is a
// weight stream with the products on the matrix cores
// (v_mfma_f32_16x16x32_bf16: 16 tokens x 16 weight rows per MFMA):
//   * Workgroup = 4 wavefronts over 64 weight rows and one part of the
//     reduction; each wavefront owns 16 rows and loads all of its weights for
//     the part into registers at once (kr = 1024: 32 x 16 bytes per lane),
//     64 contiguous bytes of one row per lane and 128-column block.
//   * The tokens' columns of the part go to LDS by DMA before the weight
//     loads are issued (rows padded by 16 bytes: the MFMA operand reads are
//     free of bank conflicts), so the wait for them leaves the weight loads in
//     flight.
//   * Inside a 128-column block the reduction order is permuted identically
//     for both operands (lane group g covers columns 32g..32g+31, k-step s its
//     elements 8s..8s+7), as in the other BF16 kernels.
// Requires kr a multiple of 512 (one 1 KB DMA per row and 512 columns), at
// most F16S_KR; tokens up to 16 TB.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int F16S_KR = 1024;     // largest reduction part
constexpr int F16S_ROWS = 64;     // weight rows per workgroup

template <int TB, int KR>
__global__ __launch_bounds__(256) void k_skinny_bf16(const uint16_t* __restrict__ x, int ldx,
                                                     const uint16_t* __restrict__ w, int ldw, int N, int T,
                                                     int nparts, float* __restrict__ out, int64_t part_stride) {
  constexpr int XS = KR / 8 + 1;          // padded LDS row, in 16-byte units
  constexpr int NKB = KR / 128;
  __shared__ uint4 xs[16 * TB * XS];
  const int nrb = (N + F16S_ROWS - 1) / F16S_ROWS;
  const int rb = blockIdx.x % nrb, q = blockIdx.x / nrb;
  if (q >= nparts) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, ln = lane & 15;
  const int64_t k0 = static_cast<int64_t>(q) * KR;

  // tokens' columns k0 .. k0 + KR of this part: one 1 KB DMA per 512 columns
  // of a token row, spread over the wavefronts
  {
    constexpr int PER_ROW = KR / 512;
    const int nins = T * PER_ROW;
    for (int i = wv; i < nins; i += 4) {
      const int t = i / PER_ROW, h = i - t * PER_ROW;
      const uint16_t* src = x + static_cast<int64_t>(t) * ldx + k0 + 512 * h + 8 * lane;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src),
                                       (void __attribute__((address_space(3)))*)(xs + t * XS + 64 * h), 16, 0, 0);
    }
  }
  asm volatile("" ::: "memory");   // the weight loads stay behind the token DMAs
  // this lane's weights: row n, columns k0 + 128 b + 32 g .. + 31 of every block b
  const int n = rb * F16S_ROWS + 16 * wv + ln;
  const uint16_t* wr = w + static_cast<int64_t>(min(n, N - 1)) * ldw + k0 + 32 * g;
  uint4 wq[NKB][4];
#pragma unroll
  for (int b = 0; b < NKB; ++b)
#pragma unroll
    for (int s = 0; s < 4; ++s) wq[b][s] = *reinterpret_cast<const uint4*>(wr + 128 * b + 8 * s);
  // the token DMAs are older than every weight load: wait for them alone
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * NKB));
  asm volatile("" ::: "memory");
  __syncthreads();

  f32x4 acc[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < NKB; ++b) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 bfrag = __builtin_bit_cast(bf16x8, wq[b][s]);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const bf16x8 af = __builtin_bit_cast(bf16x8, xs[(16 * tb + ln) * XS + 16 * b + 4 * g + s]);
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfrag, acc[tb], 0, 0, 0);
      }
    }
  }
  // lane holds tokens 16 tb + 4 g + i of weight row n
  if (n < N) {
    float* o = out + q * part_stride + n;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tb + 4 * g + i;
        if (t < T) o[static_cast<int64_t>(t) * N] = acc[tb][i];
      }
  }
}

}  // namespace moe

namespace moe {

// Routed NVFP4 down projection for a few tokens per expert (decode batches):
// y[slot][n] = g2[e] * sum_k h[pos][k] W_e[n][k] for the rows pos of expert
// e's group (expert-sorted activation rows) and slot = out_idx[pos].
//
// "Module glm5next_mlp", the routed experts' NVFP4 down projection; Constants,
// W4A16_GEMV_MODULE: with a few tokens per expert the weight bytes are the
// whole cost.  A GEMV spends a dot product per token and weight; here the
// weights are dequantised once into bf16 MFMA operands and the tokens ride
// along on the matrix cores (v_mfma_f32_16x16x32_bf16: 16 weight rows x 16
// tokens per MFMA), so the cost per weight byte does not grow with the tokens:
//   * workgroup = 4 wavefronts over 64 output rows and the whole reduction
//     (NU units of 128 columns); lane (g, l) of a wavefront holds row l's
//     codes for columns 128 b + 32 g .. + 31 of every unit b (one 16-byte
//     load per unit: with the tile-layout codes every load instruction reads
//     one contiguous 1 KB block), issued all at once before any arithmetic;
//   * the group's activation rows (up to NT per pass) reach LDS by DMA
//     before the weight loads are issued (rows padded by 16 bytes);
//   * inside a unit the reduction order is permuted identically for both
//     operands (lane group g, k-step s: columns 32 g + 8 s .. + 7);
//   * a group of more than NT tokens takes several passes over the weights
//     held in registers (dequantised again per pass).
// Requires N a multiple of 64; NU a multiple of 4 (reduction a multiple of
// 512).  Output rows are fp32, added by the combine in k order.
constexpr int SF4_ROWS = 64;   // output rows per workgroup

struct SkinnyF4Args {
  const uint8_t* wq;       // codes, expert-major: row-major [N][kdim/2] or the tile layout
  const uint8_t* ws;       // E4M3 scales, row-major [N][kdim/16] per expert
  int64_t stride_q;        // bytes of codes per expert
  int64_t stride_s;        // bytes of scales per expert
  const float* gscale;     // [E] or null (= 1)
  int N;                   // output rows
  // expert groups: (n_groups, g_expert, g_count, g_offset); or (g_count
  // null) one group per expert over positions offsets[e] .. offsets[e + 1],
  // e = g_expert[blockIdx.y] for blockIdx.y < n_groups (an expert order,
  // each expert at most once), or e = blockIdx.y when g_expert is null too
  const int32_t* n_groups;
  const int32_t* g_expert;
  const int32_t* g_count;
  const int32_t* g_offset;
  const int32_t* offsets;
  const int32_t* out_idx;  // position -> output row (slot)
  const uint16_t* in;      // [positions][kdim] bf16, expert-sorted
  float* out;              // [slots][N] fp32
};

// Wavefronts per SIMD a workgroup of 4 wavefronts with `lds` bytes of LDS
// can reach (160 KB of LDS per CU), at most 4: the register budget the
// kernels are compiled for.
constexpr int sf4_waves(int lds) { return 163840 / lds < 4 ? 163840 / lds : 4; }

template <int NU, int NT, bool CT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sf4_waves(NT * (NU * 16 + 1) * 16))))
void k_skinny_f4_down(SkinnyF4Args a) {
  static_assert(NU % 4 == 0 && NT >= 1 && NT <= 16, "whole 1 KB DMA pieces per row; one 16-token MFMA tile");
  constexpr int KD = NU * 128;        // reduction length
  constexpr int XS = KD / 8 + 1;      // LDS row in 16-byte units (padded by one)
  constexpr int DPR = KD / 512;       // 1 KB DMA instructions per activation row
  __shared__ uint4 xs[NT * XS];
  int e, cnt, off;
  if (a.g_count) {
    if (static_cast<int>(blockIdx.y) >= *a.n_groups) return;
    e = a.g_expert[blockIdx.y];
    cnt = a.g_count[blockIdx.y];
    off = a.g_offset[blockIdx.y];
  } else {
    if (a.g_expert) {
      if (static_cast<int>(blockIdx.y) >= *a.n_groups) return;
      e = a.g_expert[blockIdx.y];
    } else {
      e = blockIdx.y;
    }
    off = a.offsets[e];
    cnt = a.offsets[e + 1] - off;
  }
  if (cnt <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, ln = lane & 15;

  // rows t0 .. t0 + nt of the group into LDS rows 0 .. nt: one 1 KB DMA per
  // 512 columns of a row, spread over the wavefronts
  auto stage = [&](int t0, int nt) {
    for (int i = wv; i < nt * DPR; i += 4) {
      const int t = i / DPR, hh = i - t * DPR;
      const uint16_t* src = a.in + static_cast<int64_t>(off + t0 + t) * KD + 512 * hh + 8 * lane;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src),
                                       (void __attribute__((address_space(3)))*)(xs + t * XS + 64 * hh), 16, 0, 0);
    }
  };
  stage(0, min(cnt, NT));
  asm volatile("" ::: "memory");   // the weight loads stay behind the activation DMAs

  // this lane's weights: row n, columns 128 b + 32 g .. + 31 of every unit b
  const int n = blockIdx.x * SF4_ROWS + 16 * wv + ln;
  const int nc = min(n, a.N - 1);
  const uint8_t* wq = a.wq + static_cast<int64_t>(e) * a.stride_q;
  const uint8_t* wsr = a.ws + static_cast<int64_t>(e) * a.stride_s + static_cast<int64_t>(nc) * (KD / 16) + 2 * g;
  uint4 cw[NU];
  uint32_t sc[NU];
#pragma unroll
  for (int b = 0; b < NU; ++b) {
    cw[b] = *reinterpret_cast<const uint4*>(wq + nvfp4_code_off<CT>(nc, 4 * b + g, KD));
    sc[b] = *reinterpret_cast<const uint16_t*>(wsr + 8 * b);
  }
  // the activation DMAs are older than every weight load: wait for them alone
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NU));
  asm volatile("" ::: "memory");
  __syncthreads();

  const float gs = a.gscale ? a.gscale[e] : 1.0f;
  for (int t0 = 0; t0 < cnt; t0 += NT) {
    const int nt = min(NT, cnt - t0);
    if (t0 > 0) {
      __syncthreads();                  // every wavefront is done with the previous rows
      stage(t0, nt);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      asm volatile("" ::: "memory");
      __syncthreads();
    }
    const int xr = min(ln, nt - 1) * XS + 4 * g;   // this lane's token row (B operand column)
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < NU; ++b) {
      const float s0 = e4m3_to_f32<0>(sc[b]);
      const float s1 = e4m3_to_f32<1>(sc[b]);
      uint32_t wf[4][4];
      e2m1x8_scaled_bf16(cw[b].x, s0, wf[0]);
      e2m1x8_scaled_bf16(cw[b].y, s0, wf[1]);
      e2m1x8_scaled_bf16(cw[b].z, s1, wf[2]);
      e2m1x8_scaled_bf16(cw[b].w, s1, wf[3]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 af = __builtin_bit_cast(bf16x8, make_uint4(wf[s][0], wf[s][1], wf[s][2], wf[s][3]));
        const bf16x8 xf = __builtin_bit_cast(bf16x8, xs[xr + 16 * b + s]);
        if (s & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, xf, acc1, 0, 0, 0);
        else acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, xf, acc0, 0, 0, 0);
      }
      // one unit's operands at a time: dequantising every unit ahead of its
      // MFMAs would take the registers the in-flight weight loads need
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane (g, l) holds rows 16 wv + 4 g + i (i = 0..3) of token t0 + l
    if (ln < nt) {
      const int slot = a.out_idx[off + t0 + ln];
      const int r = blockIdx.x * SF4_ROWS + 16 * wv + 4 * g;
      if (r < a.N) {
        const float4 v = make_float4(gs * (acc0[0] + acc1[0]), gs * (acc0[1] + acc1[1]), gs * (acc0[2] + acc1[2]),
                                     gs * (acc0[3] + acc1[3]));
        *reinterpret_cast<float4*>(a.out + static_cast<int64_t>(slot) * a.N + r) = v;
      }
    }
  }
}

}  // namespace moe
