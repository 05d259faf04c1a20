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
