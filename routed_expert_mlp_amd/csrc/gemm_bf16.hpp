// BF16 GEMM for the shared expert, the dense FFN and the split-weight router
// logits on v_mfma_f32_32x32x16_bf16: out rows = activation rows (T), output
// columns = weight rows, reduction over kdim.
//
// "Module glm5next_mlp", forward_prefill_gemm (the shared expert runs beside
// the routed experts) and the page's DENSE layer (BF16 gate/up, clamped
// SwiGLU, down).
//
// Layout (same measured rules as the routed NVFP4 kernel, gemm_fp4.hpp):
//   * one workgroup of 8 wavefronts per CU, tile 256 rows x 256 weight rows
//     (gate/up: 128 gate columns and the matching 128 up columns); wavefront
//     w owns rows 128 (w / 4) .. +128 and two 32-row weight tiles (gate/up:
//     gate rows 32 (w % 4) .. +32 and the matching up rows; otherwise weight
//     rows 64 (w % 4) .. +64), i.e. 4 x 2 MFMA tiles, so every k-step reads 4
//     activation and 2 weight fragments for 8 MFMAs;
//   * both operands reach LDS by DMA with 8 lanes per 128-byte row piece (one
//     64-wide stage), the XOR swizzle of the MFMA operand reads applied on the
//     global side; a 2-stage ring of 64 KB stages (128 KB);
//   * the schedule is static (a loop over stage pairs that always issue, then
//     the tail stages), so every wait is a compile-time count, and the ring
//     slots are separate LDS arrays whose reads the compiler schedules;
//   * row tiles of one column block run back to back on an XCD, so a block of
//     weight rows is read from HBM once and reused from that XCD's L2.
// Rows past T and weight rows past the matrix edge reload row 0 (outputs
// dropped).  Requires kdim % 128 == 0.
#pragma once

#include "common.hpp"
#include "gemm.hpp"
#include "gemm_fp4.hpp"

#include <type_traits>

namespace moe {

constexpr int B16_BM = 256;        // activation rows per tile
constexpr int B16_BN = 256;        // weight rows per tile
constexpr int B16_THREADS = 512;

struct B16Lds {
  uint4* a[2];
  uint4* b[2];
};

template <int MODE, int MTV>
__device__ __forceinline__ void b16_mainloop(const B16Lds& L, const uint8_t* asrc_base, const uint32_t (&ao)[4],
                                             const uint8_t* bsrc_base, const uint32_t (&bo)[4], int wv, int lane,
                                             int kdim, f32x16 (&acc)[4][2]) {
  const int g = lane >> 5, ln = lane & 31;
  const int wm = wv >> 2, wn = wv & 3;
  const int nkb = kdim >> 6;
  // DMA: per wave per stage 4 activation and 4 weight instructions (8 rows each)
  auto issue = [&](int k, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(asrc_base + (ao[i] + 128u * k)),
                                       (void __attribute__((address_space(3)))*)(L.a[SL] + wv * 256 + i * 64),
                                       16, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(bsrc_base + (bo[i] + 128u * k)),
                                       (void __attribute__((address_space(3)))*)(L.b[SL] + wv * 256 + i * 64),
                                       16, 0, 0);
  };
  // consumer offsets (uint4 units): activation row 128 wm + 32 mt + ln; weight
  // row of n-tile nt: gate/up 32 wn + ln + 128 nt (gate j and up j in one
  // lane), otherwise 64 wn + 32 nt + ln; chunk 4 g + s sits at position
  // chunk ^ swizzle(row), and the swizzle depends on row % 16 = ln % 16 only
  constexpr int NTS = MODE == GEMM_GATEUP ? 128 * 8 : 32 * 8;
  const int sa = f4_swz_a(ln);
  const int brow0 = (MODE == GEMM_GATEUP ? 32 * wn : 64 * wn) + ln;
  int aidx[4], bidx[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    aidx[s] = (128 * wm + ln) * 8 + ((4 * g + s) ^ sa);
    bidx[s] = brow0 * 8 + ((4 * g + s) ^ sa);
  }
  // one stage: wait for its data (VM = DMA instructions allowed to stay in
  // flight), barrier, 4 k-steps of 8 MFMAs (fragments of the next k-step read
  // right after their last use), then, when ISSUE, a barrier (every wave is
  // past its reads of this slot) and the DMA of stage k + 2 into this slot
  auto stage = [&](int k, auto slot_c, auto vm_c, auto issue_c) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int VM = decltype(vm_c)::value;
    constexpr bool ISSUE = decltype(issue_c)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const uint4* As = L.a[SL];
    const uint4* Bs = L.b[SL];
    bf16x8 af[MTV], bf[2];
#pragma unroll
    for (int mt = 0; mt < MTV; ++mt) af[mt] = __builtin_bit_cast(bf16x8, As[aidx[0] + mt * 256]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) bf[nt] = __builtin_bit_cast(bf16x8, Bs[bidx[0] + nt * NTS]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int mt = 0; mt < MTV; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bf[nt], acc[mt][nt], 0, 0, 0);
        if (s < 3) af[mt] = __builtin_bit_cast(bf16x8, As[aidx[s + 1] + mt * 256]);
      }
      if (s < 3) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) bf[nt] = __builtin_bit_cast(bf16x8, Bs[bidx[s + 1] + nt * NTS]);
      }
      // keep the reads one k-step ahead (hoisting all of a stage's fragment
      // reads to its top would need 96 more registers)
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (ISSUE) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(k + 2, slot_c);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using V0 = std::integral_constant<int, 0>;
  using V8 = std::integral_constant<int, 8>;
  using Y = std::true_type;
  using N = std::false_type;
  // An even number of stages: pairs that issue the pair after next, then the
  // last pair, which issues nothing.  Stage k may leave stage k+1's 8
  // instructions in flight (always issued before stage k's wait) except the
  // last stage.  No branch in the schedule: the accumulators would otherwise
  // pass through merges that cost the register allocator dearly (measured).
  issue(0, I0{});
  issue(1, I1{});
  for (int k = 0; k + 2 < nkb; k += 2) {
    stage(k, I0{}, V8{}, Y{});
    stage(k + 1, I1{}, V8{}, Y{});
  }
  stage(nkb - 2, I0{}, V8{}, N{});
  stage(nkb - 1, I1{}, V0{}, N{});
}

// Grid: 1-D, XCD-aware (block b runs on XCD b % 8; each XCD takes a
// contiguous run of work items), row tiles of a column block back to back,
// a reduction split (ksplit parts, GEMM_DOWN_F32 only) fastest.
// n_blocks = column blocks of 256 weight rows (gate/up: 128 gate columns).
template <int MODE>
__global__ __launch_bounds__(B16_THREADS, 1) void k_gemm_bf16(GemmArgs a) {
  const int nbn = a.n_blocks;
  const int ntl = static_cast<int>(cdiv(a.T, B16_BM));
  const int ks = a.ksplit > 1 ? a.ksplit : 1;
  const int total = ntl * nbn * ks, chunk = (total + 7) >> 3;
  const int kk = blockIdx.x >> 3;
  if (kk >= chunk) return;
  const int w0 = (blockIdx.x & 7) * chunk + kk;
  if (w0 >= total) return;
  const int split = w0 % ks, w = w0 / ks;
  const int nblk = w / ntl, tile = w - nblk * ntl;
  const int p0 = tile * B16_BM;
  const int valid = min(B16_BM, a.T - p0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int kdim = a.kdim;
  const int64_t lda = a.lda ? a.lda : kdim, ldb = a.ldb ? a.ldb : kdim;

  // activation DMA: instruction i of wave wv covers tile rows 32 wv + 8 i .. +7
  uint32_t ao[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wv + 8 * i + (lane >> 3);
    const int rr = r < valid ? r : 0;
    ao[i] = static_cast<uint32_t>(((p0 + rr) * lda + 8 * ((lane & 7) ^ f4_swz_a(r))) * 2);
  }
  // weight DMA: the same for weight rows p = 32 wv + 8 i + lane / 8 of the tile
  auto wrow = [&](int p) -> int64_t {
    if (MODE == GEMM_GATEUP) {
      const int j = nblk * 128 + (p & 127);
      return j < a.half_n ? (p < 128 ? j : a.half_n + j) : 0;
    } else {
      const int n = nblk * B16_BN + p;
      return n < a.half_n ? n : 0;
    }
  };
  uint32_t bo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = 32 * wv + 8 * i + (lane >> 3);
    bo[i] = static_cast<uint32_t>((wrow(p) * ldb + 8 * ((lane & 7) ^ f4_swz_a(p))) * 2);
  }
  const uint8_t* abase = reinterpret_cast<const uint8_t*>(a.a + static_cast<int64_t>(split) * kdim);
  const uint8_t* bbase = reinterpret_cast<const uint8_t*>(a.bb + static_cast<int64_t>(split) * kdim);

  __shared__ uint4 la0[2048], la1[2048];   // activation ring (32 KB each)
  __shared__ uint4 lb0[2048], lb1[2048];   // weight ring (32 KB each)
  const B16Lds L{{la0, la1}, {lb0, lb1}};
  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mt][nt][j] = 0.0f;
  // m-tiles of this wave's 128 rows that hold valid rows
  const int wm = wv >> 2;
  const int vrows = valid - 128 * wm;
  const int mtv = vrows <= 0 ? 0 : min(4, (vrows + 31) >> 5);
  // every wave runs the same number of stages (barriers); waves without valid
  // rows still load and compute on reloaded rows, whose outputs are dropped
  switch (mtv) {
    case 0: case 1: b16_mainloop<MODE, 1>(L, abase, ao, bbase, bo, wv, lane, kdim, acc); break;
    case 2: b16_mainloop<MODE, 2>(L, abase, ao, bbase, bo, wv, lane, kdim, acc); break;
    case 3: b16_mainloop<MODE, 3>(L, abase, ao, bbase, bo, wv, lane, kdim, acc); break;
    default: b16_mainloop<MODE, 4>(L, abase, ao, bbase, bo, wv, lane, kdim, acc); break;
  }

  const int wn = wv & 3, ln = lane & 31;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (mt >= mtv) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = 128 * wm + mt * 32 + c32_row(lane, j);
      if (row >= valid) continue;
      const int64_t orow = p0 + row;
      if (MODE == GEMM_GATEUP) {
        const int jc = nblk * 128 + 32 * wn + ln;
        if (jc < a.half_n)
          static_cast<uint16_t*>(a.out)[orow * a.ldo + jc] =
              f32_to_bf16(swiglu_clamped(acc[mt][0][j], acc[mt][1][j], a.limit));
      } else {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int n = nblk * B16_BN + 64 * wn + 32 * nt + ln;
          if (n >= a.half_n) continue;
          if (MODE == GEMM_DOWN_BF16)
            static_cast<uint16_t*>(a.out)[orow * a.ldo + n] = f32_to_bf16(acc[mt][nt][j]);
          else
            static_cast<float*>(a.out)[split * a.split_out + orow * a.ldo + n] = acc[mt][nt][j];
        }
      }
    }
  }
}

}  // namespace moe
