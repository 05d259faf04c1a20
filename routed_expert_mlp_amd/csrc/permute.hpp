// Token permutation by expert id for the grouped-GEMM prefill ("Module
// glm5next_mlp", Constants, MOE_MODULE: the token sort / permute / unpermute
// family).  The T*K routing slots (slot = t*K + k) are sorted by expert id,
// stably (ascending slot within an expert), with no global atomics, in
// chunks of 256 slots:
//   1. k_perm_hist:     per chunk, a histogram over experts (LDS) and each
//                       slot's rank among the chunk's slots of its expert;
//   2. k_perm_schedule: one workgroup sums the histograms into expert counts,
//                       scans them into offsets, cuts each expert's rows into
//                       BM-row GEMM tiles and turns the histograms into the
//                       sorted position of each (chunk, expert) run;
//   3. k_perm_scatter:  one thread per slot writes it at run start + rank.
#pragma once

#include "common.hpp"

namespace moe {

struct Perm {
  int32_t* count;        // [E]
  int32_t* offset;       // [E + 1]
  int32_t* perm;         // [T*K]   sorted position -> slot
  int32_t* n_tiles;      // [1]
  int32_t* tile_expert;  // [max_tiles]
  int32_t* tile_m0;      // [max_tiles] first row of the tile within its expert
};

// Slots are taken in chunks of PERM_CHUNK (one per thread of a workgroup).
constexpr int PERM_CHUNK = 256;
constexpr int PERM_MAX_E = 1024;

// 1. One workgroup per chunk b: hist[b][e] = the chunk's slots routed to
// expert e, and rank[i] = how many earlier slots of the same chunk go to the
// same expert as slot i.
__global__ __launch_bounds__(PERM_CHUNK) void k_perm_hist(const int32_t* __restrict__ ids, int nslot, int E,
                                                          int32_t* __restrict__ hist, int32_t* __restrict__ rank) {
  __shared__ int s_id[PERM_CHUNK];
  __shared__ int s_h[PERM_MAX_E];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int i = b * PERM_CHUNK + tid;
  const int e = i < nslot ? ids[i] : -1;
  s_id[tid] = e;
  for (int x = tid; x < E; x += PERM_CHUNK) s_h[x] = 0;
  __syncthreads();
  if (e >= 0) atomicAdd(&s_h[e], 1);
  int r = 0;
  for (int j = 0; j < tid; ++j) r += s_id[j] == e;
  if (i < nslot) rank[i] = r;
  __syncthreads();
  for (int x = tid; x < E; x += PERM_CHUNK) hist[static_cast<int64_t>(b) * E + x] = s_h[x];
}

// 2. One workgroup of 1024 threads (E <= 1024): expert counts (sums over the
// chunks), their exclusive scan into offsets, the cut of each expert's rows
// into bm-row GEMM tiles, and base[b][e] = the sorted position of chunk b's
// first slot of expert e (a separate array, so the loads of both passes over
// the chunks stay in flight together).
__global__ __launch_bounds__(1024) void k_perm_schedule(int E, int nblk, int bm, const int32_t* __restrict__ hist,
                                                        int32_t* __restrict__ base, Perm p) {
  __shared__ int s_w[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int c = 0;
  if (tid < E) {
#pragma unroll 16
    for (int b = 0; b < nblk; ++b) c += hist[static_cast<int64_t>(b) * E + tid];
  }
  const int nt = static_cast<int>(cdiv(c, bm));
  int ic = c, it = nt;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int a = __shfl_up(ic, m, 64), t = __shfl_up(it, m, 64);
    if (lane >= m) {
      ic += a;
      it += t;
    }
  }
  if (lane == 63) {
    s_w[0][wv] = ic;
    s_w[1][wv] = it;
  }
  __syncthreads();
  int bc = 0, bt = 0;
  for (int w = 0; w < wv; ++w) {
    bc += s_w[0][w];
    bt += s_w[1][w];
  }
  const int off = bc + ic - c, toff = bt + it - nt;
  if (tid < E) {
    p.count[tid] = c;
    p.offset[tid] = off;
    for (int j = 0; j < nt; ++j) {
      p.tile_expert[toff + j] = tid;
      p.tile_m0[toff + j] = j * bm;
    }
    if (tid == E - 1) {
      p.offset[E] = off + c;
      *p.n_tiles = toff + nt;
    }
    int run = off;
#pragma unroll 16
    for (int b = 0; b < nblk; ++b) {
      const int64_t q = static_cast<int64_t>(b) * E + tid;
      base[q] = run;
      run += hist[q];
    }
  }
}

// 3. One thread per slot: perm[base(chunk, expert) + rank] = slot.
__global__ __launch_bounds__(256) void k_perm_scatter(const int32_t* __restrict__ ids, int nslot, int E,
                                                      const int32_t* __restrict__ base,
                                                      const int32_t* __restrict__ rank, Perm p) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= nslot) return;
  const int e = ids[i];
  p.perm[base[static_cast<int64_t>(i / PERM_CHUNK) * E + e] + rank[i]] = i;
}

}  // namespace moe
