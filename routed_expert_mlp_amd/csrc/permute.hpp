// Token permutation by expert id for the grouped-GEMM prefill ("Module
// glm5next_mlp", Constants, MOE_MODULE: the token sort / permute / unpermute
// family).  The T*K routing slots (slot = t*K + k) are sorted by expert id,
// stably (ascending slot within an expert), with no global atomics:
//   1. k_expert_count:   one workgroup per expert counts its slots;
//   2. k_schedule:       one workgroup scans the counts into offsets and cuts
//                        each expert's rows into BM-row GEMM tiles;
//   3. k_expert_scatter: one workgroup per expert writes its slots in order.
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

__global__ __launch_bounds__(256) void k_expert_count(const int32_t* __restrict__ ids, int nslot, Perm p) {
  const int e = blockIdx.x;
  int c = 0;
  for (int i = threadIdx.x; i < nslot; i += 256) c += ids[i] == e;
  __shared__ int red[4];
  for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) p.count[e] = red[0] + red[1] + red[2] + red[3];
}

// One workgroup of 1024 threads; E <= 1024.
__global__ __launch_bounds__(1024) void k_schedule(int E, int bm, Perm p) {
  __shared__ int s_w[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = tid < E ? p.count[tid] : 0;
  const int nt = static_cast<int>(cdiv(c, bm));
  int ic = c, it = nt;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int a = __shfl_up(ic, m, 64), b = __shfl_up(it, m, 64);
    if (lane >= m) {
      ic += a;
      it += b;
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
    p.offset[tid] = off;
    for (int j = 0; j < nt; ++j) {
      p.tile_expert[toff + j] = tid;
      p.tile_m0[toff + j] = j * bm;
    }
    if (tid == E - 1) {
      p.offset[E] = off + c;
      *p.n_tiles = toff + nt;
    }
  }
}

__global__ __launch_bounds__(256) void k_expert_scatter(const int32_t* __restrict__ ids, int nslot, Perm p) {
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = static_cast<int>(cdiv(cdiv(nslot, 4), 64) * 64);   // slots per wave, multiple of 64
  const int beg = wv * per, end = min(nslot, beg + per);
  int cnt = 0;
  for (int i = beg; i < end; i += 64) {
    const bool hit = (i + lane < end) && ids[i + lane] == e;
    cnt += __popcll(__ballot(hit));
  }
  __shared__ int s_c[4];
  if (lane == 0) s_c[wv] = cnt;
  __syncthreads();
  int base = p.offset[e];
  for (int w = 0; w < wv; ++w) base += s_c[w];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i = beg; i < end; i += 64) {
    const bool hit = (i + lane < end) && ids[i + lane] == e;
    const uint64_t m = __ballot(hit);
    if (hit) p.perm[base + __popcll(m & below)] = i + lane;
    base += __popcll(m);
  }
}

}  // namespace moe
