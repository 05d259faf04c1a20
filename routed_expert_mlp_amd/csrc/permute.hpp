// Token permutation by expert id for the grouped-GEMM prefill ("Module
// glm5next_mlp", Constants, MOE_MODULE: the token sort / permute / unpermute
// family).  The T*K routing slots (slot = t*K + k) are sorted by expert id,
// stably (ascending slot within an expert), with no global atomics, in
// chunks of 256 slots:
//   1. k_perm_hist:     per chunk, a histogram over experts (LDS) and each
//                       slot's rank among the chunk's slots of its expert;
//   2. k_perm_schedule: one workgroup sums the histograms into expert counts,
//                       scans them into offsets, cuts each expert's rows into
//                       BM-row GEMM tiles (those of more than small_rows rows
//                       first) and turns the histograms into the sorted
//                       position of each (chunk, expert) run;
//   3. k_perm_scatter:  one thread per slot writes it at run start + rank.
// Up to PERM_SMALL_MAX slots (decode-sized batches) k_perm_small does all
// three in one workgroup, with the order within an expert left free.
#pragma once

#include "common.hpp"

namespace moe {

struct Perm {
  int32_t* count;        // [E]
  int32_t* offset;       // [E + 1]
  int32_t* perm;         // [T*K]   sorted position -> slot
  int32_t* n_tiles;      // [2]    tiles, and how many of them (the first) hold more than small_rows rows
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

// Expert counts -> offsets, tiles and tile counts, for one workgroup of 1024
// threads (E <= 1024; thread tid < E holds expert tid's count c); returns the
// expert's offset.  s_w: LDS for the 16 wavefronts' partial sums.  Tiles of
// more than small_rows rows come first, in expert order, then the rest (an
// expert's last tile when it is that short), so that two GEMM kernels can
// each take one range; with small_rows = 0 the order is plain expert order.
__device__ __forceinline__ int perm_tiles(int c, int E, int bm, int small_rows, Perm p, int (*s_w)[16]) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nt = static_cast<int>(cdiv(c, bm));
  const int ns = (nt > 0 && c - (nt - 1) * bm <= small_rows) ? 1 : 0;   // a short last tile
  const int nb = nt - ns;
  int ic = c, ib = nb, is = ns;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int a = __shfl_up(ic, m, 64), t = __shfl_up(ib, m, 64), u = __shfl_up(is, m, 64);
    if (lane >= m) {
      ic += a;
      ib += t;
      is += u;
    }
  }
  if (lane == 63) {
    s_w[0][wv] = ic;
    s_w[1][wv] = ib;
    s_w[2][wv] = is;
  }
  __syncthreads();
  int bc = 0, bb = 0, bs = 0, nbig = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wv) {
      bc += s_w[0][w];
      bb += s_w[1][w];
      bs += s_w[2][w];
    }
    nbig += s_w[1][w];
  }
  const int off = bc + ic - c, boff = bb + ib - nb, soff = nbig + bs + is - ns;
  if (tid < E) {
    p.count[tid] = c;
    p.offset[tid] = off;
    for (int j = 0; j < nb; ++j) {
      p.tile_expert[boff + j] = tid;
      p.tile_m0[boff + j] = j * bm;
    }
    if (ns) {
      p.tile_expert[soff] = tid;
      p.tile_m0[soff] = nb * bm;
    }
    if (tid == E - 1) {
      p.offset[E] = off + c;
      p.n_tiles[0] = soff + ns;
      p.n_tiles[1] = nbig;
    }
  }
  return off;
}

// 2. One workgroup of 1024 threads: expert counts (sums over the chunks),
// offsets and tiles (perm_tiles), and base[b][e] = the sorted position of
// chunk b's first slot of expert e (a separate array, so the loads of both
// passes over the chunks stay in flight together).
__global__ __launch_bounds__(1024) void k_perm_schedule(int E, int nblk, int bm, int small_rows,
                                                        const int32_t* __restrict__ hist, int32_t* __restrict__ base,
                                                        Perm p) {
  __shared__ int s_w[3][16];
  const int tid = threadIdx.x;
  int c = 0;
  if (tid < E) {
#pragma unroll 16
    for (int b = 0; b < nblk; ++b) c += hist[static_cast<int64_t>(b) * E + tid];
  }
  const int off = perm_tiles(c, E, bm, small_rows, p, s_w);
  if (tid < E) {
    int run = off;
#pragma unroll 16
    for (int b = 0; b < nblk; ++b) {
      const int64_t q = static_cast<int64_t>(b) * E + tid;
      base[q] = run;
      run += hist[q];
    }
  }
}

// All three steps in one workgroup of 1024 threads for up to PERM_SMALL_MAX
// slots (decode-sized batches, where the three launches cost more than the
// work): LDS counts, the same offsets and tiles (perm_tiles), then each slot
// at its expert's offset plus an LDS counter.  The order of the slots within
// an expert is the order of those atomic increments, not ascending; no result
// depends on it (every row of a tile is computed alone and written back to its
// own slot).
constexpr int PERM_SMALL_MAX = 8192;

__global__ __launch_bounds__(1024) void k_perm_small(const int32_t* __restrict__ ids, int nslot, int E, int bm,
                                                     int small_rows, Perm p) {
  __shared__ int s_cnt[PERM_MAX_E];
  __shared__ int s_off[PERM_MAX_E];
  __shared__ int s_w[3][16];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) s_cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < nslot; i += 1024) atomicAdd(&s_cnt[ids[i]], 1);
  __syncthreads();
  const int c = tid < E ? s_cnt[tid] : 0;
  const int off = perm_tiles(c, E, bm, small_rows, p, s_w);
  if (tid < E) {
    s_off[tid] = off;
    s_cnt[tid] = 0;
  }
  __syncthreads();
  for (int i = tid; i < nslot; i += 1024) {
    const int e = ids[i];
    p.perm[s_off[e] + atomicAdd(&s_cnt[e], 1)] = i;
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
