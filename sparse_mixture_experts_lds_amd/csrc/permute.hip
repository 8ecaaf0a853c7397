// Grouping of (token, slot) pairs by local expert: LDS histogram, prefix sums
// and a stable scatter that keeps each pair's identity p = t*k + j.
//
// Operation (ExpertMesh README, feature list: activations grouped per expert
// with each token's identity and top-k slot kept; MoEEvolve "Architecture":
// capacity-factor dispatch, overflow dropped): pairs of each local expert are laid out in ascending p;
// with a capacity C only the first C of them are kept.
//
// Three launches, none of which depends on the order of atomic operations
// (two when the block histograms fit in one workgroup's LDS: that workgroup
// then counts too; two as well for up to 64 blocks, where every scatter
// workgroup does the scan's work for itself):
//   1. count:   one wave per block of kBlockPairs pairs builds the block's
//               per-expert histogram in LDS and writes it out;
//   2. scan:    one workgroup turns the histograms into per-block bases (an
//               exclusive scan over blocks, per expert), clamps each expert's
//               total to the capacity, scans over experts into the offsets and
//               also writes the m-tile prefix of the grouped GEMMs;
//   3. scatter: one workgroup per block, one wave per 64-pair chunk; each
//               lane finds the lanes of its chunk with the same expert by 11
//               ballots over the key bits (a wave multisplit) and takes its
//               rank from a popcount; per-wave counts become per-wave bases
//               in LDS, added to the block's base from the scan.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBlockPairs = 1024;
constexpr int kScanThreads = 1024;

// Local expert of pair p, or -1 (not resident, or an id outside [0, E)).
__device__ __forceinline__ int local_expert(const int32_t* __restrict__ ids, const int32_t* __restrict__ emap,
                                            int E, int E_loc, int p) {
  const int g = ids[p];
  if (g < 0 || g >= E) return -1;
  const int e = emap ? emap[g] : g;
  return (e >= 0 && e < E_loc) ? e : -1;
}

__global__ __launch_bounds__(256) void count_kernel(int P, const int32_t* __restrict__ ids,
                                                    const int32_t* __restrict__ emap, int E, int E_loc,
                                                    int32_t* __restrict__ counts) {
  __shared__ int32_t hist[kMaxE];
  for (int e = threadIdx.x; e < E_loc; e += 256) hist[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kBlockPairs;
  constexpr int PER = kBlockPairs / 256;
  int ev[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int p = p0 + threadIdx.x + 256 * i;
    ev[i] = p < P ? local_expert(ids, emap, E, E_loc, p) : -1;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (ev[i] >= 0) atomicAdd(&hist[ev[i]], 1);
  __syncthreads();
  int32_t* out = counts + (size_t)blockIdx.x * E_loc;
  for (int e = threadIdx.x; e < E_loc; e += 256) out[e] = hist[e];
}

// Block-wide exclusive scan of one value per thread (kScanThreads threads).
__device__ int block_exclusive_scan(int v, int* total, int* sh /* [kScanThreads/64] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kScanThreads / 64 ? sh[lane] : 0;
    int wi = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(wi, o, 64);
      if (lane >= o) wi += n;
    }
    if (lane < kScanThreads / 64) sh[lane] = wi - w;
    if (lane == kScanThreads / 64 - 1) sh[kScanThreads / 64] = wi;
  }
  __syncthreads();
  const int r = sh[wave] + incl - v;
  *total = sh[kScanThreads / 64];
  __syncthreads();
  return r;
}

// Per-m-tile table of the grouped GEMMs: {expert, first row, rows, 0}.
__device__ void write_tiles(int e, int off, int n, int BM, int mstart, int4* __restrict__ tab) {
  for (int mb = 0, r = 0; r < n; ++mb, r += BM) tab[mstart + mb] = int4{e, off + r, min(BM, n - r), 0};
}

// COUNT: the block histograms are built here, in LDS, by the one workgroup
// (the count launch is skipped); they are the same integers count_kernel
// writes, so the rest is unchanged.
// Measured on MI355X: 4 blocks (decode, 4096 pairs) 15.3 against 17.0 us for
// the grouping step; 32 blocks (granular) 25 against 16.5 us, the one
// workgroup's reads and LDS atomics then outweighing the saved launch.
constexpr int kFusedHistInts = 24576;  // blocks x local experts held in LDS
constexpr int kFusedMaxBlocks = 4;
constexpr int kScatterBasesMaxBlocks = 64;

template <bool COUNT>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(int P, const int32_t* __restrict__ ids,
                                                            const int32_t* __restrict__ emap, int E, int nblk,
                                                            int E_loc, int capacity, int BM,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ mtile_start,
                                                            int4* __restrict__ tile_tab) {
  __shared__ int sh[kScanThreads / 64 + 1];
  const int32_t* hsrc = counts;  // block histograms
  if constexpr (COUNT) {
    __shared__ int32_t hist[kFusedHistInts];
    for (int i = threadIdx.x; i < nblk * E_loc; i += kScanThreads) hist[i] = 0;
    __syncthreads();
    constexpr int U = 8;  // pairs per thread whose ids are in flight together
    for (int p0 = threadIdx.x; p0 < P; p0 += kScanThreads * U) {
      int ev[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = p0 + kScanThreads * u;
        ev[u] = p < P ? local_expert(ids, emap, E, E_loc, p) : -1;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = p0 + kScanThreads * u;
        if (ev[u] >= 0) atomicAdd(&hist[(p / kBlockPairs) * E_loc + ev[u]], 1);
      }
    }
    __syncthreads();
    hsrc = hist;
  }
  const int e = threadIdx.x;
  int kept = 0;
  if (e < E_loc) {
    int run = 0;
    constexpr int U = 16;  // blocks read per batch, all loads in flight together
    for (int b0 = 0; b0 < nblk; b0 += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = b0 + u < nblk ? hsrc[(size_t)(b0 + u) * E_loc + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b0 + u < nblk) counts[(size_t)(b0 + u) * E_loc + e] = run;  // exclusive base of the block
        run += v[u];
      }
    }
    kept = capacity > 0 ? min(run, capacity) : run;
  }
  int total;
  const int off = block_exclusive_scan(kept, &total, sh);
  if (e < E_loc) offsets[e] = off;
  if (e == 0) offsets[E_loc] = total;
  if (mtile_start != nullptr) {
    const int mt = (kept + BM - 1) / BM;
    int mtotal;
    const int moff = block_exclusive_scan(mt, &mtotal, sh);
    if (e < E_loc) mtile_start[e] = moff;
    if (e == 0) mtile_start[E_loc] = mtotal;
    if (tile_tab != nullptr && e < E_loc) write_tiles(e, off, kept, BM, moff, tile_tab);
  }
}

// One workgroup of kBlockPairs threads per block: wave w ranks chunk w (64
// pairs) by a ballot multisplit, the per-wave counts are turned into per-wave
// bases in LDS, and every lane then places its pair.
// BASES false: counts holds the scan's per-block bases and offsets the
// expert offsets.  BASES true (no scan launch): counts holds the raw block
// histograms; every workgroup sums them itself (thread e: expert e, the
// blocks before its own and all blocks) and scans the clamped totals into the
// offsets, and workgroup 0 writes the offsets and the m-tile table, the same
// integers the scan kernel writes.  Each workgroup then reads nblk x E_loc
// counts, so this form is for few blocks.
template <bool BASES>
__global__ __launch_bounds__(kBlockPairs) void scatter_kernel(int P, const int32_t* __restrict__ ids,
                                                              const int32_t* __restrict__ emap, int E, int E_loc,
                                                              int capacity, int nblk, int BM,
                                                              const int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ mtile_start,
                                                              int4* __restrict__ tile_tab,
                                                              int32_t* __restrict__ sorted_pair,
                                                              int32_t* __restrict__ pair_pos) {
  static_assert(kBlockPairs == kScanThreads, "the block scan takes every thread of the workgroup");
  constexpr int NW = kBlockPairs / 64;
  __shared__ int32_t base[kMaxE];            // block's first rank per expert (exclusive over blocks)
  __shared__ int32_t off[kMaxE];             // expert's first grouped row
  __shared__ uint16_t wbase[NW][kMaxE];      // per-wave counts, then per-wave bases within the block
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if constexpr (BASES) {
    __shared__ int sh[kScanThreads / 64 + 1];
    const int e = tid;
    int pre = 0, run = 0;
    if (e < E_loc) {
      constexpr int U = 16;  // blocks read per batch, all loads in flight together
      for (int b0 = 0; b0 < nblk; b0 += U) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = b0 + u < nblk ? counts[(size_t)(b0 + u) * E_loc + e] : 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (b0 + u == (int)blockIdx.x) pre = run;
          run += v[u];
        }
      }
    }
    const int kept = capacity > 0 ? min(run, capacity) : run;
    int total;
    const int o = block_exclusive_scan(kept, &total, sh);
    if (e < E_loc) {
      base[e] = pre;
      off[e] = o;
    }
    if (blockIdx.x == 0) {
      if (e < E_loc) offsets[e] = o;
      if (e == 0) offsets[E_loc] = total;
      if (mtile_start != nullptr) {
        int mtotal;
        const int moff = block_exclusive_scan((kept + BM - 1) / BM, &mtotal, sh);
        if (e < E_loc) mtile_start[e] = moff;
        if (e == 0) mtile_start[E_loc] = mtotal;
        if (tile_tab != nullptr && e < E_loc) write_tiles(e, o, kept, BM, moff, tile_tab);
      }
    }
  } else {
    const int32_t* cb = counts + (size_t)blockIdx.x * E_loc;
    for (int e = tid; e < E_loc; e += kBlockPairs) {
      base[e] = cb[e];
      off[e] = offsets[e];
    }
  }
  for (int i = tid; i < NW * E_loc; i += kBlockPairs) wbase[i / E_loc][i % E_loc] = 0;
  const int p = blockIdx.x * kBlockPairs + tid;
  const int e = p < P ? local_expert(ids, emap, E, E_loc, p) : -1;
  const int key = e + 1;  // 0 = not local / past the end
  uint64_t peers = ~0ull;
#pragma unroll
  for (int b = 0; b < 11; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(peers & lt_mask);
  __syncthreads();
  if (e >= 0 && rank == 0) wbase[wave][e] = (uint16_t)__popcll(peers);
  __syncthreads();
  for (int x = tid; x < E_loc; x += kBlockPairs) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = wbase[w][x];
      wbase[w][x] = (uint16_t)run;
      run += c;
    }
  }
  __syncthreads();
  if (p < P) {
    const int r = e >= 0 ? base[e] + wbase[wave][e] + rank : 0;
    const bool kept = e >= 0 && (capacity == 0 || r < capacity);
    const int pos = kept ? off[e] + r : -1;
    pair_pos[p] = pos;
    if (kept) sorted_pair[pos] = p;
  }
}

__global__ __launch_bounds__(1024) void mtile_kernel(int E_loc, int BM, const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ mtile_start, int4* __restrict__ tile_tab) {
  __shared__ int sh[kScanThreads / 64 + 1];
  const int e = threadIdx.x;
  const int n = e < E_loc ? offsets[e + 1] - offsets[e] : 0;
  int total;
  const int moff = block_exclusive_scan((n + BM - 1) / BM, &total, sh);
  if (e < E_loc) mtile_start[e] = moff;
  if (e == 0) mtile_start[E_loc] = total;
  if (e < E_loc) write_tiles(e, offsets[e], n, BM, moff, tile_tab);
}

template <typename V>
__global__ __launch_bounds__(256) void gather_kernel(int rows_max, int vec_per_row, const V* __restrict__ x,
                                                     const int32_t* __restrict__ sorted_pair, int k,
                                                     const int32_t* __restrict__ offsets_end,
                                                     V* __restrict__ x_perm) {
  const int n_rows = *offsets_end;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t r = i / vec_per_row;
  if (r >= (size_t)n_rows || r >= (size_t)rows_max) return;
  const int c = (int)(i - r * vec_per_row);
  const int t = sorted_pair[r] / k;
  x_perm[r * vec_per_row + c] = x[(size_t)t * vec_per_row + c];
}

__global__ void zero_offsets_kernel(int E_loc, int32_t* offsets, int32_t* mtile_start) {
  for (int e = threadIdx.x; e <= E_loc; e += blockDim.x) {
    offsets[e] = 0;
    if (mtile_start) mtile_start[e] = 0;
  }
}

// Owner-grouped dispatch: the composed key owner(e) * (E/n) + local(e) puts
// every expert at its place in owner-major order, so the grouping above sorts
// the pairs by (owner, local expert, p) in the same single pass.
__global__ void placement_map_kernel(int E, int n_owners, int rule, int32_t* __restrict__ map) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int per = E / n_owners;
  const int o = rule == 0 ? e % n_owners : e / per;
  const int l = rule == 0 ? e / n_owners : e % per;
  map[e] = o * per + l;
}

__global__ void owner_offsets_kernel(int n_owners, int per, const int32_t* __restrict__ eo,
                                     int32_t* __restrict__ owner_offsets, int32_t* __restrict__ recv) {
  const int total = n_owners * (per + 1);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const int o = i / (per + 1), l = i - o * (per + 1);
    if (recv) recv[i] = eo[o * per + l] - eo[o * per];
    if (i <= n_owners) owner_offsets[i] = eo[i * per];
  }
}

}  // namespace

int permute_block_pairs() { return kBlockPairs; }

size_t permute_ws_bytes(int P, int E_loc) {
  const size_t nblk = ((size_t)P + kBlockPairs - 1) / kBlockPairs;
  return (nblk > 0 ? nblk : 1) * (size_t)E_loc * sizeof(int32_t);
}

hipError_t launch_permute(int T, int k, int E, const int32_t* ids, const int32_t* expert_map, int E_loc,
                          int capacity, int BM, int32_t* offsets, int32_t* mtile_start, int4* tile_tab,
                          int32_t* sorted_pair, int32_t* pair_pos, int32_t* counts, hipStream_t s) {
  const int P = T * k;
  if (P == 0) {
    zero_offsets_kernel<<<1, 256, 0, s>>>(E_loc, offsets, mtile_start);
    return hipGetLastError();
  }
  const int nblk = (P + kBlockPairs - 1) / kBlockPairs;
  if (nblk <= kFusedMaxBlocks && (long long)nblk * E_loc <= kFusedHistInts) {
    // few blocks: one workgroup counts and scans (one launch fewer)
    scan_kernel<true><<<1, kScanThreads, 0, s>>>(P, ids, expert_map, E, nblk, E_loc, capacity, BM, counts, offsets,
                                                 mtile_start, tile_tab);
  } else if (nblk <= kScatterBasesMaxBlocks) {
    // few blocks: the scatter workgroups form their own bases (one launch fewer)
    count_kernel<<<nblk, 256, 0, s>>>(P, ids, expert_map, E, E_loc, counts);
    scatter_kernel<true><<<nblk, kBlockPairs, 0, s>>>(P, ids, expert_map, E, E_loc, capacity, nblk, BM, counts,
                                                      offsets, mtile_start, tile_tab, sorted_pair, pair_pos);
    return hipGetLastError();
  } else {
    count_kernel<<<nblk, 256, 0, s>>>(P, ids, expert_map, E, E_loc, counts);
    scan_kernel<false><<<1, kScanThreads, 0, s>>>(P, ids, expert_map, E, nblk, E_loc, capacity, BM, counts,
                                                  offsets, mtile_start, tile_tab);
  }
  scatter_kernel<false><<<nblk, kBlockPairs, 0, s>>>(P, ids, expert_map, E, E_loc, capacity, nblk, BM, counts,
                                                     offsets, mtile_start, tile_tab, sorted_pair, pair_pos);
  return hipGetLastError();
}

hipError_t launch_owner_dispatch(int T, int k, int E, int n_owners, int rule, int capacity, const int32_t* ids,
                                 int32_t* owner_offsets, int32_t* recv_offsets, int32_t* expert_offsets,
                                 int32_t* sorted_pair, int32_t* pair_pos, int32_t* map, int32_t* counts,
                                 hipStream_t s) {
  placement_map_kernel<<<(E + 255) / 256, 256, 0, s>>>(E, n_owners, rule, map);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_permute(T, k, E, ids, map, E, capacity, 16, expert_offsets, nullptr, nullptr, sorted_pair, pair_pos,
                     counts, s);
  if (e != hipSuccess) return e;
  const int total = n_owners * (E / n_owners + 1);
  owner_offsets_kernel<<<std::min((total + 255) / 256, 64), 256, 0, s>>>(n_owners, E / n_owners, expert_offsets,
                                                                          owner_offsets, recv_offsets);
  return hipGetLastError();
}

hipError_t launch_mtile_prefix(int E_loc, int BM, const int32_t* offsets, int32_t* mtile_start,
                               int4* tile_tab, hipStream_t s) {
  mtile_kernel<<<1, 1024, 0, s>>>(E_loc, BM, offsets, mtile_start, tile_tab);
  return hipGetLastError();
}

hipError_t launch_gather_rows(int rows_max, int d, bool bf16, const void* x, const int32_t* sorted_pair,
                              int k, const int32_t* offsets_end, void* x_perm, hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  const int vec = bf16 ? d / 8 : d / 4;  // 16-byte vectors per row
  const size_t n = (size_t)rows_max * vec;
  const dim3 grid((unsigned)((n + 255) / 256));
  gather_kernel<u32x4><<<grid, 256, 0, s>>>(rows_max, vec, static_cast<const u32x4*>(x), sorted_pair, k,
                                            offsets_end, static_cast<u32x4*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
