// Router by-products of one batch (moe_stream.py, MoEFFN.forward, the
// load-balancing part): per-expert token counts, the mean softmax probability
// of each expert over the batch, and the batch-local balance loss
//   count[e] = #{t : e in topk_ids[t, :]}      (a token counts once per expert)
//   P[e]     = (1/T) sum_t softmax(L[t, :])[e]  over all E experts
//   loss     = E * sum_e (count[e] / T) * P[e]
// with L = logits (+ bias).  Ids outside [0, E) match no expert.
//
// Two passes, each in a fixed order so the result does not depend on
// scheduling: each workgroup of the first pass owns a fixed strided set of
// tokens (a group of lanes per token row), keeps fp64 column sums of the
// softmax in registers and integer counts in LDS, and writes one [E] row of
// partials; the second pass adds the rows column by column (one workgroup per
// 64 experts), and the last of its workgroups folds the loss terms in expert
// order.  The logits are read once: the first pass moves
// T*E*4 + T*k*4 bytes, the partial rows at most 12*E*256 more.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kStatsMaxBlocks = 256;
constexpr int kStatsMaxPartials = 65536;  // partial rows * E, bounds the workspace
constexpr int kColWaves = 16;             // waves of a column-reduction workgroup

// First pass.  One group of G lanes per token (G = 16: one DPP row, for
// E <= 256 and k <= 16; else G = 64, the wave); lane g of a group holds experts
// g + G*i, so every lane keeps the same columns for all its tokens and adds
// their probabilities in fp64 registers.  A group takes U tokens at a time so
// the loads and reductions of the U rows overlap.  Counting a token once per
// expert: the lanes of its slots swap the token id into a per-group LDS stamp
// of the expert, and only a lane that finds another value there counts.
template <int G, int NV, int U>
__global__ __launch_bounds__(256) void stats_partial_kernel(int T, int E, int k, const float* __restrict__ logits,
                                                            const float* __restrict__ bias,
                                                            const int32_t* __restrict__ ids,
                                                            double* __restrict__ part_p,
                                                            int32_t* __restrict__ part_c, unsigned* counter) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *counter = 0;  // for the second pass's election
  constexpr int NG = 256 / G;  // groups per workgroup
  constexpr int EW = NV * G;   // expert columns covered by a group (>= E)
  __shared__ double red[NG][EW];
  __shared__ int stamp[NG][EW];
  __shared__ int cnt[EW];
  const int gl = threadIdx.x & (G - 1), grp = threadIdx.x / G;
  for (int e = threadIdx.x; e < EW; e += blockDim.x) cnt[e] = 0;
  for (int i = threadIdx.x; i < NG * EW; i += blockDim.x) (&stamp[0][0])[i] = -1;
  __syncthreads();

  float b[NV];
  double acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = gl + G * i;
    b[i] = (bias != nullptr && e < E) ? bias[e] : 0.f;
    acc[i] = 0.0;
  }
  const int stride = gridDim.x * NG;  // groups in the grid
  for (int t0 = blockIdx.x * NG + grp; t0 < T; t0 += U * stride) {
    float v[U][NV];
    float m[U], sum[U];
    int id[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * stride;  // uniform over the group
      const bool ok = t < T;
      const float* row = logits + (size_t)(ok ? t : 0) * E;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = gl + G * i;
        v[u][i] = (ok && e < E) ? row[e] + b[i] : -INFINITY;
      }
      id[u] = (ok && gl < k) ? ids[(size_t)t * k + gl] : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float mm = v[u][0];
#pragma unroll
      for (int i = 1; i < NV; ++i) mm = fmaxf(mm, v[u][i]);
      m[u] = group_max<G>(mm);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = t0 + u * stride < T;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        v[u][i] = (ok && gl + G * i < E) ? expf(v[u][i] - m[u]) : 0.f;
        ss += v[u][i];
      }
      sum[u] = group_sum<G>(ss);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t0 + u * stride < T) {  // a row past T has sum 0
        const float inv = 1.f / sum[u];  // one division per token; p within 1.5 ulp
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i] += (double)(v[u][i] * inv);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * stride;
      if (id[u] >= 0 && id[u] < E) {
        const int prev = atomicExch(&stamp[grp][id[u]], t);
        if (prev != t) atomicAdd(&cnt[id[u]], 1);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) red[grp][gl + G * i] = acc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double p = red[0][e];
#pragma unroll
    for (int g = 1; g < NG; ++g) p += red[g][e];
    part_p[(size_t)blockIdx.x * E + e] = p;
    part_c[(size_t)blockIdx.x * E + e] = cnt[e];
  }
}

// Second pass, a grid of (64-expert chunk c, row range r) workgroups: wave w
// adds the partial rows b = b0 + w, b0 + w + 16, ... of range r (at most
// kColRows, loaded together), then wave 0 adds the 16 wave sums in wave order
// into mid[r][e].  The workgroup that counts last on `counter` (zeroed by the
// first pass) finishes: thread e adds mid[0..RS-1][e] in order, writes the
// count and mean of expert e, and the workgroup folds the loss terms
// count[e] * colsum[e] in a fixed order.  Nothing waits:
// the last arrival finds every range published (release/acquire on the
// counter).
constexpr int kMaxRowSplits = kStatsMaxRowSplits;
constexpr int kColRows = 8;  // partial rows a thread of the second pass adds
static_assert(kStatsFinishMaxRows == kMaxRowSplits * 16 * kColRows, "rows of the second pass");

__global__ __launch_bounds__(64 * kColWaves) void stats_column_kernel(int T, int E, int nblk,
                                                                     const double* __restrict__ part_p,
                                                                     const int32_t* __restrict__ part_c,
                                                                     int32_t* __restrict__ counts,
                                                                     float* __restrict__ prob_mean,
                                                                     double* mid_p, int32_t* mid_c,
                                                                     unsigned* counter, float* __restrict__ loss) {
  __shared__ double rs[kColWaves][64];
  __shared__ int rc[kColWaves][64];
  __shared__ double lw[kColWaves];
  __shared__ bool last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int RS = gridDim.y, r = blockIdx.y;
  const int b0 = (int)((long long)nblk * r / RS), b1 = (int)((long long)nblk * (r + 1) / RS);
  const int e = blockIdx.x * 64 + lane;
  const int ec = e < E ? e : E - 1;
  // rows b0 + wave + 16 q: at most kColRows per wave, all loads issued together
  // (rows past the range re-read row b0 and are not added)
  double s[kColRows];
  int cv[kColRows];
#pragma unroll
  for (int q = 0; q < kColRows; ++q) {
    const int b = b0 + wave + kColWaves * q;
    const int bb = b < b1 ? b : b0;
    s[q] = part_p[(size_t)bb * E + ec];
    cv[q] = part_c[(size_t)bb * E + ec];
  }
  double sum = 0.0;
  int c = 0;
#pragma unroll
  for (int q = 0; q < kColRows; ++q)
    if (b0 + wave + kColWaves * q < b1 && e < E) {
      sum += s[q];
      c += cv[q];
    }
  rs[wave][lane] = sum;
  rc[wave][lane] = c;
  __syncthreads();
  if (wave == 0) {
    double tot = rs[0][lane];
    int ct = rc[0][lane];
#pragma unroll
    for (int w = 1; w < kColWaves; ++w) {
      tot += rs[w][lane];
      ct += rc[w][lane];
    }
    if (e < E) {
      mid_p[(size_t)r * E + e] = tot;
      mid_c[(size_t)r * E + e] = ct;
    }
    // publish this workgroup's range, then count it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane == 0) {
      const unsigned arrived = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      last = arrived == gridDim.x * gridDim.y - 1;
    }
  }
  __syncthreads();
  if (!last) return;  // the whole workgroup leaves together
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // thread t finishes expert t (E <= 1024): the ranges' sums in range order
  const int t = threadIdx.x;
  const int tc = t < E ? t : E - 1;
  double mp[kStatsMaxRowSplits];
  int mc[kStatsMaxRowSplits];
#pragma unroll
  for (int rr = 0; rr < kStatsMaxRowSplits; ++rr) {
    const int ri = rr < RS ? rr : 0;
    mp[rr] = mid_p[(size_t)ri * E + tc];
    mc[rr] = mid_c[(size_t)ri * E + tc];
  }
  double tot = 0.0;
  int ct = 0;
#pragma unroll
  for (int rr = 0; rr < kStatsMaxRowSplits; ++rr)
    if (rr < RS) {
      tot += mp[rr];
      ct += mc[rr];
    }
  double term = 0.0;
  if (t < E) {
    if (counts) counts[t] = ct;
    if (prob_mean) prob_mean[t] = T > 0 ? (float)(tot / (double)T) : 0.f;
    term = (double)ct * tot;
  }
  if (!loss) return;
  // fixed order: within each wave a shuffle tree, then the wave sums in order
  for (int m = 32; m >= 1; m >>= 1) term += __shfl_down(term, m);
  if (lane == 0) lw[wave] = term;
  __syncthreads();
  if (t == 0) {
    double l = lw[0];
#pragma unroll
    for (int w = 1; w < kColWaves; ++w) l += lw[w];
    loss[0] = T > 0 ? (float)((double)E * l / ((double)T * (double)T)) : 0.f;
  }
}

inline int stats_row_splits(int nblk) {
  return std::max(1, std::min(kMaxRowSplits, (nblk + kColWaves * kColRows - 1) / (kColWaves * kColRows)));
}

__global__ void stats_empty_kernel(int E, int32_t* __restrict__ counts, float* __restrict__ prob_mean,
                                   float* __restrict__ loss) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    if (counts) counts[e] = 0;
    if (prob_mean) prob_mean[e] = 0.f;
  }
  if (threadIdx.x == 0 && loss) loss[0] = 0.f;
}

template <int G, int NV, int U>
void launch_partial(int nblk, int T, int E, int k, const float* logits, const float* bias, const int32_t* ids,
                    double* part_p, int32_t* part_c, unsigned* counter, hipStream_t s) {
  stats_partial_kernel<G, NV, U><<<nblk, 256, 0, s>>>(T, E, k, logits, bias, ids, part_p, part_c, counter);
}

inline int stats_group(int E, int k) { return (E <= 256 && k <= 16) ? 16 : 64; }

struct StatsWs {
  double* part_p;
  int32_t* part_c;
  double* mid_p;  // [kMaxRowSplits, E]
  int32_t* mid_c;
  unsigned* counter;
};

inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

StatsWs stats_ws(void* ws, int nblk, int E) {
  const size_t n = (size_t)nblk * E;
  unsigned char* p = static_cast<unsigned char*>(ws);
  StatsWs w;
  w.part_p = reinterpret_cast<double*>(p);
  w.part_c = reinterpret_cast<int32_t*>(p + al256(n * 8));
  const size_t m = (size_t)kMaxRowSplits * E;
  w.mid_p = reinterpret_cast<double*>(p + al256(n * 8) + al256(n * 4));
  w.mid_c = reinterpret_cast<int32_t*>(p + al256(n * 8) + al256(n * 4) + al256(m * 8));
  w.counter = reinterpret_cast<unsigned*>(p + al256(n * 8) + al256(n * 4) + al256(m * 8) + al256(m * 4));
  return w;
}

}  // namespace

int router_stats_blocks(int T, int E) {
  if (T <= 0 || E <= 0) return 0;
  const int cap = std::max(1, std::min(kStatsMaxBlocks, kStatsMaxPartials / E));
  // two tokens per group at least (a 64-lane group when E > 256): fewer
  // partial rows than that would cost more to add up than they save
  const int per_block = 2 * (E <= 256 ? 16 : 4);
  return std::min(cap, (T + per_block - 1) / per_block);
}

size_t router_stats_ws_bytes(int T, int E) {
  const int nblk = router_stats_blocks(T, E);
  if (nblk == 0) return 0;  // an empty batch needs no workspace
  const size_t n = (size_t)nblk * (size_t)E;
  const size_t m = (size_t)kMaxRowSplits * E;
  return al256(n * 8) + al256(n * 4) + al256(m * 8) + al256(m * 4) + 256;
}

size_t stats_finish_bytes(int E) {
  const size_t m = (size_t)kMaxRowSplits * E;
  return al256(m * 8) + al256(m * 4) + 256;
}

hipError_t launch_stats_finish(int T, int E, int nblk, const StatsPart& sp, int32_t* counts, float* prob_mean,
                               float* loss, hipStream_t s) {
  if (nblk < 1 || nblk > kStatsFinishMaxRows) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((E + 63) / 64), (unsigned)stats_row_splits(nblk));
  stats_column_kernel<<<grid, 64 * kColWaves, 0, s>>>(T, E, nblk, sp.part_p, sp.part_c, counts, prob_mean, sp.mid_p,
                                                      sp.mid_c, sp.counter, loss);
  return hipGetLastError();
}

hipError_t launch_router_stats(int T, int E, int k, const float* logits, const float* bias, const int32_t* ids,
                               int32_t* counts, float* prob_mean, float* loss, void* ws, hipStream_t s) {
  const int nblk = router_stats_blocks(T, E);
  if (nblk == 0) {
    stats_empty_kernel<<<1, 256, 0, s>>>(E, counts, prob_mean, loss);
    return hipGetLastError();
  }
  const StatsWs w = stats_ws(ws, nblk, E);
  {
    const int G = stats_group(E, k);
    const int nv = (E + G - 1) / G;
#define MOE_STATS(Gv, NVv, Uv) \
  launch_partial<Gv, NVv, Uv>(nblk, T, E, k, logits, bias, ids, w.part_p, w.part_c, w.counter, s)
    if (G == 16) {
      if (nv <= 1) MOE_STATS(16, 1, 4);
      else if (nv <= 2) MOE_STATS(16, 2, 4);
      else if (nv <= 4) MOE_STATS(16, 4, 2);
      else if (nv <= 8) MOE_STATS(16, 8, 2);
      else MOE_STATS(16, 16, 2);
    } else {
      if (nv <= 1) MOE_STATS(64, 1, 4);
      else if (nv <= 2) MOE_STATS(64, 2, 4);
      else if (nv <= 4) MOE_STATS(64, 4, 2);
      else if (nv <= 8) MOE_STATS(64, 8, 2);
      else MOE_STATS(64, 16, 2);
    }
#undef MOE_STATS
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)((E + 63) / 64), (unsigned)stats_row_splits(nblk));
  stats_column_kernel<<<grid, 64 * kColWaves, 0, s>>>(T, E, nblk, w.part_p, w.part_c, counts, prob_mean, w.mid_p,
                                                      w.mid_c, w.counter, loss);
  return hipGetLastError();
}

}  // namespace moe
