// Router by-products of one batch (moe_stream.py, MoEFFN.forward, the
// load-balancing part): per-expert token counts, the mean softmax probability
// of each expert over the batch, and the batch-local balance loss
//   count[e] = #{t : e in topk_ids[t, :]}      (a token counts once per expert)
//   P[e]     = (1/T) sum_t softmax(L[t, :])[e]  over all E experts
//   loss     = E * sum_e (count[e] / T) * P[e]
// with L = logits (+ bias).  Ids outside [0, E) match no expert.
//
// Two passes, both in a fixed order so the result does not depend on
// scheduling: each workgroup of the first pass owns a fixed strided set of
// tokens (one wave per token row; lane l holds experts l + 64i), keeps fp64
// column sums of the softmax in registers and integer counts in LDS, and
// writes one [E] row of partials; one workgroup of the second pass adds the
// rows in block order in fp64 and forms the loss.  The logits are read once,
// so the first pass is bound by HBM at T*E*4 + T*k*4 bytes.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kStatsWaves = 4;
constexpr int kStatsMinTokensPerBlock = 32;
constexpr int kStatsMaxBlocks = 256;
constexpr int kStatsMaxPartials = 65536;  // partial rows * E, bounds the workspace

template <int NV>
__global__ __launch_bounds__(256) void stats_partial_kernel(int T, int E, int k, const float* __restrict__ logits,
                                                            const float* __restrict__ bias,
                                                            const int32_t* __restrict__ ids,
                                                            double* __restrict__ part_p,
                                                            int32_t* __restrict__ part_c) {
  constexpr int EW = NV * 64;
  __shared__ double red[kStatsWaves][EW];
  __shared__ int cnt[EW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < EW; e += blockDim.x) cnt[e] = 0;
  __syncthreads();

  float b[NV];
  double acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    b[i] = (bias != nullptr && e < E) ? bias[e] : 0.f;
    acc[i] = 0.0;
  }
  const int stride = gridDim.x * kStatsWaves;
  for (int t = blockIdx.x * kStatsWaves + wave; t < T; t += stride) {
    const float* row = logits + (size_t)t * E;
    float v[NV];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? row[e] + b[i] : -INFINITY;
      m = fmaxf(m, v[i]);
    }
    m = wave_max(m);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      v[i] = lane + 64 * i < E ? expf(v[i] - m) : 0.f;
      s += v[i];
    }
    s = wave_sum(s);
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] += (double)(v[i] / s);

    // lane j < k holds slot j; a slot whose id already appears in a lower
    // slot of the same token is not counted again
    const int id = lane < k ? ids[(size_t)t * k + lane] : -1;
    bool dup = false;
    for (int j = 0; j < k; ++j) {
      const int o = __shfl(id, j);
      dup |= (j < lane) && (o == id);
    }
    if (lane < k && !dup && id >= 0 && id < E) atomicAdd(&cnt[id], 1);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) red[wave][lane + 64 * i] = acc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double p = red[0][e];
#pragma unroll
    for (int w = 1; w < kStatsWaves; ++w) p += red[w][e];
    part_p[(size_t)blockIdx.x * E + e] = p;
    part_c[(size_t)blockIdx.x * E + e] = cnt[e];
  }
}

__global__ __launch_bounds__(1024) void stats_final_kernel(int T, int E, int nblk, const double* __restrict__ part_p,
                                                           const int32_t* __restrict__ part_c,
                                                           int32_t* __restrict__ counts, float* __restrict__ prob_mean,
                                                           float* __restrict__ loss) {
  __shared__ double red[1024];
  double tot = 0.0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    // four interleaved chains (blocks b = 0,1,2,3 mod 4) for load parallelism,
    // added in a fixed order at the end
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    int c = 0;
    int b = 0;
    for (; b + 4 <= nblk; b += 4) {
      s0 += part_p[(size_t)(b + 0) * E + e];
      s1 += part_p[(size_t)(b + 1) * E + e];
      s2 += part_p[(size_t)(b + 2) * E + e];
      s3 += part_p[(size_t)(b + 3) * E + e];
      c += part_c[(size_t)(b + 0) * E + e] + part_c[(size_t)(b + 1) * E + e] + part_c[(size_t)(b + 2) * E + e] +
           part_c[(size_t)(b + 3) * E + e];
    }
    for (; b < nblk; ++b) {
      s0 += part_p[(size_t)b * E + e];
      c += part_c[(size_t)b * E + e];
    }
    const double s = (s0 + s1) + (s2 + s3);
    if (counts) counts[e] = c;
    if (prob_mean) prob_mean[e] = T > 0 ? (float)(s / (double)T) : 0.f;
    tot += (double)c * s;
  }
  red[threadIdx.x] = tot;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0 && loss) loss[0] = T > 0 ? (float)((double)E * red[0] / ((double)T * (double)T)) : 0.f;
}

template <int NV>
void launch_partial(int nblk, int T, int E, int k, const float* logits, const float* bias, const int32_t* ids,
                    double* part_p, int32_t* part_c, hipStream_t s) {
  stats_partial_kernel<NV><<<nblk, 64 * kStatsWaves, 0, s>>>(T, E, k, logits, bias, ids, part_p, part_c);
}

}  // namespace

int router_stats_blocks(int T, int E) {
  if (T <= 0 || E <= 0) return 0;
  const int cap = std::max(1, std::min(kStatsMaxBlocks, kStatsMaxPartials / E));
  return std::min(cap, (T + kStatsMinTokensPerBlock - 1) / kStatsMinTokensPerBlock);
}

size_t router_stats_ws_bytes(int T, int E) {
  const size_t n = (size_t)router_stats_blocks(T, E) * (size_t)std::max(E, 0);
  return ((n * 8 + 255) & ~(size_t)255) + ((n * 4 + 255) & ~(size_t)255);
}

hipError_t launch_router_stats(int T, int E, int k, const float* logits, const float* bias, const int32_t* ids,
                               int32_t* counts, float* prob_mean, float* loss, void* ws, hipStream_t s) {
  const int nblk = router_stats_blocks(T, E);
  const size_t n = (size_t)nblk * E;
  double* part_p = static_cast<double*>(ws);
  int32_t* part_c = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(ws) + ((n * 8 + 255) & ~(size_t)255));
  if (nblk > 0) {
    const int nv = (E + 63) / 64;
    if (nv <= 1)
      launch_partial<1>(nblk, T, E, k, logits, bias, ids, part_p, part_c, s);
    else if (nv <= 2)
      launch_partial<2>(nblk, T, E, k, logits, bias, ids, part_p, part_c, s);
    else if (nv <= 4)
      launch_partial<4>(nblk, T, E, k, logits, bias, ids, part_p, part_c, s);
    else if (nv <= 8)
      launch_partial<8>(nblk, T, E, k, logits, bias, ids, part_p, part_c, s);
    else
      launch_partial<16>(nblk, T, E, k, logits, bias, ids, part_p, part_c, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  stats_final_kernel<<<1, 1024, 0, s>>>(T, E, nblk, part_p, part_c, counts, prob_mean, loss);
  return hipGetLastError();
}

}  // namespace moe
