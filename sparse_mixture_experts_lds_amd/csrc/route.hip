// Router step: logits GEMM on MFMA, softmax and wave-level top-k selection.
//
// Operation ("Sharding d'experts", "Deux roles": the backbone routes once,
// softmax of the router logits then the k most probable experts;
// moe_stream.py MoEFFN.forward: bias-free router, per-expert bias added before
// the softmax, softmax over all experts, top k, gates divided by their sum):
//   L[t,e]   = sum_i x[t,i] w[e,i] + b[e]           (fp32 accumulate)
//   ids[t,j] = j-th largest L[t,.], ties to the lower expert id
//   w[t,j]   = exp(L_j - m) / (renorm ? sum_sel exp(L - m) : sum_all exp(L - m))
//
// Two kernels.  The logits kernel: one workgroup (4 waves) handles 16 tokens
// and builds the logits tile [16, E] in LDS (MFMA 16x16x32 bf16 or 16x16x4 f32,
// each wave a strided set of 16-expert column fragments); it either selects
// for its tokens directly or only writes the logits.  The select kernel takes
// logits from memory with a group of G lanes per token (16 with many tokens
// and E <= 256, else the whole wave).  Selection: every lane of the group
// holds E/G logits in registers and k rounds of a (value, lower-id) group
// arg-max pick the experts.  When the activations are bf16 and E is a multiple of 64
// the logits of a whole layer come from the grouped GEMM kernel (one group,
// fp32 output) instead, which reuses each router weight slice across 16-64
// tokens per workgroup rather than 16.  Few tokens with long rows (decode)
// leave most CUs idle on either kernel; there the logits kernel splits the
// inputs into slices, each workgroup sums one slice into its own partial
// array, and the select kernel adds the partials in ascending slice order.
// When the whole router weight fits in LDS (few experts), a third logits
// kernel keeps it there and streams only the token rows.  With many tokens
// and at most 64 experts (bf16), a fourth kernel computes a 32-token tile's
// logits and selects its tokens' experts in the same launch.
#include <algorithm>

#include "ffn_wide.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokTile = 16;
constexpr int kSelectGroupMinTok = 4096;  // 16-lane selection groups from here on

// Softmax and top-k of one token held by one wave: lane l holds experts l+64i in
// v[i] (-inf past E).  Writes k ids (descending logit, ties to the lower id) and
// their gates (renormalised over the selection, or over all E).
template <int NF>
__device__ __forceinline__ void select_token(const float (&v)[NF], int E, int k, int renorm, int lane,
                                             int32_t* ids_row, float* tw_row) {
  float m = v[0];
#pragma unroll
  for (int i = 1; i < NF; ++i) m = fmaxf(m, v[i]);
  m = wave_max(m);
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < NF; ++i)
    if (lane + 64 * i < E) se += expf(v[i] - m);
  const float sum_all = wave_sum(se);

  uint32_t taken = 0;
  float my_v = -INFINITY;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int e = lane + 64 * i;
      // strict '>' keeps the lower id among this lane's equal values
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || be == 0x7fffffff)) {
        bv = v[i];
        be = e;
      }
    }
    group_argmax<64>(bv, be);
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  const float ex = lane < k ? expf(my_v - m) : 0.f;
  const float denom = renorm ? wave_sum(ex) : sum_all;
  if (lane < k) {
    ids_row[lane] = my_e;
    tw_row[lane] = ex / denom;
  }
}

// SELECT false: only the logits (without bias) are written, to logits_out.
// Without SELECT the inputs are split into gridDim.y slices of kspan: slice s
// = blockIdx.y sums inputs [s kspan, (s+1) kspan) into logits_out + s T E.
template <int NF, bool BF16, bool SELECT>
__global__ __launch_bounds__(256) void route_kernel(int T, int d, int E, int k, int kspan,
                                                    const void* __restrict__ xv, const void* __restrict__ wv,
                                                    const float* __restrict__ bias, int renorm,
                                                    int32_t* __restrict__ ids, float* __restrict__ tw,
                                                    float* __restrict__ logits_out) {
  constexpr int ES = NF * 64;  // logits row stride in LDS (E padded)
  __shared__ float Ls[kTokTile * ES];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kTokTile;
  const int kbeg = blockIdx.y * kspan;
  const int kend = kbeg + kspan;
  if (!SELECT && logits_out) logits_out += (size_t)blockIdx.y * T * E;

  {
    const int row = lane & 15;  // A row (token) / B column (expert) inside a fragment
    const int q = lane >> 4;    // K slice held by this lane group
    const int t = t0 + row;
    const bool tok_ok = t < T;
    f32x4 acc[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The k-loop runs in chunks of KC MFMA steps: every load of a chunk is
    // issued before its first MFMA, so each wave keeps KC*(NF+1) loads in flight.
    if constexpr (BF16) {
      constexpr int KC = 8;
      const uint16_t* x = static_cast<const uint16_t*>(xv);
      const uint16_t* w = static_cast<const uint16_t*>(wv);
      const uint16_t* xrow = x + (size_t)(tok_ok ? t : 0) * d + 8 * q;
      const uint16_t* wrow[NF];
      bool e_ok[NF];
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int e = 16 * (wave + 4 * i) + row;
        e_ok[i] = e < E;
        wrow[i] = w + (size_t)(e_ok[i] ? e : 0) * d + 8 * q;
      }
      for (int k0 = kbeg; k0 < kend; k0 += 32 * KC) {
        const int nk = min(KC, (kend - k0) / 32);
        u32x4 av[KC], bv[KC][NF];
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const int kk = k0 + 32 * min(c, nk - 1);  // in-bounds re-read past the end; not used
          av[c] = *reinterpret_cast<const u32x4*>(xrow + kk);
#pragma unroll
          for (int i = 0; i < NF; ++i) bv[c][i] = *reinterpret_cast<const u32x4*>(wrow[i] + kk);
        }
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          if (c < nk) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, tok_ok ? av[c] : u32x4{0, 0, 0, 0});
#pragma unroll
            for (int i = 0; i < NF; ++i)
              acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  a, __builtin_bit_cast(bf16x8, e_ok[i] ? bv[c][i] : u32x4{0, 0, 0, 0}), acc[i], 0, 0, 0);
          }
        }
      }
    } else {
      // fp32: products and sums in fp64 (each fp32 product is exact there),
      // so the logits carry only their final rounding to fp32; fp32 sums over
      // d inputs moved the gates, and through them the layer's fp32 output,
      // by up to 1e-5 of its RMS on layers whose capacity drops most rows
      constexpr int KC = 16;
      f64x4 accd[NF];
#pragma unroll
      for (int i = 0; i < NF; ++i) accd[i] = f64x4{0.0, 0.0, 0.0, 0.0};
      const float* x = static_cast<const float*>(xv);
      const float* w = static_cast<const float*>(wv);
      const float* xrow = x + (size_t)(tok_ok ? t : 0) * d + q;
      const float* wrow[NF];
      bool e_ok[NF];
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int e = 16 * (wave + 4 * i) + row;
        e_ok[i] = e < E;
        wrow[i] = w + (size_t)(e_ok[i] ? e : 0) * d + q;
      }
      for (int k0 = kbeg; k0 < kend; k0 += 4 * KC) {
        const int nk = min(KC, (kend - k0) / 4);
        float av[KC], bv[KC][NF];
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const int kk = k0 + 4 * min(c, nk - 1);
          av[c] = xrow[kk];
#pragma unroll
          for (int i = 0; i < NF; ++i) bv[c][i] = wrow[i][kk];
        }
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          if (c < nk) {
            const float a = tok_ok ? av[c] : 0.f;
#pragma unroll
            for (int i = 0; i < NF; ++i)
              accd[i] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a, (double)(e_ok[i] ? bv[c][i] : 0.f),
                                                              accd[i], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][r] = (float)accd[i][r];
    }
    // D[i][j]: lane holds column j = lane & 15 and rows 4q + r (bf16 and fp32
    // MFMAs) or q + 4r (the fp64 MFMA, checked with an in-bounds probe on the GPU)
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int e = 16 * (wave + 4 * i) + row;
      if (e < E) {
        const float bv = (SELECT && bias) ? bias[e] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) Ls[(BF16 ? 4 * q + r : q + 4 * r) * ES + e] = acc[i][r] + bv;
      }
    }
  }
  __syncthreads();

  if (logits_out != nullptr) {
    for (int i = threadIdx.x; i < kTokTile * E; i += 256) {
      const int r = i / E, e = i - r * E;
      const int t = t0 + r;
      if (t < T) logits_out[(size_t)t * E + e] = Ls[r * ES + e];
    }
  }

  if constexpr (SELECT) {
    // wave w handles tokens w, w+4, w+8, w+12 of the tile
    for (int r = wave; r < kTokTile; r += 4) {
      const int t = t0 + r;
      if (t >= T) break;
      float v[NF];
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? Ls[r * ES + e] : -INFINITY;
      }
      select_token<NF>(v, E, k, renorm, lane, ids + (size_t)t * k, tw + (size_t)t * k);
    }
  }
}

// Softmax and top-k of one token held by a group of G lanes: lane gl holds
// experts gl + G i in v[i] (-inf past E).  k rounds of a group arg-max pick
// the experts; lane j keeps the j-th pick and writes its id and gate.
// With `prob` non-null the lane also returns its experts' softmax
// probabilities (p = exp(v - m) * (1 / sum), one division per token) and, in
// `pick`, the id of its own pick (lanes >= k: -1), for the router
// by-products.
template <int G, int NV>
__device__ __forceinline__ void select_group(const float (&v)[NV], int gl, int E, int k, int renorm,
                                             int32_t* ids_row, float* tw_row, float* prob = nullptr,
                                             int* pick = nullptr) {
  float m = v[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) m = fmaxf(m, v[i]);
  m = group_max<G>(m);
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (gl + G * i < E) se += expf(v[i] - m);
  const float sum_all = group_sum<G>(se);

  uint32_t taken = 0;
  float my_v = -INFINITY;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = gl + G * i;
      // ascending e within the lane: strict '>' keeps the lower id among equal values
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || be == 0x7fffffff)) {
        bv = v[i];
        be = e;
      }
    }
    group_argmax<G>(bv, be);
    if (be % G == gl) taken |= 1u << (be / G);
    if (gl == j) {
      my_v = bv;
      my_e = be;
    }
  }
  const float ex = gl < k ? expf(my_v - m) : 0.f;
  const float denom = renorm ? group_sum<G>(ex) : sum_all;
  if (gl < k) {
    ids_row[gl] = my_e;
    tw_row[gl] = ex / denom;
  }
  if (prob) {
    const float inv = 1.f / sum_all;
#pragma unroll
    for (int i = 0; i < NV; ++i) prob[i] = gl + G * i < E ? expf(v[i] - m) * inv : 0.f;
    *pick = gl < k ? my_e : -1;
  }
}

// Router by-products from a selection workgroup (StatsPart): each group hands
// over its tokens' probabilities and picks; the workgroup adds them per expert
// (fp64, groups in order) and writes one partial row of column sums and counts.
template <int NG, int EW>
struct StatsLds {
  double red[NG][EW];
  int cnt[EW];
};

// Every thread of the workgroup calls this once, after its group's tokens
// have been added to acc (probabilities, lane's experts gl + G i) and cnt.
template <int G, int NV, int NG, int EW>
__device__ __forceinline__ void stats_flush(StatsLds<NG, EW>& L, const double (&acc)[NV], int gl, int grp, int E,
                                            const StatsPart& sp) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *sp.counter = 0;  // for the finishing pass's election
#pragma unroll
  for (int i = 0; i < NV; ++i) L.red[grp][gl + G * i] = acc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double p = L.red[0][e];
#pragma unroll
    for (int g = 1; g < NG; ++g) p += L.red[g][e];
    sp.part_p[(size_t)blockIdx.x * E + e] = p;
    sp.part_c[(size_t)blockIdx.x * E + e] = L.cnt[e];
  }
}

// One group of G lanes per token: logits row (+ bias) from memory, optionally
// written back with the bias added (logits_out may alias src).  Lane g of the
// group holds experts g + G*i in v[i]; k rounds of a group arg-max pick the
// experts, lane j of the group keeps the j-th pick.
// SPLIT: the logits come as nsplit (2 .. kMaxRouterSplits) partial arrays;
// every partial is loaded before the first addition (the loads overlap), then
// they are added in ascending slice order.
// STATS: the workgroup also writes one partial row of the router by-products
// (a group past T adds nothing; no group leaves before the workgroup's
// reduction).
template <int G, int NV, bool SPLIT, bool STATS>
__global__ __launch_bounds__(256) void select_kernel(int T, int E, int k, const float* src, int nsplit,
                                                     const float* __restrict__ bias, int renorm,
                                                     int32_t* __restrict__ ids, float* __restrict__ tw,
                                                     float* logits_out, StatsPart sp) {
  constexpr int NG = 256 / G;
  __shared__ StatsLds<STATS ? NG : 1, STATS ? G * NV : 1> sl;
  const int gl = threadIdx.x & (G - 1), grp = threadIdx.x / G;
  const int t_raw = blockIdx.x * NG + grp;
  if constexpr (STATS) {
    for (int e = threadIdx.x; e < G * NV; e += 256) sl.cnt[e] = 0;
    __syncthreads();
  } else {
    if (t_raw >= T) return;  // whole groups leave together
  }
  const bool live = t_raw < T;
  const int t = live ? t_raw : T - 1;  // (STATS) a group past T works on the last token and writes nothing
  const float* row = src + (size_t)t * E;
  float v[NV];
  if constexpr (SPLIT) {
    const size_t split_stride = (size_t)T * E;
    float part[kMaxRouterSplits][NV];
#pragma unroll
    for (int sl = 0; sl < kMaxRouterSplits; ++sl)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = gl + G * i;
        part[sl][i] = sl < nsplit ? row[sl * split_stride + (e < E ? e : E - 1)] : 0.f;
      }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float l = part[0][i];
#pragma unroll
      for (int sl = 1; sl < kMaxRouterSplits; ++sl)
        if (sl < nsplit) l += part[sl][i];
      v[i] = l;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = gl + G * i;
      v[i] = row[e < E ? e : E - 1];
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = gl + G * i;
    const int ec = e < E ? e : E - 1;
    const float x = v[i] + (bias ? bias[ec] : 0.f);
    v[i] = e < E ? x : -INFINITY;
  }
  if (logits_out && live) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = gl + G * i;
      if (e < E) logits_out[(size_t)t * E + e] = v[i];
    }
  }
  if constexpr (!STATS) {
    select_group<G, NV>(v, gl, E, k, renorm, ids + (size_t)t * k, tw + (size_t)t * k);
  } else {
    // the last token's ids and gates are written again by a group past T: the
    // same values to the same places
    float p[NV];
    int pick;
    select_group<G, NV>(v, gl, E, k, renorm, ids + (size_t)t * k, tw + (size_t)t * k, p, &pick);
    double acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = live ? (double)p[i] : 0.0;
    if (live && pick >= 0) atomicAdd(&sl.cnt[pick], 1);
    stats_flush<G, NV>(sl, acc, gl, grp, E, sp);
  }
}

template <int NF>
hipError_t launch_nf(int T, int d, int E, int k, bool bf16, const void* x, const void* wr,
                     const float* logits_in, const float* bias, int renorm, int32_t* ids, float* tw,
                     float* logits_out, hipStream_t s) {
  if (logits_in != nullptr) return launch_select(T, E, k, logits_in, 1, bias, renorm, ids, tw, logits_out, s);
  const dim3 grid((T + kTokTile - 1) / kTokTile);
  if (bf16)
    route_kernel<NF, true, true><<<grid, 256, 0, s>>>(T, d, E, k, d, x, wr, bias, renorm, ids, tw, logits_out);
  else
    route_kernel<NF, false, true><<<grid, 256, 0, s>>>(T, d, E, k, d, x, wr, bias, renorm, ids, tw, logits_out);
  return hipGetLastError();
}

template <int NF>
hipError_t logits_nf(int T, int d, int E, bool bf16, const void* x, const void* wr, float* logits, int nsplit,
                     hipStream_t s) {
  const dim3 grid((T + kTokTile - 1) / kTokTile, nsplit);
  const int kspan = d / nsplit;
  if (bf16)
    route_kernel<NF, true, false><<<grid, 256, 0, s>>>(T, d, E, 1, kspan, x, wr, nullptr, 0, nullptr, nullptr,
                                                        logits);
  else
    route_kernel<NF, false, false><<<grid, 256, 0, s>>>(T, d, E, 1, kspan, x, wr, nullptr, 0, nullptr, nullptr,
                                                         logits);
  return hipGetLastError();
}

template <int G, int NV>
hipError_t select_gn(int T, int E, int k, const float* src, int nsplit, const float* bias, int renorm,
                     int32_t* ids, float* tw, float* logits_out, const StatsPart& sp, hipStream_t s) {
  constexpr int TPB = 256 / G;  // tokens per workgroup
  const dim3 grid((T + TPB - 1) / TPB);
  const bool st = sp.part_p != nullptr;
#define MOE_GO(SPL, STA) select_kernel<G, NV, SPL, STA><<<grid, 256, 0, s>>>(T, E, k, src, nsplit, bias, renorm, \
                                                                           ids, tw, logits_out, sp)
  if (nsplit > 1) {
    if (st) MOE_GO(true, true);
    else MOE_GO(true, false);
  } else {
    if (st) MOE_GO(false, true);
    else MOE_GO(false, false);
  }
#undef MOE_GO
  return hipGetLastError();
}


// Router logits with one input slice of the router weights resident in LDS
// (bf16).  Workgroup (p, sl) loads rows 0..E-1, inputs [sl kspan, (sl+1) kspan)
// of w into LDS once, then runs over the 64-token blocks p, p + P, ...: each
// of its four waves multiplies 16 tokens' inputs (straight from memory into
// MFMA A fragments) by every 16-expert fragment from LDS and writes the
// slice's partial logits, part[sl][t][e].  Rows of the LDS copy are padded by
// 16 bytes so the 16 lanes reading one fragment hit distinct banks.
constexpr int kRouterLdsBytes = 152 * 1024;
constexpr int kRouterLdsTok = 64;  // tokens per block (4 waves x 16)

template <int NF>  // 16-expert fragments (E <= 16 NF)
__global__ __launch_bounds__(256) void router_lds_kernel(int T, int d, int E, int kspan, const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) unsigned char Wl[kRouterLdsBytes];
  const int sl = blockIdx.y;
  const int RS = kspan * 2 + 16;  // LDS row stride (bytes)
  const int cpr = kspan / 8;      // 16-byte chunks per row
  // weights: rows past E are zero
  {
    const uint16_t* wsl = w + (size_t)sl * kspan;
    const int nchunk = 16 * NF * cpr;
    constexpr int U = 8;
    for (int c0 = threadIdx.x; c0 < nchunk; c0 += 256 * U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 256 * u;
        const int e = c / cpr, cc = c - (c / cpr) * cpr;
        v[u] = (c < nchunk && e < E) ? *reinterpret_cast<const u32x4*>(wsl + (size_t)e * d + 8 * cc)
                                     : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 256 * u;
        const int e = c / cpr, cc = c - (c / cpr) * cpr;
        if (c < nchunk) *reinterpret_cast<u32x4*>(Wl + e * RS + 16 * cc) = v[u];
      }
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15;  // token in the A fragment / expert in the B fragment
  const int q = lane >> 4;
  const int nkk = kspan / 32;
  float* out = part + (size_t)sl * T * E;
  for (int blk = blockIdx.x; blk * kRouterLdsTok < T; blk += gridDim.x) {
    const int t0 = blk * kRouterLdsTok + 16 * wave;
    const int t = t0 + row;
    const bool tok_ok = t < T;
    const uint16_t* xr = x + (size_t)(tok_ok ? t : 0) * d + (size_t)sl * kspan + 8 * q;
    f32x4 acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int KC = 8;  // input steps whose loads are in flight together
    for (int k0 = 0; k0 < nkk; k0 += KC) {
      u32x4 av[KC];
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int kk = min(k0 + c, nkk - 1);  // in-bounds re-read past the end; not used
        av[c] = *reinterpret_cast<const u32x4*>(xr + 32 * kk);
      }
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if (k0 + c < nkk) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, tok_ok ? av[c] : u32x4{0, 0, 0, 0});
          const unsigned char* bp = Wl + row * RS + ((k0 + c) * 32 + 8 * q) * 2;
#pragma unroll
          for (int f = 0; f < NF; ++f)
            acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a, __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(bp + 16 * f * RS)), acc[f], 0, 0, 0);
        }
      }
    }
    // D: lane holds expert 16 f + (lane & 15) for tokens t0 + 4 q + r
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int e = 16 * f + row;
      if (e < E) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tt = t0 + 4 * q + r;
          if (tt < T) out[(size_t)tt * E + e] = acc[f][r];
        }
      }
    }
  }
}

// 16-expert fragments of the LDS-resident router kernel for E experts (the
// kernel's instantiations: 4, 8, 12, 16); its LDS copy holds 16 NF rows.
inline int router_lds_frags(int E) { return (E + 63) / 64 * 4; }

template <int NF>
hipError_t router_lds_nf(int T, int d, int E, int nsplit, const void* x, const void* wr, float* part, hipStream_t s) {
  const int kspan = d / nsplit;
  const long long blocks = ((long long)T + kRouterLdsTok - 1) / kRouterLdsTok;
  const int P = (int)std::max<long long>(1, std::min<long long>(blocks, 256 / nsplit));
  router_lds_kernel<NF><<<dim3(P, nsplit), 256, 0, s>>>(T, d, E, kspan, static_cast<const uint16_t*>(x),
                                                        static_cast<const uint16_t*>(wr), part);
  return hipGetLastError();
}

// Router logits and selection in one pass (bf16 x and router weight, E <= 256
// in 64-expert slices, NFW = ceil(E / 64)): a workgroup takes kRfTok tokens
// and every expert.  The tile's x rows and the router rows go through LDS in
// 64-input k-blocks, on a ring of NS stages filled by loads that write LDS
// directly (128-byte row pieces, 16-byte chunks XOR-swizzled by (row / 2) % 8
// so that the sixteen rows one LDS read serves fall on distinct banks), NS - 1
// k-blocks ahead of the MFMAs, one barrier per k-block.  Wave w owns the
// 16-expert fragments w, w + 4, w + 8, ... of every k-block.  The tile's
// logits (+ bias) then land in LDS (in the ring's memory); 16-lane groups
// pick each token's top k from there, and the logits are copied out in row
// order when asked for.  Against a logits GEMM followed by a selection pass
// the logits make no round trip through memory and one launch goes; every
// workgroup takes in the whole router weight, which the L2 serves.  Measured
// on MI355X (cold cache, bench timing of the routing step): 8192 tokens x 768
// inputs x 192 experts, 19.9 against 24.5 us for the grouped logits GEMM plus
// selection (each CU takes in 343 KB, at about 25 GB/s); 16384 x 768 x 32,
// 16.2 against 18.9 us for the previous one-launch kernel, which streamed the
// router rows from memory straight into MFMA registers.  Starting each
// workgroup's k-loop at a different k-block (so that the CUs of an XCD ask
// for different slices of the weight first) changed nothing measurable.
constexpr int kRfTok = 32;      // tokens per workgroup: two 16-row A fragments
constexpr int kRfKB = 64;       // inputs per k-block (two 32-deep MFMA steps)
constexpr int kRfMinTok = 4096;
constexpr int kRfMaxE = 256;
constexpr int kRfMaxD = 16384;
constexpr int kRfRing = 144 * 1024;  // LDS bytes the ring may take

template <int NFW>
struct RfGeo {
  static constexpr int XB = kRfTok * kRfKB * 2;     // token rows of one k-block (4 KB)
  static constexpr int WB = 64 * NFW * kRfKB * 2;   // router rows of one k-block
  static constexpr int STAGE = XB + WB;
  static constexpr int NS = kRfRing / STAGE < 6 ? kRfRing / STAGE : 6;
  static constexpr int LOADS = STAGE / 1024;        // 1 KB loads per stage
  static constexpr int LPW = LOADS / 4;             // per wave
  static_assert(LOADS % 4 == 0 && NS >= 3 && (NS - 2) * LPW < 64, "ring geometry");
};

// s_waitcnt vmcnt(n) for n < 64 (expcnt and lgkmcnt left alone)
template <int n>
__device__ __forceinline__ void rf_wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}

// STATS: the workgroup also writes one partial row of the router by-products.
template <int NFW, bool STATS>
__global__ __launch_bounds__(256) void router_fused_kernel(int T, int d, int E, int k,
                                                           const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w,
                                                           const float* __restrict__ bias, int renorm,
                                                           int32_t* __restrict__ ids, float* __restrict__ tw,
                                                           float* __restrict__ logits_out, StatsPart sp) {
  using G = RfGeo<NFW>;
  constexpr int NS = G::NS, LPW = G::LPW, ROWB = kRfKB * 2;
  constexpr int ES = 64 * NFW + 4;  // logits row stride in LDS (floats)
  __shared__ __attribute__((aligned(16))) unsigned char ring[NS * G::STAGE];
  // after the k-loop the ring holds the logits tile, then (STATS) the by-product sums
  using SL = StatsLds<16, 64 * NFW>;
  constexpr int LS_BYTES = (kRfTok * ES * 4 + 15) / 16 * 16;
  static_assert(LS_BYTES + sizeof(SL) <= sizeof(ring), "logits and by-product sums fit the ring");
  float* const Ls = reinterpret_cast<float*>(ring);
  SL& sl = *reinterpret_cast<SL*>(ring + LS_BYTES);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * kRfTok;
  const int nkb = d / kRfKB;

  // The wave's LPW loads of a stage: load l = wave * LPW + j fills 8 rows
  // (1 KB): token rows 8 l .. for l < 4, else router rows 8 (l - 4) ..;
  // lane takes row + lane / 8 and stores chunk lane % 8 of it, which holds
  // logical chunk (lane % 8) ^ ((row / 2) % 8).  Token rows past T re-read row
  // T - 1 and router rows past E row E - 1 (their logits are not used).
  const unsigned char* const xb = reinterpret_cast<const unsigned char*>(x) + (size_t)t0 * d * 2;
  const unsigned char* const wbp = reinterpret_cast<const unsigned char*>(w);
  uint32_t off[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int l = wave * LPW + j;
    const int r = (l < 4 ? 8 * l : 8 * (l - 4)) + (lane >> 3);
    const int src = l < 4 ? min(r, T - 1 - t0) : min(r, E - 1);
    off[j] = (uint32_t)src * (uint32_t)(d * 2) + (uint32_t)((((lane & 7) ^ ((r >> 1) & 7))) * 16);
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)&ring[0]);
  auto issue = [&](int st, int kb) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int l = wave * LPW + j;
      // x rows take the stage's first 4 KB, router rows follow: load l lands at l KB
      const uint32_t dst = lds0 + (uint32_t)(st * G::STAGE + l * 1024);
      ffn_wide::dma16(l < 4 ? xb : wbp, off[j] + (uint32_t)(kb * ROWB), dst);
    }
  };

  // fragment reads: lane (row, q) of step s needs logical chunk 4 s + q of its
  // row; fragment rows start at multiples of 16, so the swizzle is (row / 2) % 8
  f32x4 acc[2][NFW];
#pragma unroll
  for (int i = 0; i < NFW; ++i) acc[0][i] = acc[1][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < nkb) issue(p, p);
  int st = 0;
  for (int kb = 0; kb < nkb; ++kb) {
    // k-block kb landed for this wave (later ones may stay in flight), then
    // for every wave; the stage k-block kb - 1 used is free again
    if (kb + NS - 2 < nkb) rf_wait_vm<(NS - 2) * LPW>();
    else rf_wait_vm<0>();
    ffn_wide::lds_barrier();
    if (kb + NS - 1 < nkb) issue(st == 0 ? NS - 1 : st - 1, kb + NS - 1);
    const unsigned char* const S = ring + st * G::STAGE;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int co = (((4 * s + q) ^ ((row >> 1) & 7))) * 16;
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(S + row * ROWB + co));
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(S + (16 + row) * ROWB + co));
#pragma unroll
      for (int i = 0; i < NFW; ++i) {
        const bf16x8 b = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(S + G::XB + (16 * (wave + 4 * i) + row) * ROWB + co));
        acc[0][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc[0][i], 0, 0, 0);
        acc[1][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc[1][i], 0, 0, 0);
      }
    }
    st = st == NS - 1 ? 0 : st + 1;
  }
  // every wave is past its reads of the ring (and every load has landed: the
  // last k-block waited for all of them) before the logits overwrite it
  __syncthreads();
  // D: lane holds expert 16 f + row for tokens 16 m + 4 q + r
#pragma unroll
  for (int i = 0; i < NFW; ++i) {
    const int e = 16 * (wave + 4 * i) + row;
    const float be = (bias && e < E) ? bias[e] : 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) Ls[(16 * m + 4 * q + r) * ES + e] = acc[m][i][r] + be;
  }
  if constexpr (STATS)
    for (int e = threadIdx.x; e < 64 * NFW; e += 256) sl.cnt[e] = 0;
  __syncthreads();

  // selection: 16 groups of 16 lanes, two tokens each
  const int gl = threadIdx.x & 15, grp = threadIdx.x >> 4;
  double pacc[4 * NFW];
#pragma unroll
  for (int i = 0; i < 4 * NFW; ++i) pacc[i] = 0.0;
#pragma unroll
  for (int hh = 0; hh < kRfTok / 16; ++hh) {
    const int r = grp + 16 * hh, t = t0 + r;
    if (t < T) {  // uniform over the group
      float v[4 * NFW];
#pragma unroll
      for (int i = 0; i < 4 * NFW; ++i) {
        const int e = gl + 16 * i;
        v[i] = e < E ? Ls[r * ES + e] : -INFINITY;
      }
      if constexpr (STATS) {
        float p[4 * NFW];
        int pick;
        select_group<16, 4 * NFW>(v, gl, E, k, renorm, ids + (size_t)t * k, tw + (size_t)t * k, p, &pick);
#pragma unroll
        for (int i = 0; i < 4 * NFW; ++i) pacc[i] += (double)p[i];
        if (pick >= 0) atomicAdd(&sl.cnt[pick], 1);
      } else {
        select_group<16, 4 * NFW>(v, gl, E, k, renorm, ids + (size_t)t * k, tw + (size_t)t * k);
      }
    }
  }
  if constexpr (STATS) stats_flush<16, 4 * NFW>(sl, pacc, gl, grp, E, sp);
  if (logits_out) {
    const int n = min(kRfTok, T - t0) * E;
    for (int c = threadIdx.x; c < n; c += 256) {
      const int r = c / E;
      logits_out[(size_t)(t0 + r) * E + (c - r * E)] = Ls[r * ES + (c - r * E)];
    }
  }
}

template <int NFW>
hipError_t router_fused_nf(int T, int d, int E, int k, const void* x, const void* wr, const float* bias,
                           int renorm, int32_t* ids, float* tw, float* logits_out, const StatsPart& sp,
                           hipStream_t s) {
  const dim3 grid((unsigned)((T + kRfTok - 1) / kRfTok));
  if (sp.part_p)
    router_fused_kernel<NFW, true><<<grid, 256, 0, s>>>(T, d, E, k, static_cast<const uint16_t*>(x),
                                                        static_cast<const uint16_t*>(wr), bias, renorm, ids, tw,
                                                        logits_out, sp);
  else
    router_fused_kernel<NFW, false><<<grid, 256, 0, s>>>(T, d, E, k, static_cast<const uint16_t*>(x),
                                                         static_cast<const uint16_t*>(wr), bias, renorm, ids, tw,
                                                         logits_out, sp);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_route(int T, int d, int E, int k, bool bf16, const void* x, const void* wr,
                        const float* logits_in, const float* bias, int renorm, int32_t* ids,
                        float* tw, float* logits_out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!logits_in && router_fused_ok(T, d, E, k, bf16))
    return launch_router_fused(T, d, E, k, x, wr, bias, renorm, ids, tw, logits_out, s);
  // Many experts and a logits buffer from the caller: the layer's two passes
  // (logits GEMM on its own tiles into the buffer, then the selection) rather
  // than 16-token tiles that each hold every expert's logits.  Measured on
  // MI355X, 512 tokens x 896 experts x 7168 inputs: 0.79 ms in one pass.
  if (!logits_in && logits_out && E > 256) {
    hipError_t e = launch_router_logits(T, d, E, bf16, x, wr, logits_out, 1, s);
    if (e != hipSuccess) return e;
    return launch_select(T, E, k, logits_out, 1, bias, renorm, ids, tw, logits_out, s);
  }
  const int nf = (E + 63) / 64;
#define MOE_CALL(NFv) launch_nf<NFv>(T, d, E, k, bf16, x, wr, logits_in, bias, renorm, ids, tw, logits_out, s)
  if (nf <= 1) return MOE_CALL(1);
  if (nf <= 2) return MOE_CALL(2);
  if (nf <= 4) return MOE_CALL(4);
  if (nf <= 8) return MOE_CALL(8);
  return MOE_CALL(16);
#undef MOE_CALL
}

int router_logits_tile_m(int T, int E) {
  const long long nb = E / 64;
  // the largest tile that still gives every CU one: the tiles' operand bytes
  // (tile rows of x plus 64 router rows) are what a CU has to take in
  for (int bm : {64, 32})
    if ((long long)((T + bm - 1) / bm) * nb >= 256) return bm;
  return 16;
}

// The LDS-resident router kernel takes the layer's logits when the whole
// router weight fits in LDS (bf16, up to 256 experts).  Measured on MI355X:
// 32 experts x 768 inputs, 23 against 28 us for logits + selection; sliced
// weights (192 x 768 in two slices, 128 x 3072 in six) lost to the grouped
// GEMM and to the sliced register kernel, whose partial logits also cost the
// selection a second read.
bool router_lds_whole(int d, int E, bool bf16) {
  return bf16 && E <= 256 && d % 32 == 0 && (long long)16 * router_lds_frags(E) * (d * 2 + 16) <= kRouterLdsBytes;
}

int router_logits_splits(int T, int d, int E, bool bf16) {
  if (T == 0 || router_lds_whole(d, E, bf16)) return 1;
  // workgroups without a split: the grouped GEMM's tiles, else 16-token tiles
  const long long tiles16 = ((long long)T + kTokTile - 1) / kTokTile;
  const long long wgs = (bf16 && E % 64 == 0) ? ((long long)T + router_logits_tile_m(T, E) - 1) /
                                                    router_logits_tile_m(T, E) * (E / 64)
                                              : tiles16;
  if (T == 0 || wgs >= 256) return 1;
  // few tokens and long rows: split the inputs until 16-token tiles fill the
  // CUs, keeping every slice a multiple of 32 inputs and at least 256 long
  int ns = 1;
  while (ns < kMaxRouterSplits && tiles16 * ns < 256 && d % (64 * ns) == 0 && d / (2 * ns) >= 256) ns *= 2;
  return ns;
}

hipError_t launch_router_logits(int T, int d, int E, bool bf16, const void* x, const void* wr, float* logits,
                                int nsplit, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (nsplit < 1 || d % nsplit || (d / nsplit) % (bf16 ? 32 : 4)) return hipErrorInvalidValue;
  if (nsplit == 1 && router_lds_whole(d, E, bf16)) {
    const int nf = router_lds_frags(E);
#define MOE_CALL(NFv) router_lds_nf<NFv>(T, d, E, nsplit, x, wr, logits, s)
    if (nf == 4) return MOE_CALL(4);
    if (nf == 8) return MOE_CALL(8);
    if (nf == 12) return MOE_CALL(12);
    return MOE_CALL(16);
#undef MOE_CALL
  }
  if (nsplit > 1) {
    const int nf = (E + 63) / 64;
#define MOE_CALL(NFv) logits_nf<NFv>(T, d, E, bf16, x, wr, logits, nsplit, s)
    if (nf <= 1) return MOE_CALL(1);
    if (nf <= 2) return MOE_CALL(2);
    if (nf <= 4) return MOE_CALL(4);
    if (nf <= 8) return MOE_CALL(8);
    return MOE_CALL(16);
#undef MOE_CALL
  }
  if (bf16 && E % 64 == 0) {
    FfnGemmArgs g{};
    g.A = x;
    g.row_div = 1;
    g.W0 = wr;
    g.out = logits;
    g.E_loc = 1;
    g.rows_max = T;
    g.a_rows = T;
    g.K = d;
    g.N = E;
    g.out_f32 = 1;
    return launch_ffn_gemm(g, false, W_BF16, false, router_logits_tile_m(T, E), 1, s);
  }
  const int nf = (E + 63) / 64;
#define MOE_CALL(NFv) logits_nf<NFv>(T, d, E, bf16, x, wr, logits, 1, s)
  if (nf <= 1) return MOE_CALL(1);
  if (nf <= 2) return MOE_CALL(2);
  if (nf <= 4) return MOE_CALL(4);
  if (nf <= 8) return MOE_CALL(8);
  return MOE_CALL(16);
#undef MOE_CALL
}

bool router_fused_ok(int T, int d, int E, int k, bool bf16) {
  return bf16 && T >= kRfMinTok && E >= 1 && E <= kRfMaxE && k >= 1 && k <= 16 && d >= kRfKB &&
         d % kRfKB == 0 && d <= kRfMaxD;
}

hipError_t launch_router_fused(int T, int d, int E, int k, const void* x, const void* wr, const float* bias,
                               int renorm, int32_t* ids, float* tw, float* logits_out, hipStream_t s,
                               const StatsPart* stats) {
  if (!router_fused_ok(T, d, E, k, true)) return hipErrorInvalidValue;
  const StatsPart sp = stats ? *stats : StatsPart{};
  const int nf = (E + 63) / 64;
#define MOE_CALL(NFv) router_fused_nf<NFv>(T, d, E, k, x, wr, bias, renorm, ids, tw, logits_out, sp, s)
  if (nf <= 1) return MOE_CALL(1);
  if (nf <= 2) return MOE_CALL(2);
  if (nf <= 3) return MOE_CALL(3);
  return MOE_CALL(4);
#undef MOE_CALL
}

int select_stats_rows(int T, int E, int k, bool fused) {
  if (fused) return (T + kRfTok - 1) / kRfTok;
  const int tpb = (E <= 256 && k <= 16 && T >= kSelectGroupMinTok) ? 16 : 4;  // tokens per select workgroup
  return (T + tpb - 1) / tpb;
}

hipError_t launch_select(int T, int E, int k, const float* src, int nsplit, const float* bias, int renorm,
                         int32_t* ids, float* tw, float* logits_out, hipStream_t s, const StatsPart* stats) {
  const StatsPart sp = stats ? *stats : StatsPart{};
  if (T == 0) return hipSuccess;
  if (nsplit < 1 || nsplit > kMaxRouterSplits) return hipErrorInvalidValue;
  // 16 lanes per token while a lane holds at most 16 logits, the k picks fit in
  // the group and there are tokens enough for a wave per SIMD; the whole wave
  // otherwise.  Measured on MI355X, routing step: 8192 tokens x 192 experts,
  // 24.6 us with 16 lanes against 28.3 with 64; 512 x 128 (four partial
  // arrays), 34.5 against 30.0.
  if (E <= 256 && k <= 16 && T >= kSelectGroupMinTok) {
    const int nv = (E + 15) / 16;
#define MOE_CALL(NVv) select_gn<16, NVv>(T, E, k, src, nsplit, bias, renorm, ids, tw, logits_out, sp, s)
    if (nv <= 2) return MOE_CALL(2);
    if (nv <= 4) return MOE_CALL(4);
    if (nv <= 8) return MOE_CALL(8);
    if (nv <= 12) return MOE_CALL(12);
    return MOE_CALL(16);
#undef MOE_CALL
  }
  const int nv = (E + 63) / 64;
#define MOE_CALL(NVv) select_gn<64, NVv>(T, E, k, src, nsplit, bias, renorm, ids, tw, logits_out, sp, s)
  if (nv <= 1) return MOE_CALL(1);
  if (nv <= 2) return MOE_CALL(2);
  if (nv <= 4) return MOE_CALL(4);
  if (nv <= 8) return MOE_CALL(8);
  return MOE_CALL(16);
#undef MOE_CALL
}

}  // namespace moe
