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
// logits from memory with one wave per token.  Selection: every lane holds
// E/64 logits in registers and k rounds of a (value, lower-id) wave arg-max
// pick the experts.  When the activations are bf16 and E is a multiple of 64
// the logits of a whole layer come from the grouped GEMM kernel (one group,
// fp32 output) instead, which reuses each router weight slice across 16-64
// tokens per workgroup rather than 16.  Few tokens with long rows (decode)
// leave most CUs idle on either kernel; there the logits kernel splits the
// inputs into slices, each workgroup sums one slice into its own partial
// array, and the select kernel adds the partials in ascending slice order.
// When the whole router weight fits in LDS (few experts), a third logits
// kernel keeps it there and streams only the token rows.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokTile = 16;

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
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) {
      const float ov = wave_shfl_xor(bv, msk);
      const int oe = wave_shfl_xor(be, msk);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
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
      constexpr int KC = 16;
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
              acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, e_ok[i] ? bv[c][i] : 0.f, acc[i], 0, 0, 0);
          }
        }
      }
    }
    // D[i][j]: lane holds column j = lane & 15 and rows 4q + r.
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int e = 16 * (wave + 4 * i) + row;
      if (e < E) {
        const float bv = (SELECT && bias) ? bias[e] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) Ls[(4 * q + r) * ES + e] = acc[i][r] + bv;
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

__device__ __forceinline__ void take_better(float& v, int& e, float ov, int oe) {
  if (ov > v || (ov == v && oe < e)) {
    v = ov;
    e = oe;
  }
}
template <int G>
__device__ __forceinline__ void group_argmax(float& v, int& e) {  // larger value, then lower id
  take_better(v, e, dppf<kRowRor8>(v), dpp<kRowRor8>(e));
  take_better(v, e, dppf<kRowRor4>(v), dpp<kRowRor4>(e));
  take_better(v, e, dppf<kQuadSwap2>(v), dpp<kQuadSwap2>(e));
  take_better(v, e, dppf<kQuadSwap1>(v), dpp<kQuadSwap1>(e));
  if constexpr (G == 64) {
    take_better(v, e, wave_shfl_xor(v, 16), wave_shfl_xor(e, 16));
    take_better(v, e, wave_shfl_xor(v, 32), wave_shfl_xor(e, 32));
  }
}

// One group of G lanes per token: logits row (+ bias) from memory, optionally
// written back with the bias added (logits_out may alias src).  Lane g of the
// group holds experts g + G*i in v[i]; k rounds of a group arg-max pick the
// experts, lane j of the group keeps the j-th pick.
// SPLIT: the logits come as nsplit (2 .. kMaxRouterSplits) partial arrays;
// every partial is loaded before the first addition (the loads overlap), then
// they are added in ascending slice order.
template <int G, int NV, bool SPLIT>
__global__ __launch_bounds__(256) void select_kernel(int T, int E, int k, const float* src, int nsplit,
                                                     const float* __restrict__ bias, int renorm,
                                                     int32_t* __restrict__ ids, float* __restrict__ tw,
                                                     float* logits_out) {
  const int gl = threadIdx.x & (G - 1);
  const int t = blockIdx.x * (256 / G) + threadIdx.x / G;
  if (t >= T) return;  // whole groups leave together
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
  if (logits_out) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = gl + G * i;
      if (e < E) logits_out[(size_t)t * E + e] = v[i];
    }
  }
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
    ids[(size_t)t * k + gl] = my_e;
    tw[(size_t)t * k + gl] = ex / denom;
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
                     int32_t* ids, float* tw, float* logits_out, hipStream_t s) {
  constexpr int TPB = 256 / G;  // tokens per workgroup
  const dim3 grid((T + TPB - 1) / TPB);
  if (nsplit > 1)
    select_kernel<G, NV, true><<<grid, 256, 0, s>>>(T, E, k, src, nsplit, bias, renorm, ids, tw, logits_out);
  else
    select_kernel<G, NV, false><<<grid, 256, 0, s>>>(T, E, k, src, 1, bias, renorm, ids, tw, logits_out);
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

}  // namespace

hipError_t launch_route(int T, int d, int E, int k, bool bf16, const void* x, const void* wr,
                        const float* logits_in, const float* bias, int renorm, int32_t* ids,
                        float* tw, float* logits_out, hipStream_t s) {
  if (T == 0) return hipSuccess;
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
  for (int bm : {64, 32})
    if ((long long)((T + bm - 1) / bm) * nb >= 512) return bm;
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

hipError_t launch_select(int T, int E, int k, const float* src, int nsplit, const float* bias, int renorm,
                         int32_t* ids, float* tw, float* logits_out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (nsplit < 1 || nsplit > kMaxRouterSplits) return hipErrorInvalidValue;
  // 16 lanes per token while a lane holds at most 16 logits and the k picks fit
  // in the group; the whole wave otherwise
  if (E <= 256 && k <= 16) {
    const int nv = (E + 15) / 16;
#define MOE_CALL(NVv) select_gn<16, NVv>(T, E, k, src, nsplit, bias, renorm, ids, tw, logits_out, s)
    if (nv <= 2) return MOE_CALL(2);
    if (nv <= 4) return MOE_CALL(4);
    if (nv <= 8) return MOE_CALL(8);
    if (nv <= 12) return MOE_CALL(12);
    return MOE_CALL(16);
#undef MOE_CALL
  }
  const int nv = (E + 63) / 64;
#define MOE_CALL(NVv) select_gn<64, NVv>(T, E, k, src, nsplit, bias, renorm, ids, tw, logits_out, s)
  if (nv <= 1) return MOE_CALL(1);
  if (nv <= 2) return MOE_CALL(2);
  if (nv <= 4) return MOE_CALL(4);
  if (nv <= 8) return MOE_CALL(8);
  return MOE_CALL(16);
#undef MOE_CALL
}

}  // namespace moe
