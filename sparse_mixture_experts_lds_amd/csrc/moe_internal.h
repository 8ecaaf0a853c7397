// Internal declarations of the gfx950 MoE kernels: device helpers, kernel
// argument blocks and the host-side launchers used by the C ABI (abi.hip).
// Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

enum WType { W_F32 = 0, W_BF16 = 1, W_I4 = 2 };

constexpr int kWave = 64;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kI4Group = 128;

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even float -> bf16 bit pattern (finite inputs).
// fp32 -> bf16, rounded to nearest even (gfx950's v_cvt_pk_bf16_f32, one
// instruction per pair)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// fp32 -> fp16 bit pattern, rounded to nearest even (v_cvt_f16_f32)
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// The xor-16 and xor-32 lane exchanges of a wave in registers (gfx950's
// v_permlane16_swap / v_permlane32_swap) rather than through LDS permutes.
// Lane mapping, checked on the GPU: from r = permlane32_swap(x, x) lane l
// takes r[1] for l < 32 and r[0] above; from r = permlane16_swap(x, x), r[1]
// in the even 16-lane rows and r[0] in the odd ones.
__device__ __forceinline__ int xor32_lanes(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (__lane_id() & 32) ? r[0] : r[1];
}
__device__ __forceinline__ int xor16_lanes(int x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return (__lane_id() & 16) ? r[0] : r[1];
}
__device__ __forceinline__ float xor32_lanes(float x) { return __int_as_float(xor32_lanes(__float_as_int(x))); }
__device__ __forceinline__ float xor16_lanes(float x) { return __int_as_float(xor16_lanes(__float_as_int(x))); }

// SiLU from the hardware base-2 exponential and reciprocal (v_exp_f32,
// v_rcp_f32, about 1 ulp each): g / (1 + e^-g) = g * rcp(1 + 2^(-g log2 e)).
// Large positive g gives g, large negative g gives -0.  Five instructions
// against about twenty for expf and an IEEE division; the result feeds a z
// that is rounded to bf16, or kept in fp32 where outputs are held to 1e-5 of
// their RMS.
__device__ __forceinline__ float sigmoid_hw(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}
__device__ __forceinline__ float silu_hw(float g) { return g * sigmoid_hw(g); }

// Exact-erf GELU, 0.5 g (1 + erf(g / sqrt 2)), with erf from Abramowitz and
// Stegun's rational approximation 7.1.26 (Handbook of Mathematical
// Functions; |error| <= 1.5e-7 for x >= 0, erf odd):
//   1 - erf(x) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^(-x^2),
//   t = 1 / (1 + p x).
// With c = 1 - erf(|g| / sqrt 2) the result is g - g c / 2 for g >= 0 and
// g c / 2 below, which avoids the cancellation in 1 + erf for negative g.
// gelu_tail returns c = 1 - erf(|g| / sqrt 2) and sets e = exp(-g^2 / 2),
// which the derivative reuses (GELU'(g) = Phi(g) + g e / sqrt(2 pi)).
__device__ __forceinline__ float gelu_tail(float g, float& e) {
  const float x = fabsf(g) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float p = fmaf(t, 1.061405429f, -1.453152027f);
  p = fmaf(t, p, 1.421413741f);
  p = fmaf(t, p, -0.284496736f);
  p = fmaf(t, p, 0.254829592f);
  e = __builtin_amdgcn_exp2f(x * x * -1.4426950408889634f);
  return t * p * e;
}
__device__ __forceinline__ float gelu_hw(float g) {
  float e;
  const float h = 0.5f * g * gelu_tail(g, e);
  return g >= 0.f ? g - h : h;
}

// Gate backward at one hidden unit of a pair row with gate w (ACT 0 SiLU, 1
// GELU, each as the forward's epilogue forms it): a = act(g), a' = act'(g),
// z = a u (rounded to bf16 when BF16, as the forward stores it); dg =
// w dz' u a', du = w dz' a, zw = w z.  Returns z, whose products with dz'
// sum to the pair's gate gradient.
template <int ACT, bool BF16>
__device__ __forceinline__ float gate_bwd_point(float g, float u, float dz1, float w, float& dg, float& du,
                                                float& zw) {
  float a, ad;
  if constexpr (ACT == 0) {
    const float sg = sigmoid_hw(g);
    a = g * sg;
    ad = sg * (1.f + g * (1.f - sg));
  } else {
    float e;
    const float c = gelu_tail(g, e);
    const float h = 0.5f * g * c;
    a = g >= 0.f ? g - h : h;
    const float phi = g >= 0.f ? 1.f - 0.5f * c : 0.5f * c;
    ad = phi + g * e * 0.39894228040143268f;
  }
  float z = a * u;
  if constexpr (BF16) z = bf16_bits_to_f32(f32_to_bf16_bits(z));
  const float dzw = w * dz1;
  dg = dzw * u * ad;
  du = dzw * a;
  zw = w * z;
  return z;
}

// Reductions over a group of G lanes (G = 16: one DPP row; G = 64: the wave).
// Every lane of the group ends with the result.
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}
constexpr int kRowRor8 = 0x128, kRowRor4 = 0x124, kQuadSwap2 = 0x4E, kQuadSwap1 = 0xB1;

template <int G>
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, dppf<kRowRor8>(x));
  x = fmaxf(x, dppf<kRowRor4>(x));
  x = fmaxf(x, dppf<kQuadSwap2>(x));
  x = fmaxf(x, dppf<kQuadSwap1>(x));
  if constexpr (G == 64) {
    x = fmaxf(x, xor16_lanes(x));
    x = fmaxf(x, xor32_lanes(x));
  }
  return x;
}
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += dppf<kRowRor8>(x);
  x += dppf<kRowRor4>(x);
  x += dppf<kQuadSwap2>(x);
  x += dppf<kQuadSwap1>(x);
  if constexpr (G == 64) {
    x += xor16_lanes(x);
    x += xor32_lanes(x);
  }
  return x;
}
// Arg-max over a group of G lanes: the larger value, then the lower id among
// equal values; every lane of the group ends with the winner.  Two reductions
// (the maximum value, then the minimum id of the lanes that hold it) of one
// DPP or lane-swap move and one min/max each per step.
template <int G>
__device__ __forceinline__ int group_min(int x) {
  x = min(x, dpp<kRowRor8>(x));
  x = min(x, dpp<kRowRor4>(x));
  x = min(x, dpp<kQuadSwap2>(x));
  x = min(x, dpp<kQuadSwap1>(x));
  if constexpr (G == 64) {
    x = min(x, xor16_lanes(x));
    x = min(x, xor32_lanes(x));
  }
  return x;
}
template <int G>
__device__ __forceinline__ void group_argmax(float& v, int& e) {
  const float m = group_max<G>(v);
  e = group_min<G>(v == m ? e : 0x7fffffff);
  v = m;
}
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already checked.

// Router: logits GEMM (or given logits) + bias, softmax, top-k.
hipError_t launch_route(int T, int d, int E, int k, bool bf16, const void* x, const void* wr,
                        const float* logits_in, const float* bias, int renorm, int32_t* ids,
                        float* tw, float* logits_out, hipStream_t s);
// Router logits without bias, L[t,e] = sum_i x[t,i] w[e,i] in fp32, written
// as nsplit partial sums over consecutive input slices: part[s][t][e], [nsplit,
// T, E] (nsplit 1: the logits themselves).  router_logits_splits picks nsplit
// (1 .. kMaxRouterSplits) for the shape.
constexpr int kMaxRouterSplits = 8;
int router_logits_splits(int T, int d, int E, bool bf16);
hipError_t launch_router_logits(int T, int d, int E, bool bf16, const void* x, const void* wr, float* part,
                                int nsplit, hipStream_t s);
// Per-workgroup partial rows of the router by-products, written by a
// selection launch that is handed one: softmax column sums (fp64) and pick
// counts of the workgroup's tokens, one [E] row per workgroup.
constexpr int kStatsMaxRowSplits = 8;      // row ranges of the by-products' finishing pass
constexpr int kStatsFinishMaxRows = 1024;  // partial rows it adds at most (128 per range)
struct StatsPart {
  double* part_p;
  int32_t* part_c;
  double* mid_p;      // the finishing pass's per-row-range sums (stats_finish_bytes(E) with mid_c and counter)
  int32_t* mid_c;
  unsigned* counter;  // zeroed by the selection launch, counted by the finishing pass
};

// Router logits (+ bias), softmax and top-k in one launch for bf16 layers with
// many tokens (router_fused_ok); logits_out (NULL allowed) receives the biased
// logits.
bool router_fused_ok(int T, int d, int E, int k, bool bf16);
hipError_t launch_router_fused(int T, int d, int E, int k, const void* x, const void* wr, const float* bias,
                               int renorm, int32_t* ids, float* tw, float* logits_out, hipStream_t s,
                               const StatsPart* stats = nullptr);
// Softmax + top-k from logits given as nsplit partial arrays src[s][T][E]
// (added in ascending s) plus bias; logits_out (NULL, or aliasing the first
// partial array: every element is read and written by the same lane) receives
// the sum + bias.
hipError_t launch_select(int T, int E, int k, const float* src, int nsplit, const float* bias, int renorm,
                         int32_t* ids, float* tw, float* logits_out, hipStream_t s,
                         const StatsPart* stats = nullptr);
// Partial rows a selection launch writes with StatsPart (one per workgroup):
// launch_select's, or the fused router's when fused.
int select_stats_rows(int T, int E, int k, bool fused);
// Counts, means and loss from nblk partial rows (workgroups over 64-expert
// chunks and row ranges; the last to finish folds the loss).
size_t stats_finish_bytes(int E);
hipError_t launch_stats_finish(int T, int E, int nblk, const StatsPart& sp, int32_t* counts, float* prob_mean,
                               float* loss, hipStream_t s);

// Router by-products: per-expert token counts, mean softmax probabilities and
// the balance loss from logits (+ bias) and top-k ids; ws holds
// router_stats_ws_bytes(T, E) bytes of per-block partials.  Any of counts,
// prob_mean, loss may be NULL.
int router_stats_blocks(int T, int E);
size_t router_stats_ws_bytes(int T, int E);
hipError_t launch_router_stats(int T, int E, int k, const float* logits, const float* bias, const int32_t* ids,
                               int32_t* counts, float* prob_mean, float* loss, void* ws, hipStream_t s);

// Grouping of pairs by local expert.
struct PermuteWs {
  int32_t* counts;       // [nblk * E_loc] per-block counts, then per-block bases
  int nblk;
};
size_t permute_ws_bytes(int P, int E_loc);
int permute_block_pairs();
// mtile_start/tile_tab (may be NULL): the m-tile prefix and per-m-tile table of
// the grouped GEMMs for tiles of BM rows.
hipError_t launch_permute(int T, int k, int E, const int32_t* ids, const int32_t* expert_map, int E_loc,
                          int capacity, int BM, int32_t* offsets, int32_t* mtile_start, int4* tile_tab,
                          int32_t* sorted_pair, int32_t* pair_pos, int32_t* counts, hipStream_t s);
// Pairs grouped by (owner, local expert, p) under a placement rule (0 round
// robin, 1 contiguous); map holds E ints and counts permute_ws_bytes(T*k, E).
hipError_t launch_owner_dispatch(int T, int k, int E, int n_owners, int rule, int capacity, const int32_t* ids,
                                 int32_t* owner_offsets, int32_t* recv_offsets, int32_t* expert_offsets,
                                 int32_t* sorted_pair, int32_t* pair_pos, int32_t* map, int32_t* counts,
                                 hipStream_t s);
hipError_t launch_gather_rows(int rows_max, int d, bool bf16, const void* x, const int32_t* sorted_pair,
                              int k, const int32_t* offsets_end, void* x_perm, hipStream_t s);
hipError_t launch_mtile_prefix(int E_loc, int BM, const int32_t* offsets, int32_t* mtile_start,
                               int4* tile_tab, hipStream_t s);

// Grouped GEMMs.
// Where a gate/up launch that recomputes g and u for the backward sends its
// results instead of z (per problem): for grouped row r with gate w =
// w_row[r] (or 1) it writes dGU[r] = [dg | du] and ZW[r] = w z (bf16), and
// part[r][j] = the sum of dz'[r, c] z[r, c] over hidden units c of 64-wide
// block j.
struct GateBwdOut {
  const float* dZ;     // [rows, h] dz' = dout Wd per grouped row
  const float* w_row;  // [rows] gate of each grouped row's pair, NULL: 1
  uint16_t* dGU;       // [rows, 2h]
  uint16_t* ZW;        // [rows, h]
  float* part;         // [rows, h / 64]
};

struct FfnGemmArgs {
  const void* A;             // activations [rows, K] (bf16 or f32)
  const int32_t* row_index;  // NULL: A row = grouped row; else A row = row_index[r] / row_div
  int row_div;
  const void* W0;            // [E_loc, N, K] (I4: bytes [E_loc, N, K/2])
  const void* W1;            // second matrix (up projection) for gate/up, else NULL
  const uint16_t* S0;        // I4 scales [E_loc, N, K/128]
  const uint16_t* S1;
  void* out;                 // [rows, N]
  const int32_t* offsets;    // [E_loc+1] or NULL (single group of rows_max rows)
  const int32_t* mtile_start;// [E_loc+1] m-tile prefix, or NULL with offsets == NULL
  const int4* tile_tab;      // per m-tile {expert, first row, rows, 0}, or NULL with offsets == NULL
  int E_loc, rows_max, K, N;
  int a_rows;                // rows of A as addressed (a_rows * K elements must stay below 4 GiB)
  int act;                   // 0 SiLU, 1 GELU (gate/up only)
  int out_f32;               // 1: store the output as fp32 whatever the operand type
  int out_f16;               // 1 (with out_f32 0): store the output as fp16
  void* ev_start;            // hipEvent_t pair carried by the launch itself (NULL: none):
  void* ev_stop;             //   they time exactly this kernel and add no packet to the stream
};

struct FfnPlan {
  int BM;                    // rows per tile (16 * MF)
  int NF_up, NF_down;        // 16-col fragments per wave
  bool z_f16;                // INT4: z stored in fp16, the down projection on the fp16 MFMA
  int BM_down;               // rows per tile of the down GEMM when it differs (its own m-tile table), else 0
};
// avg_rows: expected rows per group (local expert); groups: number of groups.
FfnPlan plan_ffn(double avg_rows, int groups, int d, int h, int w_type);
int ffn_max_mtiles(int E_loc, int rows_max, int BM);
// z16: (INT4 down projections only) A is fp16 and is multiplied on the fp16 MFMA.
hipError_t launch_ffn_gemm(const FfnGemmArgs& a, bool gateup, int w_type, bool z16, int BM,
                           int NF, hipStream_t s);
// Two problems of the same kind, K and N on the narrow kernel (fp32 or bf16
// weights, BM rows per tile), problem 0's tiles dispatched first; a0's events,
// if any, time the launch.
hipError_t launch_ffn_gemm_pair(const FfnGemmArgs& a0, const FfnGemmArgs& a1, bool gateup, int w_type, int BM,
                                int NF, hipStream_t s);
// Two problems of the same kind (bf16 weights, wide 256-row tiles, 64 * NF
// weight rows per tile, same activation and output type) in one launch, the
// tiles of a0 dispatched first; the events, if any, time the launch.
// The wide gate/up GEMM (bf16, 256-row tiles of 128 outputs; K and N
// multiples of 128) of np problems with the gate backward in its epilogue
// (GateBwdOut) instead of the z store; a's out is not written.
bool gateup_bwd_wide_ok(const FfnGemmArgs& a);
hipError_t launch_gateup_bwd_wide(const FfnGemmArgs* a, const GateBwdOut* gb, int np, hipStream_t s);
hipError_t launch_ffn_gemm_wide_pair(const FfnGemmArgs& a0, const FfnGemmArgs& a1, bool gateup, int NF,
                                     void* ev_start, void* ev_stop, hipStream_t s);

// Weighted combine.
// Storage type of the expert outputs y and shared_y: the output dtype, fp32,
// or fp16 (bf16 outputs only).
enum YType { Y_OUT = 0, Y_F32 = 1, Y_F16 = 2 };
hipError_t launch_combine(int T, int k, int d, bool out_bf16, int ytype, const void* y, const int32_t* pair_pos,
                          const float* tw, const void* shared_y, void* out, hipStream_t s);

// Hierarchical routing down an expert tree (tree_route.hip).
constexpr int kTreeMaxBranch = 64;
constexpr int kTreeMaxLevels = 16;
struct TreeShape {
  int n[kTreeMaxLevels + 1];          // existing nodes per depth (n[0] = 1, n[L] = E)
  long long first[kTreeMaxLevels + 1];// first gate row of each depth's children
  long long rows;                     // gate rows of the table
};
// false unless 2 <= B <= kTreeMaxBranch, 1 <= L <= kTreeMaxLevels, 1 <= E <= B^L
bool tree_shape(int E, int B, int L, TreeShape* sh);
size_t tree_ws_bytes(int T, int d, int k, int B, int L, bool bf16, const TreeShape& sh);
hipError_t launch_route_tree(int T, int d, int E, int k, int B, int L, bool bf16, const void* x, const void* w,
                             int renorm, int32_t* ids, float* tw, void* ws, hipStream_t s);

// INT4 quantiser.
hipError_t launch_quantize_int4(int rows, int K, const float* w, uint8_t* packed, uint16_t* scales,
                                hipStream_t s);

}  // namespace moe
