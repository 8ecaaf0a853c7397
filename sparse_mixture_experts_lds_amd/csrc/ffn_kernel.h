// Grouped expert GEMM kernel template on MFMA: the gate/up projection fused with the gated
// activation, and the down projection.
//
// Operation ("Sharding d'experts", "Deux roles": the three matrix products a
// worker runs per expert;
// MoEEvolve "Architecture": SwiGLU experts; kieve-moe "Features": GeGLU
// experts; ExpertMesh README: group-scaled signed INT4 routed experts):
//   gate/up:  z[r, n] = act(sum_k a[r,k] Wg[e,n,k]) * (sum_k a[r,k] Wu[e,n,k])
//   down:     y[r, n] = sum_k z[r,k] Wd[e,n,k]
// for every grouped row r of local expert e (rows offsets[e] .. offsets[e+1]).
//
// Two problems per launch.  A launch covers one or two GEMM problems with the
// same K and N (the routed experts' grouped rows and the shared expert's dense
// rows, when the shared hidden width equals the routed one); each XCD takes a
// contiguous range of problem 0's tiles, then of problem 1's, so both spread
// evenly over the XCDs.
//
// Work decomposition.  A tile is (expert e, 16*MF rows, 64*NF output columns);
// the four waves of a workgroup split the columns, 16*NF each, and share the
// activation rows.  Tiles of one expert are consecutive, rows fastest, so the
// workgroups that re-read a weight slice run side by side; workgroup ids are
// remapped so that each XCD gets one contiguous range of tiles and those
// re-reads hit its own L2.  The number of tiles is read on the device (from
// the m-tile prefix of the grouping step): the grid is an upper bound and
// surplus workgroups exit at once, so the host never waits for routing.
//
// Data path per k-block (64 inputs, 128 for INT4):
//   activations  global -> registers -> LDS (double buffered, one barrier per
//                k-block), read back as MFMA A fragments (16 B per lane);
//   weights      global -> registers directly in the MFMA B-fragment layout,
//                prefetched one k-block ahead; each lane reads a contiguous
//                run of one weight row, so each weight byte is fetched once
//                per tile and never passes through LDS.
// Inside a k-block the lane group q (lanes 16q..16q+15) owns a contiguous
// slice of 1/4 of the inputs; A and B use the same slice, which is all the
// MFMA's K-sum needs.
//
// INT4: each lane loads 16 bytes = 32 codes of one 128-input group.  A code
// nibble c (two's complement) becomes the bf16 value 136 + c exactly by
// flipping bit 3 and OR-ing it into the mantissa of 128.0 (0x4300), two codes
// per 32-bit operation; the MFMA then accumulates sum a*(136+c) for the group,
// and the epilogue of the group applies  acc += scale * (sum - 136 * sum(a)),
// with sum(a) per row taken while the activations are staged.  Codes come
// out of a word in the order 0,4,1,5,2,6,3,7; the activations are staged in
// LDS in the same order.
#pragma once

#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace ffn_detail {

// Workgroup barrier that orders LDS accesses only (outstanding global loads
// stay in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

#ifndef MOE_FFN_STAGES
#define MOE_FFN_STAGES 4
#endif
constexpr int kStages = MOE_FFN_STAGES;
#ifndef MOE_I4_DOWN_STAGES
#define MOE_I4_DOWN_STAGES 4
#endif
constexpr int kI4DownStages = MOE_I4_DOWN_STAGES;
constexpr int kGroupM = 8;

template <int WT>
struct Traits;
template <>
struct Traits<W_BF16> {
  static constexpr int KB = 64;    // inputs per k-block
  static constexpr int QS = 16;    // inputs per lane group per k-block
  static constexpr int EPS = 8;    // inputs per lane per MFMA
  static constexpr int VPB = 2;    // 16-byte weight vectors per lane per fragment per k-block
  static constexpr int AELT = 2;   // activation bytes
};
template <>
struct Traits<W_F32> {
  static constexpr int KB = 64;
  static constexpr int QS = 16;
  static constexpr int EPS = 1;
  static constexpr int VPB = 4;
  static constexpr int AELT = 4;
};
template <>
struct Traits<W_I4> {
  static constexpr int KB = 128;
  static constexpr int QS = 32;
  static constexpr int EPS = 8;
  static constexpr int VPB = 1;
  static constexpr int AELT = 2;
};

__device__ __forceinline__ float act_fn(float g, int act) {
  if (act == 0) return silu_hw(g);
  return gelu_hw(g);
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Four bf16 pairs (codes 0,4 / 1,5 / 2,6 / 3,7 of the word) as 136 + code.
__device__ __forceinline__ u32x4 i4_word_to_bf16x8(uint32_t w) {
  const uint32_t v = w ^ 0x88888888u;
  u32x4 o;
  o[0] = (v & 0x000F000Fu) | 0x43004300u;
  o[1] = ((v >> 4) & 0x000F000Fu) | 0x43004300u;
  o[2] = ((v >> 8) & 0x000F000Fu) | 0x43004300u;
  o[3] = ((v >> 12) & 0x000F000Fu) | 0x43004300u;
  return o;
}

// The same four pairs as fp16, 1032 + code: 0x6400 is 1024, where the unit in
// the last place of fp16 is 1.
__device__ __forceinline__ u32x4 i4_word_to_f16x8(uint32_t w) {
  const uint32_t v = w ^ 0x88888888u;
  u32x4 o;
  o[0] = (v & 0x000F000Fu) | 0x64006400u;
  o[1] = ((v >> 4) & 0x000F000Fu) | 0x64006400u;
  o[2] = ((v >> 8) & 0x000F000Fu) | 0x64006400u;
  o[3] = ((v >> 12) & 0x000F000Fu) | 0x64006400u;
  return o;
}

// Reorder 8 16-bit values (a0..a7) to a0,a4,a1,a5,a2,a6,a3,a7.
__device__ __forceinline__ u32x4 perm_04152637(u32x4 d) {
  u32x4 o;
  o[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
  o[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
  o[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
  o[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
  return o;
}

__device__ __forceinline__ float sum_bf16x8(u32x4 d) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += bf16_bits_to_f32(d[i] & 0xFFFFu) + bf16_bits_to_f32(d[i] >> 16);
  return s;
}

__device__ __forceinline__ float sum_f16x8(u32x4 d) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += half_bits_to_f32(d[i] & 0xFFFFu) + half_bits_to_f32(d[i] >> 16);
  return s;
}

// Tiles one workgroup can hold decoded in LDS (row sources of NT_MAX tiles: 8 KB).
template <int BM>
struct TileCap {
  static constexpr int NT_MAX = 2048 / BM;
};

// One or two problems of one launch (same K, N, activation and output type).
struct GemmPair {
  FfnGemmArgs p[2];
  int np;  // 1 or 2
};

template <int WT, int MF, int NF, bool GATEUP, bool A16>
__global__ __launch_bounds__(256) void ffn_gemm_kernel(GemmPair gp) {
  const FfnGemmArgs& args = gp.p[0];  // K, N, act, out_f32: common to both problems
  using Tr = Traits<WT>;
  constexpr int BM = 16 * MF;
  constexpr int BN = 64 * NF;
  constexpr int NB_FR = GATEUP ? 2 * NF : NF;          // B fragments per wave
  constexpr int KB = Tr::KB;
  constexpr bool F32 = WT == W_F32;
  constexpr bool I4 = WT == W_I4;
  static_assert(!A16 || (I4 && !GATEUP), "fp16 activations: INT4 down projections only");
  // A16: the activations (the z of an INT4 layer) are fp16; the codes are
  // then decoded to fp16 and multiplied on the fp16 MFMA (else bf16).
  constexpr int LELT = F32 ? 4 : 2;                    // LDS element bytes
  constexpr int GELT = F32 ? 4 : 2;                    // global activation element bytes
  constexpr int AS = KB + 16 / LELT;                   // LDS row stride in elements (+16 B)
  constexpr int CHE = 16 / LELT;                       // elements per staged chunk (16 B of LDS)
  constexpr int CPR = KB / CHE;                        // chunks per staged row
  constexpr int GV = CHE * GELT / 16;                  // 16-byte global loads per chunk
  constexpr int NCH = (BM * CPR + 255) / 256;          // chunks per thread
  constexpr int STEPS = Tr::QS / Tr::EPS;
  // register stages (prefetch distance NS-1); the largest tiles keep one stage
  // less so that two workgroups still fit on a CU
  constexpr int NS = A16 ? kI4DownStages : (MF * NB_FR >= 16 ? 3 : kStages);
  constexpr int NT_MAX = TileCap<BM>::NT_MAX;

  // LDS: the activation double buffer, reused after each tile's k-loop as the
  // output staging tile; the decoded tiles of this workgroup.
  constexpr int ABUF = BM * AS * LELT;
  constexpr int RING = 2 * ABUF;
  constexpr int OS_MAX = BN * 4 + 16;  // output row stride in bytes for fp32 outputs (+16 B pad)
  constexpr int LDS_BYTES = RING > BM * OS_MAX ? RING : BM * OS_MAX;
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float lds_s[2][I4 ? BM : 4];
  __shared__ int4 lds_tile[NT_MAX];      // {expert, row0, rows, n-block}
  __shared__ int lds_src[NT_MAX][BM];    // source activation row of every tile row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 15;
  const int q = lane >> 4;
  const int N = args.N, K = args.K;
  const int NBLK = N / BN;

  // ---------------- work range of this workgroup
  // Tiles of a problem are numbered R = 0..total-1 in grouped-M order; XCD
  // x = blockIdx % 8 owns the contiguous range [x*per, (x+1)*per) of each
  // problem (n0x tiles of problem 0, then n1x of problem 1: its local slots
  // 0..n0x+n1x-1) and its S workgroups stride through those slots, so the
  // tiles that share a weight slice or activation rows run side by side on
  // one XCD and hit its L2.
  auto total_mtiles = [&](const FfnGemmArgs& a) -> int {
    return a.offsets ? a.mtile_start[a.E_loc] : (a.rows_max + BM - 1) / BM;
  };
  const int total0 = total_mtiles(gp.p[0]) * NBLK;
  const int total1 = gp.np > 1 ? total_mtiles(gp.p[1]) * NBLK : 0;
  const int S = gridDim.x >> 3;  // grid is a multiple of 8
  const int xcd = blockIdx.x & 7;
  const int per0 = (total0 + 7) / 8, per1 = (total1 + 7) / 8;
  const int n0x = max(0, min(per0, total0 - xcd * per0));
  const int n1x = max(0, min(per1, total1 - xcd * per1));
  const int first = blockIdx.x >> 3;
  const int nx = n0x + n1x;
  const int ntiles = first < nx ? min((nx - first + S - 1) / S, NT_MAX) : 0;
  if (ntiles == 0) return;

  // ---------------- decode every tile of this workgroup into LDS (once);
  // the problem index rides in bits 24+ of the n-block field
  if (tid < ntiles) {
    const int sl = first + tid * S;
    const int pi = sl < n0x ? 0 : 1;
    const FfnGemmArgs& a = gp.p[pi];
    const int R = pi ? xcd * per1 + (sl - n0x) : xcd * per0 + sl;
    const int total_mt = (pi ? total1 : total0) / NBLK;
    // groups of GM m-tiles, m-tile fastest inside a group: GM = kGroupM
    // shares each weight tile between neighbouring m-tiles of one expert;
    // where experts average fewer than two m-tiles there is little of that to
    // share, and GM = 1 puts an expert's n-tiles side by side instead, so its
    // activation rows are fetched into one XCD's L2 once
    const int GM = (a.offsets && total_mt < 2 * a.E_loc) ? 1 : kGroupM;
    const int grp = R / (GM * NBLK);
    const int t0 = grp * GM;
    const int gm = min(GM, total_mt - t0);
    const int rr = R - grp * GM * NBLK;
    const int nb = rr / gm;
    const int t = t0 + (rr - nb * gm);
    int4 ti;
    if (a.tile_tab) {
      ti = a.tile_tab[t];
    } else {
      ti.x = 0;
      ti.y = t * BM;
      ti.z = min(BM, a.rows_max - t * BM);
    }
    ti.w = nb | (pi << 24);
    lds_tile[tid] = ti;
  }
  __syncthreads();
  for (int idx = tid; idx < ntiles * BM; idx += 256) {
    const int i = idx / BM;
    const int r = idx - i * BM;
    const int4 ti = lds_tile[i];
    const FfnGemmArgs& a = gp.p[ti.w >> 24];
    const int gr = ti.y + min(r, max(ti.z - 1, 0));
    lds_src[i][r] = a.row_index ? a.row_index[gr] / a.row_div : gr;
  }
  __syncthreads();

  // ---------------- per-tile operand addresses
  // Every lane issues the same loads every k-block (no branches around loads,
  // so the compiler can count outstanding loads exactly).  Rows past the tile
  // end re-read the tile's last row: a row of the product depends only on the
  // same row of the activations, and those rows are never stored.  k-blocks
  // past the end (padding) re-read the last block and are zeroed.  Activation
  // rows are 32-bit byte offsets (the activation matrix is below 4 GiB); the
  // weight slice of a tile is a uniform base plus a fixed per-lane offset.
  constexpr int CH_TOT = BM * CPR;
  int a_dst[NCH];
  int a_row[NCH];
  uint32_t a_col[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + 256 * j;
    const int ce = c % CH_TOT;
    a_row[j] = ce / CPR;
    const int cc = ce - a_row[j] * CPR;
    a_col[j] = (uint32_t)(cc * CHE * GELT);
    a_dst[j] = c < CH_TOT ? (a_row[j] * AS + cc * CHE) * LELT : -1;
  }
  uint32_t b_lane[NB_FR];  // lane offset of fragment f inside a tile's weight slice (bytes)
  uint32_t s_lane[NB_FR];  // INT4: lane offset into the scales (elements)
#pragma unroll
  for (int f = 0; f < NB_FR; ++f) {
    const int fl = (GATEUP && f >= NF) ? f - NF : f;
    const int nl = 16 * (NF * wave + fl) + lrow;
    if constexpr (I4) {
      b_lane[f] = (uint32_t)(nl * (K / 2) + q * 16);
      s_lane[f] = (uint32_t)(nl * (K / kI4Group));
    } else {
      b_lane[f] = (uint32_t)((nl * K + q * Tr::QS) * Tr::AELT);
      s_lane[f] = 0;
    }
  }
  struct Ptrs {
    const unsigned char* abase;
    uint32_t a[NCH];
    const unsigned char* w0;
    const unsigned char* w1;
    const uint16_t* s0;
    const uint16_t* s1;
  };
  auto setup = [&](int i, Ptrs& P) {
    const int4 ti = lds_tile[i];
    const int e = __builtin_amdgcn_readfirstlane(ti.x);
    const int pi = __builtin_amdgcn_readfirstlane(ti.w) >> 24;
    const int n0 = (__builtin_amdgcn_readfirstlane(ti.w) & 0xFFFFFF) * BN;
    const FfnGemmArgs& args = gp.p[pi];
    P.abase = static_cast<const unsigned char*>(args.A);
#pragma unroll
    for (int j = 0; j < NCH; ++j) P.a[j] = (uint32_t)lds_src[i][a_row[j]] * (uint32_t)(K * GELT) + a_col[j];
    const size_t row_first = (size_t)e * N + n0;  // first weight row of the tile
    if constexpr (I4) {
      P.w0 = static_cast<const unsigned char*>(args.W0) + row_first * (size_t)(K / 2);
      P.w1 = GATEUP ? static_cast<const unsigned char*>(args.W1) + row_first * (size_t)(K / 2) : P.w0;
      P.s0 = args.S0 + row_first * (size_t)(K / kI4Group);
      P.s1 = GATEUP ? args.S1 + row_first * (size_t)(K / kI4Group) : P.s0;
    } else {
      P.w0 = static_cast<const unsigned char*>(args.W0) + row_first * (size_t)K * Tr::AELT;
      P.w1 = GATEUP ? static_cast<const unsigned char*>(args.W1) + row_first * (size_t)K * Tr::AELT : P.w0;
      P.s0 = P.s1 = nullptr;
    }
  };

  u32x4 a_reg[NS][NCH][GV];
  u32x4 bbuf[NS][NB_FR][Tr::VPB];
  float sbuf[NS][NB_FR];
  auto load_a = [&](int st, const Ptrs& P, int kb) {
    const bool kin = kb < K;
    const unsigned char* base = P.abase + (size_t)(kin ? kb : K - KB) * GELT;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
#pragma unroll
      for (int v = 0; v < GV; ++v) {
        const u32x4 t = *reinterpret_cast<const u32x4*>(base + P.a[j] + 16 * v);
        a_reg[st][j][v] = kin ? t : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto load_b = [&](int st, const Ptrs& P, int kb) {
    const int kbe = min(kb, K - KB);  // past the end: re-read the last block (its activations are zero)
#pragma unroll
    for (int f = 0; f < NB_FR; ++f) {
      const bool second = GATEUP && f >= NF;
      if constexpr (I4) {
        const unsigned char* w = (second ? P.w1 : P.w0) + kbe / 2;
        bbuf[st][f][0] = *reinterpret_cast<const u32x4*>(w + b_lane[f]);
        sbuf[st][f] = half_bits_to_f32(((second ? P.s1 : P.s0) + kbe / kI4Group)[s_lane[f]]);
      } else {
        const unsigned char* w = (second ? P.w1 : P.w0) + (size_t)kbe * Tr::AELT;
#pragma unroll
        for (int v = 0; v < Tr::VPB; ++v) bbuf[st][f][v] = *reinterpret_cast<const u32x4*>(w + b_lane[f] + 16 * v);
      }
    }
  };
  auto lds_a_at = [&](int lb) -> unsigned char* { return lds_raw + lb * ABUF; };
  auto store_a = [&](int st, int lb) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (a_dst[j] < 0) continue;
      u32x4 v = a_reg[st][j][0];
      if constexpr (I4) {
        // per-row sum of the group (16 lanes hold one row's 16 chunks)
        float sm = A16 ? sum_f16x8(v) : sum_bf16x8(v);
        sm += wave_shfl_xor(sm, 1);
        sm += wave_shfl_xor(sm, 2);
        sm += wave_shfl_xor(sm, 4);
        sm += wave_shfl_xor(sm, 8);
        if ((lane & 15) == 0) lds_s[lb][(tid + 256 * j) / CPR] = sm;
        v = perm_04152637(v);
      }
      *reinterpret_cast<u32x4*>(lds_a_at(lb) + a_dst[j]) = v;
    }
  };

  f32x4 acc[MF][NB_FR];

  auto compute = [&](int st, int lb) {
    const unsigned char* As = lds_a_at(lb);
    if constexpr (WT == W_F32) {
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        float a[MF];
#pragma unroll
        for (int mi = 0; mi < MF; ++mi)
          a[mi] = *reinterpret_cast<const float*>(As + ((16 * mi + lrow) * AS + Tr::QS * q + s) * LELT);
#pragma unroll
        for (int f = 0; f < NB_FR; ++f) {
          const u32x4 bv = bbuf[st][f][s >> 2];
          const float b = __uint_as_float(bv[s & 3]);
#pragma unroll
          for (int mi = 0; mi < MF; ++mi) acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mi], b, acc[mi][f], 0, 0, 0);
        }
      }
    } else if constexpr (WT == W_BF16) {
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        bf16x8 a[MF];
#pragma unroll
        for (int mi = 0; mi < MF; ++mi) {
          const int off = ((16 * mi + lrow) * AS + Tr::QS * q + 8 * s) * 2;
          a[mi] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(As + off));
        }
#pragma unroll
        for (int f = 0; f < NB_FR; ++f) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, bbuf[st][f][s]);
#pragma unroll
          for (int mi = 0; mi < MF; ++mi)
            acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b, acc[mi][f], 0, 0, 0);
        }
      }
    } else {  // INT4
      f32x4 gacc[MF][NB_FR];
#pragma unroll
      for (int mi = 0; mi < MF; ++mi)
#pragma unroll
        for (int f = 0; f < NB_FR; ++f) gacc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        u32x4 a[MF];
#pragma unroll
        for (int mi = 0; mi < MF; ++mi) {
          const int off = ((16 * mi + lrow) * AS + Tr::QS * q + 8 * s) * 2;
          a[mi] = *reinterpret_cast<const u32x4*>(As + off);
        }
#pragma unroll
        for (int f = 0; f < NB_FR; ++f) {
          const uint32_t w = bbuf[st][f][0][s];
#pragma unroll
          for (int mi = 0; mi < MF; ++mi) {
            if constexpr (A16)
              gacc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[mi]),
                                                                   __builtin_bit_cast(f16x8, i4_word_to_f16x8(w)),
                                                                   gacc[mi][f], 0, 0, 0);
            else
              gacc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mi]),
                                                                    __builtin_bit_cast(bf16x8, i4_word_to_bf16x8(w)),
                                                                    gacc[mi][f], 0, 0, 0);
          }
        }
      }
      // gacc = sum a (offset + code), the offset 1032 (fp16) or 136 (bf16)
      constexpr float kOff = A16 ? -1032.0f : -136.0f;
#pragma unroll
      for (int mi = 0; mi < MF; ++mi) {
        const f32x4 rs = *reinterpret_cast<const f32x4*>(&lds_s[lb][16 * mi + 4 * q]);
#pragma unroll
        for (int f = 0; f < NB_FR; ++f) {
          const float sc = sbuf[st][f];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mi][f][r] = fmaf(sc, fmaf(kOff, rs[r], gacc[mi][f][r]), acc[mi][f][r]);
        }
      }
    }
  };

  // ---------------- tile loop with a continuous NS-stage software pipeline.
  // Loads for k-block j+NS-1 are issued before k-block j is computed, so the
  // in-order vmcnt waits that guard each use leave the newer prefetches in
  // flight; the barrier orders LDS only (a plain __syncthreads would also drain
  // every outstanding global load).  During the last NS-1 k-blocks of a tile
  // the prefetches already fetch the first k-blocks of the workgroup's next
  // tile (of the same tile again after the last one; never computed), so the
  // epilogue overlaps those loads.  k-block j of a tile sits in register stage
  // j % NS; consecutive k-blocks of the whole sequence alternate between the
  // two LDS buffers.
  const int NKB = K / KB;
  const int NIT = (NKB + NS - 1) / NS * NS;  // padded with all-zero activation blocks
  const bool f32out = F32 || args.out_f32;
  const bool f16out = !f32out && args.out_f16;
  const int osz = f32out ? 4 : 2;
  const int OS = BN * osz + 16;
  const int cpr = BN * osz / 16;  // 16-byte chunks per output row

  Ptrs cur, nxt;
  setup(0, cur);
  setup(min(1, ntiles - 1), nxt);
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) {
    load_a(st, cur, st * KB);
    load_b(st, cur, st * KB);
  }
  int par = 0;  // LDS buffer of the tile's k-block 0
  for (int it = 0; it < ntiles; ++it) {
#pragma unroll
    for (int mi = 0; mi < MF; ++mi)
#pragma unroll
      for (int f = 0; f < NB_FR; ++f) acc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    store_a(0, par);
    lds_barrier();
    for (int i = 0; i < NIT - NS; i += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int pf = (u + NS - 1) % NS;
        const int lb = (par + i + u) & 1;
        load_a(pf, cur, (i + u + NS - 1) * KB);
        load_b(pf, cur, (i + u + NS - 1) * KB);
        compute(u, lb);
        store_a((u + 1) % NS, lb ^ 1);
        lds_barrier();
      }
    }
    // last NS k-blocks: the first prefetch is this tile's last k-block, the
    // others are k-blocks 0..NS-2 of the next tile
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int pf = (u + NS - 1) % NS;
      const int lb = (par + NIT - NS + u) & 1;
      if (u == 0) {
        load_a(pf, cur, (NIT - 1) * KB);
        load_b(pf, cur, (NIT - 1) * KB);
      } else {
        load_a(pf, nxt, (u - 1) * KB);
        load_b(pf, nxt, (u - 1) * KB);
      }
      compute(u, lb);
      if (u + 1 < NS) store_a(u + 1, lb ^ 1);
      lds_barrier();
    }
    par = (par + NIT) & 1;

    // epilogue: results -> LDS tile (output dtype) -> 16-byte row stores
    {
      const int4 ti = lds_tile[it];
      const int row0 = ti.y, nrows = ti.z, n0 = (ti.w & 0xFFFFFF) * BN;
      void* const out = gp.p[__builtin_amdgcn_readfirstlane(ti.w) >> 24].out;
#pragma unroll
      for (int mi = 0; mi < MF; ++mi) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int col = 16 * (NF * wave + f) + lrow;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * mi + 4 * q + r;
            float v = acc[mi][f][r];
            if constexpr (GATEUP) v = act_fn(v, args.act) * acc[mi][NF + f][r];
            unsigned char* dst = lds_raw + row * OS + col * osz;
            if (f32out) *reinterpret_cast<float*>(dst) = v;
            else if (f16out) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)f32_to_f16_bits(v);
            else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)f32_to_bf16_bits(v);
          }
        }
      }
      lds_barrier();
      unsigned char* obase = static_cast<unsigned char*>(out) + ((size_t)row0 * N + n0) * osz;
      for (int c = tid; c < nrows * cpr; c += 256) {
        const int row = c / cpr;
        const int cc = c - row * cpr;
        *reinterpret_cast<u32x4*>(obase + (size_t)row * N * osz + cc * 16) =
            *reinterpret_cast<const u32x4*>(lds_raw + row * OS + cc * 16);
      }
      lds_barrier();
    }
    cur = nxt;
    setup(min(it + 2, ntiles - 1), nxt);
  }
}

template <int WT, int MF, int NF, bool GU, bool A16>
int resident_groups(int& cus) {
  static int cached_occ = -1, cached_cus = -1;
  if (cached_occ < 0) {
    int dev = 0, occ = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, ffn_gemm_kernel<WT, MF, NF, GU, A16>, 256, 0) !=
            hipSuccess) {
      occ = 1;
      n = 256;
    }
    cached_cus = n > 0 ? n : 256;
    cached_occ = occ > 0 ? occ : 1;
  }
  cus = cached_cus;
  return cached_occ;
}

template <int WT, int MF, int NF, bool GU, bool A16>
hipError_t launch_one(const FfnGemmArgs* a, int np, hipStream_t s) {
  const int BM = 16 * MF, BN = 64 * NF;
  GemmPair gp{};
  gp.np = np;
  long long per_ub = 0;  // per-XCD tiles, upper bound
  for (int i = 0; i < np; ++i) {
    const FfnGemmArgs& p = a[i];
    if (p.N % BN || (i > 0 && (p.K != a[0].K || p.N != a[0].N || p.act != a[0].act || p.out_f32 != a[0].out_f32 ||
                               p.out_f16 != a[0].out_f16)))
      return hipErrorInvalidValue;
    const int mt = p.offsets ? ffn_max_mtiles(p.E_loc, p.rows_max, BM) : (p.rows_max + BM - 1) / BM;
    per_ub += ((long long)mt * (p.N / BN) + 7) / 8;
    gp.p[i] = p;
  }
  if (per_ub == 0) return hipSuccess;
  // Persistent grid: every resident slot once, but no more than the tiles there
  // can be, and enough workgroups that none holds more than NT_MAX tiles.
  int cus = 256;
  const int occ = resident_groups<WT, MF, NF, GU, A16>(cus);
  constexpr int NT_MAX = TileCap<16 * MF>::NT_MAX;
  const long long slots = (long long)occ * cus / 8;
  long long S = std::max<long long>(slots, (per_ub + NT_MAX - 1) / NT_MAX);
  S = std::min<long long>(S, per_ub);
  const long long g = 8 * S;
  const dim3 grid((unsigned)g), block(256);
  auto kernel = ffn_gemm_kernel<WT, MF, NF, GU, A16>;
  if (a[0].ev_start || a[0].ev_stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, static_cast<hipEvent_t>(a[0].ev_start),
                          static_cast<hipEvent_t>(a[0].ev_stop), 0, gp);
  else
    kernel<<<grid, block, 0, s>>>(gp);
  return hipGetLastError();
}

// np problems (1 or 2) of the same K and N in one launch, problem 0's tiles
// dispatched first
template <int WT, bool GU, bool A16>
hipError_t launch_mf_nf(const FfnGemmArgs* a, int np, int BM, int NF, hipStream_t s) {
  if (np < 1 || np > 2) return hipErrorInvalidValue;
#define MOE_CASE(MFv, NFv) \
  if (BM == 16 * MFv && NF == NFv) return launch_one<WT, MFv, NFv, GU, A16>(a, np, s);
  if constexpr (WT == W_F32) {
    MOE_CASE(1, 1) MOE_CASE(1, 2) MOE_CASE(2, 1) MOE_CASE(2, 2)
  } else if constexpr (WT == W_I4) {
    MOE_CASE(1, 1) MOE_CASE(1, 2) MOE_CASE(2, 1) MOE_CASE(2, 2) MOE_CASE(4, 1) MOE_CASE(4, 2)
  } else {
    MOE_CASE(1, 1) MOE_CASE(1, 2) MOE_CASE(2, 1) MOE_CASE(2, 2) MOE_CASE(4, 1) MOE_CASE(4, 2)
    MOE_CASE(8, 1) MOE_CASE(8, 2)
  }
#undef MOE_CASE
  return hipErrorInvalidValue;
}

}  // namespace ffn_detail
}  // namespace moe
