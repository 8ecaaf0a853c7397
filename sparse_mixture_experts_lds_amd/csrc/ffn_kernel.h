// Grouped expert GEMM kernel template on MFMA: the gate/up projection fused with the gated
// activation, and the down projection.
//
// Operation ("Sharding d'experts", "Deux roles": the worker's "3 mat-muls";
// MoEEvolve "Architecture": SwiGLU experts; kieve-moe "Features": GeGLU
// experts; ExpertMesh README: group-scaled signed INT4 routed experts):
//   gate/up:  z[r, n] = act(sum_k a[r,k] Wg[e,n,k]) * (sum_k a[r,k] Wu[e,n,k])
//   down:     y[r, n] = sum_k z[r,k] Wd[e,n,k]
// for every grouped row r of local expert e (rows offsets[e] .. offsets[e+1]).
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
  if (act == 0) return g / (1.0f + expf(-g));
  return 0.5f * g * (1.0f + erff(g * 0.70710678118654752f));
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

// Reorder 8 bf16 (a0..a7) to a0,a4,a1,a5,a2,a6,a3,a7.
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

template <int WT, int MF, int NF, bool GATEUP, bool SPLIT>
__global__ __launch_bounds__(256) void ffn_gemm_kernel(FfnGemmArgs args) {
  using Tr = Traits<WT>;
  constexpr int BM = 16 * MF;
  constexpr int BN = 64 * NF;
  constexpr int NB_FR = GATEUP ? 2 * NF : NF;          // B fragments per wave
  constexpr int KB = Tr::KB;
  constexpr bool F32 = WT == W_F32;
  constexpr bool I4 = WT == W_I4;
  static_assert(!(SPLIT && F32), "fp32 operands need no split");
  // SPLIT: the activations arrive in fp32 and are staged as two bf16 planes,
  // hi = bf16(v) and lo = bf16(v - hi), each multiplied by the weights.
  constexpr int LELT = F32 ? 4 : 2;                    // LDS element bytes
  constexpr int GELT = (F32 || SPLIT) ? 4 : 2;         // global activation element bytes
  constexpr int NPL = SPLIT ? 2 : 1;                   // LDS planes
  constexpr int AS = KB + 16 / LELT;                   // LDS row stride in elements (+16 B)
  constexpr int CHE = 16 / LELT;                       // elements per staged chunk (16 B of LDS)
  constexpr int CPR = KB / CHE;                        // chunks per staged row
  constexpr int GV = CHE * GELT / 16;                  // 16-byte global loads per chunk
  constexpr int NCH = (BM * CPR + 255) / 256;          // chunks per thread
  constexpr int STEPS = Tr::QS / Tr::EPS;
  constexpr int NS = kStages;                          // pipeline depth (prefetch distance NS-1)

  __shared__ __attribute__((aligned(16))) unsigned char lds_a[NS][NPL][BM * AS * LELT];
  __shared__ __attribute__((aligned(16))) float lds_s[NS][I4 ? BM : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 15;
  const int q = lane >> 4;

  // ---------------- tile decode (device-side tile count, XCD-contiguous ranges)
  const int N = args.N, K = args.K;
  const int NBLK = N / BN;
  int total_mt;
  if (args.offsets) total_mt = args.mtile_start[args.E_loc];
  else total_mt = (args.rows_max + BM - 1) / BM;
  const int total = total_mt * NBLK;
  const int G = gridDim.x;  // multiple of 8
  const int per = (total + 7) / 8;
  const int slot = blockIdx.x >> 3;
  if (slot >= per) return;
  const int R = (blockIdx.x & 7) * per + slot;
  if (R >= total) return;
  (void)G;

  // Tile order: groups of kGroupM m-tiles, m-tile fastest inside a group, so a
  // weight slice is re-read by the group's tiles side by side and the group's
  // activation rows stay in L2 across its n-blocks.
  int e = 0, row0, nrows, nb;
  {
    const int grp = R / (kGroupM * NBLK);
    const int t0 = grp * kGroupM;
    const int gm = min(kGroupM, total_mt - t0);
    const int rr = R - grp * kGroupM * NBLK;
    nb = rr / gm;
    const int t = t0 + (rr - nb * gm);
    if (args.tile_tab) {
      const int4 ti = args.tile_tab[t];
      e = ti.x;
      row0 = ti.y;
      nrows = ti.z;
    } else {
      row0 = t * BM;
      nrows = min(BM, args.rows_max - row0);
    }
  }
  const int n0 = nb * BN;

  // ---------------- activation staging setup
  // Every lane issues the same loads every k-block (no branches around loads,
  // so the compiler can count outstanding loads exactly): rows past the tile
  // end re-read the last valid row and are zeroed, k-blocks past the end re-read
  // the last block and are zeroed, and lanes without a chunk duplicate one.
  constexpr int CH_TOT = BM * CPR;
  const unsigned char* a_src[NCH];
  int a_dst[NCH];
  bool a_ok[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + 256 * j;
    const int ce = c % CH_TOT;
    const int r = ce / CPR;
    const int cc = ce - r * CPR;
    a_dst[j] = c < CH_TOT ? (r * AS + cc * CHE) * LELT : -1;
    a_ok[j] = r < nrows;
    const int gr = row0 + min(r, nrows - 1);
    const int srow = args.row_index ? args.row_index[gr] / args.row_div : gr;
    a_src[j] = static_cast<const unsigned char*>(args.A) + ((size_t)srow * K + cc * CHE) * GELT;
  }
  u32x4 a_reg[NS][NCH][GV];
  auto load_a = [&](int st, int kb) {
    const bool kin = kb < K;
    const int kbe = kin ? kb : K - KB;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
#pragma unroll
      for (int v = 0; v < GV; ++v) {
        const u32x4 t = *reinterpret_cast<const u32x4*>(a_src[j] + (size_t)kbe * GELT + 16 * v);
        a_reg[st][j][v] = (kin && a_ok[j]) ? t : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_a = [&](int st, int buf) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (a_dst[j] < 0) continue;
      u32x4 hi = a_reg[st][j][0], lo = u32x4{0, 0, 0, 0};
      if constexpr (SPLIT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v0 = __uint_as_float(a_reg[st][j][i >> 1][2 * (i & 1)]);
          const float v1 = __uint_as_float(a_reg[st][j][i >> 1][2 * (i & 1) + 1]);
          const uint32_t h0 = f32_to_bf16_bits(v0), h1 = f32_to_bf16_bits(v1);
          hi[i] = h0 | (h1 << 16);
          lo[i] = pack_bf16x2(v0 - bf16_bits_to_f32(h0), v1 - bf16_bits_to_f32(h1));
        }
      }
      if constexpr (I4) {
        // per-row sum of the group (16 lanes hold one row's 16 chunks)
        float sm = sum_bf16x8(hi);
        if constexpr (SPLIT) sm += sum_bf16x8(lo);
        sm += wave_shfl_xor(sm, 1);
        sm += wave_shfl_xor(sm, 2);
        sm += wave_shfl_xor(sm, 4);
        sm += wave_shfl_xor(sm, 8);
        if ((lane & 15) == 0) lds_s[buf][(tid + 256 * j) / CPR] = sm;
        hi = perm_04152637(hi);
        if constexpr (SPLIT) lo = perm_04152637(lo);
      }
      *reinterpret_cast<u32x4*>(&lds_a[buf][0][a_dst[j]]) = hi;
      if constexpr (SPLIT) *reinterpret_cast<u32x4*>(&lds_a[buf][NPL - 1][a_dst[j]]) = lo;
    }
  };

  // ---------------- weight fragment pointers
  const unsigned char* b_ptr[NB_FR];
  const uint16_t* s_ptr[NB_FR];
#pragma unroll
  for (int f = 0; f < NB_FR; ++f) {
    const bool second = GATEUP && f >= NF;
    const int fl = second ? f - NF : f;
    const int n = n0 + 16 * (NF * wave + fl) + lrow;
    const void* W = second ? args.W1 : args.W0;
    if constexpr (I4) {
      b_ptr[f] = static_cast<const unsigned char*>(W) + ((size_t)e * N + n) * (size_t)(K / 2) + q * 16;
      s_ptr[f] = (second ? args.S1 : args.S0) + ((size_t)e * N + n) * (size_t)(K / kI4Group);
    } else {
      b_ptr[f] = static_cast<const unsigned char*>(W) + (((size_t)e * N + n) * (size_t)K + q * Tr::QS) * Tr::AELT;
      s_ptr[f] = nullptr;
    }
  }
  u32x4 bbuf[NS][NB_FR][Tr::VPB];
  float sbuf[NS][NB_FR];
  auto load_b = [&](int buf, int kb) {
    const int kbe = min(kb, K - KB);  // past the end: re-read the last block (its activations are zero)
#pragma unroll
    for (int f = 0; f < NB_FR; ++f) {
      if constexpr (I4) {
        bbuf[buf][f][0] = *reinterpret_cast<const u32x4*>(b_ptr[f] + (size_t)kbe / 2);
        sbuf[buf][f] = half_bits_to_f32(s_ptr[f][kbe / kI4Group]);
      } else {
#pragma unroll
        for (int v = 0; v < Tr::VPB; ++v)
          bbuf[buf][f][v] = *reinterpret_cast<const u32x4*>(b_ptr[f] + (size_t)kbe * Tr::AELT + 16 * v);
      }
    }
  };

  f32x4 acc[MF][NB_FR];
#pragma unroll
  for (int mi = 0; mi < MF; ++mi)
#pragma unroll
    for (int f = 0; f < NB_FR; ++f) acc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    const unsigned char* As = lds_a[buf][0];
    const unsigned char* Al = lds_a[buf][NPL - 1];
    if constexpr (WT == W_F32) {
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        float a[MF];
#pragma unroll
        for (int mi = 0; mi < MF; ++mi)
          a[mi] = *reinterpret_cast<const float*>(As + ((16 * mi + lrow) * AS + Tr::QS * q + s) * LELT);
#pragma unroll
        for (int f = 0; f < NB_FR; ++f) {
          const u32x4 bv = bbuf[buf][f][s >> 2];
          const float b = __uint_as_float(bv[s & 3]);
#pragma unroll
          for (int mi = 0; mi < MF; ++mi) acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mi], b, acc[mi][f], 0, 0, 0);
        }
      }
    } else if constexpr (WT == W_BF16) {
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        bf16x8 a[MF], al[MF];
#pragma unroll
        for (int mi = 0; mi < MF; ++mi) {
          const int off = ((16 * mi + lrow) * AS + Tr::QS * q + 8 * s) * 2;
          a[mi] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(As + off));
          if constexpr (SPLIT) al[mi] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Al + off));
        }
#pragma unroll
        for (int f = 0; f < NB_FR; ++f) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, bbuf[buf][f][s]);
#pragma unroll
          for (int mi = 0; mi < MF; ++mi) {
            acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b, acc[mi][f], 0, 0, 0);
            if constexpr (SPLIT) acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[mi], b, acc[mi][f], 0, 0, 0);
          }
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
        bf16x8 a[MF], al[MF];
#pragma unroll
        for (int mi = 0; mi < MF; ++mi) {
          const int off = ((16 * mi + lrow) * AS + Tr::QS * q + 8 * s) * 2;
          a[mi] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(As + off));
          if constexpr (SPLIT) al[mi] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Al + off));
        }
#pragma unroll
        for (int f = 0; f < NB_FR; ++f) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, i4_word_to_bf16x8(bbuf[buf][f][0][s]));
#pragma unroll
          for (int mi = 0; mi < MF; ++mi) {
            gacc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b, gacc[mi][f], 0, 0, 0);
            if constexpr (SPLIT) gacc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[mi], b, gacc[mi][f], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int mi = 0; mi < MF; ++mi) {
        const f32x4 rs = *reinterpret_cast<const f32x4*>(&lds_s[buf][16 * mi + 4 * q]);
#pragma unroll
        for (int f = 0; f < NB_FR; ++f) {
          const float sc = sbuf[buf][f];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mi][f][r] = fmaf(sc, fmaf(-136.0f, rs[r], gacc[mi][f][r]), acc[mi][f][r]);
        }
      }
    }
  };

  // ---------------- main loop: NS-stage software pipeline, one LDS barrier per k-block.
  // Loads for k-block j+NS-1 are issued before k-block j is computed (activations
  // first, then weights), so the in-order vmcnt waits that guard each use leave
  // the newer prefetches in flight.  The barrier orders LDS only: a plain
  // __syncthreads would also drain every outstanding global load.
  const int NKB = K / KB;
  const int NIT = (NKB + NS - 1) / NS * NS;  // padded with all-zero activation blocks
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) {
    load_a(st, st * KB);
    load_b(st, st * KB);
  }
  store_a(0, 0);
  lds_barrier();
  for (int i = 0; i < NIT; i += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int j = i + u;
      const int pf = (u + NS - 1) % NS;
      load_a(pf, (j + NS - 1) * KB);
      load_b(pf, (j + NS - 1) * KB);
      compute(u);
      store_a((u + 1) % NS, (u + 1) % NS);
      lds_barrier();
    }
  }

  // ---------------- epilogue
  const bool f32out = F32 || args.out_f32;
#pragma unroll
  for (int mi = 0; mi < MF; ++mi) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int n = n0 + 16 * (NF * wave + f) + lrow;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mi + 4 * q + r;
        if (row >= nrows) continue;
        float v = acc[mi][f][r];
        if constexpr (GATEUP) v = act_fn(v, args.act) * acc[mi][NF + f][r];
        const size_t o = (size_t)(row0 + row) * N + n;
        if (f32out) static_cast<float*>(args.out)[o] = v;
        else static_cast<uint16_t*>(args.out)[o] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
  }
}

template <int WT, int MF, int NF, bool GU, bool SPLIT>
hipError_t launch_one(const FfnGemmArgs& a, hipStream_t s) {
  const int BM = 16 * MF, BN = 64 * NF;
  const int mt = a.offsets ? ffn_max_mtiles(a.E_loc, a.rows_max, BM) : (a.rows_max + BM - 1) / BM;
  long long g = (long long)mt * (a.N / BN);
  g = (g + 7) / 8 * 8;
  if (g == 0) return hipSuccess;
  ffn_gemm_kernel<WT, MF, NF, GU, SPLIT><<<dim3((unsigned)g), 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int WT, bool GU, bool SPLIT>
hipError_t launch_mf_nf(const FfnGemmArgs& a, int BM, int NF, hipStream_t s) {
#define MOE_CASE(MFv, NFv) \
  if (BM == 16 * MFv && NF == NFv) return launch_one<WT, MFv, NFv, GU, SPLIT>(a, s);
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
