// Grouped GEMMs of the layer backward on MFMA (gfx950).
//
//   nn_kernel (data gradients)   C[r, n]   = sum_k A[row(r), k] * B_g[k, n]
//       rows r grouped by expert g (m-tile table), A rows optionally gathered,
//       B_g row-major [K, N] (n contiguous), split along k over two matrices
//       (k < K1 from B1_g, else row k - K1 of B2_g): dz = dy Wd, dx = [dg du] [Wg; Wu]
//   tn_kernel (weight gradients) C_g[m, n] = sum_{r in group g} A[row_a(r), m] * B[row_b(r), n]
//       contraction over the rows of a group (a segment of the grouped rows,
//       or a slice of all rows), both operands row-major with the output
//       dimension contiguous: dWd = dy^T z, [dWg; dWu] = [dg du]^T x
//
// The operand whose contiguous dimension is an output dimension (B of
// nn_kernel, both operands of tn_kernel) is staged in LDS as it lies in
// memory, [k][mn], and read into MFMA fragments with the transposing LDS read
// ds_read_b64_tr_b16: lane a of a 16-lane group points at 4 consecutive
// 16-bit values of row k0 + (a >> 2), columns x0 + 4 (a & 3); lane l then
// receives the values of column x0 + l for rows k0 .. k0 + 3, i.e. one
// quarter of the 8-value k-run the 16x16x32 bf16 MFMA takes per lane.  Two
// such reads (rows k0 and k0 + 4) make the fragment.
//
// Tiles: 256 threads, 4 waves; nn: BM 64 or 128 rows x 128 columns, tn: 128 x
// 128; 32 (bf16) or 16 (fp32) contraction steps per k-block; global ->
// registers -> LDS, two LDS buffers, one barrier per k-block.  Accumulation in fp32; fp32 operands use
// the 16x16x4 fp32 MFMA.
#pragma once

#include "bwd.h"

namespace moe {
namespace bwdg {

constexpr int BN = 128;  // output columns per tile
constexpr int NTH = 256;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

template <typename T>
struct Elt {
  static constexpr int V = 16 / (int)sizeof(T);          // elements per 16-byte vector
  static constexpr int PAD = sizeof(T) == 2 ? 16 : 4;    // [k][mn] row padding (elements)
  static constexpr int KB = sizeof(T) == 2 ? 32 : 16;    // contraction elements per k-block
};

// One bf16 fragment (8 consecutive k for column x0 + lane % 16) from a [k][mn]
// tile: rows k0 .. k0 + 7 of group q = lane / 16 start at k0 = kb0 + 8 q.
__device__ __forceinline__ bf16x8 frag_tr(const uint16_t* tile, int stride, int kb0, int x0, int lane) {
  const int q = lane >> 4, a = lane & 15;
  const uint16_t* p = tile + (kb0 + 8 * q + (a >> 2)) * stride + x0 + 4 * (a & 3);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * stride));
  const v8s c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// ------------------------------------------------------------------ nn
template <typename T, int BM>
__global__ __launch_bounds__(NTH) void nn_kernel(NnArgs a) {
  constexpr int V = Elt<T>::V;
  constexpr int KB = Elt<T>::KB;
  constexpr int BS = BN + Elt<T>::PAD;  // B tile row stride
  constexpr int WM = BM / 64, WN = 4 / WM;
  constexpr int FN = BN / WN / 16;  // 2 (BM 64) or 4 (BM 128) fragments across
  constexpr int A_CH = KB / V;      // vectors per A row per k-block
  constexpr int A_VEC = BM * A_CH / NTH;
  constexpr int B_CH = BN / V;
  constexpr int B_VEC = KB * B_CH / NTH;
  __shared__ __attribute__((aligned(16))) T As[2][BM * KB];
  __shared__ __attribute__((aligned(16))) T Bs[2][KB * BS];

  int g = 0, row0, nrows;
  if (a.tile_tab) {
    if ((int)blockIdx.x >= a.mtile_start[a.groups]) return;
    const int4 tt = a.tile_tab[blockIdx.x];
    g = tt.x;
    row0 = tt.y;
    nrows = tt.z;
  } else {
    row0 = blockIdx.x * BM;
    nrows = min(BM, a.rows - row0);
    if (nrows <= 0) return;
  }
  const int n0 = blockIdx.y * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const T* Ab = static_cast<const T*>(a.A);
  const T* a_src[A_VEC];
  bool a_ok[A_VEC];
#pragma unroll
  for (int i = 0; i < A_VEC; ++i) {
    const int lr = tid / A_CH + i * (NTH / A_CH);
    a_ok[i] = lr < nrows;
    const int r = row0 + (a_ok[i] ? lr : 0);
    const int src = a.a_index ? a.a_index[r] / a.a_div : r;
    a_src[i] = Ab + (size_t)src * a.lda + (tid % A_CH) * V;
  }
  const int b_col = n0 + (tid % B_CH) * V;
  const bool b_col_ok = b_col < a.N;
  const T* B1 = static_cast<const T*>(a.B1) + (size_t)g * a.b_stride;
  const T* B2 = a.B2 ? static_cast<const T*>(a.B2) + (size_t)g * a.b_stride : nullptr;

  u32x4 ra[A_VEC], rb[B_VEC];
  auto load = [&](int kb) {
#pragma unroll
    for (int i = 0; i < A_VEC; ++i)
      ra[i] = a_ok[i] ? *reinterpret_cast<const u32x4*>(a_src[i] + kb * KB) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < B_VEC; ++i) {
      const int k = kb * KB + tid / B_CH + i * (NTH / B_CH);
      const bool ok = b_col_ok && k < a.K_valid;
      const T* p = k < a.K1 ? B1 + (size_t)k * a.ldb : B2 + (size_t)(k - a.K1) * a.ldb;
      rb[i] = ok ? *reinterpret_cast<const u32x4*>(p + b_col) : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_VEC; ++i) {
      const int lr = tid / A_CH + i * (NTH / A_CH);
      *reinterpret_cast<u32x4*>(&As[buf][lr * KB + (tid % A_CH) * V]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_VEC; ++i) {
      const int kr = tid / B_CH + i * (NTH / B_CH);
      *reinterpret_cast<u32x4*>(&Bs[buf][kr * BS + (tid % B_CH) * V]) = rb[i];
    }
  };

  f32x4 acc[4][FN];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int f = 0; f < FN; ++f) acc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    const int lr = lane & 15, q = lane >> 4;
    if constexpr (sizeof(T) == 2) {
      bf16x8 fa[4], fb[FN];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        fa[mi] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm * 64 + 16 * mi + lr) * KB + 8 * q]);
#pragma unroll
      for (int f = 0; f < FN; ++f)
        fb[f] = frag_tr(reinterpret_cast<const uint16_t*>(Bs[buf]), BS, 0, wn * (BN / WN) + 16 * f, lane);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int f = 0; f < FN; ++f) acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mi], fb[f], acc[mi][f], 0, 0, 0);
    } else {
#pragma unroll
      for (int s = 0; s < KB / 4; ++s) {
        float fa[4], fb[FN];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) fa[mi] = As[buf][(wm * 64 + 16 * mi + lr) * KB + 4 * s + q];
#pragma unroll
        for (int f = 0; f < FN; ++f) fb[f] = Bs[buf][(4 * s + q) * BS + wn * (BN / WN) + 16 * f + lr];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int f = 0; f < FN; ++f) acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[mi], fb[f], acc[mi][f], 0, 0, 0);
      }
    }
  };

  const int nkb = a.K / KB;
  load(0);
  store(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) load(kb + 1);
    compute(kb & 1);
    if (kb + 1 < nkb) store((kb + 1) & 1);
    __syncthreads();
  }

  const int lr = lane & 15, q = lane >> 4;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int col = n0 + wn * (BN / WN) + 16 * f + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lrow = wm * 64 + 16 * mi + 4 * q + r;
        if (lrow < nrows && col < a.N) a.C[(size_t)(row0 + lrow) * a.ldc + col] = acc[mi][f][r];
      }
    }
  }
}

// ------------------------------------------------------------------ tn
template <typename T>
__global__ __launch_bounds__(NTH) void tn_kernel(TnArgs a) {
  constexpr int BM = 128;
  constexpr int V = Elt<T>::V;
  constexpr int KB = Elt<T>::KB;
  constexpr int S = 128 + Elt<T>::PAD;  // tile row stride (both operands)
  constexpr int CH = 128 / V;           // vectors per tile row
  constexpr int VEC = KB * CH / NTH;
  __shared__ __attribute__((aligned(16))) T At[2][KB * S];
  __shared__ __attribute__((aligned(16))) T Bt[2][KB * S];

  const int z = blockIdx.y;
  const int mt = blockIdx.x % a.mtiles, nt = blockIdx.x / a.mtiles;
  const int m0 = mt * BM, n0 = nt * BN;
  int r0, r1;
  if (a.offsets) {
    r0 = a.offsets[z];
    r1 = a.offsets[z + 1];
  } else {
    r0 = z * a.slice;
    r1 = min(a.rows, r0 + a.slice);
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int col_a = m0 + (tid % CH) * V, col_b = n0 + (tid % CH) * V;
  const bool a_col_ok = col_a < a.M, b_col_ok = col_b < a.N;
  const T* Ab = static_cast<const T*>(a.A);
  const T* Bb = static_cast<const T*>(a.B);

  u32x4 ra[VEC], rb[VEC];
  auto load = [&](int kb) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const int r = r0 + kb * KB + tid / CH + i * (NTH / CH);
      const bool in = r < r1;
      const int ra_row = in ? (a.a_index ? a.a_index[r] / a.a_div : r) : 0;
      const int rb_row = in ? (a.b_index ? a.b_index[r] / a.b_div : r) : 0;
      ra[i] = (in && a_col_ok) ? *reinterpret_cast<const u32x4*>(Ab + (size_t)ra_row * a.lda + col_a)
                               : u32x4{0, 0, 0, 0};
      rb[i] = (in && b_col_ok) ? *reinterpret_cast<const u32x4*>(Bb + (size_t)rb_row * a.ldb + col_b)
                               : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const int kr = tid / CH + i * (NTH / CH);
      *reinterpret_cast<u32x4*>(&At[buf][kr * S + (tid % CH) * V]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bt[buf][kr * S + (tid % CH) * V]) = rb[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    if constexpr (sizeof(T) == 2) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        fa[mi] = frag_tr(reinterpret_cast<const uint16_t*>(At[buf]), S, 0, wm * 64 + 16 * mi, lane);
#pragma unroll
      for (int f = 0; f < 4; ++f)
        fb[f] = frag_tr(reinterpret_cast<const uint16_t*>(Bt[buf]), S, 0, wn * 64 + 16 * f, lane);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mi], fb[f], acc[mi][f], 0, 0, 0);
    } else {
      const int lr = lane & 15, q = lane >> 4;
#pragma unroll
      for (int s = 0; s < KB / 4; ++s) {
        float fa[4], fb[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) fa[mi] = At[buf][(4 * s + q) * S + wm * 64 + 16 * mi + lr];
#pragma unroll
        for (int f = 0; f < 4; ++f) fb[f] = Bt[buf][(4 * s + q) * S + wn * 64 + 16 * f + lr];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[mi], fb[f], acc[mi][f], 0, 0, 0);
      }
    }
  };

  const int nkb = r1 > r0 ? (r1 - r0 + KB - 1) / KB : 0;
  if (nkb > 0) {
    load(0);
    store(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
      if (kb + 1 < nkb) load(kb + 1);
      compute(kb & 1);
      if (kb + 1 < nkb) store((kb + 1) & 1);
      __syncthreads();
    }
  }
  // an empty group still writes its (zero) gradient
  const int lr = lane & 15, q = lane >> 4;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + 16 * mi + 4 * q + r;
      if (m >= a.M) continue;
      float* crow = m < a.M1 ? a.C1 + (size_t)z * a.c_stride + (size_t)m * a.ldc
                             : a.C2 + (size_t)z * a.c_stride + (size_t)(m - a.M1) * a.ldc;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int n = n0 + wn * 64 + 16 * f + lr;
        if (n < a.N) crow[n] = acc[mi][f][r];
      }
    }
  }
}

}  // namespace bwdg
}  // namespace moe
