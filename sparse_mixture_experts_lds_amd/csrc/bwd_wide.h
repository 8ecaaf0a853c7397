// Wide-tile grouped GEMMs of the layer backward (bf16 operands, fp32 out):
// 256 x 256 output tiles, eight waves, operands loaded straight into LDS.
//
//   wide_nn_kernel (data gradients)   C[r, n] = sum_k A[row(r), k] * B_g[k, n]
//   wide_tn_kernel (weight gradients) C_g[m, n] = sum_{r in group g} A[row_a(r), m] * B[row_b(r), n]
//
// Same operations and argument blocks as bwd_gemm.h (bwdg::NnArgs, TnArgs);
// the pipeline is the forward's wide kernel (ffn_wide.h): a ring of five
// 32-deep k-block stages of 32 KB filled by direct-to-LDS loads, exact vmcnt
// waits, one LDS barrier per k-block, MFMA fragments double-buffered in
// registers, eight waves in a 4 x 2 grid of 64 x 128 accumulator blocks.
//
// Operand stages.  An operand whose contraction dimension is contiguous (A of
// nn) is staged like the forward's: 256 rows x 64 B, 16-byte chunks
// XOR-swizzled by (row / 2) % 4.  An operand whose output dimension is
// contiguous (B of nn, both of tn) is staged as it lies, 32 k-rows x 512 B
// (256 bf16 outputs): one load instruction fills two k-rows (lanes 0-31 and
// 32-63), chunk c of k-row kr holding the operand's chunk c ^ 2 (kr % 4), so
// the four k-rows a transposing read touches (ds_read_b64_tr_b16, as in
// bwd_gemm.h) sit in distinct banks.
//
// Contraction rows of tn.  The rows of a k-block are a run of a group's rows;
// the two rows an instruction fills are the same for a half-wave, so their
// gathered indices are wave-uniform scalar loads, issued one stage ahead
// (the barrier's lgkmcnt(0) has them in registers by their use).  Rows past
// the group's end contribute zero: A reads a row of zeros, B a valid row.  A
// group with an odd number of k-blocks gets one more, all zero.
#pragma once

#include "bwd.h"
#include "ffn_wide.h"

namespace moe {
namespace bwdw {

using ffn_wide::dma16;
using ffn_wide::lds_barrier;
using ffn_wide::wait_vm;

constexpr int BT = 256;              // tile rows and columns
constexpr int KB = 32;               // contraction per k-block
constexpr int OP = 16384;            // one operand of a stage
constexpr int STAGE = 2 * OP;
constexpr int NS = (160 * 1024) / STAGE;  // 5
constexpr int LPS = 4;               // loads per thread per stage (two per operand)
constexpr int MF = 4, NF = 8;        // 16 x 16 fragments per wave (64 rows x 128 columns)
constexpr int kGroupM = 4;

// 512 zero bytes: the A row of contraction rows past a group's end (tn)
__device__ __attribute__((aligned(16))) const uint16_t g_zero_row[BT] = {};

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// p[i] for a wave-uniform i, read through the scalar cache (s_load): the
// gathered row indices of tn must not enter the vector memory counter, whose
// waits the pipeline counts exactly.  The index arrays are written by earlier
// launches only.
__device__ __forceinline__ int uload(const int32_t* p, int i) {
  typedef __attribute__((address_space(4))) const int32_t cint;
  return reinterpret_cast<cint*>(reinterpret_cast<uintptr_t>(p))[i];
}

// 16-byte chunk swizzle of a k-row of a [k][256] stage
__device__ __forceinline__ int kswz(int kr) { return 2 * (kr & 3); }

// One MFMA fragment (8 consecutive k for column x0 + lane % 16, k rows 8 q ..
// 8 q + 7 of the stage for lane group q) from a [k][256] stage.
__device__ __forceinline__ bf16x8 frag_k(const unsigned char* stage, int x0, int lane) {
  const int q = lane >> 4, a = lane & 15;
  const int kr = 8 * q + (a >> 2);
  const int chunk = (x0 >> 3) + ((a & 3) >> 1);
  const int off = kr * 512 + ((chunk ^ kswz(kr)) << 4) + 8 * (a & 1);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(stage + off));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(stage + off + 4 * 512));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One fragment of a [256 rows][64 B] stage (forward layout): lane (lrow, q)
// takes logical chunk q of row r0 + lrow.
__device__ __forceinline__ bf16x8 frag_r(const unsigned char* stage, int r0, int lane) {
  const int lrow = lane & 15, q = lane >> 4;
  const int row = r0 + lrow;
  return __builtin_bit_cast(bf16x8,
                            *reinterpret_cast<const u32x4*>(stage + row * 64 + ((q ^ ((row >> 1) & 3)) << 4)));
}

// Tile R of `total` in XCD-contiguous ranges (blockIdx -> XCD round robin);
// -1 when this workgroup has none.
__device__ __forceinline__ int xcd_tile(int total) {
  const int per = (total + 7) / 8;
  const int slot = blockIdx.x >> 3;
  if (slot >= per) return -1;
  const int R = (blockIdx.x & 7) * per + slot;
  return R < total ? R : -1;
}

// The k-loop shared by both kernels.  issue(st, kb, real) fills stage st with
// k-block kb (real false: a dummy load of a fixed valid address, never read);
// frags(st, fa, fb) reads a stage's fragments.  nkb is even and positive.
template <typename Issue, typename Frags>
__device__ __forceinline__ void kloop(int nkb, bool active, f32x4 (&acc)[MF][NF], Issue&& issue, Frags&& frags) {
  bf16x8 fa0[MF], fb0[NF], fa1[MF], fb1[NF];
  auto mfmas = [&](const bf16x8(&fa)[MF], const bf16x8(&fb)[NF]) {
    if (!active) return;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int mi = 0; mi < MF; ++mi)
        acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mi], fb[f], acc[mi][f], 0, 0, 0);
  };
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) issue(st, st, st < nkb);
  wait_vm<(NS - 2) * LPS>();
  lds_barrier();
  frags(0, fa0, fb0);
  int cst = 0;
  for (int j = 0; j < nkb; j += 2) {
    wait_vm<(NS - 3) * LPS>();
    lds_barrier();
    const int st0 = cst == 0 ? NS - 1 : cst - 1;
    cst = cst + 1 == NS ? 0 : cst + 1;
    frags(cst, fa1, fb1);
    issue(st0, j + NS - 1, j + NS - 1 < nkb);
    mfmas(fa0, fb0);

    wait_vm<(NS - 3) * LPS>();
    lds_barrier();
    const int st1 = cst == 0 ? NS - 1 : cst - 1;
    cst = cst + 1 == NS ? 0 : cst + 1;
    frags(cst, fa0, fb0);
    issue(st1, j + NS, j + NS < nkb);
    mfmas(fa1, fb1);
  }
  wait_vm<0>();
  lds_barrier();
}

// Every wave stages its 64 x 128 fp32 block through a private LDS region in
// two halves of 64 columns and stores 16-byte row chunks; row_ptr(r) gives
// the destination of tile row r (0..255) at the tile's first column, or
// nullptr to skip the row.
template <typename RowPtr>
__device__ __forceinline__ void store_tile(unsigned char* lds, const f32x4 (&acc)[MF][NF], bool active,
                                           RowPtr&& row_ptr) {
  constexpr int QC = 64;             // columns per half
  constexpr int OS = QC * 4 + 16;    // LDS row stride (bytes)
  constexpr int cpr = QC * 4 / 16;   // 16-byte chunks per row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave & 3, wc = wave >> 2, lrow = lane & 15, q = lane >> 4;
  unsigned char* const wl = lds + wave * 64 * OS;
  if (!active) return;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int mi = 0; mi < MF; ++mi)
#pragma unroll
      for (int ff = 0; ff < NF / 2; ++ff)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<float*>(wl + (16 * mi + 4 * q + r) * OS + (16 * ff + lrow) * 4) =
              acc[mi][(NF / 2) * hh + ff][r];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    for (int c = lane; c < 64 * cpr; c += 64) {
      const int row = c / cpr, cc = c - (c / cpr) * cpr;
      float* dst = row_ptr(64 * wr + row);
      if (dst)
        *reinterpret_cast<u32x4*>(dst + 128 * wc + QC * hh + 4 * cc) =
            *reinterpret_cast<const u32x4*>(wl + row * OS + cc * 16);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// ------------------------------------------------------------------ nn
__global__ __launch_bounds__(512) void wide_nn_kernel(bwdg::NnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char stg[NS][STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave & 3, wc = wave >> 2;
  const int NBLK = a.N / BT;
  const int total_mt = a.tile_tab ? a.mtile_start[a.groups] : (a.rows + BT - 1) / BT;
  const int R = xcd_tile(total_mt * NBLK);
  if (R < 0) return;
  int g = 0, row0, nrows, nb;
  {
    const int grp = R / (kGroupM * NBLK);
    const int t0 = grp * kGroupM;
    const int gm = min(kGroupM, total_mt - t0);
    const int rr = R - grp * kGroupM * NBLK;
    nb = rr / gm;
    const int t = t0 + (rr - nb * gm);
    if (a.tile_tab) {
      const int4 ti = a.tile_tab[t];
      g = ti.x;
      row0 = ti.y;
      nrows = ti.z;
    } else {
      row0 = t * BT;
      nrows = min(BT, a.rows - row0);
    }
  }
  g = __builtin_amdgcn_readfirstlane(g);
  nrows = __builtin_amdgcn_readfirstlane(nrows);
  const int n0 = nb * BT;

  // A: rows gathered once per tile; rows past the tile end re-read its last row
  const unsigned char* a_ptr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * (2 * wave + i) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 1) & 3);
    const int gr = row0 + min(row, nrows - 1);
    const int src = a.a_index ? a.a_index[gr] / a.a_div : gr;
    a_ptr[i] = static_cast<const unsigned char*>(a.A) + ((size_t)src * a.lda + chunk * 8) * 2;
  }
  // B: k-row kr = 2 (2 wave + i) + lane / 32 of the stage, chunk lane % 32
  const uint16_t* B1 = static_cast<const uint16_t*>(a.B1) + (size_t)g * a.b_stride;
  const uint16_t* B2 = a.B2 ? static_cast<const uint16_t*>(a.B2) + (size_t)g * a.b_stride : B1;
  const int c = lane & 31;
  const unsigned char* const dummy = static_cast<const unsigned char*>(a.A);
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)&stg[0][0]);
  auto issue = [&](int st, int kb, bool real) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16(real ? a_ptr[i] + kb * KB * 2 : dummy, lds_base + (uint32_t)(st * STAGE + (2 * wave + i) * 1024));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kr = 2 * (2 * wave + i) + (lane >> 5);
      const int k = min(kb * KB + kr, a.K_valid - 1);
      const uint16_t* brow = k < a.K1 ? B1 + (size_t)k * a.ldb : B2 + (size_t)(k - a.K1) * a.ldb;
      const unsigned char* src = reinterpret_cast<const unsigned char*>(brow + n0 + 8 * (c ^ kswz(kr)));
      dma16(real ? src : dummy, lds_base + (uint32_t)(st * STAGE + OP + (2 * wave + i) * 1024));
    }
  };
  const int a_rd = 64 * wr;
  auto frags = [&](int st, bf16x8(&fa)[MF], bf16x8(&fb)[NF]) {
    const unsigned char* A = &stg[0][0] + st * STAGE;
    const unsigned char* B = A + OP;
#pragma unroll
    for (int mi = 0; mi < MF; ++mi) fa[mi] = frag_r(A, a_rd + 16 * mi, lane);
#pragma unroll
    for (int f = 0; f < NF; ++f) fb[f] = frag_k(B, 128 * wc + 16 * f, lane);
  };
  const bool active = 64 * wr < nrows;
  f32x4 acc[MF][NF];
#pragma unroll
  for (int mi = 0; mi < MF; ++mi)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop(a.K / KB, active, acc, issue, frags);
  store_tile(&stg[0][0], acc, active, [&](int r) -> float* {
    return r < nrows ? a.C + (size_t)(row0 + r) * a.ldc + n0 : nullptr;
  });
}

// ------------------------------------------------------------------ tn
__global__ __launch_bounds__(512) void wide_tn_kernel(bwdg::TnArgs a, int groups) {
  __shared__ __attribute__((aligned(16))) unsigned char stg[NS][STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave & 3, wc = wave >> 2;
  const int MT = a.M / BT, NT = a.N / BT;
  // tiles in dispatch order (round robin over the XCDs, then as CUs free up):
  // a tile's work follows its group's row count, which routing can skew, so
  // contiguous per-XCD ranges would load some XCDs with the largest groups
  const int R = blockIdx.x;
  if (R >= groups * MT * NT) return;
  const int z = R / (MT * NT);
  const int rem = R - z * (MT * NT);
  const int mt = rem / NT, nt = rem - (rem / NT) * NT;
  const int m0 = mt * BT, n0 = nt * BT;
  int r0, r1, g = z, slot = -1;
  if (a.chunks) {
    const int4 ck = a.chunks[z];
    g = __builtin_amdgcn_readfirstlane(ck.x);
    if (g < 0) return;  // past the virtual groups
    r0 = ck.y;
    r1 = ck.z;
    slot = __builtin_amdgcn_readfirstlane(ck.w);
  } else if (a.offsets) {
    r0 = a.offsets[z];
    r1 = a.offsets[z + 1];
  } else {
    r0 = z * a.slice;
    r1 = min(a.rows, r0 + a.slice);
  }
  r0 = __builtin_amdgcn_readfirstlane(r0);
  r1 = __builtin_amdgcn_readfirstlane(r1);
  const int nkb = r1 > r0 ? ((r1 - r0 + 2 * KB - 1) / (2 * KB)) * 2 : 0;

  const int c = lane & 31;
  const int hi = lane >> 5;
  const unsigned char* Ab = static_cast<const unsigned char*>(a.A);
  const unsigned char* Bb = static_cast<const unsigned char*>(a.B);
  const unsigned char* const zero = reinterpret_cast<const unsigned char*>(g_zero_row);
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)&stg[0][0]);
  // source rows of the two k-rows instruction i fills (wave-uniform pairs)
  struct Rows {
    int a[2][2], b[2][2];  // [instruction][half] source row, a: -1 = zero row
  };
  auto rows_of = [&](int kb) {
    Rows s;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = r0 + kb * KB + 2 * (2 * wave + i) + h;
        const int rb = min(r, r1 - 1);
        s.a[i][h] = r < r1 ? (a.a_index ? uload(a.a_index, r) / a.a_div : r) : -1;
        s.b[i][h] = a.b_index ? uload(a.b_index, rb) / a.b_div : rb;
      }
    return s;
  };
  const unsigned char* const dummy = Bb;
  auto issue_rows = [&](int st, const Rows& s, bool real) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kr = 2 * (2 * wave + i) + hi;
      const int ra = hi ? s.a[i][1] : s.a[i][0];
      const int col = 8 * (c ^ kswz(kr));
      const unsigned char* src = ra >= 0 ? Ab + ((size_t)ra * a.lda + m0 + col) * 2 : zero + col * 2;
      dma16(real ? src : dummy, lds_base + (uint32_t)(st * STAGE + (2 * wave + i) * 1024));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kr = 2 * (2 * wave + i) + hi;
      const int rb = hi ? s.b[i][1] : s.b[i][0];
      const unsigned char* src = Bb + ((size_t)rb * a.ldb + n0 + 8 * (c ^ kswz(kr))) * 2;
      dma16(real ? src : dummy, lds_base + (uint32_t)(st * STAGE + OP + (2 * wave + i) * 1024));
    }
  };
  auto frags = [&](int st, bf16x8(&fa)[MF], bf16x8(&fb)[NF]) {
    const unsigned char* A = &stg[0][0] + st * STAGE;
    const unsigned char* B = A + OP;
#pragma unroll
    for (int mi = 0; mi < MF; ++mi) fa[mi] = frag_k(A, 64 * wr + 16 * mi, lane);
#pragma unroll
    for (int f = 0; f < NF; ++f) fb[f] = frag_k(B, 128 * wc + 16 * f, lane);
  };
  f32x4 acc[MF][NF];
#pragma unroll
  for (int mi = 0; mi < MF; ++mi)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nkb > 0) {
    // the rows of the next stage to fill are looked up one stage ahead: real
    // fills come with k-blocks 0, 1, 2, ... and dummy ones only after them
    Rows next = rows_of(0);
    auto issue = [&](int st, int kb, bool real) {
      issue_rows(st, next, real);
      if (real) next = rows_of(kb + 1);
    };
    kloop(nkb, true, acc, issue, frags);
  }
  // an empty group still writes its (zero) gradient
  store_tile(&stg[0][0], acc, true, [&](int r) -> float* {
    const int m = m0 + r;
    if (slot >= 0) return a.part + (size_t)slot * a.M * a.N + (size_t)m * a.N + n0;
    return m < a.M1 ? a.C1 + (size_t)g * a.c_stride + (size_t)m * a.ldc + n0
                    : a.C2 + (size_t)g * a.c_stride + (size_t)(m - a.M1) * a.ldc + n0;
  });
}

}  // namespace bwdw
}  // namespace moe
