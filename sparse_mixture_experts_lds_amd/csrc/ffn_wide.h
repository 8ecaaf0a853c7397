// Wide-tile grouped expert GEMM for bf16 weights: tiles of 256 grouped rows by
// 256 weight rows, eight waves, both operands loaded straight into LDS.
//
// Same operation as ffn_kernel.h ("Sharding d'experts", "Deux roles": the
// three matrix products a worker runs per expert; MoEEvolve "Architecture":
// SwiGLU experts; kieve-moe "Features": GeGLU experts):
//   gate/up:  z[r, n] = act(sum_k a[r,k] Wg[e,n,k]) * (sum_k a[r,k] Wu[e,n,k])
//   down:     y[r, n] = sum_k z[r,k] Wd[e,n,k]
//
// Why a second tile shape.  The narrow kernel's time follows the bytes its
// workgroups pull through the CU caches: a 128x128 tile loads 32 KB per 64-deep
// k-block for 2.1 MFLOP.  This tile loads 32 KB per 32-deep k-block for
// 4.2 MFLOP, half the bytes per FLOP, and it is tall enough that an expert with
// up to 256 rows reads each weight slice once.  It pays when experts get at
// least ~100 rows.
//
// Layout.  A tile has BW = 256 (or 128) weight rows.  Waves form a 4 x 2
// grid: wave (wr, wc) owns rows 64*wr..64*wr+63 and BW/2 of the weight rows,
// as 4 x BW/32 MFMA 16x16x32 fragments (up to 128 fp32 accumulators per lane).
// For gate/up the tile's weight rows are BW/2 gate rows then the BW/2 up rows
// of the same outputs, and wave wc takes gate and up rows of the same output
// columns, so g and u of an output meet in one lane; its MFMAs take the
// weight fragment as the A operand, so a lane ends with four consecutive
// outputs of one row and stores their z straight from registers.  For down
// the weight rows are output columns, BW/2 per wave column, and the output
// goes out through LDS as whole row pieces.  The half-width tile exists
// for workloads whose full-width tiles would leave the last round of
// workgroups mostly empty.
//
// Pipeline.  Operands go global -> LDS with loads that write LDS directly
// (global_load_lds_dwordx4, no staging registers), into as many stages as
// LDS holds (A 256 x 64 B plus B BW x 64 B each: 5 stages for BW 256, 6 for
// 128); the MFMA fragments are double-buffered in registers, so a k-block's
// LDS reads overlap the previous k-block's MFMAs.  Every thread issues the
// same loads per stage, so an explicit vmcnt wait plus
// an LDS barrier marks a stage complete.  Inside a 64-byte row the four
// 16-byte chunks are stored XOR-swizzled by (row / 2) % 4, so the eight lanes
// served per LDS cycle (eight consecutive rows, one chunk each) hit eight
// distinct groups of four banks.  Activation rows are gathered on load
// (row_index); rows past the tile end re-read its last row.  A wave whose 64
// rows all lie past the tile end skips its MFMAs.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace ffn_wide {

constexpr int BM = 256;            // grouped rows per tile
constexpr int KB = 32;             // inputs per k-block (one MFMA K step)
constexpr int ROWB = KB * 2;       // bytes per operand row per k-block
constexpr int OPA = BM * ROWB;     // the A operand of one stage (16 KB)
constexpr int kGroupM = 4;         // m-tiles per group in the tile order

// Geometry for BW weight rows per tile (256 or 128).
template <int BW>
struct Geo {
  static constexpr int OPB = BW * ROWB;                   // B operand of one stage
  static constexpr int STAGE = OPA + OPB;                 // A then B
  static constexpr int NS = (160 * 1024) / STAGE;         // LDS stages: 5 (BW 256) or 6 (BW 128)
  static constexpr int LB = BW / 128;                     // B loads per thread per stage
  static constexpr int LPS = 2 + LB;                      // loads per thread per stage
  static constexpr int NF = BW / 32;                      // 16-row B fragments per wave
};

// Workgroup barrier that orders LDS only: the compiler sees the lgkmcnt wait
// (so it knows every LDS read has landed) and outstanding global loads stay in
// flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_barrier();
}

// s_waitcnt vmcnt(n) (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their no-wait maxima)
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 16, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}

template <int ACT>  // 0 SiLU, 1 exact-erf GELU
__device__ __forceinline__ float act_fn(float g) {
  if constexpr (ACT == 0) return silu_hw(g);
  else return gelu_hw(g);
}

// 16 bytes per lane from base + off (base uniform, off a per-lane 32-bit byte
// offset) into LDS at byte address lds_addr + 16 * lane (lds_addr uniform).
// Written as asm so that the compiler, which cannot tell the stages apart,
// adds no waits of its own; the kernel waits explicitly (wait_vm +
// lds_barrier) before it reads a stage.  The asm has no register outputs, and
// the "memory" clobber keeps every LDS access on its side.
__device__ __forceinline__ void dma16(const unsigned char* base, uint32_t off, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  // the base is uniform; readfirstlane keeps it in scalar registers (the
  // builtin returns int: each half goes through uint32_t before widening, or
  // the low half would be sign-extended into the high one)
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t ub = ((uint64_t)hi << 32) | (uint64_t)lo;
  base = reinterpret_cast<const unsigned char*>(ub);
  // one wait state between the SALU write of M0 and the LDS-writing load
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}

// The same from a per-lane 64-bit address.
__device__ __forceinline__ void dma16(const unsigned char* src, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}

// p[i] for a wave-uniform i, read through the scalar cache (s_load, counted by
// lgkmcnt): the tile table and gathered row indices of a workgroup's next tile
// are read while its operand loads are in flight, and those loads' vmcnt waits
// are counted exactly.  The arrays are written by earlier launches only.
__device__ __forceinline__ int sload(const int32_t* p, int i) {
  typedef __attribute__((address_space(4))) const int32_t cint;
  return reinterpret_cast<cint*>(reinterpret_cast<uintptr_t>(p))[i];
}
__device__ __forceinline__ int4 sload4(const int4* p, int i) {
  const int32_t* w = reinterpret_cast<const int32_t*>(p) + 4 * i;
  int4 r;
  r.x = sload(w, 0);
  r.y = sload(w, 1);
  r.z = sload(w, 2);
  r.w = sload(w, 3);
  return r;
}

// One launch covers one or two GEMM problems of the same kind (the routed
// experts' grouped rows and the shared expert's dense rows): each XCD takes a
// contiguous range of problem 0's tiles, then of problem 1's, so both spread
// evenly over the XCDs and problem 0's tiles are dispatched first.
struct WideArgs {
  FfnGemmArgs p[2];
  int np;  // 1 or 2
  GateBwdOut gb[2];  // gate/up launches with the gate backward in their epilogue only
};

// tiles of one problem: m-tiles x weight-row blocks
__device__ __forceinline__ int wide_tiles(const FfnGemmArgs& a, int NBLK) {
  const int mt = a.offsets ? sload(a.mtile_start, a.E_loc) : (a.rows_max + BM - 1) / BM;
  return mt * NBLK;
}

// A tile: problem, expert, first grouped row, rows, first output column.
struct Tile {
  int pi, e, row0, nrows, n0;
};

// A tile's operand addresses: uniform bases, per-lane A row offsets.
struct Ops {
  const unsigned char* abase;
  const unsigned char* bbase;
  uint32_t a_off[2];
};

template <bool GATEUP, int OUT, int ACT, int BW>
__global__ __launch_bounds__(512) void wide_kernel(WideArgs wa) {
  using G = Geo<BW>;
  constexpr int OPB = G::OPB, STAGE = G::STAGE, NS = G::NS, LPS = G::LPS, LB = G::LB;
  constexpr int BNO = GATEUP ? BW / 2 : BW;  // output columns per tile
  constexpr int MF = 4, NF = G::NF;
  constexpr int HW = BW / 2;                 // weight rows per wave column
  __shared__ __attribute__((aligned(16))) unsigned char stg[NS][STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in scalar registers
  const int lrow = lane & 15;
  const int q = lane >> 4;
  const int wr = wave & 3;
  const int wc = wave >> 2;
  static_assert(NS >= 4, "the loop keeps two k-blocks out of the load window");

  // ---------------- slots.  XCD x = blockIdx % 8 owns a contiguous range of
  // each problem's tiles (grouped-M order within a problem): slot s < per0 is
  // problem 0's tile x per0 + s, slot per0 + s problem 1's tile x per1 + s.
  // Workgroup b takes slots b / 8, b / 8 + S, ... (S = workgroups per XCD).
  // Down launches one workgroup per slot.  Gate/up launches one per CU, and
  // each carries its operand pipeline from one tile into the next: the next
  // tile's first k-blocks are loaded during the current tile's last ones, and
  // the epilogue stores from registers, leaving the stages to those loads.
  const int xcd = blockIdx.x & 7;
  const int S = gridDim.x >> 3;
  const int total0 = wide_tiles(wa.p[0], wa.p[0].N / BNO);
  const int total1 = wa.np > 1 ? wide_tiles(wa.p[1], wa.p[1].N / BNO) : 0;
  const int per0 = (total0 + 7) / 8, per1 = (total1 + 7) / 8;
  const int nslots = per0 + per1;
  auto decode = [&](int sl, Tile& t) -> bool {
    const int pi = sl < per0 ? 0 : 1;
    const int R = pi ? xcd * per1 + (sl - per0) : xcd * per0 + sl;
    const int total = pi ? total1 : total0;
    if (R >= total) return false;
    const FfnGemmArgs& a = wa.p[pi];
    const int NBLK = a.N / BNO;
    const int total_mt = total / NBLK;
    const int grp = R / (kGroupM * NBLK);
    const int t0 = grp * kGroupM;
    const int gm = min(kGroupM, total_mt - t0);
    const int rr = R - grp * kGroupM * NBLK;
    const int nb = rr / gm;
    const int mt = t0 + (rr - nb * gm);
    if (a.tile_tab) {
      const int4 ti = sload4(a.tile_tab, mt);
      t.e = ti.x;
      t.row0 = ti.y;
      t.nrows = ti.z;
    } else {
      t.e = 0;
      t.row0 = mt * BM;
      t.nrows = min(BM, a.rows_max - t.row0);
    }
    t.pi = pi;
    t.n0 = nb * BNO;
    return true;
  };
  // the first slot from sl on (in steps of S) that holds a tile, else nslots
  auto next_slot = [&](int sl, Tile& t) -> int {
    while (sl < nslots && !decode(sl, t)) sl += S;
    return sl;
  };

  // ---------------- load addresses.  Load i (0, 1) of wave w fills 1 KB = 16
  // rows of an operand: rows 16 (2w + i) + lane / 4, stored chunk lane % 4,
  // holding logical chunk (lane % 4) ^ ((row / 2) % 4) of the row.  Rows
  // past the tile end re-read the tile's last row (their results are never
  // stored; a row of the product depends only on the same row of A).  The
  // A offsets are 32-bit (the launcher checks the matrix size); a B load is
  // the tile's weight base plus a fixed per-lane offset.
  Tile tc, tn;
  int sl = next_slot(blockIdx.x >> 3, tc);
  if (sl >= nslots) return;
  // K of this workgroup's tiles (a gate/up workgroup with several tiles only
  // runs where both problems have the same K; the launcher checks)
  const int K = wa.p[tc.pi].K;
  const int NKB = K / KB;
  // per-lane offset of B load i in the tile's weight rows (recomputed at each
  // issue rather than held: registers are the scarce resource here)
  auto b_off = [&](int i) -> uint32_t {
    const int row = 16 * (LB * wave + i) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 1) & 3);
    // gate/up: tile rows 0..BW/2-1 are gate rows, BW/2..BW-1 the up rows of the same outputs
    return (uint32_t)(((GATEUP ? row % (BW / 2) : row) * K + chunk * 8) * 2);
  };
  const bool up_rows = GATEUP && 16 * LB * wave >= BW / 2;  // this wave's B rows (wave-uniform)
  auto make_ops = [&](const Tile& t, Ops& o) {
    const FfnGemmArgs& a = wa.p[t.pi];
    o.abase = static_cast<const unsigned char*>(a.A);
    o.bbase = static_cast<const unsigned char*>(up_rows ? a.W1 : a.W0) + ((size_t)t.e * a.N + t.n0) * (size_t)K * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 16 * (2 * wave + i) + (lane >> 2);
      const int chunk = (lane & 3) ^ ((row >> 1) & 3);
      int src;
      if (a.row_index) {
        // the 16 rows of this load, read wave-uniformly; lane keeps row lane / 4
        int v = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = sload(a.row_index, t.row0 + min(16 * (2 * wave + i) + j, t.nrows - 1));
          v = (lane >> 2) == j ? r : v;
        }
        src = v / a.row_div;
      } else {
        src = t.row0 + min(row, t.nrows - 1);
      }
      o.a_off[i] = (uint32_t)src * (uint32_t)(K * 2) + (uint32_t)(chunk * 16);
    }
  };

  Ops cur, nxt;
  make_ops(tc, cur);
  int sln = GATEUP ? next_slot(sl + S, tn) : nslots;
  bool has_next = sln < nslots;
  nxt = cur;
  if (has_next) make_ops(tn, nxt);

  // k-block qb of the running sequence into stage st: block qb of the current
  // tile, block qb - NKB of the next one, and past both every lane reads the
  // same 16 bytes (one cached line) into the stage, which is never read again,
  // so that every step issues the same loads and the wait counts never change
  const unsigned char* const dummy = static_cast<const unsigned char*>(wa.p[0].A);
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)&stg[0][0]);
  // load l of a stage: A rows (l = 0, 1), then B rows (l = 2 .. 1 + LB)
  auto issue_one = [&](int l, int st, int qb) {
    const uint32_t dst = l < 2 ? lds_base + (uint32_t)(st * STAGE + (2 * wave + l) * 1024)
                               : lds_base + (uint32_t)(st * STAGE + OPA + (LB * wave + l - 2) * 1024);
    const bool in_cur = qb < NKB;
    const bool in_next = !in_cur && has_next && qb < 2 * NKB;
    // field by field (uniform selects), no branches
    const unsigned char* const base_c = l < 2 ? cur.abase : cur.bbase;
    const unsigned char* const base_n = l < 2 ? nxt.abase : nxt.bbase;
    const uint32_t off_c = l < 2 ? cur.a_off[l & 1] : b_off(l - 2);
    const uint32_t off_n = l < 2 ? nxt.a_off[l & 1] : b_off(l - 2);
    const unsigned char* const base = in_cur ? base_c : (in_next ? base_n : dummy);
    const uint32_t off = in_cur ? off_c + (uint32_t)(qb * KB * 2)
                                : (in_next ? off_n + (uint32_t)((qb - NKB) * KB * 2) : 0u);
    dma16(base, off, dst);
  };
  auto issue = [&](int st, int qb) {
#pragma unroll
    for (int l = 0; l < LPS; ++l) issue_one(l, st, qb);
  };

  // fragment reads: lane (lrow, q) needs logical chunk q of its row; rows of a
  // fragment start at multiples of 16, so the stored chunk is q ^ ((lrow / 2) % 4)
  const int rd = lrow * ROWB + ((q ^ ((lrow >> 1) & 3)) * 16);
  const int a_rd = 64 * wr * ROWB + rd;
  // wave column wc: gate/up -> gate rows [BW/4 wc, BW/4 (wc+1)) and the same up
  // rows at +BW/2; down -> rows [BW/2 wc, BW/2 (wc+1))
  const int b_rd = (GATEUP ? HW / 2 : HW) * wc * ROWB + rd;

  f32x4 acc[MF][NF];
  // MFMA fragments of one k-block, double-buffered in registers (two named
  // sets): the fragments of k-block j+1 are read from LDS while k-block j's
  // MFMAs run
  bf16x8 fa0[MF], fb0[NF], fa1[MF], fb1[NF];
  auto read_frags = [&](bf16x8 (&fa)[MF], bf16x8 (&fb)[NF], int st) {
    const unsigned char* A = &stg[0][0] + st * STAGE;
    const unsigned char* B = A + OPA;
#pragma unroll
    for (int mi = 0; mi < MF; ++mi)
      fa[mi] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(A + a_rd + 16 * mi * ROWB));
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      // B row offset of fragment f: gate/up -> gate fragments then the up ones
      const int fo = GATEUP ? (f >= NF / 2 ? BW / 2 : 0) + 16 * (f % (NF / 2)) : 16 * f;
      fb[f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(B + b_rd + fo * ROWB));
    }
  };
  // The MFMAs of one k-block in four groups, with one of the stage's four loads
  // issued after each group: a load issue that waits for the address unit
  // (64 B/clk per CU) then overlaps the MFMAs already in the matrix pipe
  // instead of holding up the whole k-block.
  bool active = false;  // this wave has rows in the current tile (wave-uniform)
  auto mfmas_issue = [&](const bf16x8 (&fa)[MF], const bf16x8 (&fb)[NF], int st, int qb) {
    if (!active) {
      issue(st, qb);
      return;
    }
#pragma unroll
    for (int g = 0; g < LPS; ++g) {
#pragma unroll
      for (int f = g * NF / LPS; f < (g + 1) * NF / LPS; ++f)
#pragma unroll
        for (int mi = 0; mi < MF; ++mi)
          // gate/up: the weight fragment is the A operand (rows of D are
          // outputs); down: the activation fragment is (rows of D are tokens)
          acc[mi][f] = GATEUP ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[f], fa[mi], acc[mi][f], 0, 0, 0)
                              : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mi], fb[f], acc[mi][f], 0, 0, 0);
      issue_one(g, st, qb);
    }
  };

  // ---------------- k-loop.  k-block q of the running sequence sits in stage
  // q % NS.  At the top of k-block j the fragments of j are in registers and
  // the k-blocks j+1..j+NS-2 are in flight; waiting until at most NS-3
  // stages' loads remain, then a barrier, makes stage j+1 complete for every
  // wave and frees stage j-1 (last read one iteration ago), which then
  // receives k-block j+NS-1.  The fragments of j+1 are read while j's MFMAs
  // run (past the tile's last k-block they read a stage that is not complete
  // and are never used).  K / KB is even.  A tile starts with k-blocks
  // 0..NS-2 in flight (issued here for the first tile, during the previous
  // tile's last k-blocks for the others); the global stores of an epilogue
  // are counted by vmcnt as well, which only makes the next waits stricter.
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) issue(st, st);
  int cst = 0;  // stage of the tile's k-block j
  for (;;) {
    const FfnGemmArgs& args = wa.p[tc.pi];
    const int N = args.N, nrows = tc.nrows;
    active = 64 * wr < nrows;
#pragma unroll
    for (int mi = 0; mi < MF; ++mi)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    wait_vm<(NS - 2) * LPS>();
    lds_barrier();
    read_frags(fa0, fb0, cst);
    for (int j = 0; j < NKB; j += 2) {
      wait_vm<(NS - 3) * LPS>();
      lds_barrier();
      const int st0 = cst == 0 ? NS - 1 : cst - 1;  // free stage (k-block j-1)
      cst = cst + 1 == NS ? 0 : cst + 1;             // stage of k-block j+1
      read_frags(fa1, fb1, cst);
      mfmas_issue(fa0, fb0, st0, j + NS - 1);

      wait_vm<(NS - 3) * LPS>();
      lds_barrier();
      const int st1 = cst == 0 ? NS - 1 : cst - 1;
      cst = cst + 1 == NS ? 0 : cst + 1;  // stage of k-block j+2
      read_frags(fa0, fb0, cst);
      mfmas_issue(fa1, fb1, st1, j + NS);
    }
    // cst is now the stage of the next tile's k-block 0

    unsigned char* obase = static_cast<unsigned char*>(args.out) + ((size_t)tc.row0 * N + tc.n0) * (OUT == 1 ? 4 : 2);
    if constexpr (GATEUP) {
      // ---------------- gate/up epilogue.  Lane (lrow, q) holds, for tile row
      // 64 wr + 16 mi + lrow, g (fragment f) and u (fragment f + NF / 2) of the
      // four consecutive outputs 16 f + 4 q .. 16 f + 4 q + 3: z = act(g) u
      // goes out straight from registers, 8 bytes per lane and 4 lanes side by
      // side per row.  Rows past the tile end are not stored.
      if (active) {
#pragma unroll
        for (int mi = 0; mi < MF; ++mi) {
          const int row = 64 * wr + 16 * mi + lrow;
          if (row < nrows) {
            uint16_t* orow = reinterpret_cast<uint16_t*>(obase) + (size_t)row * N + HW / 2 * wc + 4 * q;
#pragma unroll
            for (int f = 0; f < NF / 2; ++f) {
              float z[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) z[r] = act_fn<ACT>(acc[mi][f][r]) * acc[mi][f + NF / 2][r];
              *reinterpret_cast<uint2*>(orow + 16 * f) = uint2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
            }
          }
        }
      }
      if (!has_next) break;
      // the next tile becomes the current one; the one after is decoded
      // through the scalar cache while the next tile's loads are in flight
      tc = tn;
      cur = nxt;
      sln = next_slot(sln + S, tn);
      has_next = sln < nslots;
      if (has_next) make_ops(tn, nxt);
    } else {
      // ---------------- down epilogue (lane (lrow, q) holds output column
      // 16 f + lrow of tile rows 64 wr + 16 mi + 4 q + r).  Straight 64-byte
      // row pieces from registers ran slower here than full rows staged in LDS.
      // One tile per workgroup: the dummy loads land before the stages become
      // the staging buffer.
      wait_vm<0>();
      lds_barrier();
      unsigned char* const lds = &stg[0][0];
      // every wave stages its own 64 x HW block of the output through a private
      // LDS region, in two halves of HW/2 columns, and stores 16-byte row
      // chunks; a wave's LDS accesses complete in order, so no workgroup barrier
      // is needed between the writes and the reads
      constexpr int osz = OUT == 1 ? 4 : 2;
      constexpr int QC = HW / 2;          // output columns per half
      constexpr int OS = QC * osz + 16;   // LDS row stride of a wave's block (bytes)
      constexpr int cpr = QC * osz / 16;  // 16-byte chunks per row
      static_assert(8 * 64 * OS <= NS * STAGE, "the waves' blocks fit the stage memory");
      unsigned char* const wl = lds + wave * 64 * OS;
      const int rows_w = min(64, nrows - 64 * wr);
      if (active) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int mi = 0; mi < MF; ++mi)
#pragma unroll
            for (int ff = 0; ff < NF / 2; ++ff)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float v = acc[mi][(NF / 2) * hh + ff][r];
                unsigned char* dst = wl + (16 * mi + 4 * q + r) * OS + (16 * ff + lrow) * osz;
                if constexpr (OUT == 1) *reinterpret_cast<float*>(dst) = v;
                else if constexpr (OUT == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)f32_to_f16_bits(v);
                else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)f32_to_bf16_bits(v);
              }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          unsigned char* const ob = obase + ((size_t)(64 * wr) * N + HW * wc + QC * hh) * osz;
          for (int c = lane; c < rows_w * cpr; c += 64) {
            const int row = c / cpr;
            const int cc = c - row * cpr;
            *reinterpret_cast<u32x4*>(ob + (size_t)row * N * osz + cc * 16) =
                *reinterpret_cast<const u32x4*>(wl + row * OS + cc * 16);
          }
          // the reads land before the next half overwrites the block
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
      }
      break;
    }
  }
  wait_vm<0>();  // every load has landed in LDS before the workgroup ends
}

// compute units per XCD of the current device (8 XCDs), at least 1
inline int cus_per_xcd() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8)
      n = 256;
    cached = n / 8;
  }
  return cached;
}

template <bool GATEUP, int BW>
hipError_t launch_bw(const FfnGemmArgs* a, int np, void* ev_start, void* ev_stop, hipStream_t s) {
  constexpr int BNO = GATEUP ? BW / 2 : BW;
  WideArgs w{};
  w.np = np;
  long long slots = 0;
  for (int i = 0; i < np; ++i) {
    const FfnGemmArgs& p = a[i];
    if (p.N % BNO || p.K % (2 * KB) || (size_t)p.N * p.K * 2 > 0x7FFFFFFFull) return hipErrorInvalidValue;
    if (i > 0 && (p.out_f32 != a[0].out_f32 || p.out_f16 != a[0].out_f16 || p.act != a[0].act))
      return hipErrorInvalidValue;
    const int mt = p.offsets ? ffn_max_mtiles(p.E_loc, p.rows_max, BM) : (p.rows_max + BM - 1) / BM;
    slots += ((long long)mt * (p.N / BNO) + 7) / 8;  // per-XCD slots of problem i
    w.p[i] = p;
  }
  long long g = 8 * slots;
  if (g == 0) return hipSuccess;
  if (g > 0x7FFFFFFFll) return hipErrorInvalidValue;
  // gate/up: one workgroup per CU, each running several tiles back to back,
  // where the pipeline can run from tile to tile (the same K in every problem
  // and at least NS - 1 k-blocks per tile); otherwise one workgroup per tile
  if (GATEUP) {
    bool same_k = true;
    for (int i = 1; i < np; ++i) same_k = same_k && a[i].K == a[0].K;
    if (same_k && a[0].K / KB >= Geo<BW>::NS - 1 && g > 8LL * cus_per_xcd()) g = 8LL * cus_per_xcd();
  }
  auto go = [&](auto kernel) {
    if (ev_start || ev_stop)
      hipExtLaunchKernelGGL(kernel, dim3((unsigned)g), dim3(512), 0, s, static_cast<hipEvent_t>(ev_start),
                            static_cast<hipEvent_t>(ev_stop), 0, w);
    else
      kernel<<<dim3((unsigned)g), dim3(512), 0, s>>>(w);
  };
  if (!GATEUP && a[0].out_f32) go(wide_kernel<false, 1, 0, BW>);
  else if (!GATEUP && a[0].out_f16) go(wide_kernel<false, 2, 0, BW>);
  else if (GATEUP && a[0].act == 1) go(wide_kernel<GATEUP, 0, 1, BW>);
  else go(wide_kernel<GATEUP, 0, 0, BW>);
  return hipGetLastError();
}

// bw: weight rows per tile (256 or 128); np problems of the same kind in one
// launch (their tiles in the order given); the events, if any, are attached to
// the launch
template <bool GATEUP>
hipError_t launch_wide(const FfnGemmArgs* a, int np, int bw, void* ev_start, void* ev_stop, hipStream_t s) {
  if (np < 1 || np > 2) return hipErrorInvalidValue;
  // gate/up writes z in bf16 (the fp32 z of the INT4 path never comes here)
  if (GATEUP && a[0].out_f32) return hipErrorInvalidValue;
  if (bw == 256) return launch_bw<GATEUP, 256>(a, np, ev_start, ev_stop, s);
  if (bw == 128) return launch_bw<GATEUP, 128>(a, np, ev_start, ev_stop, s);
  return hipErrorInvalidValue;
}

}  // namespace ffn_wide
}  // namespace moe
