// Wide-tile grouped expert GEMM with 64-deep k-blocks: tiles of 256 grouped
// rows by 256 weight rows, eight waves, both operands loaded straight into
// LDS as 128-byte row pieces, two LDS stages.
//
// Same operation and tile layout as ffn_wide.h ("Sharding d'experts", "Deux
// roles": the three matrix products a worker runs per expert; MoEEvolve
// "Architecture": SwiGLU experts; kieve-moe "Features": GeGLU experts):
//   gate/up:  z[r, n] = act(sum_k a[r,k] Wg[e,n,k]) * (sum_k a[r,k] Wu[e,n,k])
//   down:     y[r, n] = sum_k z[r,k] Wd[e,n,k]
//
// Why 64-deep k-blocks.  The loads that write LDS directly move a wave's
// 1 KB per instruction as row pieces; measured on MI355X with operands that
// live beyond the L2, 128-byte pieces stream about 1.5x faster than 64-byte
// ones (26 against 17 TB/s over the chip), because each L1 -> L2 request then
// carries a whole 128-byte line and the number of requests a CU keeps in
// flight is what bounds its rate.  A 64-deep stage of both operands is 64 KB,
// so LDS holds two.
//
// Pipeline (two stages, k-block j in stage j % 2, K / 64 even).  In k-block j
// the MFMAs of its first 32-deep step run while the fragments of its second
// step are read from LDS; then every wave waits for its loads of k-block j+1
// and meets the others at one barrier, after which stage j % 2 is free: the
// loads of k-block j+2 are issued into it, and the MFMAs of the second step
// run while the fragments of k-block j+1's first step are read.  So global ->
// LDS loads run one k-block ahead and LDS -> register reads half a step ahead,
// with one barrier per k-block.  Past a tile's last k-blocks the loads fetch
// the first k-blocks of the workgroup's next tile (gate/up runs one workgroup
// per CU over several tiles), and past both every lane re-reads one valid
// 16-byte piece, so every iteration issues the same loads and the vmcnt waits
// stay exact.
//
// LDS layout.  A stage is A (256 rows x 128 B) then B (256 rows x 128 B).
// Inside a row the eight 16-byte chunks are stored XOR-swizzled by
// (row / 2) % 8, so the sixteen lanes an LDS read serves at once (sixteen
// consecutive rows, one chunk each) hit sixteen distinct groups of banks.
#pragma once

#include <type_traits>

#include "ffn_wide.h"

namespace moe {
namespace ffn_wide64 {

using ffn_wide::act_fn;
using ffn_wide::dma16;
using ffn_wide::lds_barrier;
using ffn_wide::sload;
using ffn_wide::sload4;
using ffn_wide::Tile;
using ffn_wide::wait_vm;
using ffn_wide::WideArgs;

constexpr int BM = 256;            // grouped rows per tile
constexpr int BW = 256;            // weight rows per tile
constexpr int KB = 64;             // inputs per k-block (two MFMA K steps)
constexpr int ROWB = KB * 2;       // bytes per operand row per k-block
constexpr int OPA = BM * ROWB;     // the A operand of one stage (32 KB)
constexpr int OPB = BW * ROWB;     // the B operand of one stage (32 KB)
constexpr int STAGE = OPA + OPB;
constexpr int NS = 2;
constexpr int LA = OPA / (8 * 1024);   // A loads per wave per stage (4)
constexpr int LB = OPB / (8 * 1024);   // B loads per wave per stage (4)
constexpr int LPS = LA + LB;
constexpr int kGroupM = 4;             // m-tiles per group in the tile order

struct Ops {
  const unsigned char* abase;
  const unsigned char* bbase;
  uint32_t a_off[LA];
};

// GBWD (gate/up only): the epilogue does the gate backward (GateBwdOut)
// instead of storing z.
template <bool GATEUP, int OUT, int ACT, bool GBWD = false>
__global__ __launch_bounds__(512) void wide64_kernel(WideArgs wa) {
  constexpr int BNO = GATEUP ? BW / 2 : BW;  // output columns per tile
  constexpr int MF = 4, NF = BW / 32;
  constexpr int HW = BW / 2;                 // weight rows per wave column
  __shared__ __attribute__((aligned(16))) unsigned char stg[NS][STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15;
  const int q = lane >> 4;
  const int wr = wave & 3;
  const int wc = wave >> 2;

  // ---------------- slots (as ffn_wide.h): XCD x = blockIdx % 8 owns a
  // contiguous range of each problem's tiles, grouped-M order; workgroup b
  // takes slots b / 8, b / 8 + S, ...
  const int xcd = blockIdx.x & 7;
  const int S = gridDim.x >> 3;
  const int total0 = ffn_wide::wide_tiles(wa.p[0], wa.p[0].N / BNO);
  const int total1 = wa.np > 1 ? ffn_wide::wide_tiles(wa.p[1], wa.p[1].N / BNO) : 0;
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
  auto next_slot = [&](int sl, Tile& t) -> int {
    while (sl < nslots && !decode(sl, t)) sl += S;
    return sl;
  };

  // ---------------- load addresses.  Load i of wave w fills 1 KB = 8 rows of
  // an operand: rows 32 w + 8 i + lane / 8, stored chunk lane % 8, holding
  // logical chunk (lane % 8) ^ ((row / 2) % 8) of the row.  Rows past the tile
  // end re-read the tile's last row (their results are never stored).
  Tile tc, tn;
  int sl = next_slot(blockIdx.x >> 3, tc);
  if (sl >= nslots) return;
  const int K = wa.p[tc.pi].K;  // the launcher checks that every problem of a persistent launch has this K
  const int NKB = K / KB;       // even
  auto lrow_of = [&](int i) { return 32 * wave + 8 * i + (lane >> 3); };
  auto chunk_of = [&](int row) { return (lane & 7) ^ ((row >> 1) & 7); };
  auto b_off = [&](int i) -> uint32_t {
    const int row = lrow_of(i);
    // gate/up: tile rows 0..127 are gate rows, 128..255 the up rows of the same outputs
    return (uint32_t)(((GATEUP ? row % (BW / 2) : row) * K + chunk_of(row) * 8) * 2);
  };
  const bool up_rows = GATEUP && 32 * wave >= BW / 2;  // this wave's B rows (wave-uniform)
  auto make_ops = [&](const Tile& t, Ops& o) {
    const FfnGemmArgs& a = wa.p[t.pi];
    o.abase = static_cast<const unsigned char*>(a.A);
    o.bbase = static_cast<const unsigned char*>(up_rows ? a.W1 : a.W0) + ((size_t)t.e * a.N + t.n0) * (size_t)K * 2;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int row = lrow_of(i);
      int src;
      if (a.row_index) {
        // the 8 rows of this load, read wave-uniformly; lane keeps row lane / 8
        int v = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = sload(a.row_index, t.row0 + min(32 * wave + 8 * i + j, t.nrows - 1));
          v = (lane >> 3) == j ? r : v;
        }
        src = v / a.row_div;
      } else {
        src = t.row0 + min(row, t.nrows - 1);
      }
      o.a_off[i] = (uint32_t)src * (uint32_t)(K * 2) + (uint32_t)(chunk_of(row) * 16);
    }
  };

  Ops cur, nxt;
  make_ops(tc, cur);
  int sln = GATEUP ? next_slot(sl + S, tn) : nslots;
  bool has_next = sln < nslots;
  nxt = cur;
  if (has_next) make_ops(tn, nxt);

  const unsigned char* const dummy = static_cast<const unsigned char*>(wa.p[0].A);
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)&stg[0][0]);
  // load l of a stage (A rows for l < LA, then B rows) of k-block qb of the
  // running sequence: block qb of the current tile, qb - NKB of the next, and
  // past both the same valid 16 bytes for every lane
  auto issue_one = [&](int l, int st, int qb) {
    const bool isa = l < LA;
    const int li = isa ? l : l - LA;
    const uint32_t dst = lds_base + (uint32_t)(st * STAGE + (isa ? 0 : OPA) + (32 * wave + 8 * li) * ROWB);
    const bool in_cur = qb < NKB;
    const bool in_next = !in_cur && has_next && qb < 2 * NKB;
    const unsigned char* const base_c = isa ? cur.abase : cur.bbase;
    const unsigned char* const base_n = isa ? nxt.abase : nxt.bbase;
    const uint32_t off_c = isa ? cur.a_off[li] : b_off(li);
    const uint32_t off_n = isa ? nxt.a_off[li] : b_off(li);
    const unsigned char* const base = in_cur ? base_c : (in_next ? base_n : dummy);
    const uint32_t off = in_cur ? off_c + (uint32_t)(qb * ROWB) : (in_next ? off_n + (uint32_t)((qb - NKB) * ROWB) : 0u);
    dma16(base, off, dst);
  };
  auto issue = [&](int st, int qb) {
#pragma unroll
    for (int l = 0; l < LPS; ++l) issue_one(l, st, qb);
  };

  // fragment reads: lane (lrow, q) of step s needs logical chunk 4 s + q of
  // its row; fragment rows start at multiples of 16, so the swizzle is (lrow / 2) % 8
  auto rd_off = [&](int s) { return lrow * ROWB + (((4 * s + q) ^ ((lrow >> 1) & 7)) * 16); };
  const int a_row0 = 64 * wr;
  const int b_row0 = (GATEUP ? HW / 2 : HW) * wc;

  f32x4 acc[MF][NF];
  // A fragments double-buffered in registers; B fragments single-buffered and
  // refilled in place, each right after its last MFMA of a step (this keeps
  // the kernel within 256 registers at two waves per SIMD)
  bf16x8 fa0[MF], fa1[MF], fb[NF];
  auto read_a = [&](bf16x8 (&fa)[MF], int st, int s) {
    const unsigned char* A = &stg[0][0] + st * STAGE;
    const int ro = rd_off(s);
#pragma unroll
    for (int mi = 0; mi < MF; ++mi)
      fa[mi] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(A + (a_row0 + 16 * mi) * ROWB + ro));
  };
  auto read_b = [&](int f, int st, int s) {
    const unsigned char* B = &stg[0][0] + st * STAGE + OPA;
    // gate/up: gate fragments then the up ones (tile rows +128)
    const int fo = GATEUP ? (f >= NF / 2 ? BW / 2 : 0) + 16 * (f % (NF / 2)) : 16 * f;
    fb[f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(B + (b_row0 + fo) * ROWB + rd_off(s)));
  };
  bool active = false;  // this wave has rows in the current tile (wave-uniform)
  // The MFMAs of one 32-deep step on (fa, fb), group by group (one B fragment
  // each), and after each group the reads of the next step's fragments (stage
  // st, step s): B fragment f in place into fb[f] (its last use just issued),
  // the A fragments into fan (one after each of the first MF groups).  Every
  // read of a step is issued after the step's first MFMAs, so a step starts by
  // waiting only for the previous step's reads, which had a whole step to
  // land.  With qb >= 0 the loads of k-block qb go into stage lst, one after
  // each group: a load issue waits for the address unit (one 1 KB load per 16
  // clocks per CU), and eight waves issuing one load per group of four MFMAs
  // keep it about as busy as the matrix cores.  Waves whose rows all lie past
  // the tile end run the MFMAs on re-read rows too (results never stored):
  // both waves of their SIMD are in that state, and every wave waits for the
  // busiest SIMD at the next barrier anyway.
  static_assert(LPS == NF && MF <= NF, "one load and at most one A read per group of MFMAs");
  auto step = [&](const bf16x8 (&fa)[MF], bf16x8 (&fan)[MF], int st, int s, int lst, int qb, auto with_loads) {
    const unsigned char* const A = &stg[0][0] + st * STAGE;
    const int ro = rd_off(s);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      // down: a wave that starts a group of MFMAs keeps issue priority over
      // the other wave of its SIMD until the group is in (measured on the
      // wide GeGLU down, K = 4096: 0.242 -> 0.234 ms; the gate/up ran slower
      // with it, 0.544 -> 0.552 ms, and goes without)
      if constexpr (!GATEUP) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mi = 0; mi < MF; ++mi)
        acc[mi][f] = GATEUP ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[f], fa[mi], acc[mi][f], 0, 0, 0)
                            : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mi], fb[f], acc[mi][f], 0, 0, 0);
      if constexpr (!GATEUP) __builtin_amdgcn_s_setprio(0);
      read_b(f, st, s);
      if (f < MF)
        fan[f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(A + (a_row0 + 16 * f) * ROWB + ro));
      if constexpr (decltype(with_loads)::value) issue_one(f, lst, qb);
    }
  };
  using no_loads = std::false_type;
  using loads = std::true_type;

  // ---------------- prologue: k-blocks 0 and 1 of the first tile in flight,
  // then the first step's fragments of k-block 0
  issue(0, 0);
  issue(1, 1);
  wait_vm<LPS>();
  lds_barrier();
  read_a(fa0, 0, 0);
#pragma unroll
  for (int f = 0; f < NF; ++f) read_b(f, 0, 0);
  for (;;) {
    const FfnGemmArgs& args = wa.p[tc.pi];
    const int N = args.N, nrows = tc.nrows;
    active = 64 * wr < nrows;
#pragma unroll
    for (int mi = 0; mi < MF; ++mi)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    // step 0 of k-block 0; the fragments of its step 1 are read meanwhile
    step(fa0, fa1, 0, 1, 0, 0, no_loads{});
    // (the loop is rotated so that its back edge meets the barrier's own wait
    // for outstanding LDS reads)
    for (int j = 0; j < NKB; ++j) {
      const int st = j & 1;
      // k-block j+1 complete for every wave, stage st free
      wait_vm<0>();
      lds_barrier();
      // step 1 of k-block j; the first fragments of k-block j+1 are read and
      // the loads of k-block j+2 issued into stage st meanwhile
      step(fa1, fa0, st ^ 1, 0, st, j + 2, loads{});
      // step 0 of k-block j+1; the fragments of its step 1 are read meanwhile
      if (j + 1 < NKB) step(fa0, fa1, st ^ 1, 1, 0, 0, no_loads{});
    }

    unsigned char* obase = static_cast<unsigned char*>(args.out) + ((size_t)tc.row0 * N + tc.n0) * (OUT == 1 ? 4 : 2);
    if constexpr (GATEUP && GBWD) {
      // ---------------- gate backward epilogue: lane (lrow, q) holds g and u
      // of hidden units c0 + 16 f + 0..3 of tile row 64 wr + 16 mi + lrow
      // (c0 = n0 + 64 wc + 4 q); with that row's dz' it writes [dg | du] and
      // w z, and the four lanes q of the row add their 16 products dz' z in a
      // fixed order into the row's partial of the 64-wide block n0 / 64 + wc
      if (active) {
        const GateBwdOut& gb = wa.gb[tc.pi];
        const int nbk = N / 64;
#pragma unroll
        for (int mi = 0; mi < MF; ++mi) {
          const int row = 64 * wr + 16 * mi + lrow;
          float part = 0.f;
          if (row < nrows) {
            const int rg = tc.row0 + row;
            const int c0 = tc.n0 + HW / 2 * wc + 4 * q;
            // the row's gate and its dz' loaded together (one row at a time:
            // the next tile's first fragments hold registers too)
            const float w = gb.w_row ? gb.w_row[rg] : 1.f;
            const float* dzr = gb.dZ + (size_t)rg * N + c0;
            f32x4 dz[NF / 2];
#pragma unroll
            for (int f = 0; f < NF / 2; ++f) dz[f] = *reinterpret_cast<const f32x4*>(dzr + 16 * f);
            uint16_t* dgr = gb.dGU + (size_t)rg * 2 * N + c0;
            uint16_t* zwr = gb.ZW + (size_t)rg * N + c0;
#pragma unroll
            for (int f = 0; f < NF / 2; ++f) {
              float dg[4], du[4], zw[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float z = gate_bwd_point<ACT, true>(acc[mi][f][r], acc[mi][f + NF / 2][r], dz[f][r], w, dg[r],
                                                          du[r], zw[r]);
                part += dz[f][r] * z;
              }
              *reinterpret_cast<uint2*>(dgr + 16 * f) = uint2{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
              *reinterpret_cast<uint2*>(dgr + N + 16 * f) =
                  uint2{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
              *reinterpret_cast<uint2*>(zwr + 16 * f) = uint2{pack_bf16x2(zw[0], zw[1]), pack_bf16x2(zw[2], zw[3])};
            }
          }
          part += __shfl_xor(part, 16, 64);
          part += __shfl_xor(part, 32, 64);
          if (q == 0 && row < nrows) gb.part[(size_t)(tc.row0 + row) * nbk + tc.n0 / 64 + wc] = part;
        }
      }
      if (!has_next) break;
      tc = tn;
      cur = nxt;
      sln = next_slot(sln + S, tn);
      has_next = sln < nslots;
      if (has_next) make_ops(tn, nxt);
    } else if constexpr (GATEUP) {
      // ---------------- gate/up epilogue (as ffn_wide.h): lane (lrow, q)
      // holds g (fragment f) and u (fragment f + NF/2) of four consecutive
      // outputs of tile row 64 wr + 16 mi + lrow; z goes out from registers
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
      tc = tn;
      cur = nxt;
      sln = next_slot(sln + S, tn);
      has_next = sln < nslots;
      if (has_next) make_ops(tn, nxt);
    } else {
      // ---------------- down epilogue: every wave stages its own 64 x HW
      // block through a private LDS region in parts of 128 bytes per row and
      // stores 16-byte row chunks (a wave's LDS accesses complete in order, so
      // no workgroup barrier is needed between its writes and reads).  One
      // tile per workgroup: the trailing loads land before the stages become
      // the staging buffer.
      wait_vm<0>();
      lds_barrier();
      unsigned char* const lds = &stg[0][0];
      constexpr int osz = OUT == 1 ? 4 : 2;
      constexpr int NPART = HW * osz / 128;  // 4 (fp32) or 2 (bf16)
      constexpr int QC = HW / NPART;         // output columns per part
      constexpr int FPP = NF / NPART;        // fragments per part
      constexpr int OS = QC * osz + 16;      // LDS row stride of a wave's block (bytes)
      constexpr int cpr = QC * osz / 16;     // 16-byte chunks per row and part
      static_assert(8 * 64 * OS <= NS * STAGE, "the waves' blocks fit the stage memory");
      unsigned char* const wl = lds + wave * 64 * OS;
      const int rows_w = min(64, nrows - 64 * wr);
      if (active) {
#pragma unroll
        for (int hh = 0; hh < NPART; ++hh) {
#pragma unroll
          for (int mi = 0; mi < MF; ++mi)
#pragma unroll
            for (int ff = 0; ff < FPP; ++ff)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float v = acc[mi][FPP * hh + ff][r];
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
          // the reads land before the next part overwrites the block
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
      }
      break;
    }
  }
  wait_vm<0>();  // every load has landed in LDS before the workgroup ends
}

// np problems (1 or 2) of the same kind in one launch, problem 0's tiles first;
// the events, if any, are attached to the launch.  Every K must be a multiple
// of 128 (an even number of 64-deep k-blocks).
template <bool GATEUP, bool GBWD = false>
hipError_t launch(const FfnGemmArgs* a, int np, void* ev_start, void* ev_stop, hipStream_t s,
                  const GateBwdOut* gb = nullptr) {
  constexpr int BNO = GATEUP ? BW / 2 : BW;
  if (np < 1 || np > 2) return hipErrorInvalidValue;
  if (GATEUP && a[0].out_f32) return hipErrorInvalidValue;  // gate/up writes z in bf16
  WideArgs w{};
  w.np = np;
  if (GBWD) {
    if (!GATEUP || !gb) return hipErrorInvalidValue;
    for (int i = 0; i < np; ++i) {
      if (!gb[i].dZ || !gb[i].dGU || !gb[i].ZW || !gb[i].part) return hipErrorInvalidValue;
      w.gb[i] = gb[i];
    }
  }
  long long slots = 0;
  for (int i = 0; i < np; ++i) {
    const FfnGemmArgs& p = a[i];
    if (p.N % BNO || p.K % (2 * KB) || (size_t)p.N * p.K * 2 > 0x7FFFFFFFull) return hipErrorInvalidValue;
    if (i > 0 && (p.out_f32 != a[0].out_f32 || p.out_f16 != a[0].out_f16 || p.act != a[0].act))
      return hipErrorInvalidValue;
    const int mt = p.offsets ? ffn_max_mtiles(p.E_loc, p.rows_max, BM) : (p.rows_max + BM - 1) / BM;
    slots += ((long long)mt * (p.N / BNO) + 7) / 8;
    w.p[i] = p;
  }
  long long g = 8 * slots;
  if (g == 0) return hipSuccess;
  if (g > 0x7FFFFFFFll) return hipErrorInvalidValue;
  // gate/up: one workgroup per CU running several tiles back to back where
  // every problem has the same K; otherwise one workgroup per tile
  if (GATEUP) {
    bool same_k = true;
    for (int i = 1; i < np; ++i) same_k = same_k && a[i].K == a[0].K;
    if (same_k && g > 8LL * ffn_wide::cus_per_xcd()) g = 8LL * ffn_wide::cus_per_xcd();
  }
  auto go = [&](auto kernel) {
    if (ev_start || ev_stop)
      hipExtLaunchKernelGGL(kernel, dim3((unsigned)g), dim3(512), 0, s, static_cast<hipEvent_t>(ev_start),
                            static_cast<hipEvent_t>(ev_stop), 0, w);
    else
      kernel<<<dim3((unsigned)g), dim3(512), 0, s>>>(w);
  };
  if constexpr (GBWD) {
    if (a[0].act == 1) go(wide64_kernel<true, 0, 1, true>);
    else go(wide64_kernel<true, 0, 0, true>);
  } else {
    if (!GATEUP && a[0].out_f32) go(wide64_kernel<false, 1, 0>);
    else if (!GATEUP && a[0].out_f16) go(wide64_kernel<false, 2, 0>);
    else if (GATEUP && a[0].act == 1) go(wide64_kernel<GATEUP, 0, 1>);
    else go(wide64_kernel<GATEUP, 0, 0>);
  }
  return hipGetLastError();
}

}  // namespace ffn_wide64
}  // namespace moe
