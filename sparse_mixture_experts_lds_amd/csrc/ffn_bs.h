// Grouped gate/up GEMM for bf16 expert weights and few rows per expert that
// streams the weights through LDS: tiles of 32 or 64 grouped rows by 64 or 128
// outputs (twice as many weight rows: the gate rows, then the up rows of the
// same outputs), sixteen waves, both operands loaded straight into LDS.
//
// Operation ("Sharding d'experts", "Deux roles": the gate and up products of a
// worker; MoEEvolve "Architecture" / kieve-moe "Features": SwiGLU / GeGLU
// experts):
//   z[r, n] = act(sum_k a[r,k] Wg[e,n,k]) * (sum_k a[r,k] Wu[e,n,k])
// for every grouped row r of local expert e; z is written in bf16.
//
// Why.  With a few dozen rows per expert (a decode batch) the gate/up GEMM is
// a weight stream.  The register-loaded kernel (ffn_kernel.h) reads each weight
// row in 16-byte pieces spread over the k-steps, so one load instruction
// touches 64 weight rows; here a load that writes LDS directly covers eight
// rows with 128 bytes each (whole L2 lines), as the INT4 streaming kernel
// (ffn_i4s.h) does for packed codes.
//
// Data per k-block (64 inputs) and stage:
//   A  BM rows x 128 B of bf16 activations, gathered by row_index, loaded as
//      4-byte pieces (each instruction two rows), so every wave issues the
//      same number of loads;
//   B  2 BNO weight rows x 128 B;
// the 16-byte chunks of every 128-byte row stored XOR-swizzled by (row/2) % 8.
// Three stages; the loads of k-block j+2 are issued after the one barrier of
// k-block j, so every k-block has two k-blocks' time to land; the loads past
// a tile's end fetch the workgroup's next tile (one workgroup per CU runs its
// tiles back to back), past both every lane re-reads one valid piece, so each
// k-block issues the same loads and the vmcnt waits are exact.
//
// Waves.  A wave takes one group of 16 outputs (their gate and up rows), one
// 32-input half of every k-block and, with 64-output tiles, one half of the
// tile's rows; the two waves of an output group and row part add their sums
// through LDS at the end of a tile.
//
// Two problems per launch (the routed experts and the shared expert, same K
// and N), each XCD taking a contiguous range of problem 0's tiles, then of
// problem 1's, as in ffn_kernel.h.
#pragma once

#include "ffn_kernel.h"
#include "ffn_wide.h"

namespace moe {
namespace ffn_bs {

using ffn_wide::act_fn;
using ffn_wide::dma16;
using ffn_wide::lds_barrier;
using ffn_wide::sload;
using ffn_wide::sload4;
using ffn_wide::wait_vm;

// 4 bytes per lane from base + off (base uniform, off a per-lane 32-bit byte
// offset) into LDS at lds_addr + 4 * lane (lds_addr uniform); as dma16.
__device__ __forceinline__ void dma4(const unsigned char* base, uint32_t off, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  base = reinterpret_cast<const unsigned char*>(((uint64_t)hi << 32) | (uint64_t)lo);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}

constexpr int KB = 64;                // inputs per k-block
constexpr int ROWB = KB * 2;          // bytes per row per k-block (128)
constexpr int NS = 3;
constexpr int NWAVE = 16;
constexpr int kGroupM = 8;

// Tiles of 16 MF rows by BNO outputs (128 or 64).  The 16 waves split the
// outputs into OG groups of 16, the k-block into two halves of 32 inputs, and
// the rows into MH parts of MFW fragments.
template <int MF, int BNO>
struct Geo {
  static constexpr int BM = 16 * MF;
  static constexpr int OG = BNO / 16;
  static constexpr int MH = NWAVE / (2 * OG);
  static constexpr int MFW = MF / MH;
  static constexpr int OPA = BM * ROWB;
  static constexpr int OPB = 2 * BNO * ROWB;
  static constexpr int STAGE = OPA + OPB;
  static constexpr int LA = OPA / (NWAVE * 256);   // A loads (256 bytes each) per wave per stage
  static constexpr int LB = OPB / (NWAVE * 1024);  // B loads (1 KB each) per wave per stage
  static constexpr int LPS = LA + LB;
  static_assert(LA >= 1 && OPA == LA * NWAVE * 256, "A loads cover the stage");
  static_assert(LB >= 1 && OPB == LB * NWAVE * 1024, "B loads cover the stage");
  static_assert(MH >= 1 && MFW >= 1 && MFW * MH == MF, "waves cover the rows");
  static_assert(8 * 64 * 8 * 4 <= STAGE, "a round of the k-half exchange fits one stage");
};

struct Tile {
  int pi, e, row0, nrows, n0;
};

struct BsArgs {
  FfnGemmArgs p[2];
  int np;
};

struct Ops {
  const unsigned char* bb;  // this wave's weight matrix (gate or up) at the tile's first output row
  uint32_t a_off[4];        // per-lane byte offsets of the A loads in the activation matrix
  const unsigned char* abase;
};

template <int MF, int BNO, int ACT>
__global__ __launch_bounds__(1024) void bs_gateup_kernel(BsArgs args) {
  using G = Geo<MF, BNO>;
  constexpr int BM = G::BM, OPA = G::OPA, STAGE = G::STAGE, LA = G::LA, LB = G::LB, LPS = G::LPS;
  constexpr int OG = G::OG, MFW = G::MFW;
  __shared__ __attribute__((aligned(16))) unsigned char stg[NS][STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15;
  const int q = lane >> 4;
  const int og = wave % OG;            // output group: outputs 16 og .. 16 og + 15
  const int kh = (wave / OG) & 1;      // 32-input half of each k-block this wave takes
  const int mh = wave / (2 * OG);      // row part: fragments MFW mh .. MFW mh + MFW - 1
  const int K = args.p[0].K, N = args.p[0].N;
  const int NKB = K / KB;
  const int NBLK = N / BNO;

  // ---------------- tiles: XCD x = blockIdx % 8 owns a contiguous range of
  // each problem's tiles (problem 0's, then problem 1's: its local slots), and
  // its S workgroups stride through them
  const int xcd = blockIdx.x & 7;
  const int S = gridDim.x >> 3;
  auto total_mtiles = [&](const FfnGemmArgs& a) -> int {
    return a.offsets ? sload(a.mtile_start, a.E_loc) : (a.rows_max + BM - 1) / BM;
  };
  const int mt0 = total_mtiles(args.p[0]);
  const int mt1 = args.np > 1 ? total_mtiles(args.p[1]) : 0;
  const int total0 = mt0 * NBLK, total1 = mt1 * NBLK;
  const int per0 = (total0 + 7) / 8, per1 = (total1 + 7) / 8;
  const int n0x = max(0, min(per0, total0 - xcd * per0));
  const int n1x = max(0, min(per1, total1 - xcd * per1));
  auto decode = [&](int sl, Tile& t) -> bool {
    if (sl >= n0x + n1x) return false;
    const int pi = sl < n0x ? 0 : 1;
    const FfnGemmArgs& a = args.p[pi];
    const int R = pi ? xcd * per1 + (sl - n0x) : xcd * per0 + sl;
    const int total_mt = pi ? mt1 : mt0;
    // groups of GM m-tiles, m-tile fastest inside a group (GM = 1 where
    // experts average fewer than two m-tiles: an expert's n-tiles side by side)
    const int GM = (a.offsets && total_mt < 2 * a.E_loc) ? 1 : kGroupM;
    const int grp = R / (GM * NBLK);
    const int t0 = grp * GM;
    const int gm = min(GM, total_mt - t0);
    const int rr = R - grp * GM * NBLK;
    const int nb = rr / gm;
    const int mt = t0 + (rr - nb * gm);
    t.pi = pi;
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
    t.n0 = nb * BNO;
    return true;
  };
  Tile tc, tn;
  int sl = blockIdx.x >> 3;
  if (!decode(sl, tc)) return;

  // ---------------- load addresses.  A load i of wave w: rows 2 (LA w + i) +
  // lane / 32, 4-byte piece lane % 32 of the row: stored chunk (lane % 32) / 4
  // holding logical chunk ((lane % 32) / 4) ^ ((row / 2) % 8).  B load i:
  // weight rows 8 LB w + 8 i + lane / 8 (0..BNO-1 gate, BNO..2 BNO-1 up of the
  // same outputs), stored chunk lane % 8 holding logical chunk (lane % 8) ^
  // ((row / 2) % 8).  Rows past the tile end re-read its last row (never
  // stored).
  const bool up_rows = 8 * LB * wave >= BNO;
  auto b_off = [&](int i) -> uint32_t {
    const int row = 8 * LB * wave + 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    return (uint32_t)((row % BNO) * (K * 2) + chunk * 16);
  };
  auto make_ops = [&](const Tile& t, Ops& o) {
    const FfnGemmArgs& a = args.p[t.pi];
    const size_t row_first = (size_t)t.e * N + t.n0;
    o.bb = static_cast<const unsigned char*>(up_rows ? a.W1 : a.W0) + row_first * (size_t)(K * 2);
    o.abase = static_cast<const unsigned char*>(a.A);
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r0 = 2 * (LA * wave + i);
      const int row = r0 + (lane >> 5);
      int src;
      if (a.row_index) {
        const int s0 = sload(a.row_index, t.row0 + min(r0, t.nrows - 1));
        const int s1 = sload(a.row_index, t.row0 + min(r0 + 1, t.nrows - 1));
        src = ((lane >> 5) ? s1 : s0) / a.row_div;
      } else {
        src = t.row0 + min(row, t.nrows - 1);
      }
      const int piece = lane & 31;
      const int chunk = (piece >> 2) ^ ((row >> 1) & 7);
      o.a_off[i] = (uint32_t)src * (uint32_t)(K * 2) + (uint32_t)(chunk * 16 + (piece & 3) * 4);
    }
  };
  Ops cur, nxt;
  make_ops(tc, cur);
  int sln = sl + S;
  bool has_next = decode(sln, tn);
  nxt = cur;
  if (has_next) make_ops(tn, nxt);

  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)&stg[0][0]);
  // the loads of k-block kb of the tile whose addresses o holds into stage st;
  // real = false (past the last tile): every lane re-reads the same valid bytes
  auto issue = [&](const Ops& o, bool real, int st, int kb) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const uint32_t dst = lds_base + (uint32_t)(st * STAGE + 2 * (LA * wave + i) * ROWB);
      dma4(o.abase, real ? o.a_off[i] + (uint32_t)(kb * ROWB) : 0u, dst);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const uint32_t dst = lds_base + (uint32_t)(st * STAGE + OPA + (8 * LB * wave + 8 * i) * ROWB);
      dma16(real ? o.bb : o.abase, real ? b_off(i) + (uint32_t)(kb * ROWB) : 0u, dst);
    }
  };

  f32x4 acc[MFW][2];  // [m fragment of this wave's part][gate, up]

  // ---------------- prologue: k-blocks 0 and 1 in flight (NKB >= 2)
  issue(cur, true, 0, 0);
  issue(cur, true, 1, 1);
  int st = 0;  // stage of the current tile's k-block j
  // this lane's fragment chunk (same for A and B: rows 16 m + lrow)
  const int fchunk = (4 * kh + q) ^ ((lrow >> 1) & 7);
  for (;;) {
    const int nrows = tc.nrows;
#pragma unroll
    for (int mi = 0; mi < MFW; ++mi) acc[mi][0] = acc[mi][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < NKB; ++j) {
      // k-block j complete for this wave; the barrier makes it complete for
      // all and frees stage (j + 2) % NS (k-block j - 1)
      wait_vm<LPS>();
      lds_barrier();
      const int st2 = st >= 1 ? st - 1 : NS - 1;
      // k-block j + 2 of this tile, else k-block j + 2 - NKB of the next one
      if (j + 2 < NKB) issue(cur, true, st2, j + 2);
      else issue(nxt, has_next, st2, j + 2 - NKB);
      const unsigned char* const As = &stg[0][0] + st * STAGE;
      const unsigned char* const Bs = As + OPA;
      bf16x8 bf[2], af[MFW];
#pragma unroll
      for (int f = 0; f < 2; ++f)
        bf[f] = *reinterpret_cast<const bf16x8*>(Bs + (BNO * f + 16 * og + lrow) * ROWB + fchunk * 16);
#pragma unroll
      for (int mi = 0; mi < MFW; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8*>(As + (16 * (MFW * mh + mi) + lrow) * ROWB + fchunk * 16);
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int mi = 0; mi < MFW; ++mi)
          acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bf[f], acc[mi][f], 0, 0, 0);
      st = st + 1 == NS ? 0 : st + 1;
    }
    // ---------------- epilogue.  The waves of k-half 1 hand their sums to the
    // waves of k-half 0 (same output group and row part) through the stage
    // that held the tile's last k-block (free until the next k-block's
    // barrier; the first barrier below waits until every wave has finished
    // reading it), one m fragment per round (16 KB).  Lane (lrow, q) then
    // holds g (f = 0) and u (f = 1) of output n0 + 16 og + lrow for tile rows
    // 16 (MFW mh + mi) + 4 q + r; z goes out in bf16.
    {
      const int st_free = st >= 1 ? st - 1 : NS - 1;
      float* const xch =
          reinterpret_cast<float*>(&stg[0][0] + st_free * STAGE) + ((mh * OG + og) * 64 + lane) * 8;
#pragma unroll
      for (int mi = 0; mi < MFW; ++mi) {
        lds_barrier();
        if (kh == 1) {
#pragma unroll
          for (int f = 0; f < 2; ++f) *reinterpret_cast<f32x4*>(xch + f * 4) = acc[mi][f];
        }
        lds_barrier();
        if (kh == 0) {
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            const f32x4 o = *reinterpret_cast<const f32x4*>(xch + f * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mi][f][r] += o[r];
          }
        }
      }
      if (kh == 0) {
        uint16_t* const out = static_cast<uint16_t*>(args.p[tc.pi].out);
#pragma unroll
        for (int mi = 0; mi < MFW; ++mi)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * (MFW * mh + mi) + 4 * q + r;
            if (row < nrows) {
              const float z = act_fn<ACT>(acc[mi][0][r]) * acc[mi][1][r];
              out[(size_t)(tc.row0 + row) * N + tc.n0 + 16 * og + lrow] = (uint16_t)f32_to_bf16_bits(z);
            }
          }
      }
    }
    if (!has_next) break;
    tc = tn;
    cur = nxt;
    sln += S;
    has_next = decode(sln, tn);
    if (has_next) make_ops(tn, nxt);
  }
  wait_vm<0>();  // every load has landed before the workgroup ends
}

// Whether the streaming kernel takes these gate/up problems (bf16 weights and
// activations, z in bf16, tiles of 16 MF rows by 64 or 128 outputs).
inline bool ok(const FfnGemmArgs* a, int np) {
  if (np < 1 || np > 2) return false;
  for (int i = 0; i < np; ++i) {
    const FfnGemmArgs& p = a[i];
    if (p.K % KB || p.K < 2 * KB || p.N % 64 || p.out_f32 || p.out_f16 || !p.W1) return false;
    if ((size_t)p.a_rows * p.K * 2 > 0xFFFFFFFFull || (size_t)128 * p.K * 2 > 0x7FFFFFFFull) return false;
    if (i > 0 && (p.K != a[0].K || p.N != a[0].N || p.act != a[0].act)) return false;
  }
  return true;
}

inline hipError_t launch(const FfnGemmArgs* a, int np, int MF, int bno, hipStream_t s) {
  if (!ok(a, np) || (MF != 2 && MF != 4) || (bno != 64 && bno != 128) || a[0].N % bno) return hipErrorInvalidValue;
  const int BM = 16 * MF;
  BsArgs w{};
  w.np = np;
  long long per_ub = 0;  // per-XCD tiles, upper bound
  for (int i = 0; i < np; ++i) {
    const int mt = a[i].offsets ? ffn_max_mtiles(a[i].E_loc, a[i].rows_max, BM) : (a[i].rows_max + BM - 1) / BM;
    per_ub += ((long long)mt * (a[i].N / bno) + 7) / 8;
    w.p[i] = a[i];
  }
  if (per_ub == 0) return hipSuccess;
  // one workgroup per CU, each running its tiles back to back
  long long g = 8 * std::min<long long>(per_ub, ffn_wide::cus_per_xcd());
  const bool gelu = a[0].act == 1;
  auto go = [&](auto kernel) {
    if (a[0].ev_start || a[0].ev_stop)
      hipExtLaunchKernelGGL(kernel, dim3((unsigned)g), dim3(1024), 0, s, static_cast<hipEvent_t>(a[0].ev_start),
                            static_cast<hipEvent_t>(a[0].ev_stop), 0, w);
    else
      kernel<<<dim3((unsigned)g), dim3(1024), 0, s>>>(w);
  };
#define MOE_GO(MFv, BNOv) gelu ? go(bs_gateup_kernel<MFv, BNOv, 1>) : go(bs_gateup_kernel<MFv, BNOv, 0>)
  if (MF == 2) {
    if (bno == 128) MOE_GO(2, 128);
    else MOE_GO(2, 64);
  } else {
    if (bno == 128) MOE_GO(4, 128);
    else MOE_GO(4, 64);
  }
#undef MOE_GO
  return hipGetLastError();
}

}  // namespace ffn_bs
}  // namespace moe
