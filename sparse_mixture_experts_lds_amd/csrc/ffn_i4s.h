// Grouped gate/up GEMM for signed INT4 expert weights that streams the packed
// codes through LDS: tiles of 32 grouped rows by 128 outputs (256 weight rows:
// 128 gate then 128 up), sixteen waves, both operands loaded straight into LDS.
//
// Operation (ExpertMesh README: routed experts with group-scaled signed INT4
// weights, FP16 scales per 128 inputs, [expert, output, packed_input] layout;
// MoEEvolve "Architecture" / kieve-moe "Features": SwiGLU / GeGLU experts):
//   z[r, n] = act(sum_k a[r,k] Wg[e,n,k]) * (sum_k a[r,k] Wu[e,n,k]),
//   W[n, k] = scale[n, k / 128] * code[n, k]
// for every grouped row r of local expert e; z is written in fp16 (as INT4
// layers keep it for their down projection) or in fp32.
//
// Why a second INT4 kernel.  A share with a few dozen rows per expert is a
// weight stream: its time is the time to move the packed codes.  Loaded into
// registers in the MFMA fragment layout, a wave's 1 KB load covers sixteen
// weight rows with 64 bytes each, and the counters show the address unit
// stalled by the L1 for 42 % of the kernel.  Here a load that writes LDS
// directly covers eight rows with 128 bytes each (whole L2 lines), and the
// fragments are read from LDS afterwards.
//
// Data per k-block (256 inputs, two scale groups) and stage:
//   A  32 rows x 512 B of bf16 activations, gathered by row_index; the 16-byte
//      chunks of a row are stored XOR-swizzled by row % 16;
//   B  256 weight rows x 128 B of packed codes, chunks swizzled by (row/2) % 8;
//   S  the two fp16 scales (both groups) of each of the 256 weight rows, one
//      32-bit word per row, in a 4 KB block (each wave loads 16 rows' words;
//      its other 48 lanes load the same words again).
// Three stages (52 KB each); the loads of k-block j+2 are issued after the one
// barrier of k-block j, so every k-block has two k-blocks' time to land; the
// loads past a tile's end fetch the workgroup's next tile (one workgroup per
// CU runs its tiles back to back), past both every lane re-reads one valid
// piece, so each k-block issues the same loads and the vmcnt waits are exact.
//
// Dequantisation (as ffn_kernel.h): a 32-bit word of eight codes becomes four
// bf16 pairs 136 + code (codes 0,4 / 1,5 / 2,6 / 3,7; two instructions a pair),
// and the activations are permuted the same way: each wave permutes the
// 16-byte chunks it loaded itself, in place in LDS, once its loads have
// landed and before the barrier that publishes them.  Per 128-input group the
// MFMAs accumulate sum a (136 + code) plus, against a fragment of -136s,
// -136 sum a in fresh registers, which then hold sum a code exactly as the
// definition has it, and acc += scale * that.
// Lane group q (lanes 16q..16q+15) owns inputs 32q..32q+31 of a group: one
// 16-byte B read is four MFMA steps of eight codes.
//
// Waves.  Wave w takes outputs 16 (w % 8) .. +15 (their gate and up rows) and
// scale group w / 8 of every k-block, so no code is dequantised twice; the two
// waves of an output group add their sums through LDS at the end of a tile.
// Sixteen waves (four per SIMD) let one wave's dequantisation overlap
// another's MFMAs and loads.
#pragma once

#include "ffn_kernel.h"
#include "ffn_wide.h"

namespace moe {
namespace ffn_i4s {

using ffn_detail::half_bits_to_f32;
using ffn_detail::i4_word_to_bf16x8;
using ffn_detail::perm_04152637;
using ffn_wide::dma16;
using ffn_wide::lds_barrier;
using ffn_wide::sload;
using ffn_wide::sload4;
using ffn_wide::wait_vm;

// 4 bytes per lane from a per-lane address into LDS at lds_addr + 4 * lane
// (lds_addr uniform); as ffn_wide.h's dma16, asm so that the kernel's own
// vmcnt waits are the only ones.
__device__ __forceinline__ void dma4(const unsigned char* src, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}

// (x & mask) | magic in one instruction (the compiler splits it in two)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(magic));
  return r;
}

// Eight signed codes of a word as four bf16 pairs 136 + code (codes 0,4 / 1,5
// / 2,6 / 3,7), as ffn_kernel.h's i4_word_to_bf16x8; magic = 0x43004300 held
// in a register.
__device__ __forceinline__ u32x4 i4_word_to_bf16x8_v(uint32_t w, uint32_t magic) {
  const uint32_t v = w ^ 0x88888888u;
  u32x4 o;
  o[0] = and_or(v, 0x000F000Fu, magic);
  o[1] = and_or(v >> 4, 0x000F000Fu, magic);
  o[2] = and_or(v >> 8, 0x000F000Fu, magic);
  o[3] = and_or(v >> 12, 0x000F000Fu, magic);
  return o;
}

constexpr int BM = 32;              // grouped rows per tile
constexpr int BNO = 128;            // outputs per tile
constexpr int KB = 256;             // inputs per k-block (two scale groups)
constexpr int AROWB = KB * 2;       // activation bytes per row per k-block
constexpr int BROWB = KB / 2;       // packed code bytes per weight row per k-block
constexpr int OPA = BM * AROWB;     // 16 KB
constexpr int OPB = 2 * BNO * BROWB;  // 32 KB
constexpr int OPS = 4096;             // scale words: 16 waves x 64 lanes x 4 B
constexpr int STAGE = OPA + OPB + OPS;
constexpr int NS = 3;
constexpr int NWAVE = 16;
constexpr int LA = OPA / (NWAVE * 1024);  // A loads per wave per stage (1)
constexpr int LB = OPB / (NWAVE * 1024);  // B loads per wave per stage (2)
constexpr int LPS = LA + LB + 1;          // + the scale load
constexpr int kGroupM = 8;

struct Tile {
  int e, row0, nrows, n0;
};

struct Ops {
  const unsigned char* bg;   // gate codes of the tile's first output row
  const unsigned char* bu;   // up codes
  const uint16_t* sp;        // scales of the weight row whose word this lane loads
  uint32_t a_off[LA];        // per-lane byte offsets of the A loads in the activation matrix
};

template <int ACT>
__global__ __launch_bounds__(1024) void i4s_gateup_kernel(FfnGemmArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char stg[NS][STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15;
  const int q = lane >> 4;
  const int og = wave & 7;   // output group: outputs 16 og .. 16 og + 15
  const int kh = wave >> 3;  // scale group of each k-block this wave takes
  const int K = a.K, N = a.N;
  const int NKB = K / KB;
  const int NBLK = N / BNO;
  const int KG = K / kI4Group;  // scale groups per weight row

  // ---------------- tiles: XCD x = blockIdx % 8 owns a contiguous range of
  // the tiles (grouped-M order), workgroup b takes slots b / 8, b / 8 + S, ...
  const int xcd = blockIdx.x & 7;
  const int S = gridDim.x >> 3;
  const int total_mt = a.offsets ? sload(a.mtile_start, a.E_loc) : (a.rows_max + BM - 1) / BM;
  const int total = total_mt * NBLK;
  const int per = (total + 7) / 8;
  // groups of GM m-tiles, m-tile fastest inside a group: kGroupM shares a
  // weight slice between neighbouring m-tiles of one expert; where experts
  // average fewer than two m-tiles, GM = 1 puts an expert's n-tiles side by
  // side instead, so its activation rows are fetched into one XCD's L2 once
  const int GM = (a.offsets && total_mt < 2 * a.E_loc) ? 1 : kGroupM;
  auto decode = [&](int sl, Tile& t) -> bool {
    const int R = xcd * per + sl;
    if (sl >= per || R >= total) return false;
    const int grp = R / (GM * NBLK);
    const int t0 = grp * GM;
    const int gm = min(GM, total_mt - t0);
    const int rr = R - grp * GM * NBLK;
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
    t.n0 = nb * BNO;
    return true;
  };
  Tile tc, tn;
  int sl = blockIdx.x >> 3;
  if (!decode(sl, tc)) return;

  // ---------------- load addresses.  A load of wave w: rows 2 w + lane / 32,
  // lane % 32 the stored chunk, holding logical chunk (lane % 32) ^ (row % 16).
  // B load i: weight rows 16 w + 8 i + lane / 8 (0..127 gate, 128..255 up of
  // the same outputs), stored chunk lane % 8 holding logical chunk (lane % 8)
  // ^ ((row / 2) % 8).  Scale load: the word of weight row 16 w + lane % 16.
  // Rows past the tile end re-read its last row (never stored).
  const bool up_rows = 16 * wave >= BNO;
  auto b_off = [&](int i) -> uint32_t {
    const int row = 16 * wave + 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    return (uint32_t)((row % BNO) * (K / 2) + chunk * 16);
  };
  auto make_ops = [&](const Tile& t, Ops& o) {
    const size_t row_first = (size_t)t.e * N + t.n0;
    o.bg = static_cast<const unsigned char*>(a.W0) + row_first * (size_t)(K / 2);
    o.bu = static_cast<const unsigned char*>(a.W1) + row_first * (size_t)(K / 2);
    o.sp = (up_rows ? a.S1 : a.S0) + (row_first + ((16 * wave + (lane & 15)) % BNO)) * (size_t)KG;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int row = 2 * wave + 2 * i + (lane >> 5);
      int src;
      if (a.row_index) {
        const int r0 = sload(a.row_index, t.row0 + min(2 * wave + 2 * i, t.nrows - 1));
        const int r1 = sload(a.row_index, t.row0 + min(2 * wave + 2 * i + 1, t.nrows - 1));
        src = ((lane >> 5) ? r1 : r0) / a.row_div;
      } else {
        src = t.row0 + min(row, t.nrows - 1);
      }
      const int chunk = (lane & 31) ^ (row & 15);
      o.a_off[i] = (uint32_t)src * (uint32_t)(K * 2) + (uint32_t)(chunk * 16);
    }
  };
  Ops cur, nxt;
  make_ops(tc, cur);
  int sln = sl + S;
  bool has_next = decode(sln, tn);
  nxt = cur;
  if (has_next) make_ops(tn, nxt);

  const unsigned char* const abase = static_cast<const unsigned char*>(a.A);
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)&stg[0][0]);
  // the loads of k-block kb of the tile whose addresses o holds into stage st;
  // real = false (past the last tile): every lane re-reads the same valid bytes
  auto issue = [&](const Ops& o, bool real, int st, int kb) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const uint32_t dst = lds_base + (uint32_t)(st * STAGE + (2 * wave + 2 * i) * AROWB);
      dma16(abase, real ? o.a_off[i] + (uint32_t)(kb * AROWB) : 0u, dst);
    }
    const unsigned char* const bb = real ? (up_rows ? o.bu : o.bg) : abase;
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const uint32_t dst = lds_base + (uint32_t)(st * STAGE + OPA + (16 * wave + 8 * i) * BROWB);
      dma16(bb, real ? b_off(i) + (uint32_t)(kb * BROWB) : 0u, dst);
    }
    // the scale word (groups 2 kb and 2 kb + 1) of weight row 16 w + lane % 16
    const unsigned char* const sp = real ? reinterpret_cast<const unsigned char*>(o.sp + 2 * kb) : abase;
    dma4(sp, lds_base + (uint32_t)(st * STAGE + OPA + OPB + wave * 256));
  };

  // -136 in bf16 (0xC308, exact), and the dequantisation's magic in a register
  const bf16x8 m136 = __builtin_bit_cast(bf16x8, u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u});
  const uint32_t magic = __builtin_amdgcn_readfirstlane(0x43004300u);
  f32x4 acc[2][2];  // [m fragment][gate, up]

  // ---------------- prologue: k-blocks 0 and 1 in flight
  issue(cur, true, 0, 0);
  issue(cur, true, 1, 1);
  int st = 0;  // stage of the current tile's k-block j
  for (;;) {
    const int nrows = tc.nrows;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) acc[mi][0] = acc[mi][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < NKB; ++j) {
      // k-block j complete for every wave; stage (j + 2) % NS (k-block j - 1) free
      wait_vm<LPS>();
      {
        // this wave's own A chunks of k-block j (landed): codes come out of a
        // word in the order 0,4,1,5,2,6,3,7, and the activations are stored
        // permuted the same way (the swizzle moves whole chunks, so it holds)
        u32x4* const mine = reinterpret_cast<u32x4*>(&stg[0][0] + st * STAGE + 2 * wave * AROWB) + lane;
        *mine = perm_04152637(*mine);
      }
      lds_barrier();
      const int st2 = st >= 1 ? st - 1 : NS - 1;
      // k-block j + 2 of this tile, else k-block j + 2 - NKB of the next one
      if (j + 2 < NKB) issue(cur, true, st2, j + 2);
      else issue(nxt, has_next, st2, j + 2 - NKB);
      const unsigned char* const As = &stg[0][0] + st * STAGE;
      const unsigned char* const Bs = As + OPA;
      {
        const int g = kh;  // this wave's scale group of the k-block
        // this lane's 32 codes of the group for its gate and up output rows
        u32x4 bw[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int row = BNO * f + 16 * og + lrow;
          const int chunk = (4 * g + q) ^ ((lrow >> 1) & 7);
          bw[f] = *reinterpret_cast<const u32x4*>(Bs + row * BROWB + chunk * 16);
        }
        // the scales of this lane's gate and up output rows (row f*128 + 16 og +
        // lrow: word lrow of wave 8 f + og's block), group g
        float sc[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const uint32_t wd = *reinterpret_cast<const uint32_t*>(Bs + OPB + (8 * f + og) * 256 + lrow * 4);
          sc[f] = half_bits_to_f32((uint16_t)(wd >> (16 * g)));
        }
        f32x4 gacc[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) gacc[mi][0] = gacc[mi][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          bf16x8 af[2];
#pragma unroll
          for (int mi = 0; mi < 2; ++mi) {
            const int chunk = (16 * g + 4 * q + t) ^ lrow;
            af[mi] = *reinterpret_cast<const bf16x8*>(As + (16 * mi + lrow) * AROWB + chunk * 16);
          }
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            const bf16x8 b = __builtin_bit_cast(bf16x8, i4_word_to_bf16x8_v(bw[f][t], magic));
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
              gacc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], b, gacc[mi][f], 0, 0, 0);
              gacc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], m136, gacc[mi][f], 0, 0, 0);
            }
          }
        }
        // gacc = sum a (136 + code) - 136 sum a = sum a code; acc += scale * gacc
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mi][f][r] = fmaf(sc[f], gacc[mi][f][r], acc[mi][f][r]);
      }
      st = st + 1 == NS ? 0 : st + 1;
    }
    // ---------------- epilogue.  The waves of scale group 1 hand their sums
    // to the waves of group 0 through the stage that held the tile's last
    // k-block (free until the next k-block's barrier; the first barrier below
    // waits until every wave has finished reading it).  Lane (lrow, q) then
    // holds g (f = 0) and u (f = 1) of output n0 + 16 og + lrow for tile rows
    // 16 mi + 4 q + r; z goes out in fp16 (out_f16) or fp32.
    {
      const int st_free = st >= 1 ? st - 1 : NS - 1;
      float* const xch = reinterpret_cast<float*>(&stg[0][0] + st_free * STAGE) + (og * 64 + lane) * 16;
      lds_barrier();
      if (kh == 1) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int f = 0; f < 2; ++f) *reinterpret_cast<f32x4*>(xch + (2 * mi + f) * 4) = acc[mi][f];
      }
      lds_barrier();
      if (kh == 0) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            const f32x4 o = *reinterpret_cast<const f32x4*>(xch + (2 * mi + f) * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mi][f][r] += o[r];
          }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * mi + 4 * q + r;
            if (row < nrows) {
              const float gv = acc[mi][0][r];
              const float z = (ACT == 0 ? silu_hw(gv) : gelu_hw(gv)) * acc[mi][1][r];
              const size_t o = (size_t)(tc.row0 + row) * N + tc.n0 + 16 * og + lrow;
              if (a.out_f16) static_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_f16_bits(z);
              else static_cast<float*>(a.out)[o] = z;
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

// Whether the streaming kernel takes this INT4 gate/up GEMM.  The loads run
// two k-blocks ahead within a tile, so a tile has at least two.
inline bool ok(const FfnGemmArgs& a) {
  return a.K % KB == 0 && a.K >= 2 * KB && a.N % BNO == 0 && (a.out_f32 || a.out_f16) &&
         (size_t)a.a_rows * a.K * 2 <= 0xFFFFFFFFull &&
         (size_t)a.N * (a.K / 2) <= 0x7FFFFFFFull;
}

inline hipError_t launch(const FfnGemmArgs& a, hipStream_t s) {
  if (!ok(a)) return hipErrorInvalidValue;
  const int mt = a.offsets ? ffn_max_mtiles(a.E_loc, a.rows_max, BM) : (a.rows_max + BM - 1) / BM;
  const long long tiles = (long long)mt * (a.N / BNO);
  if (tiles == 0) return hipSuccess;
  // one workgroup per CU (three 52 KB stages), each running its tiles back to back
  long long g = 8LL * ((tiles + 7) / 8);
  const long long cap = 8LL * ffn_wide::cus_per_xcd();
  if (g > cap) g = cap;
  auto kernel = a.act == 1 ? i4s_gateup_kernel<1> : i4s_gateup_kernel<0>;
  if (a.ev_start || a.ev_stop)
    hipExtLaunchKernelGGL(kernel, dim3((unsigned)g), dim3(1024), 0, s, static_cast<hipEvent_t>(a.ev_start),
                          static_cast<hipEvent_t>(a.ev_stop), 0, a);
  else
    kernel<<<dim3((unsigned)g), dim3(1024), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ffn_i4s
}  // namespace moe
