// Plans and launches of the grouped expert GEMMs for fp32 and bf16 weights
// (the kernel template is in ffn_kernel.h; INT4 weights are in ffn_i4.hip).
// Built with the MFMA "VGPR form": accumulators carried across the k-loop stay
// in ordinary VGPRs instead of being shuffled between register files.
#include "ffn_bs.h"
#include "ffn_kernel.h"
#include "ffn_wide.h"
#include "ffn_wide64.h"

namespace moe {

using ffn_detail::launch_mf_nf;

#ifndef MOE_BS_BNO
#define MOE_BS_BNO 64
#endif
// outputs per tile of the weight-streaming gate/up kernel
constexpr int kBsBno = MOE_BS_BNO;
#ifndef MOE_I4_BM_DOWN
#define MOE_I4_BM_DOWN 32
#endif
#ifndef MOE_I4_NF_DOWN
#define MOE_I4_NF_DOWN 2
#endif
// rows and 64-column fragments per tile of the INT4 down projection
constexpr int kI4BmDown = MOE_I4_BM_DOWN;
constexpr int kI4NfDown = MOE_I4_NF_DOWN;

hipError_t launch_ffn_gemm_i4(const FfnGemmArgs& a, bool gateup, bool z16, int BM, int NF, hipStream_t s);

int ffn_max_mtiles(int E_loc, int rows_max, int BM) {
  // sum_e ceil(n_e / BM) <= ceil(rows / BM) + (number of non-empty groups - 1)
  const long long a = ((long long)rows_max + BM - 1) / BM + (E_loc > 0 ? E_loc - 1 : 0);
  const long long b = rows_max;  // each non-empty group has at least one row
  return (int)(a < b ? a : b);
}

FfnPlan plan_ffn(double avg_rows, int groups, int d, int h, int w_type) {
  // Tile shapes from measurements on MI355X: tiles as tall as the typical
  // expert (weights are then re-read from L2 at most a few times), 64-column
  // gate/up tiles once tiles are tall (halves the live accumulators), 128-column
  // down tiles whenever d allows.
  FfnPlan p{};
  // Wide tiles (256 rows x 256 weight rows, bf16): half the bytes per FLOP of
  // the narrow tiles; worth it once experts average ~100 rows and there are
  // enough tiles to give every CU one.
  if (w_type == W_BF16 && avg_rows >= 96 && h % 128 == 0 && d % 256 == 0) {
    const double mt = (double)groups * (double)(int)((avg_rows + 255) / 256);
    if (mt * (h / 128) >= 256) {
      // 256 weight rows per tile (the 128-row variant, reachable through the
      // tile hints, measured slower on every workload here: a k-block's fixed
      // costs do not shrink with the tile)
      p.BM = 256;
      p.NF_up = p.NF_down = 4;
      p.z_f16 = false;
      return p;
    }
  }
  int BM;
  if (avg_rows <= 16) BM = 16;
  else if (avg_rows <= 24) BM = 32;
  else if (avg_rows <= 112) BM = 64;
  else BM = 128;
  if (w_type == W_I4 && BM > 64) BM = 64;
  // INT4 with up to ~32 rows per expert: gate/up on 32-row tiles of 64
  // columns (each weight slice read once per expert, two workgroups per CU),
  // down on the same 32-row tiles, 128 columns wide (with its fp16 z the
  // kernel keeps two workgroups per CU).  Measured on MI355X (INT4 share, 25
  // touched experts of 1 to 472 rows): down 0.114-0.119 ms against
  // 0.124-0.127 on 16-row tiles and 0.138-0.141 on 16 x 64 tiles.
  if (w_type == W_I4 && avg_rows <= 32) {
    p.BM = 32;
    p.NF_up = 1;
    p.BM_down = kI4BmDown == p.BM ? 0 : kI4BmDown;
    p.NF_down = d % (64 * kI4NfDown) == 0 ? kI4NfDown : 1;
    p.z_f16 = true;
    return p;
  }
  if (w_type == W_F32 && BM > 32) BM = 32;
  p.BM = BM;
  p.NF_up = (BM <= 64 && h % 128 == 0) ? 2 : 1;
  p.NF_down = (d % 128 == 0) ? 2 : 1;
  if (w_type == W_F32) p.NF_up = p.NF_down = 1;
  // INT4 shares carry the gated activations into the down projection in fp16
  // (three more significand bits than bf16, half the bytes of fp32)
  p.z_f16 = w_type == W_I4;
  return p;
}

hipError_t launch_ffn_gemm(const FfnGemmArgs& a, bool gateup, int w_type, bool z16, int BM, int NF,
                           hipStream_t s) {
  // z16: fp16 activations (the z of INT4 layers), INT4 down projections only
  if (z16 && (gateup || w_type != W_I4)) return hipErrorInvalidValue;
  // activation rows are addressed with 32-bit byte offsets
  const size_t gelt = w_type == W_F32 ? 4 : 2;
  if (a.a_rows < 0 || (size_t)a.a_rows * (size_t)a.K * gelt > 0xFFFFFFFFull) return hipErrorInvalidValue;
  if (BM == ffn_wide::BM) {
    if (w_type != W_BF16) return hipErrorInvalidValue;
    // NF: weight rows per tile / 64 (4 -> 256, 2 -> 128); 256 weight rows and
    // K a multiple of 128 take the 64-deep k-blocks
    if (NF == 4 && a.K % 128 == 0)
      return gateup ? ffn_wide64::launch<true>(&a, 1, a.ev_start, a.ev_stop, s)
                    : ffn_wide64::launch<false>(&a, 1, a.ev_start, a.ev_stop, s);
    return gateup ? ffn_wide::launch_wide<true>(&a, 1, 64 * NF, a.ev_start, a.ev_stop, s)
                  : ffn_wide::launch_wide<false>(&a, 1, 64 * NF, a.ev_start, a.ev_stop, s);
  }
  if (w_type == W_F32)
    return gateup ? launch_mf_nf<W_F32, true, false>(&a, 1, BM, NF, s) : launch_mf_nf<W_F32, false, false>(&a, 1, BM, NF, s);
  if (w_type == W_I4) return launch_ffn_gemm_i4(a, gateup, z16, BM, NF, s);
  // few rows per expert: the weight-streaming kernel (its tiles are always 128
  // outputs wide)
  if (gateup && (BM == 32 || BM == 64) && ffn_bs::ok(&a, 1)) return ffn_bs::launch(&a, 1, BM / 16, kBsBno, s);
  if (gateup) return launch_mf_nf<W_BF16, true, false>(&a, 1, BM, NF, s);
  return launch_mf_nf<W_BF16, false, false>(&a, 1, BM, NF, s);
}

hipError_t launch_ffn_gemm_pair(const FfnGemmArgs& a0, const FfnGemmArgs& a1, bool gateup, int w_type, int BM,
                                int NF, hipStream_t s) {
  const FfnGemmArgs a[2] = {a0, a1};
  const size_t gelt = w_type == W_F32 ? 4 : 2;
  for (const FfnGemmArgs& p : a)
    if (p.a_rows < 0 || (size_t)p.a_rows * (size_t)p.K * gelt > 0xFFFFFFFFull) return hipErrorInvalidValue;
  if (BM == ffn_wide::BM || (w_type != W_F32 && w_type != W_BF16)) return hipErrorInvalidValue;
  if (w_type == W_F32)
    return gateup ? launch_mf_nf<W_F32, true, false>(a, 2, BM, NF, s) : launch_mf_nf<W_F32, false, false>(a, 2, BM, NF, s);
  if (gateup && (BM == 32 || BM == 64) && ffn_bs::ok(a, 2)) return ffn_bs::launch(a, 2, BM / 16, kBsBno, s);
  return gateup ? launch_mf_nf<W_BF16, true, false>(a, 2, BM, NF, s) : launch_mf_nf<W_BF16, false, false>(a, 2, BM, NF, s);
}

bool gateup_bwd_wide_ok(const FfnGemmArgs& a) {
  return a.K % (2 * ffn_wide64::KB) == 0 && a.N % (ffn_wide64::BW / 2) == 0 && !a.out_f32 && a.W1 &&
         a.a_rows >= 0 && (size_t)a.a_rows * (size_t)a.K * 2 <= 0xFFFFFFFFull;
}

hipError_t launch_gateup_bwd_wide(const FfnGemmArgs* a, const GateBwdOut* gb, int np, hipStream_t s) {
  if (np < 1 || np > 2) return hipErrorInvalidValue;
  for (int i = 0; i < np; ++i)
    if (!gateup_bwd_wide_ok(a[i])) return hipErrorInvalidValue;
  return ffn_wide64::launch<true, true>(a, np, nullptr, nullptr, s, gb);
}

hipError_t launch_ffn_gemm_wide_pair(const FfnGemmArgs& a0, const FfnGemmArgs& a1, bool gateup, int NF,
                                     void* ev_start, void* ev_stop, hipStream_t s) {
  const FfnGemmArgs a[2] = {a0, a1};
  for (const FfnGemmArgs& p : a)
    if (p.a_rows < 0 || (size_t)p.a_rows * (size_t)p.K * 2 > 0xFFFFFFFFull) return hipErrorInvalidValue;
  if (NF == 4 && a0.K % 128 == 0 && a1.K % 128 == 0)
    return gateup ? ffn_wide64::launch<true>(a, 2, ev_start, ev_stop, s)
                  : ffn_wide64::launch<false>(a, 2, ev_start, ev_stop, s);
  return gateup ? ffn_wide::launch_wide<true>(a, 2, 64 * NF, ev_start, ev_stop, s)
                : ffn_wide::launch_wide<false>(a, 2, 64 * NF, ev_start, ev_stop, s);
}

}  // namespace moe
