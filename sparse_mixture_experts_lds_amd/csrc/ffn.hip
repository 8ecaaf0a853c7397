// Plans and launches of the grouped expert GEMMs for fp32 and bf16 weights
// (the kernel template is in ffn_kernel.h; INT4 weights are in ffn_i4.hip).
// Built with the MFMA "VGPR form": accumulators carried across the k-loop stay
// in ordinary VGPRs instead of being shuffled between register files.
#include "ffn_kernel.h"
#include "ffn_wide.h"

namespace moe {

using ffn_detail::launch_mf_nf;

hipError_t launch_ffn_gemm_i4(const FfnGemmArgs& a, bool gateup, bool split, int BM, int NF, hipStream_t s);

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
      p.split_z = false;
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
  // down on 16-row tiles of 128 columns, whose 32-row version holds one
  // workgroup per CU.  Measured on MI355X (28-of-896-expert share, ~26 rows
  // per expert): 0.40 against 0.50 ms per layer.
  if (w_type == W_I4 && avg_rows <= 32) {
    p.BM = 32;
    p.NF_up = 1;
    p.BM_down = 16;
    p.NF_down = d % 128 == 0 ? 2 : 1;
    p.split_z = true;
    return p;
  }
  if (w_type == W_F32 && BM > 32) BM = 32;
  p.BM = BM;
  p.NF_up = (BM <= 64 && h % 128 == 0) ? 2 : 1;
  p.NF_down = (d % 128 == 0) ? 2 : 1;
  if (w_type == W_F32) p.NF_up = p.NF_down = 1;
  // INT4 shares carry the gated activations in fp32 into the down projection
  // (hi/lo bf16 split): their weight stream leaves the matrix cores idle
  // enough to afford the second MFMA.
  p.split_z = w_type == W_I4;
  return p;
}

hipError_t launch_ffn_gemm(const FfnGemmArgs& a, bool gateup, int w_type, bool split, int BM, int NF,
                           hipStream_t s) {
  // activation rows are addressed with 32-bit byte offsets
  const size_t gelt = (w_type == W_F32 || split) ? 4 : 2;
  if (a.a_rows < 0 || (size_t)a.a_rows * (size_t)a.K * gelt > 0xFFFFFFFFull) return hipErrorInvalidValue;
  if (BM == ffn_wide::BM) {
    if (w_type != W_BF16 || split) return hipErrorInvalidValue;
    // NF: weight rows per tile / 64 (4 -> 256, 2 -> 128)
    return gateup ? ffn_wide::launch_wide<true>(&a, 1, 64 * NF, a.ev_start, a.ev_stop, s)
                  : ffn_wide::launch_wide<false>(&a, 1, 64 * NF, a.ev_start, a.ev_stop, s);
  }
  if (w_type == W_F32) return gateup ? launch_mf_nf<W_F32, true, false>(a, BM, NF, s) : launch_mf_nf<W_F32, false, false>(a, BM, NF, s);
  if (w_type == W_I4) return launch_ffn_gemm_i4(a, gateup, split, BM, NF, s);
  if (gateup) return launch_mf_nf<W_BF16, true, false>(a, BM, NF, s);
  return split ? launch_mf_nf<W_BF16, false, true>(a, BM, NF, s) : launch_mf_nf<W_BF16, false, false>(a, BM, NF, s);
}

hipError_t launch_ffn_gemm_wide_pair(const FfnGemmArgs& a0, const FfnGemmArgs& a1, bool gateup, int NF,
                                     void* ev_start, void* ev_stop, hipStream_t s) {
  const FfnGemmArgs a[2] = {a0, a1};
  for (const FfnGemmArgs& p : a)
    if (p.a_rows < 0 || (size_t)p.a_rows * (size_t)p.K * 2 > 0xFFFFFFFFull) return hipErrorInvalidValue;
  return gateup ? ffn_wide::launch_wide<true>(a, 2, 64 * NF, ev_start, ev_stop, s)
                : ffn_wide::launch_wide<false>(a, 2, 64 * NF, ev_start, ev_stop, s);
}

}  // namespace moe
