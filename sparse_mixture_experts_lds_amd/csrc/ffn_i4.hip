// Launches of the grouped expert GEMMs for signed INT4 weights (kernel
// template in ffn_kernel.h).  Kept in its own translation unit: the INT4
// kernels accumulate each 128-input group in fresh registers and are built
// with the compiler's default MFMA register form.
#include "ffn_kernel.h"

namespace moe {

using ffn_detail::launch_mf_nf;

hipError_t launch_ffn_gemm_i4(const FfnGemmArgs& a, bool gateup, bool split, int BM, int NF, hipStream_t s) {
  if (gateup) return launch_mf_nf<W_I4, true, false>(a, BM, NF, s);
  return split ? launch_mf_nf<W_I4, false, true>(a, BM, NF, s) : launch_mf_nf<W_I4, false, false>(a, BM, NF, s);
}

}  // namespace moe
