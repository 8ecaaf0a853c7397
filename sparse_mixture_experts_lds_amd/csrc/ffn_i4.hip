// Launches of the grouped expert GEMMs for signed INT4 weights (kernel
// template in ffn_kernel.h).  Kept in its own translation unit: the INT4
// kernels accumulate each 128-input group in fresh registers and are built
// with the compiler's default MFMA register form.
#include "ffn_i4s.h"
#include "ffn_kernel.h"

namespace moe {

using ffn_detail::launch_mf_nf;

// z16: the down projection's activations are fp16 (else bf16)
hipError_t launch_ffn_gemm_i4(const FfnGemmArgs& a, bool gateup, bool z16, int BM, int NF, hipStream_t s) {
  // 32-row gate/up tiles: the weight-streaming kernel (packed codes through LDS)
  if (gateup && BM == ffn_i4s::BM && ffn_i4s::ok(a)) return ffn_i4s::launch(a, s);
  if (gateup) return launch_mf_nf<W_I4, true, false>(&a, 1, BM, NF, s);
  return z16 ? launch_mf_nf<W_I4, false, true>(&a, 1, BM, NF, s) : launch_mf_nf<W_I4, false, false>(&a, 1, BM, NF, s);
}

}  // namespace moe
