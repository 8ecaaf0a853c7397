// Weight preparation: signed INT4 codes with fp16 scales per 128-input group.
//
// Operation (ExpertMesh README: group-scaled signed INT4 weights, FP16 group
// scales, [expert, output, packed_input] layout, a bit-exact quantiser):
//   scale = fp16_rne(fp32(max |w|) / 7)
//   code  = clip(rint_even(w / fp32(scale)), -8, 7), 0 when scale == 0
//   byte i of a packed row = code[2i] (low nibble) | code[2i+1] << 4
// The divisions are IEEE float32 round-to-nearest (__fdiv_rn), so the result
// is bit-identical to any correct float32 implementation.
#include "moe_internal.h"

namespace moe {
namespace {

// One wave per (row, group): lane i handles inputs 2i, 2i+1 of the group.
__global__ __launch_bounds__(256) void quantize_kernel(int rows, int K, const float* __restrict__ w,
                                                       uint8_t* __restrict__ packed,
                                                       uint16_t* __restrict__ scales) {
  const int groups = K / kI4Group;
  const size_t gid = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gid >= (size_t)rows * groups) return;
  const int lane = threadIdx.x & 63;
  const size_t row = gid / groups;
  const int g = (int)(gid - row * groups);
  const float2 v = *reinterpret_cast<const float2*>(w + row * K + (size_t)g * kI4Group + 2 * lane);
  const float amax = wave_max(fmaxf(fabsf(v.x), fabsf(v.y)));
  const _Float16 s16 = (_Float16)__fdiv_rn(amax, 7.0f);  // float -> half rounds to nearest even
  const float sf = (float)s16;
  int c0 = 0, c1 = 0;
  if (sf > 0.f) {
    c0 = (int)fminf(fmaxf(rintf(__fdiv_rn(v.x, sf)), -8.f), 7.f);
    c1 = (int)fminf(fmaxf(rintf(__fdiv_rn(v.y, sf)), -8.f), 7.f);
  }
  packed[row * (K / 2) + (size_t)g * (kI4Group / 2) + lane] = (uint8_t)((c0 & 0xF) | ((c1 & 0xF) << 4));
  if (lane == 0) scales[row * groups + g] = __builtin_bit_cast(uint16_t, s16);
}

}  // namespace

hipError_t launch_quantize_int4(int rows, int K, const float* w, uint8_t* packed, uint16_t* scales,
                                hipStream_t s) {
  const size_t n = (size_t)rows * (K / kI4Group);
  if (n == 0) return hipSuccess;
  quantize_kernel<<<dim3((unsigned)((n + 3) / 4)), 256, 0, s>>>(rows, K, w, packed, scales);
  return hipGetLastError();
}

}  // namespace moe
