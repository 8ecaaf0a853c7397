// Weighted top-k combine.
//
// Operation ("Sharding d'experts", "Deux roles": gate-weighted sum of the
// partial outputs plus the shared expert; ExpertMesh data-flow figure: expert
// outputs reduced with the top-k weights; moe_stream.py MoEFFN.forward: each
// expert's output scaled by its gate and added back into its token's row):
//   out[t] = sum_{j ascending, pair_pos[t*k+j] >= 0} w[t,j] * y[pair_pos[t*k+j]] + shared_y[t]
// in fp32, rounded once to the output type.
//
// A gather, not a scatter: each thread owns 8 consecutive values of one
// output row and reads the k expert rows of that token, so no atomics are
// needed and the result does not depend on scheduling.  Consecutive threads
// cover consecutive pieces of a row: every load and store is coalesced.
// Inside a bf16 layer the expert rows and the shared expert's output arrive in
// fp16 (a bf16 layer's y rounded once to fp16's 11-bit significand, then
// summed in fp32 and rounded once to bf16), inside an fp32 layer in fp32; the
// standalone entry point takes them in the output dtype.
#include "moe_internal.h"

namespace moe {
namespace {

// 8 consecutive values of a row: fp32 (two 16-byte vectors), bf16 or fp16
// (one).  TY: 0 bf16, 1 fp32, 2 fp16.
template <int TY>
__device__ __forceinline__ void load8(const void* base, size_t idx8, float* v) {
  if constexpr (TY == 1) {
    const u32x4* p = static_cast<const u32x4*>(base) + 2 * idx8;
    const u32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
    }
  } else {
    const u32x4 a = static_cast<const u32x4*>(base)[idx8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (TY == 2) {
        v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(a[i] & 0xFFFFu));
        v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(a[i] >> 16));
      } else {
        v[2 * i] = bf16_bits_to_f32(a[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_bits_to_f32(a[i] >> 16);
      }
    }
  }
}

// TY: storage of y and shared_y (0 bf16, 1 fp32, 2 fp16)
template <bool OUT_BF16, int TY>
__global__ __launch_bounds__(256) void combine_kernel(int T, int k, int v8_per_row, const void* __restrict__ y,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ tw,
                                                      const void* __restrict__ shared_y, void* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t t = i / v8_per_row;
  if (t >= (size_t)T) return;
  const int c = (int)(i - t * v8_per_row);
  float acc[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) acc[v] = 0.f;
  // the shared row's load is issued first; slots go four at a time: their
  // indices and gates, then the rows of the kept ones, all in flight together,
  // then the sums in ascending slot order (the order of the definition)
  float sv[8];
  if (shared_y) load8<TY>(shared_y, t * v8_per_row + c, sv);
  for (int j0 = 0; j0 < k; j0 += 4) {
    int pos[4];
    float w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u;
      pos[u] = j < k ? pair_pos[t * k + j] : -1;
      w[u] = pos[u] >= 0 ? tw[t * k + j] : 0.f;
    }
    float yv[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (pos[u] >= 0) {
        load8<TY>(y, (size_t)pos[u] * v8_per_row + c, yv[u]);
      } else {
#pragma unroll
        for (int v = 0; v < 8; ++v) yv[u][v] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (pos[u] >= 0) {
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[v] = fmaf(w[u], yv[u][v], acc[v]);
      }
    }
  }
  if (shared_y) {
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[v] += sv[v];
  }
  if constexpr (OUT_BF16) {
    u32x4 o;
#pragma unroll
    for (int v = 0; v < 4; ++v) o[v] = pack_bf16x2(acc[2 * v], acc[2 * v + 1]);
    static_cast<u32x4*>(out)[t * v8_per_row + c] = o;
  } else {
    u32x4* o = static_cast<u32x4*>(out) + 2 * (t * v8_per_row + c);
    o[0] = u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]), __float_as_uint(acc[3])};
    o[1] = u32x4{__float_as_uint(acc[4]), __float_as_uint(acc[5]), __float_as_uint(acc[6]), __float_as_uint(acc[7])};
  }
}

}  // namespace

hipError_t launch_combine(int T, int k, int d, bool out_bf16, int ytype, const void* y, const int32_t* pair_pos,
                          const float* tw, const void* shared_y, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int v8 = d / 8;
  const size_t n = (size_t)T * v8;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (!out_bf16)  // fp32 layers keep y in fp32
    combine_kernel<false, 1><<<grid, 256, 0, s>>>(T, k, v8, y, pair_pos, tw, shared_y, out);
  else if (ytype == Y_F32)
    combine_kernel<true, 1><<<grid, 256, 0, s>>>(T, k, v8, y, pair_pos, tw, shared_y, out);
  else if (ytype == Y_F16)
    combine_kernel<true, 2><<<grid, 256, 0, s>>>(T, k, v8, y, pair_pos, tw, shared_y, out);
  else
    combine_kernel<true, 0><<<grid, 256, 0, s>>>(T, k, v8, y, pair_pos, tw, shared_y, out);
  return hipGetLastError();
}

}  // namespace moe
