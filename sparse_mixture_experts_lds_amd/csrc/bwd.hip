// Backward pass of the layer: launchers of the grouped GEMMs and the
// element-wise, router and assembly kernels.
//
// The gradients are the chain rule of the forward (the trainers of moe_stream.py,
// MoEEvolve and kieve-moe differentiate this layer): per kept pair p of token
// t with gate w and expert e, the expert sees dy = w dout[t]; the gate gets
// <dout[t], y_p> = <dout[t] Wd_e, z_p>, so y is never materialised; the
// softmax and top-k gate normalisation pass it on to the router logits.
#include <algorithm>

#include "bwd_gemm.h"
#include "bwd_wide.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- gate
// One wave per grouped row r (pair p = sorted_pair[r], or r itself for the
// shared expert), four consecutive hidden units per lane per step:
//   a = act(g), a' = act'(g), z = round_T(a * u)   (the forward's z)
//   dgate[p] = sum_c dz'[c] z[c]   (wave sum, fixed butterfly order)
//   dz = w dz';  dg = dz u a';  du = dz a
//   dGU[r] = [dg | du] (T),  ZW[r] = round_T(w z) (T)
template <typename T, int ACT>
__global__ __launch_bounds__(256) void gate_bwd_kernel(int rows, int h, const int32_t* __restrict__ n_rows,
                                                       const float* __restrict__ G, const float* __restrict__ U,
                                                       const float* __restrict__ dZ,
                                                       const int32_t* __restrict__ sorted_pair,
                                                       const float* __restrict__ tw, T* __restrict__ dGU,
                                                       T* __restrict__ ZW, float* __restrict__ dgate) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n = n_rows ? *n_rows : rows;
  if (r >= n || r >= rows) return;
  const int p = sorted_pair ? sorted_pair[r] : r;
  const float w = tw ? tw[p] : 1.f;
  const size_t o = (size_t)r * h;
  float part = 0.f;
  for (int c = lane * 4; c < h; c += 256) {
    const f32x4 g = *reinterpret_cast<const f32x4*>(G + o + c);
    const f32x4 u = *reinterpret_cast<const f32x4*>(U + o + c);
    const f32x4 dz1 = *reinterpret_cast<const f32x4*>(dZ + o + c);
    float dg[4], du[4], zw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float z = gate_bwd_point<ACT, sizeof(T) == 2>(g[i], u[i], dz1[i], w, dg[i], du[i], zw[i]);
      part += dz1[i] * z;
    }
    T* dgu = dGU + (size_t)r * 2 * h;
    if constexpr (sizeof(T) == 2) {
      uint2 vg, vu, vz;
      vg.x = pack_bf16x2(dg[0], dg[1]);
      vg.y = pack_bf16x2(dg[2], dg[3]);
      vu.x = pack_bf16x2(du[0], du[1]);
      vu.y = pack_bf16x2(du[2], du[3]);
      vz.x = pack_bf16x2(zw[0], zw[1]);
      vz.y = pack_bf16x2(zw[2], zw[3]);
      *reinterpret_cast<uint2*>(dgu + c) = vg;
      *reinterpret_cast<uint2*>(dgu + h + c) = vu;
      *reinterpret_cast<uint2*>(ZW + o + c) = vz;
    } else {
      *reinterpret_cast<f32x4*>(dgu + c) = f32x4{dg[0], dg[1], dg[2], dg[3]};
      *reinterpret_cast<f32x4*>(dgu + h + c) = f32x4{du[0], du[1], du[2], du[3]};
      *reinterpret_cast<f32x4*>(ZW + o + c) = f32x4{zw[0], zw[1], zw[2], zw[3]};
    }
  }
  part = wave_sum(part);
  if (lane == 0 && dgate) dgate[p] = part;
}

// The gate gradient of each grouped row from the partial sums a fused gate/up
// launch wrote (one per 64-wide block of hidden units): a 16-lane group per
// row adds its nb partials lane-strided, then across the group in a fixed
// shuffle order.
__global__ __launch_bounds__(256) void gate_part_sum_kernel(int rows, int nb, const int32_t* __restrict__ n_rows,
                                                            const float* __restrict__ part,
                                                            const int32_t* __restrict__ sorted_pair,
                                                            float* __restrict__ dgate) {
  const int gl = threadIdx.x & 15;
  const int r = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int n = n_rows ? *n_rows : rows;
  if (r >= n || r >= rows) return;  // whole groups leave together
  float v = 0.f;
  for (int j = gl; j < nb; j += 16) v += part[(size_t)r * nb + j];
  v = group_sum<16>(v);
  if (gl == 0) dgate[sorted_pair ? sorted_pair[r] : r] = v;
}

// The gate of each grouped row's pair, w_row[r] = tw[sorted_pair[r]].
__global__ __launch_bounds__(256) void row_gates_kernel(int rows, const int32_t* __restrict__ n_rows,
                                                        const int32_t* __restrict__ sorted_pair,
                                                        const float* __restrict__ tw, float* __restrict__ w_row) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r < rows && r < *n_rows) w_row[r] = tw[sorted_pair[r]];
}

// ---------------------------------------------------------------- router
// One group of G lanes per token (lane g holds experts g + G i); lane j < k
// holds slot j.  pi = softmax(L[t]); dw_j = dgate[t k + j] for kept slots,
// else 0; with renorm (S = sum_j pi_{id_j}): dsel_j = dw_j / S -
// (sum_j dw_j pi_{id_j}) / S^2, else dsel_j = dw_j; dpi_e = sum_{j: id_j = e}
// dsel_j + bal * count[e]; dL = pi (dpi - <dpi, pi>).
template <typename T, int G, int NV>
__global__ __launch_bounds__(256) void router_bwd_kernel(int Tn, int E, int Epad, int k, int renorm,
                                                         const float* __restrict__ L,
                                                         const int32_t* __restrict__ ids,
                                                         const int32_t* __restrict__ pair_pos,
                                                         const float* __restrict__ dgate,
                                                         const int32_t* __restrict__ count, float bal,
                                                         float* __restrict__ dL, T* __restrict__ dLc,
                                                         float* __restrict__ dgates_out) {
  const int gl = threadIdx.x & (G - 1);
  const int t = blockIdx.x * (256 / G) + threadIdx.x / G;
  if (t >= Tn) return;  // whole groups leave together
  const int base = (threadIdx.x & 63) & ~(G - 1);  // first lane of the group in the wave
  const float* row = L + (size_t)t * E;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = gl + G * i;
    v[i] = e < E ? row[e] : -INFINITY;
  }
  float m = v[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) m = fmaxf(m, v[i]);
  m = group_max<G>(m);
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i] = gl + G * i < E ? expf(v[i] - m) : 0.f;
    se += v[i];
  }
  const float inv = 1.f / group_sum<G>(se);
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] *= inv;  // pi

  int id = -1;
  float dw = 0.f, pj = 0.f;
  if (gl < k) {
    const size_t pidx = (size_t)t * k + gl;
    id = ids[pidx];
    dw = pair_pos[pidx] >= 0 ? dgate[pidx] : 0.f;
    pj = expf(row[id] - m) * inv;
    if (dgates_out) dgates_out[pidx] = dw;
  }
  float dsel = dw;
  if (renorm) {
    const float S = group_sum<G>(pj);
    const float A = group_sum<G>(dw * pj);
    dsel = dw / S - A / (S * S);
  }
  float dpi[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = gl + G * i;
    dpi[i] = (count != nullptr && e < E) ? bal * (float)count[e] : 0.f;
  }
  for (int j = 0; j < k; ++j) {
    const int idj = __shfl(id, base + j);
    const float dj = __shfl(dsel, base + j);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (gl + G * i == idj) dpi[i] += dj;
  }
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) dot += dpi[i] * v[i];
  dot = group_sum<G>(dot);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = gl + G * i;
    const float g = v[i] * (dpi[i] - dot);
    if (e < E && dL) dL[(size_t)t * E + e] = g;
    if (e < Epad) {
      if constexpr (sizeof(T) == 2)
        dLc[(size_t)t * Epad + e] = (T)(e < E ? f32_to_bf16_bits(g) : 0u);
      else
        dLc[(size_t)t * Epad + e] = e < E ? g : 0.f;
    }
  }
}

// ---------------------------------------------------------------- reductions
__global__ __launch_bounds__(256) void sum_slices_kernel(int S, int M, int N, int M1, const float* __restrict__ part,
                                                         float* __restrict__ C1, float* __restrict__ C2, int ldc) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t MN = (size_t)M * N;
  if (i >= MN) return;
  const int m = (int)(i / N), n = (int)(i % N);
  float acc = 0.f;
  for (int z = 0; z < S; ++z) acc += part[(size_t)z * MN + i];
  if (m < M1)
    C1[(size_t)m * ldc + n] = acc;
  else
    C2[(size_t)(m - M1) * ldc + n] = acc;
}

// Virtual groups of a chunked weight gradient (one workgroup; E <= 1024):
// c_e = max(1, ceil(n_e / CH)) chunks per group, numbered in group order by
// an inclusive scan; the j-th chunk of group e (j >= 1) takes partial slot
// v0_e - e + j - 1 (the chunks past the first of the groups before it).  The
// groups with more than one chunk are listed in group order (a second scan).
__global__ __launch_bounds__(1024) void tn_chunk_table_kernel(int E, const int32_t* __restrict__ offsets, int CH,
                                                              int Vmax, int Xmax, int4* __restrict__ chunks,
                                                              int4* __restrict__ ext) {
  __shared__ int scan[2][1024];
  const int e = threadIdx.x;
  int n = 0, c = 0;
  if (e < E) {
    n = offsets[e + 1] - offsets[e];
    c = n > CH ? (n + CH - 1) / CH : 1;
  }
  scan[0][e] = c;
  scan[1][e] = c > 1 ? 1 : 0;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = e >= off ? scan[0][e - off] : 0;
    const int w = e >= off ? scan[1][e - off] : 0;
    __syncthreads();
    scan[0][e] += v;
    scan[1][e] += w;
    __syncthreads();
  }
  const int v0 = scan[0][e] - c;
  const int V = scan[0][1023], X = scan[1][1023];
  if (e < E) {
    const int r0 = offsets[e];
    for (int j = 0; j < c && v0 + j < Vmax; ++j)
      chunks[v0 + j] = int4{e, r0 + j * CH, min(r0 + (j + 1) * CH, r0 + n), j == 0 ? -1 : v0 - e + j - 1};
    const int xi = scan[1][e] - 1;
    if (c > 1 && xi < Xmax) ext[xi] = int4{v0 - e, c - 1, e, 0};
  }
  for (int v = V + e; v < Vmax; v += 1024) chunks[v] = int4{-1, 0, 0, -1};
  for (int i = X + e; i < Xmax; i += 1024) ext[i] = int4{0, 0, -1, 0};
}

// Workgroup (x, i) adds listed group i's partial slots, in slot order.
__global__ __launch_bounds__(256) void tn_chunk_add_kernel(int M, int N, int M1, float* __restrict__ C1,
                                                           float* __restrict__ C2, int ldc, long long c_stride,
                                                           const float* __restrict__ part,
                                                           const int4* __restrict__ ext) {
  const int4 x = ext[blockIdx.y];
  const int e = x.z;
  if (e < 0 || x.y <= 0) return;
  const size_t MN = (size_t)M * N;
  for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; i < MN; i += (size_t)gridDim.x * 1024) {
    const int m = (int)(i / N), n = (int)(i - (size_t)m * N);
    float* const dst = m < M1 ? C1 + (size_t)e * c_stride + (size_t)m * ldc + n
                              : C2 + (size_t)e * c_stride + (size_t)(m - M1) * ldc + n;
    f32x4 v = *reinterpret_cast<const f32x4*>(dst);
    for (int j = 0; j < x.y; ++j) {
      const f32x4 p = *reinterpret_cast<const f32x4*>(part + (size_t)(x.x + j) * MN + i);
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] += p[t];
    }
    *reinterpret_cast<f32x4*>(dst) = v;
  }
}

constexpr int kColRows = 64;  // rows per partial of the column sum

__global__ __launch_bounds__(256) void colsum_part_kernel(int Tn, int E, const float* __restrict__ X,
                                                          float* __restrict__ part) {
  const int r0 = blockIdx.x * kColRows, r1 = min(Tn, r0 + kColRows);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    float acc = 0.f;
    for (int r = r0; r < r1; ++r) acc += X[(size_t)r * E + e];
    part[(size_t)blockIdx.x * E + e] = acc;
  }
}

__global__ __launch_bounds__(256) void colsum_final_kernel(int nb, int E, const float* __restrict__ part,
                                                           float* __restrict__ out) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  float acc = 0.f;
  for (int b = 0; b < nb; ++b) acc += part[(size_t)b * E + e];
  out[e] = acc;
}

// ---------------------------------------------------------------- dx
template <typename T>
__global__ __launch_bounds__(256) void dx_assemble_kernel(int Tn, int k, int d, const float* __restrict__ dXp,
                                                          const int32_t* __restrict__ pair_pos,
                                                          const float* __restrict__ dXs,
                                                          const float* __restrict__ dXr, T* __restrict__ dx) {
  const int d4 = d / 4;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)Tn * d4) return;
  const int t = (int)(i / d4), c = (int)(i % d4) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // slots four at a time: their positions, then the rows of the kept ones,
  // all in flight together, then the sums in ascending slot order
  for (int j0 = 0; j0 < k; j0 += 4) {
    int pos[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pos[u] = j0 + u < k ? pair_pos[(size_t)t * k + j0 + u] : -1;
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = pos[u] >= 0 ? *reinterpret_cast<const f32x4*>(dXp + (size_t)pos[u] * d + c) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (pos[u] >= 0) acc += v[u];
  }
  if (dXs) acc += *reinterpret_cast<const f32x4*>(dXs + (size_t)t * d + c);
  if (dXr) acc += *reinterpret_cast<const f32x4*>(dXr + (size_t)t * d + c);
  if constexpr (sizeof(T) == 2) {
    uint2 v;
    v.x = pack_bf16x2(acc[0], acc[1]);
    v.y = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<uint2*>(dx + (size_t)t * d + c) = v;
  } else {
    *reinterpret_cast<f32x4*>(dx + (size_t)t * d + c) = acc;
  }
}

template <typename T, int G, int NV>
hipError_t router_bwd_gn(int Tn, int E, int Epad, int k, int renorm, const float* L, const int32_t* ids,
                         const int32_t* pp, const float* dg, const int32_t* cnt, float bal, float* dL, void* dLc,
                         float* dgo, hipStream_t s) {
  constexpr int TPB = 256 / G;
  router_bwd_kernel<T, G, NV><<<(Tn + TPB - 1) / TPB, 256, 0, s>>>(Tn, E, Epad, k, renorm, L, ids, pp, dg, cnt, bal,
                                                                    dL, static_cast<T*>(dLc), dgo);
  return hipGetLastError();
}

template <typename T>
hipError_t router_bwd_t(int Tn, int E, int Epad, int k, int renorm, const float* L, const int32_t* ids,
                        const int32_t* pp, const float* dg, const int32_t* cnt, float bal, float* dL, void* dLc,
                        float* dgo, hipStream_t s) {
  // every lane of a group must also cover the padded columns up to Epad
  if (Epad <= 256 && k <= 16) {
    const int nv = (Epad + 15) / 16;
#define MOE_CALL(NVv) router_bwd_gn<T, 16, NVv>(Tn, E, Epad, k, renorm, L, ids, pp, dg, cnt, bal, dL, dLc, dgo, s)
    if (nv <= 1) return MOE_CALL(1);
    if (nv <= 2) return MOE_CALL(2);
    if (nv <= 4) return MOE_CALL(4);
    if (nv <= 8) return MOE_CALL(8);
    return MOE_CALL(16);
#undef MOE_CALL
  }
  const int nv = (Epad + 63) / 64;
#define MOE_CALL(NVv) router_bwd_gn<T, 64, NVv>(Tn, E, Epad, k, renorm, L, ids, pp, dg, cnt, bal, dL, dLc, dgo, s)
  if (nv <= 1) return MOE_CALL(1);
  if (nv <= 2) return MOE_CALL(2);
  if (nv <= 4) return MOE_CALL(4);
  if (nv <= 8) return MOE_CALL(8);
  return MOE_CALL(16);
#undef MOE_CALL
}

}  // namespace

hipError_t launch_bwd_nn(bool bf16, const bwdg::NnArgs& a, int BM, int grid_m, hipStream_t s) {
  if (grid_m <= 0) return hipSuccess;
  const dim3 grid(grid_m, (a.N + bwdg::kNnBN - 1) / bwdg::kNnBN);
  if (bf16) {
    if (BM == 128)
      bwdg::nn_kernel<uint16_t, 128><<<grid, bwdg::NTH, 0, s>>>(a);
    else
      bwdg::nn_kernel<uint16_t, 64><<<grid, bwdg::NTH, 0, s>>>(a);
  } else {
    bwdg::nn_kernel<float, 64><<<grid, bwdg::NTH, 0, s>>>(a);
  }
  return hipGetLastError();
}

bool bwd_nn_wide_ok(const bwdg::NnArgs& a) {
  return a.N % bwdw::BT == 0 && a.K % (2 * bwdw::KB) == 0 && a.K1 % bwdw::KB == 0 && a.K_valid > 0;
}

hipError_t launch_bwd_nn_wide(const bwdg::NnArgs& a, hipStream_t s) {
  if (!bwd_nn_wide_ok(a)) return hipErrorInvalidValue;
  const long long mt = a.tile_tab ? ffn_max_mtiles(a.groups, a.rows, bwdw::BT) : (a.rows + bwdw::BT - 1) / bwdw::BT;
  const long long g = (mt * (a.N / bwdw::BT) + 7) / 8 * 8;
  if (g == 0) return hipSuccess;
  if (g > 0x7FFFFFFFll) return hipErrorInvalidValue;
  bwdw::wide_nn_kernel<<<dim3((unsigned)g), 512, 0, s>>>(a);
  return hipGetLastError();
}

bool bwd_tn_wide_ok(const bwdg::TnArgs& a) {
  return a.M % bwdw::BT == 0 && a.N % bwdw::BT == 0 && (a.M1 % bwdw::BT == 0 || a.M1 >= a.M);
}

hipError_t launch_bwd_tn_wide(const bwdg::TnArgs& a, int grid_z, hipStream_t s) {
  if (!bwd_tn_wide_ok(a)) return hipErrorInvalidValue;
  if (grid_z <= 0) return hipSuccess;
  const long long total = (long long)grid_z * (a.M / bwdw::BT) * (a.N / bwdw::BT);
  const long long g = (total + 7) / 8 * 8;
  if (g > 0x7FFFFFFFll) return hipErrorInvalidValue;
  bwdw::wide_tn_kernel<<<dim3((unsigned)g), 512, 0, s>>>(a, grid_z);
  return hipGetLastError();
}

hipError_t launch_bwd_tn(bool bf16, const bwdg::TnArgs& a, int grid_z, hipStream_t s) {
  if (grid_z <= 0) return hipSuccess;
  const int nt = (a.N + bwdg::kTnTile - 1) / bwdg::kTnTile;
  const dim3 grid(a.mtiles * nt, grid_z);
  if (bf16)
    bwdg::tn_kernel<uint16_t><<<grid, bwdg::NTH, 0, s>>>(a);
  else
    bwdg::tn_kernel<float><<<grid, bwdg::NTH, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_row_gates(int rows, const int32_t* n_rows, const int32_t* sorted_pair, const float* tw,
                            float* w_row, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  row_gates_kernel<<<dim3((unsigned)((rows + 255) / 256)), 256, 0, s>>>(rows, n_rows, sorted_pair, tw, w_row);
  return hipGetLastError();
}

hipError_t launch_gate_part_sum(int rows, int h, const int32_t* n_rows, const float* part,
                                const int32_t* sorted_pair, float* dgate, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (h % 64) return hipErrorInvalidValue;
  gate_part_sum_kernel<<<dim3((unsigned)((rows + 15) / 16)), 256, 0, s>>>(rows, h / 64, n_rows, part, sorted_pair,
                                                                         dgate);
  return hipGetLastError();
}

hipError_t launch_gate_bwd(bool bf16, int act, int rows, int h, const int32_t* n_rows, const float* G,
                           const float* U, const float* dZ, const int32_t* sorted_pair, const float* tw, void* dGU,
                           void* ZW, float* dgate, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int grid = (rows + 3) / 4;
#define MOE_CALL(T, A)                                                                                           \
  gate_bwd_kernel<T, A><<<grid, 256, 0, s>>>(rows, h, n_rows, G, U, dZ, sorted_pair, tw, static_cast<T*>(dGU), \
                                             static_cast<T*>(ZW), dgate)
  if (bf16) {
    if (act == 0) MOE_CALL(uint16_t, 0);
    else MOE_CALL(uint16_t, 1);
  } else {
    if (act == 0) MOE_CALL(float, 0);
    else MOE_CALL(float, 1);
  }
#undef MOE_CALL
  return hipGetLastError();
}

hipError_t launch_router_bwd(bool bf16, int Tn, int E, int Epad, int k, int renorm, const float* L,
                             const int32_t* ids, const int32_t* pair_pos, const float* dgate, const int32_t* count,
                             float bal_scale, float* dL, void* dLc, float* dgates_out, hipStream_t s) {
  if (Tn <= 0) return hipSuccess;
  return bf16 ? router_bwd_t<uint16_t>(Tn, E, Epad, k, renorm, L, ids, pair_pos, dgate, count, bal_scale, dL, dLc,
                                       dgates_out, s)
              : router_bwd_t<float>(Tn, E, Epad, k, renorm, L, ids, pair_pos, dgate, count, bal_scale, dL, dLc,
                                    dgates_out, s);
}

hipError_t launch_sum_slices(int S, int M, int N, int M1, const float* part, float* C1, float* C2, int ldc,
                             hipStream_t s) {
  const size_t n = (size_t)M * N;
  if (n == 0) return hipSuccess;
  sum_slices_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(S, M, N, M1, part, C1, C2, ldc);
  return hipGetLastError();
}

int tn_chunk_rows(int rows_max, int group_max, int M, int N) {
  // an even share of a launch's rows x tiles over the 256 CUs of an MI355X
  const long long tiles = (long long)(M / bwdw::BT) * (N / bwdw::BT);
  long long ch = ((long long)rows_max * tiles / 256 + 255) / 256 * 256;
  if (ch < 2048) ch = 2048;
  if (rows_max <= ch || group_max <= ch) return 0;
  return (int)ch;
}

hipError_t launch_tn_chunk_table(int E, const int32_t* offsets, int CH, int Vmax, int Xmax, int4* chunks,
                                 int4* ext, hipStream_t s) {
  if (E <= 0 || E > 1024 || CH <= 0 || Vmax < E || Xmax < 1) return hipErrorInvalidValue;
  tn_chunk_table_kernel<<<1, 1024, 0, s>>>(E, offsets, CH, Vmax, Xmax, chunks, ext);
  return hipGetLastError();
}

hipError_t launch_tn_chunk_add(int Xmax, int M, int N, int M1, float* C1, float* C2, int ldc, long long c_stride,
                               const float* part, const int4* ext, hipStream_t s) {
  if (Xmax <= 0 || (size_t)M * N == 0) return hipSuccess;
  if (N % 4 || ldc % 4) return hipErrorInvalidValue;
  const size_t blocks = std::min<size_t>(((size_t)M * N + 1023) / 1024, 256);
  tn_chunk_add_kernel<<<dim3((unsigned)blocks, (unsigned)Xmax), 256, 0, s>>>(M, N, M1, C1, C2, ldc, c_stride,
                                                                            part, ext);
  return hipGetLastError();
}

size_t colsum_ws_floats(int Tn, int E) { return (size_t)std::max(1, (Tn + kColRows - 1) / kColRows) * E; }

hipError_t launch_colsum(int Tn, int E, const float* X, float* part, float* out, hipStream_t s) {
  const int nb = (Tn + kColRows - 1) / kColRows;
  if (nb > 0) {
    colsum_part_kernel<<<nb, 256, 0, s>>>(Tn, E, X, part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  colsum_final_kernel<<<(E + 255) / 256, 256, 0, s>>>(nb, E, part, out);
  return hipGetLastError();
}

hipError_t launch_dx_assemble(bool bf16, int Tn, int k, int d, const float* dXp, const int32_t* pair_pos,
                              const float* dXs, const float* dXr, void* dx, hipStream_t s) {
  const size_t n = (size_t)Tn * (d / 4);
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (bf16)
    dx_assemble_kernel<uint16_t><<<grid, 256, 0, s>>>(Tn, k, d, dXp, pair_pos, dXs, dXr, static_cast<uint16_t*>(dx));
  else
    dx_assemble_kernel<float><<<grid, 256, 0, s>>>(Tn, k, d, dXp, pair_pos, dXs, dXr, static_cast<float*>(dx));
  return hipGetLastError();
}

}  // namespace moe
