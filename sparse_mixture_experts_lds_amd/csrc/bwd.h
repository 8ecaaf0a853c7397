// Backward pass of the layer: argument blocks of its grouped GEMMs and the
// launchers of its kernels (implemented in bwd.hip).
#pragma once

#include "moe_internal.h"

namespace moe {
namespace bwdg {

// Data-gradient GEMM: C[r, n] = sum_k A[row(r), k] * B_g[k, n].
struct NnArgs {
  const void* A;  // [*, lda]; row of grouped row r: a_index ? a_index[r] / a_div : r
  int lda;
  const int32_t* a_index;
  int a_div;
  const void* B1;  // [groups][K1][ldb]
  const void* B2;  // [groups][K - K1][ldb] or NULL (K1 == K)
  int K1, ldb;
  long long b_stride;  // elements between groups' matrices
  int K_valid;         // rows of B that exist (k >= K_valid read as zero)
  float* C;            // [rows][ldc] fp32
  int ldc;
  const int32_t* mtile_start;  // grouped rows: m-tile prefix [groups+1] and table, else NULL
  const int4* tile_tab;
  int groups;
  int rows;  // without a tile table: one group of `rows` rows
  int N, K;  // K a multiple of the k-block (32 bf16, 16 fp32), N % 8 == 0
};


// Weight-gradient GEMM: C_g[m, n] = sum_{r in group g} A[row_a(r), m] * B[row_b(r), n].
struct TnArgs {
  const void* A;  // [*, lda]; contraction row r: a_index ? a_index[r] / a_div : r
  int lda;
  const int32_t* a_index;
  int a_div;
  const void* B;  // [*, ldb]
  int ldb;
  const int32_t* b_index;
  int b_div;
  const int32_t* offsets;  // group g contracts rows [offsets[g], offsets[g+1]); NULL: slices of `rows`
  int rows, slice;         // without offsets: blockIdx.y = z takes rows [z*slice, min(rows, (z+1)*slice))
  float* C1;               // rows m < M1 of C_g (group or slice z): C1 + z * c_stride + m * ldc
  float* C2;               // rows m >= M1: C2 + z * c_stride + (m - M1) * ldc
  int M1, ldc;
  long long c_stride;
  int M, N;  // M % 8 == 0, N % 8 == 0
  int mtiles;
  // (wide kernel only) virtual groups: blockIdx z takes chunks[z] = {group g
  // (< 0: none), first row, end row, slot}; slot < 0 writes C_g as above,
  // else the [M][N] block part + slot * M * N
  const int4* chunks;
  float* part;
};


constexpr int kTnTile = 128;  // tn tiles are 128 x 128
constexpr int kNnBN = 128;    // nn tiles are BM x 128

}  // namespace bwdg

// grid_m: m-tiles to launch (table size, or ceil(rows / BM) without a table)
hipError_t launch_bwd_nn(bool bf16, const bwdg::NnArgs& a, int BM, int grid_m, hipStream_t s);
// grid_z: groups (with offsets) or row slices
hipError_t launch_bwd_tn(bool bf16, const bwdg::TnArgs& a, int grid_z, hipStream_t s);
// The same two GEMMs on 256 x 256 tiles (bf16 operands only; ok tells whether
// the shapes fit: N a multiple of 256, K of 64 and K1 of 32 for nn; M, N and
// M1 multiples of 256 for tn).  The nn tile table, if any, is for 256-row tiles.
bool bwd_nn_wide_ok(const bwdg::NnArgs& a);
hipError_t launch_bwd_nn_wide(const bwdg::NnArgs& a, hipStream_t s);
bool bwd_tn_wide_ok(const bwdg::TnArgs& a);
hipError_t launch_bwd_tn_wide(const bwdg::TnArgs& a, int grid_z, hipStream_t s);
// Per grouped row: dgate (pair gradient), dGU = [dg | du], ZW = w * z.
hipError_t launch_gate_bwd(bool bf16, int act, int rows, int h, const int32_t* n_rows, const float* G,
                           const float* U, const float* dZ, const int32_t* sorted_pair, const float* tw,
                           void* dGU, void* ZW, float* dgate, hipStream_t s);
// w_row[r] = tw[sorted_pair[r]] for grouped rows r < *n_rows.
hipError_t launch_row_gates(int rows, const int32_t* n_rows, const int32_t* sorted_pair, const float* tw,
                            float* w_row, hipStream_t s);
// dgate[pair of r] = the sum, in a fixed order, of part[r][0 .. h/64) (the
// partials of a gate/up launch with the gate backward in its epilogue).
hipError_t launch_gate_part_sum(int rows, int h, const int32_t* n_rows, const float* part,
                                const int32_t* sorted_pair, float* dgate, hipStream_t s);
// Softmax / gate / balance backward per token: dL (fp32 [T, E], may be NULL),
// dLc (compute dtype, [T, Epad], zero past E) and the pair gradients of the
// gates (fp32 [T, k], 0 for pairs not kept; may be NULL).
hipError_t launch_router_bwd(bool bf16, int T, int E, int Epad, int k, int renorm, const float* L,
                             const int32_t* ids, const int32_t* pair_pos, const float* dgate,
                             const int32_t* count, float bal_scale, float* dL, void* dLc, float* dgates_out,
                             hipStream_t s);
// Rows per chunk of a grouped weight gradient on the wide kernel (M x N per
// group, at most rows_max rows in all, at most group_max in one group): a
// group with more rows is cut into chunks of at most that many, so that no
// tile runs much longer than an even share of the launch; 0 when no group
// can need it.
int tn_chunk_rows(int rows_max, int group_max, int M, int N);
// Virtual groups for chunk size CH (tn_chunk_rows): chunks[v] = {e, first
// row, end row, slot} for every chunk of every group e < E (slot -1 for a
// group's first chunk, else its partial slot), {-1, 0, 0, -1} up to Vmax;
// ext[i] = {first slot, number of slots, e, 0} for the i-th group with more
// than one chunk, {0, 0, -1, 0} up to Xmax.  Vmax >= E + rows / CH and
// Xmax >= rows / CH.
hipError_t launch_tn_chunk_table(int E, const int32_t* offsets, int CH, int Vmax, int Xmax, int4* chunks,
                                 int4* ext, hipStream_t s);
// C_e += the partial slots of each listed group e, in slot order (layout as
// TnArgs C1, C2, M1).
hipError_t launch_tn_chunk_add(int Xmax, int M, int N, int M1, float* C1, float* C2, int ldc, long long c_stride,
                               const float* part, const int4* ext, hipStream_t s);
// C = sum over S slices of part[z][M][N] in slice order (rows m >= M1 to C2).
hipError_t launch_sum_slices(int S, int M, int N, int M1, const float* part, float* C1, float* C2, int ldc,
                             hipStream_t s);
// out[e] = sum_t X[t, e] in a fixed order; part holds colsum_ws_floats(T, E) floats.
size_t colsum_ws_floats(int T, int E);
hipError_t launch_colsum(int T, int E, const float* X, float* part, float* out, hipStream_t s);
// dx[t] = sum_{kept slots} dXp[pair_pos] + dXs[t] + dXr[t] (the last two may be NULL).
hipError_t launch_dx_assemble(bool bf16, int T, int k, int d, const float* dXp, const int32_t* pair_pos,
                              const float* dXs, const float* dXr, void* dx, hipStream_t s);

}  // namespace moe
