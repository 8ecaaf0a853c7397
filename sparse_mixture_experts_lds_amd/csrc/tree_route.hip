// Hierarchical routing down an expert tree (kieve-moe "Features": fractal
// tiling routing, self-similar routing over a branch^levels expert tree, the
// cheap router of very large expert pools).
//
// Operation (the page gives no formula; this is the reading the library
// implements).  The E experts are the leaves of a tree with B children per
// node and L levels; leaf e is reached by the base-B digits of e, most
// significant first, and depth l holds n_l = ceil(E / B^(L-l)) nodes (those
// with a leaf below them).  Every internal node scores its existing children
// with its own gate rows (row first_l + j for child j of depth l+1, first_l =
// B (n_0 + ... + n_{l-1})) and takes the softmax over them; a leaf's
// probability is the product along its path.  Selection is a beam search of
// width k: at each depth the kept nodes' children are ranked by path
// log-probability (ties to the lower node id) and the best min(k, n_{l+1})
// are kept.  The k leaves kept last are the experts; a gate is the path
// probability, renormalised over the k on request.
//
// GPU design, per depth (L rounds of two to four launches):
//   * dense depths (where the beam holds at least a quarter of the depth's
//     nodes, always at the root): the scores of every child of the depth at
//     once, x times the depth's block of gate rows, on the scores kernel's
//     dense tiles (64 tokens by up to 64 children; for many tokens and bf16
//     the grouped-GEMM kernel's 128 x 128 tiles): x is read once per column
//     block, and the unneeded columns cost less than re-reading x for every
//     kept node;
//   * grouped depths (wide trees, beams that touch few nodes): the (token,
//     beam slot) pairs are grouped by node with the LDS histogram / prefix
//     sum / stable scatter of the expert grouping, and the scores kernel runs
//     on 64-pair tiles of one node (the tile's gathered activation rows by the
//     node's child rows);
//   * the scores kernel: MFMA 16x16x32 (bf16) or 16x16x4 (fp32); the four
//     waves of a tile share its rows and split its k-range (interleaved
//     64-element pieces, 128 bytes of a bf16 row), so every activation and
//     gate byte is loaded once per tile, and their partial scores meet in
//     LDS; with few tiles the width is also split over gridDim.y;
//   * selection: one wave per token sums the candidates' partial scores into
//     LDS, forms each kept node's log-normaliser with a group of lanes per
//     node, and picks the best of the k*B candidates by k rounds of a DPP
//     arg-max (higher path log-probability, then the lower node id).
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTreeBM = 64;           // pair rows per grouped tile (4 A fragments)
constexpr int kTreeMaxSplit = 16;     // width slices of the grouped scores at most
constexpr int kTreeSelTok = 4;        // tokens (waves) per selection workgroup
constexpr int kTreeDenseMaxCols = 4096;  // children of a dense depth at most

struct TreeScores {
  const void* x;               // [T, d] activations
  const void* w;               // gate table [rows, d]
  float* out;                  // [nsplit][rows_p, B]: pair p's child c at p * B + c
  const int32_t* sorted_pair;  // grouped row -> pair p = t * width + slot (NULL in dense mode: row = token)
  const int32_t* n_tiles;      // device tile count (NULL in dense mode)
  const int4* tile_tab;        // per tile {node, first row, rows, 0} (NULL in dense mode: 64-token tiles
                               // by column blocks of the depth's children)
  int d, B, width;             // width: pairs per token at this depth
  int row_base;                // first gate row of this depth's children
  int n_next;                  // nodes at the next depth
  int rows_p;                  // pairs at this depth (T * width); tokens in dense mode
  int kp_per_split;            // 64-element k-pieces per width slice
  int ncols;                   // dense mode (no tile table): children of the depth, scores [rows_p, ncols]
  int ncb;                     // dense mode: column blocks of 16 * NB children
};

// Grouped scores.  Lane (lrow, q) of every wave holds row lrow of each of the
// four 16-row A fragments and column lrow of each 16-column B fragment; of a
// 64-element k-piece it holds elements 16q .. 16q+15 (32 contiguous bytes of
// bf16: two MFMA k-steps of 8).  Both operands use the same element map, so
// the products pair up; wave w takes the pieces w, w+4, ... of the slice.
template <bool BF16, int NB>
__global__ __launch_bounds__(256) void tree_scores_kernel(TreeScores a) {
  constexpr int NC = 16 * NB;
  __shared__ float part[4][kTreeBM][NC + 1];
  int node = 0, first, nrows, col0 = 0;
  if (a.tile_tab) {
    if ((int)blockIdx.x >= *a.n_tiles) return;  // whole workgroup, before any barrier
    const int4 tt = a.tile_tab[blockIdx.x];
    node = tt.x;
    first = tt.y;
    nrows = tt.z;
  } else {
    const int mt = blockIdx.x / a.ncb;
    col0 = (blockIdx.x - mt * a.ncb) * NC;
    first = mt * kTreeBM;
    nrows = min(kTreeBM, a.rows_p - first);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lrow = lane & 15, q = lane >> 4;
  // A rows (rows past the tile's end re-read its first row; MFMA rows are
  // independent and those are not stored)
  size_t xoff[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int rl = 16 * m + lrow;
    const int r = first + (rl < nrows ? rl : 0);
    const int p = a.sorted_pair ? a.sorted_pair[r] : r;
    xoff[m] = (size_t)(p / a.width) * a.d + 16 * q;
  }
  // B columns: child 16 f + lrow of the node (dense mode: child col0 + 16 f +
  // lrow of the depth); one past the end or missing reads the first column's
  // row (which exists) and is not stored
  const int child0 = a.tile_tab ? node * a.B : col0;
  const int cend = a.tile_tab ? min(a.B, a.n_next - child0) : a.ncols - col0;
  size_t woff[NB];
#pragma unroll
  for (int f = 0; f < NB; ++f) {
    const int c = 16 * f + lrow;
    woff[f] = (size_t)(a.row_base + child0 + (c < cend ? c : 0)) * a.d + 16 * q;
  }
  const int kp0 = blockIdx.y * a.kp_per_split;
  const int kp1 = min(a.d / 64, kp0 + a.kp_per_split);
  f32x4 acc[4][NB];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int f = 0; f < NB; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (BF16) {
    const uint16_t* X = static_cast<const uint16_t*>(a.x);
    const uint16_t* W = static_cast<const uint16_t*>(a.w);
    constexpr int KC = NB <= 2 ? 2 : 1;  // pieces whose loads are issued before their MFMAs
    for (int kp = kp0 + wave; kp < kp1; kp += 4 * KC) {
      const int nk = min(KC, (kp1 - kp + 3) / 4);
      u32x4 av[KC][4][2], bv[KC][NB][2];
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const size_t kk = (size_t)64 * (kp + 4 * min(c, nk - 1));  // in-bounds re-read past the end; unused
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int m = 0; m < 4; ++m) av[c][m][h] = *reinterpret_cast<const u32x4*>(X + xoff[m] + kk + 8 * h);
#pragma unroll
          for (int f = 0; f < NB; ++f) bv[c][f][h] = *reinterpret_cast<const u32x4*>(W + woff[f] + kk + 8 * h);
        }
      }
#pragma unroll
      for (int c = 0; c < KC; ++c)
        if (c < nk) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
              for (int f = 0; f < NB; ++f)
                acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, av[c][m][h]), __builtin_bit_cast(bf16x8, bv[c][f][h]), acc[m][f], 0,
                    0, 0);
        }
    }
  } else {
    // fp32: of a 64-element piece the lane holds elements 16q .. 16q+15; the
    // 16x16x4 MFMA number j takes element 16q + j from every lane
    const float* X = static_cast<const float*>(a.x);
    const float* W = static_cast<const float*>(a.w);
    for (int kp = kp0 + wave; kp < kp1; kp += 4) {
      const size_t kk = (size_t)64 * kp;
      u32x4 av[4][4], bv[NB][4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
#pragma unroll
        for (int m = 0; m < 4; ++m) av[m][h] = *reinterpret_cast<const u32x4*>(X + xoff[m] + kk + 4 * h);
#pragma unroll
        for (int f = 0; f < NB; ++f) bv[f][h] = *reinterpret_cast<const u32x4*>(W + woff[f] + kk + 4 * h);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int f = 0; f < NB; ++f)
            acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av[m][j >> 2][j & 3]),
                                                             __uint_as_float(bv[f][j >> 2][j & 3]), acc[m][f], 0, 0,
                                                             0);
    }
  }
  // the four waves' partial scores meet in LDS (D layout: lane (lrow, q)
  // holds column lrow of rows 4q .. 4q+3 of each fragment)
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int f = 0; f < NB; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wave][16 * m + 4 * q + i][16 * f + lrow] = acc[m][f][i];
  __syncthreads();
  // wave w sums rows 16w .. 16w+15 in wave order and stores them
  const int row = 16 * wave + lrow;
  if (row < nrows) {
    const size_t pr = a.sorted_pair ? (size_t)a.sorted_pair[first + row] : (size_t)(first + row);
    const int ld = a.tile_tab ? a.B : a.ncols;  // scores row length
    const int cn = a.tile_tab ? a.B : a.ncols - col0;
    float* out = a.out + (size_t)blockIdx.y * a.rows_p * ld + pr * ld + col0;
#pragma unroll
    for (int j = 0; j < 4 * NB; ++j) {
      const int c = q + 4 * j;
      if (c < cn) out[c] = ((part[0][row][c] + part[1][row][c]) + part[2][row][c]) + part[3][row][c];
    }
  }
}

struct TreeSelect {
  const float* scores;    // grouped: [nsplit][T * width, B]; dense: [nsplit][T, dense_N] (column = child id)
  int dense_N;            // 0 for the grouped layout
  const int32_t* beam;    // [T, width] node ids at this depth (NULL: the root)
  const float* beam_lp;   // [T, width] their path log-probabilities (NULL: 0)
  int32_t* next;          // [T, keep] kept nodes of the next depth (the experts at the last)
  float* next_lp;         // [T, keep] their path log-probabilities (NULL at the last depth)
  float* tw;              // [T, keep] gates (last depth only, else NULL)
  int T, B, width, n_next, keep, nsplit, renorm;
};

template <int NJ>
__global__ __launch_bounds__(64 * kTreeSelTok) void tree_select_kernel(TreeSelect a) {
  __shared__ float zs[kTreeSelTok][64 * NJ];  // the token's candidate scores, slot-major
  __shared__ float base_s[kTreeSelTok][kMaxK];
  __shared__ int node_s[kTreeSelTok][kMaxK];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t_raw = blockIdx.x * kTreeSelTok + w;
  const bool live = t_raw < a.T;  // a wave past the end works on the last token and writes nothing
  const int t = live ? t_raw : a.T - 1;
  const int ncand = a.width * a.B;
  // the beam slot's node and path log-probability (lane b < width: slot b)
  const float lp_lane = (a.beam_lp && lane < a.width) ? a.beam_lp[(size_t)t * a.width + lane] : 0.f;
  if (lane < a.width) node_s[w][lane] = a.beam ? a.beam[(size_t)t * a.width + lane] : 0;
  __syncthreads();
  // 1. candidate i = b B + c (child c of beam slot b): partial scores summed in
  //    slice order, four slices' loads in flight at a time
  const size_t split_stride = a.dense_N ? (size_t)a.T * a.dense_N : (size_t)a.T * ncand;
  const float* src[NJ];
  float acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = min(lane + 64 * j, ncand - 1);  // lanes past the end re-read the last candidate; unused
    const int b = i / a.B;
    src[j] = a.dense_N ? a.scores + (size_t)t * a.dense_N + node_s[w][b] * a.B + (i - b * a.B)
                       : a.scores + (size_t)t * ncand + i;
    acc[j] = 0.f;
  }
  for (int s0 = 0; s0 < a.nsplit; s0 += 4) {
    float part[4][NJ];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t off = (size_t)min(s0 + u, a.nsplit - 1) * split_stride;  // unconditional loads
#pragma unroll
      for (int j = 0; j < NJ; ++j) part[u][j] = src[j][off];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < NJ; ++j) part[u][j] = s0 + u < a.nsplit ? part[u][j] : 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] += part[u][j];
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (lane + 64 * j < ncand) zs[w][lane + 64 * j] = acc[j];
  __syncthreads();
  // 2. G lanes per beam slot (G a power of two, G * width <= 64): each kept
  //    node's log-normaliser over its existing children
  int G = 64;
  while (G * a.width > 64) G >>= 1;
  {
    const int b = lane / G, sub = lane & (G - 1);
    const int nc = b < a.width ? min(a.B, a.n_next - node_s[w][b] * a.B) : 0;
    const float* zb = &zs[w][(b < a.width ? b : 0) * a.B];
    float m = -INFINITY;
#pragma unroll 8
    for (int c = sub; c < nc; c += G) m = fmaxf(m, zb[c]);
    for (int o = 1; o < G; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    float sum = 0.f;
#pragma unroll 8
    for (int c = sub; c < nc; c += G) sum += __expf(zb[c] - m);
    for (int o = 1; o < G; o <<= 1) sum += __shfl_xor(sum, o);
    const float lp = __shfl(lp_lane, b < a.width ? b : 0);
    if (sub == 0 && b < a.width) base_s[w][b] = lp - (m + __logf(sum));
  }
  __syncthreads();
  // 3. path log-probabilities of the existing children
  float v[NJ];
  int id[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = lane + 64 * j;
    v[j] = -INFINITY;
    id[j] = 0x7fffffff;
    if (i < ncand) {
      const int b = i / a.B;
      const int child = node_s[w][b] * a.B + (i - b * a.B);
      if (child < a.n_next) {
        v[j] = base_s[w][b] + zs[w][i];
        id[j] = child;
      }
    }
  }
  // 4. keep rounds of a wave arg-max; lane r keeps the r-th pick
  uint32_t taken = 0;
  float my_v = -INFINITY;
  int my_id = 0;
  for (int r = 0; r < a.keep; ++r) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (!((taken >> j) & 1u) && (v[j] > bv || (v[j] == bv && id[j] < be))) {
        bv = v[j];
        be = id[j];
      }
    group_argmax<64>(bv, be);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (id[j] == be) taken |= 1u << j;
    if (lane == r) {
      my_v = bv;
      my_id = be;
    }
  }
  const size_t o = (size_t)t * a.keep + lane;
  if (!a.tw) {
    if (live && lane < a.keep) {
      a.next[o] = my_id;
      a.next_lp[o] = my_v;
    }
    return;
  }
  float g = lane < a.keep ? __expf(my_v) : 0.f;
  if (a.renorm) g = g / wave_sum(g);
  if (live && lane < a.keep) {
    a.next[o] = my_id;
    a.tw[o] = g;
  }
}

template <bool BF16>
hipError_t launch_scores(const TreeScores& a, int NB, int grid_x, int nsplit, hipStream_t s) {
  const dim3 grid((unsigned)grid_x, (unsigned)nsplit), block(256);
#define MOE_CASE(NBv)                                        \
  if (NB == NBv) {                                           \
    tree_scores_kernel<BF16, NBv><<<grid, block, 0, s>>>(a); \
    return hipGetLastError();                                \
  }
  MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4)
#undef MOE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_tree_select(const TreeSelect& a, hipStream_t s) {
  const int nj = (a.width * a.B + 63) / 64;
  const dim3 grid((unsigned)((a.T + kTreeSelTok - 1) / kTreeSelTok)), block(64 * kTreeSelTok);
#define MOE_CASE(NJv)                                  \
  if (nj <= NJv) {                                     \
    tree_select_kernel<NJv><<<grid, block, 0, s>>>(a); \
    return hipGetLastError();                          \
  }
  MOE_CASE(1) MOE_CASE(2) MOE_CASE(4) MOE_CASE(8) MOE_CASE(16)
#undef MOE_CASE
  return hipErrorInvalidValue;
}

size_t al(size_t v) { return (v + 255) & ~(size_t)255; }

int grouped_splits(int tiles, int d) {
  // few tiles: split the width until tiles x slices reach ~512 workgroups,
  // keeping at least two 64-element pieces per wave (8 per slice)
  const int kp = d / 64;
  int ns = 1;
  while (ns < kTreeMaxSplit && (long long)tiles * ns < 512 && kp / (2 * ns) >= 8) ns *= 2;
  return ns;
}

enum DepthKind { kDense = 0, kDenseGemm = 1, kGrouped = 2 };

struct TreePlan {
  int kind[kTreeMaxLevels];
  int width[kTreeMaxLevels], keep[kTreeMaxLevels], tiles[kTreeMaxLevels], nsplit[kTreeMaxLevels];
  int nb[kTreeMaxLevels];   // 16-column fragments per scores tile
  int n_perm_max;           // largest node count grouped (0: no grouping)
  int tiles_max;            // largest grouped tile count
  long long score_floats;
};

// The scores of one depth:
//   dense       where the beam holds at least a quarter of the depth's nodes
//               (always at the root): every child of the depth at once, x
//               times the depth's block of gate rows, on the scores kernel's
//               dense tiles (64 tokens by 64 children, the width split over
//               workgroups when tiles are few): x is read once per column
//               block, and the unneeded columns cost less than re-reading x
//               for every kept node;
//   dense GEMM  the same product for many tokens (bf16, 128-multiple widths)
//               on the grouped-GEMM kernel's 128 x 128 tiles;
//   grouped     otherwise: the pairs grouped by node, then the scores kernel
//               on 64-pair tiles of one node.
TreePlan plan_tree(int T, int d, int k, int B, int L, bool bf16, const TreeShape& sh) {
  TreePlan p{};
  for (int l = 0; l < L; ++l) {
    p.width[l] = l == 0 ? 1 : std::min(k, sh.n[l]);
    p.keep[l] = std::min(k, sh.n[l + 1]);
    const long long N = (long long)sh.n[l] * B;  // children of the depth's nodes (gate rows of its block)
    const int P = T * p.width[l];
    const bool wide_beam = 4LL * p.width[l] >= sh.n[l] && N <= kTreeDenseMaxCols;
    if (l == 0 || wide_beam) {
      p.kind[l] = (bf16 && T >= 2048 && N % 128 == 0 && (unsigned long long)T * d * 2 <= 0xFFFFFFFFull)
                      ? kDenseGemm : kDense;
    } else {
      p.kind[l] = kGrouped;
    }
    if (p.kind[l] == kDenseGemm) {
      p.nsplit[l] = 1;
      p.score_floats = std::max(p.score_floats, (long long)T * N);
    } else if (p.kind[l] == kDense) {
      p.nb[l] = N >= 64 ? 4 : (int)((N + 15) / 16);
      p.tiles[l] = (T + kTreeBM - 1) / kTreeBM * (int)((N + 16 * p.nb[l] - 1) / (16 * p.nb[l]));
      p.nsplit[l] = grouped_splits(p.tiles[l], d);
      p.score_floats = std::max(p.score_floats, (long long)T * N * p.nsplit[l]);
    } else {
      p.nb[l] = (B + 15) / 16;
      p.tiles[l] = ffn_max_mtiles(sh.n[l], P, kTreeBM);
      p.nsplit[l] = grouped_splits((P + kTreeBM - 1) / kTreeBM, d);
      p.n_perm_max = std::max(p.n_perm_max, sh.n[l]);
      p.tiles_max = std::max(p.tiles_max, p.tiles[l]);
      p.score_floats = std::max(p.score_floats, (long long)P * B * p.nsplit[l]);
    }
  }
  return p;
}

}  // namespace

bool tree_shape(int E, int B, int L, TreeShape* sh) {
  if (B < 2 || B > kTreeMaxBranch || L < 1 || L > kTreeMaxLevels || E < 1) return false;
  long long pw = 1;  // B^(L - l), no longer multiplied once it exceeds E
  long long pows[kTreeMaxLevels + 1];
  for (int l = L; l >= 0; --l) {
    pows[l] = pw;
    pw = pw > E ? pw : pw * B;
  }
  if (pows[0] < E) return false;  // E > B^L
  long long first = 0;
  for (int l = 0; l <= L; ++l) {
    sh->n[l] = (int)((E + pows[l] - 1) / pows[l]);
    sh->first[l] = first;
    first += (long long)B * sh->n[l];
  }
  sh->rows = sh->first[L];
  return true;
}

size_t tree_ws_bytes(int T, int d, int k, int B, int L, bool bf16, const TreeShape& sh) {
  const TreePlan p = plan_tree(T, d, k, B, L, bf16, sh);
  const size_t tk = (size_t)T * k * 4;
  size_t b = al((size_t)p.score_floats * 4) + 4 * al(tk);  // scores, beam nodes x2, beam lp x2
  if (p.n_perm_max > 0)
    b += 2 * al((size_t)(kMaxE + 1) * 4) + al((size_t)p.tiles_max * sizeof(int4)) + 2 * al(tk) +
         al(permute_ws_bytes(T * k, p.n_perm_max));
  return b;
}

hipError_t launch_route_tree(int T, int d, int E, int k, int B, int L, bool bf16, const void* x, const void* w,
                             int renorm, int32_t* ids, float* tw, void* ws, hipStream_t s) {
  TreeShape sh;
  if (!tree_shape(E, B, L, &sh) || d % 64) return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  const TreePlan p = plan_tree(T, d, k, B, L, bf16, sh);
  unsigned char* base = static_cast<unsigned char*>(ws);
  size_t used = 0;
  auto take = [&](size_t bytes) {
    void* r = base + used;
    used += al(bytes);
    return r;
  };
  const size_t tk = (size_t)T * k * 4;
  float* scores = static_cast<float*>(take((size_t)p.score_floats * 4));
  int32_t* beam[2] = {static_cast<int32_t*>(take(tk)), static_cast<int32_t*>(take(tk))};
  float* blp[2] = {static_cast<float*>(take(tk)), static_cast<float*>(take(tk))};
  int32_t *offsets = nullptr, *mtile_start = nullptr, *sorted_pair = nullptr, *pair_pos = nullptr, *counts = nullptr;
  int4* tile_tab = nullptr;
  if (p.n_perm_max > 0) {
    offsets = static_cast<int32_t*>(take((size_t)(kMaxE + 1) * 4));
    mtile_start = static_cast<int32_t*>(take((size_t)(kMaxE + 1) * 4));
    tile_tab = static_cast<int4*>(take((size_t)p.tiles_max * sizeof(int4)));
    sorted_pair = static_cast<int32_t*>(take(tk));
    pair_pos = static_cast<int32_t*>(take(tk));
    counts = static_cast<int32_t*>(take(permute_ws_bytes(T * k, p.n_perm_max)));
  }
  const size_t elt = bf16 ? 2 : 4;
  for (int l = 0; l < L; ++l) {
    const int width = p.width[l];
    const int32_t* cur = l == 0 ? nullptr : beam[(l - 1) & 1];
    const float* cur_lp = l == 0 ? nullptr : blp[(l - 1) & 1];
    const int N = sh.n[l] * B;
    hipError_t e = hipSuccess;
    if (p.kind[l] == kDenseGemm) {
      FfnGemmArgs g{};
      g.A = x;
      g.row_div = 1;
      g.W0 = static_cast<const unsigned char*>(w) + (size_t)sh.first[l] * d * elt;
      g.out = scores;
      g.E_loc = 1;
      g.rows_max = T;
      g.a_rows = T;
      g.K = d;
      g.N = N;
      g.out_f32 = 1;
      e = launch_ffn_gemm(g, false, W_BF16, false, 128, 2, s);
    } else {
      TreeScores a{};
      if (p.kind[l] == kGrouped) {
        e = launch_permute(T, width, sh.n[l], cur, nullptr, sh.n[l], 0, kTreeBM, offsets, mtile_start, tile_tab,
                           sorted_pair, pair_pos, counts, s);
        if (e != hipSuccess) return e;
        a.sorted_pair = sorted_pair;
        a.n_tiles = mtile_start + sh.n[l];
        a.tile_tab = tile_tab;
        a.rows_p = T * width;
      } else {
        a.rows_p = T;
        a.ncols = N;
        a.ncb = (N + 16 * p.nb[l] - 1) / (16 * p.nb[l]);
      }
      a.x = x;
      a.w = w;
      a.out = scores;
      a.d = d;
      a.B = B;
      a.width = p.kind[l] == kGrouped ? width : 1;
      a.row_base = (int)sh.first[l];
      a.n_next = sh.n[l + 1];
      a.kp_per_split = (d / 64 + p.nsplit[l] - 1) / p.nsplit[l];
      e = bf16 ? launch_scores<true>(a, p.nb[l], p.tiles[l], p.nsplit[l], s)
               : launch_scores<false>(a, p.nb[l], p.tiles[l], p.nsplit[l], s);
    }
    if (e != hipSuccess) return e;
    TreeSelect q{};
    q.scores = scores;
    q.dense_N = p.kind[l] == kGrouped ? 0 : N;
    q.beam = cur;
    q.beam_lp = cur_lp;
    q.T = T;
    q.B = B;
    q.width = width;
    q.n_next = sh.n[l + 1];
    q.keep = p.keep[l];
    q.nsplit = p.nsplit[l];
    q.renorm = renorm;
    if (l == L - 1) {
      q.next = ids;
      q.tw = tw;
    } else {
      q.next = beam[l & 1];
      q.next_lp = blp[l & 1];
    }
    if ((e = launch_tree_select(q, s)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
