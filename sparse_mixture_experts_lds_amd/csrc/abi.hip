// C ABI of the MoE layer forward (declared in include/moe_lds.h): argument
// checks, workspace carving and the launch sequence on the caller's stream.
#include "moe_lds.h"

#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "bwd.h"
#include "moe_internal.h"

using namespace moe;

namespace {

thread_local std::string g_last_error;

int hip_fail(hipError_t e) {
  g_last_error = hipGetErrorString(e);
  return MOE_EHIP;
}

#define MOE_HIP(call)                          \
  do {                                         \
    const hipError_t e_ = (call);              \
    if (e_ != hipSuccess) return hip_fail(e_); \
  } while (0)

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

inline size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

inline size_t elt_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }

// A bump allocator over the caller's workspace.
struct Carver {
  unsigned char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<unsigned char*>(b)) {}
  template <typename T>
  T* take(size_t bytes) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += align_up(bytes);
    return p;
  }
};

bool act_ok(int a) { return a == MOE_SWIGLU || a == MOE_GEGLU; }
bool act_dtype_ok(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }

// Weight/activation mixes the kernels implement.
bool mix_ok(int act_dtype, int w_dtype) {
  if (act_dtype == MOE_F32) return w_dtype == MOE_F32;
  if (act_dtype == MOE_BF16) return w_dtype == MOE_BF16 || w_dtype == MOE_I4G128;
  return false;
}

int wtype_of(int w_dtype) { return w_dtype == MOE_F32 ? W_F32 : (w_dtype == MOE_BF16 ? W_BF16 : W_I4); }

int check_width(int v, int w_dtype) {
  if (v <= 0) return MOE_EINVAL;
  if (v % 64) return MOE_EUNSUPPORTED;
  if (w_dtype == MOE_I4G128 && v % 128) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int check_route_dims(int T, int E, int k) {
  if (T < 0 || E <= 0 || k <= 0) return MOE_EINVAL;
  if (k > E) return MOE_EINVAL;
  if (E > kMaxE || k > kMaxK) return MOE_EUNSUPPORTED;
  if ((long long)T * k >= (1LL << 31) || (long long)T * E >= (1LL << 40)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// The layer's router by-products come from its selection launch (one partial
// row per selection workgroup) unless that makes more than this many
// partial entries; then the standalone passes read the logits again.
constexpr long long kSelStatsMaxEntries = 1LL << 21;

long long sel_stats_rows(int T, int E, int k) {
  return std::max(select_stats_rows(T, E, k, true), select_stats_rows(T, E, k, false));
}

size_t sel_stats_bytes(int T, int E, int k) {
  const long long rows = sel_stats_rows(T, E, k), n = rows * E;
  if (T <= 0 || rows > kStatsFinishMaxRows || n > kSelStatsMaxEntries) return 0;
  return align_up((size_t)n * 8) + align_up((size_t)n * 4) + stats_finish_bytes(E);
}

// Argument blocks of the gate/up GEMM (z = act(A Wg^T) * (A Wu^T) over
// grouped rows; `offsets` NULL means one group) and of the down GEMM that
// follows it (y = z Wd^T).
FfnGemmArgs gate_up_args(int E_loc, int rows_max, int d, int h, int act, const void* A, int a_rows,
                         const int32_t* row_index, int row_div, const int32_t* offsets, const int32_t* mtile,
                         const int4* tile_tab, const FfnPlan& plan, const void* wg, const void* wu,
                         const void* sg, const void* su, void* z) {
  FfnGemmArgs g{};
  g.A = A;
  g.row_index = row_index;
  g.row_div = row_div > 0 ? row_div : 1;
  g.W0 = wg;
  g.W1 = wu;
  g.S0 = static_cast<const uint16_t*>(sg);
  g.S1 = static_cast<const uint16_t*>(su);
  g.out = z;
  g.offsets = offsets;
  g.mtile_start = mtile;
  g.tile_tab = tile_tab;
  g.E_loc = E_loc;
  g.rows_max = rows_max;
  g.a_rows = a_rows;
  g.K = d;
  g.N = h;
  g.act = act == MOE_GEGLU ? 1 : 0;
  g.out_f16 = plan.z_f16 ? 1 : 0;
  return g;
}

// ytype: storage of y (YType: the operand dtype, fp32, or fp16)
FfnGemmArgs down_args(const FfnGemmArgs& gu, const void* wd, const void* sd, void* y, int ytype) {
  FfnGemmArgs dn = gu;
  dn.A = gu.out;
  dn.row_index = nullptr;
  dn.row_div = 1;
  dn.W0 = wd;
  dn.W1 = nullptr;
  dn.S0 = static_cast<const uint16_t*>(sd);
  dn.S1 = nullptr;
  dn.out = y;
  dn.out_f32 = ytype == Y_F32 ? 1 : 0;
  dn.out_f16 = ytype == Y_F16 ? 1 : 0;
  dn.a_rows = gu.rows_max;
  dn.K = gu.N;
  dn.N = gu.K;
  return dn;
}

// Gate/up then down over grouped rows; `offsets` NULL means one group.
// With plan.BM_down set, the down GEMM takes its own tile height and m-tile
// tables (mtile_dn, tiles_dn, for grouped rows).
int run_ffn(int E_loc, int rows_max, int d, int h, int act, int w_dtype, const void* A, int a_rows,
            const int32_t* row_index, int row_div, const int32_t* offsets, const int32_t* mtile,
            const int4* tile_tab, int BM,
            const FfnPlan& plan, const void* wg, const void* wu, const void* wd, const void* sg,
            const void* su, const void* sd, void* z, void* y, int ytype, hipStream_t s,
            void* mid_event = nullptr, void* const* kernel_events = nullptr,
            const int32_t* mtile_dn = nullptr, const int4* tiles_dn = nullptr) {
  const int wt = wtype_of(w_dtype);
  FfnGemmArgs g = gate_up_args(E_loc, rows_max, d, h, act, A, a_rows, row_index, row_div, offsets, mtile,
                               tile_tab, plan, wg, wu, sg, su, z);
  if (kernel_events) {
    g.ev_start = kernel_events[0];
    g.ev_stop = kernel_events[1];
  }
  MOE_HIP(launch_ffn_gemm(g, true, wt, false, BM, plan.NF_up, s));
  if (mid_event) MOE_HIP(hipEventRecord(static_cast<hipEvent_t>(mid_event), s));
  FfnGemmArgs dn = down_args(g, wd, sd, y, ytype);
  dn.ev_start = kernel_events ? kernel_events[2] : nullptr;
  dn.ev_stop = kernel_events ? kernel_events[3] : nullptr;
  int BMd = BM;
  if (plan.BM_down && plan.BM_down != BM) {
    BMd = plan.BM_down;
    if (offsets) {
      if (!mtile_dn || !tiles_dn) return MOE_EINVAL;
      dn.mtile_start = mtile_dn;
      dn.tile_tab = tiles_dn;
    }
  }
  MOE_HIP(launch_ffn_gemm(dn, false, wt, plan.z_f16, BMd, plan.NF_down, s));
  return MOE_OK;
}

constexpr int kSharedWideMinRows = 2048;

// The shared expert is one group of T rows.  With bf16 weights and enough
// rows it takes the wide 256-row tiles: they finish its GEMMs in fewer, fuller
// workgroups that slot in beside the routed GEMMs' own wide tiles.
FfnPlan shared_plan(int T, int d, int hs, int wt) {
  if (wt == W_BF16 && T >= kSharedWideMinRows && hs % 128 == 0 && d % 256 == 0) return FfnPlan{256, 4, 4, false};
  return plan_ffn((double)T, 1, d, hs, wt);
}

// How the layer forward runs the shared expert.  Its GEMMs ride in the routed
// GEMMs' own launches as a second problem whenever one kernel can take both:
//  - the wide kernel, when both take its tiles with the same tile widths
//    (granular: 384 + 128 gate/up tiles, exactly two rounds of 256 CUs);
//  - the narrow kernel at the routed tile shape, when the weights are of the
//    activation dtype and the shared hidden width equals the routed one (both
//    problems then have the same K and N; decode: 768 tiles of routed gate/up
//    plus 48 shared ones).
// Otherwise (an INT4 share with a bf16 shared expert, or other widths) the
// shared expert runs after the routed experts on the same stream.  There is
// no second stream and no fork or join event: the layer is one stream's work.
enum class SharedMode { kNone, kWidePair, kNarrowPair, kSerial };
SharedMode shared_mode(const moe_layer_desc* L, const FfnPlan& plan, const FfnPlan& sp) {
  if (L->h_shared <= 0) return SharedMode::kNone;
  if (L->w_dtype == MOE_BF16 && L->act_dtype == MOE_BF16 && plan.BM == 256 && sp.BM == 256 && !plan.z_f16 &&
      plan.NF_up == sp.NF_up && plan.NF_down == sp.NF_down)
    return SharedMode::kWidePair;
  if (plan.BM != 256 && L->w_dtype == L->act_dtype && L->w_dtype != MOE_I4G128 && L->h_shared == L->h &&
      !plan.z_f16 && (!plan.BM_down || plan.BM_down == plan.BM))
    return SharedMode::kNarrowPair;
  return SharedMode::kSerial;
}

// Rows a grouped GEMM may see: at most T*k pairs, and at most capacity per expert.
int layer_rows_max(const moe_layer_desc* L) {
  long long r = (long long)L->T * L->k;
  if (L->capacity > 0) {
    const long long c = (long long)L->capacity * L->E_loc;
    if (c < r) r = c;
  }
  return (int)r;
}

// The kernels read and write activations, weights, expert and layer outputs,
// their gradients and the workspaces with 16-byte accesses (row chunks, MFMA
// fragments, loads straight into LDS), so those arrays must start at a
// multiple of 16 bytes; the others (indices, offsets, gates, logits, biases,
// scales, counts) at a multiple of 4.  hipMalloc and torch allocations are
// 256-byte aligned; NULL passes.
template <typename... P>
inline bool all_a16(const P*... p) {
  return ((reinterpret_cast<uintptr_t>(p) % 16 == 0) && ...);
}
template <typename... P>
inline bool all_a4(const P*... p) {
  return ((reinterpret_cast<uintptr_t>(p) % 4 == 0) && ...);
}

int check_layer(const moe_layer_desc* L) {
  if (!L) return MOE_EINVAL;
  if (!all_a16(L->w_router, L->w_gate, L->w_up, L->w_down, L->ws_gate, L->ws_up, L->ws_down) ||
      !all_a4(L->expert_map, L->expert_bias, L->s_gate, L->s_up, L->s_down))
    return MOE_EINVAL;
  int rc = check_route_dims(L->T, L->E, L->k);
  if (rc) return rc;
  if (!act_ok(L->act) || !act_dtype_ok(L->act_dtype)) return MOE_EUNSUPPORTED;
  if (L->w_dtype < MOE_F32 || L->w_dtype > MOE_I4G128) return MOE_EUNSUPPORTED;
  if (!mix_ok(L->act_dtype, L->w_dtype)) return MOE_EUNSUPPORTED;
  if ((rc = check_width(L->d, L->w_dtype)) || (rc = check_width(L->h, L->w_dtype))) return rc;
  if (L->E_loc <= 0 || L->E_loc > L->E || L->capacity < 0 || L->h_shared < 0) return MOE_EINVAL;
  if (!L->expert_map && L->E_loc != L->E) return MOE_EINVAL;
  if (!L->w_gate || !L->w_up || !L->w_down) return MOE_EINVAL;
  if (L->w_dtype == MOE_I4G128 && (!L->s_gate || !L->s_up || !L->s_down)) return MOE_EINVAL;
  if (L->h_shared > 0) {
    if (L->h_shared % 64) return MOE_EUNSUPPORTED;
    if (!L->ws_gate || !L->ws_up || !L->ws_down) return MOE_EINVAL;
  }
  // the grouped GEMMs address activation rows with 32-bit byte offsets
  const size_t lim = 0xFFFFFFFFull;
  if ((size_t)L->T * L->d * 4 > lim || (size_t)layer_rows_max(L) * L->h * 4 > lim) return MOE_EUNSUPPORTED;
  if (L->tile_m) {
    const int m = L->tile_m;
    const int mmax = L->w_dtype == MOE_I4G128 ? 64 : (L->w_dtype == MOE_F32 ? 32 : 256);
    if ((m != 16 && m != 32 && m != 64 && m != 128 && m != 256) || m > mmax) return MOE_EUNSUPPORTED;
    // 256-row tiles are the wide bf16 kernel: 64- or 128-column gate/up and
    // 128- or 256-column down tiles
    if (m == 256) {
      if (L->h % 128 || L->d % 256) return MOE_EUNSUPPORTED;
      if (L->tile_n_up && L->tile_n_up != 64 && L->tile_n_up != 128) return MOE_EUNSUPPORTED;
      if (L->tile_n_down && L->tile_n_down != 128 && L->tile_n_down != 256) return MOE_EUNSUPPORTED;
      return MOE_OK;
    }
  }
  if (L->tile_n_up && (L->tile_n_up != 64 && L->tile_n_up != 128)) return MOE_EUNSUPPORTED;
  if (L->tile_n_down && (L->tile_n_down != 64 && L->tile_n_down != 128)) return MOE_EUNSUPPORTED;
  if (L->tile_n_up == 128 && L->h % 128) return MOE_EUNSUPPORTED;
  if (L->tile_n_down == 128 && L->d % 128) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// The automatic plan, overridden by the descriptor's tile hints.
FfnPlan layer_plan(const moe_layer_desc* L, int rows) {
  (void)rows;
  const int wt = wtype_of(L->w_dtype);
  FfnPlan p = plan_ffn((double)L->T * L->k / L->E, L->E_loc, L->d, L->h, wt);
  const bool hints = L->tile_m || L->tile_n_up || L->tile_n_down;
  if (!hints) return p;
  if (L->tile_m == 256) {
    // wide tiles: tile_n_up = output columns of gate/up (64 or 128 -> 128 or 256
    // weight rows), tile_n_down = output columns of down (128 or 256)
    FfnPlan w = p.BM == 256 ? p : FfnPlan{256, 4, 4, false};
    if (L->tile_n_up) w.NF_up = 2 * L->tile_n_up / 64;
    if (L->tile_n_down) w.NF_down = L->tile_n_down / 64;
    return w;
  }
  // narrow tiles: the hinted sizes, the planner's choice for the rest (one
  // tile height for both GEMMs)
  if (p.BM == 256) p = FfnPlan{128, 1, L->d % 128 == 0 ? 2 : 1, false};
  p.BM_down = 0;
  if (L->tile_m) p.BM = L->tile_m;
  if (L->tile_n_up) p.NF_up = L->tile_n_up / 64;
  if (L->tile_n_down) p.NF_down = L->tile_n_down / 64;
  p.z_f16 = wt == W_I4;
  return p;
}

struct LayerBufs {
  int4* tiles;
  int32_t *ids, *offsets, *mtile, *sorted_pair, *pair_pos, *counts, *mtile_dn;
  int4* tiles_dn;
  float *tw, *logits;
  void *z, *y, *zs, *ys, *stats;
};

size_t carve_layer(const moe_layer_desc* L, void* ws, LayerBufs* b) {
  Carver c(ws);
  const size_t P = (size_t)L->T * L->k;
  const size_t rows = (size_t)layer_rows_max(L);
  const size_t eb = elt_bytes(L->act_dtype);
  b->ids = c.take<int32_t>(P * 4);
  b->tw = c.take<float>(P * 4);
  // router GEMM output: its partial arrays over input slices
  b->logits = c.take<float>(L->w_router ? (size_t)router_logits_splits(L->T, L->d, L->E, L->act_dtype == MOE_BF16) *
                                              L->T * L->E * 4
                                        : 0);
  b->offsets = c.take<int32_t>((L->E_loc + 1) * 4);
  b->mtile = c.take<int32_t>((L->E_loc + 1) * 4);
  b->tiles = c.take<int4>((size_t)ffn_max_mtiles(L->E_loc, (int)rows, 16) * sizeof(int4));
  // the down GEMM's own m-tiles when its tile height differs
  const bool own_dn = layer_plan(L, (int)rows).BM_down > 0;
  b->mtile_dn = c.take<int32_t>(own_dn ? (L->E_loc + 1) * 4 : 0);
  b->tiles_dn = c.take<int4>(own_dn ? (size_t)ffn_max_mtiles(L->E_loc, (int)rows, 16) * sizeof(int4) : 0);
  b->sorted_pair = c.take<int32_t>(P * 4);
  b->pair_pos = c.take<int32_t>(P * 4);
  b->counts = c.take<int32_t>(permute_ws_bytes((int)P, L->E_loc));
  b->z = c.take<void>(rows * L->h * 4);  // room for the fp32 z of fp32 layers
  // expert outputs: fp16 in bf16 layers (one rounding to an 11-bit significand
  // before the combine's fp32 sum), fp32 in fp32 layers
  b->y = c.take<void>(rows * L->d * 4);
  b->zs = c.take<void>(L->h_shared > 0 ? (size_t)L->T * L->h_shared * eb : 0);
  b->ys = c.take<void>(L->h_shared > 0 ? (size_t)L->T * L->d * 4 : 0);
  // router by-product partials: from the selection's workgroups, or the
  // standalone passes' blocks
  b->stats = c.take<void>(std::max(router_stats_ws_bytes(L->T, L->E), sel_stats_bytes(L->T, L->E, L->k)));
  return c.used;
}

// ---------------------------------------------------------------- backward
struct BwdBufs {
  int32_t *ids, *offsets, *mtile, *sorted_pair, *pair_pos, *counts, *mtile_rc, *cnt;
  int4 *tiles, *tiles_rc, *chunks, *chunk_ext;
  float *tw, *Lraw, *Lw, *G, *U, *dZ, *dgate, *dXp, *Gs, *Us, *dZs, *dXs, *dL, *dXr, *part, *colpart;
  void *dGU, *ZW, *dGUs, *ZWs, *dLc, *stats;
};

// Grouped rows per tile of the backward's expert GEMMs (and of the gate/up
// recompute): 128 once experts average 96 rows or more (granular, 0.80 against
// 0.86 ms per backward), else 64 (decode, 1.93 against 1.99 ms).  The
// workspace is sized for 64, the larger tile count.
constexpr int kBwdBM = 64;
inline int bwd_bm(const moe_layer_desc* L, bool bf16) {
  return (bf16 && (double)L->T * L->k / L->E >= 96.0) ? 128 : kBwdBM;
}

inline int round_up(int v, int m) { return (v + m - 1) / m * m; }

// Weight rows per tile (64 * NF) of the wide recompute of g and u for hidden
// width h (N = h), or 0 when the wide kernel does not take it.
inline int wide_rc_nf(bool bf16, int d, int h) {
  if (!bf16 || d % 64) return 0;
  return h % 256 == 0 ? 4 : (h % 128 == 0 ? 2 : 0);
}

// The backward recomputes the routed g and u on the wide kernel when the
// forward's routed gate/up runs on it (bf16 weights).
inline bool bwd_wide_rc(const moe_layer_desc* L) {
  return L->act_dtype == MOE_BF16 && L->w_dtype == MOE_BF16 && layer_plan(L, layer_rows_max(L)).BM == 256 &&
         wide_rc_nf(true, L->d, L->h) > 0;
}

// Row slices of a single-group weight gradient: enough workgroups to fill the
// chip, at least 256 rows per slice.
int tn_slices(int rows, int M, int N) {
  const int tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int S = (512 + tiles - 1) / tiles;
  S = std::min(S, std::max(1, rows / 256));
  return std::max(1, std::min(S, 64));
}

// Most grouped rows one local expert can hold: a token selects an expert at
// most once, and the capacity (when > 0) caps it.
inline int bwd_group_max(const moe_layer_desc* L) {
  return L->capacity > 0 ? std::min(L->capacity, L->T) : L->T;
}

size_t carve_bwd(const moe_layer_desc* L, void* ws, BwdBufs* b) {
  Carver c(ws);
  const size_t T = L->T, P = T * L->k, E = L->E, d = L->d, h = L->h, hs = L->h_shared;
  const size_t rows = (size_t)layer_rows_max(L);
  const size_t eb = elt_bytes(L->act_dtype);
  const size_t Epad = (size_t)round_up(L->E, 32);
  const bool f32 = L->act_dtype == MOE_F32;
  b->ids = c.take<int32_t>(P * 4);
  b->tw = c.take<float>(P * 4);
  b->Lraw = c.take<float>(L->w_router ? (size_t)router_logits_splits(L->T, L->d, L->E, L->act_dtype == MOE_BF16) *
                                            T * E * 4
                                      : 0);
  b->Lw = c.take<float>(T * E * 4);
  b->offsets = c.take<int32_t>((L->E_loc + 1) * 4);
  b->mtile = c.take<int32_t>((L->E_loc + 1) * 4);
  b->tiles = c.take<int4>((size_t)ffn_max_mtiles(L->E_loc, (int)rows, kBwdBM) * sizeof(int4));
  // m-tiles of the recompute of g and u when they differ from the backward's own
  // (fp32: at most 32 rows; wide bf16: 256 rows)
  const bool own_rc = f32 || bwd_wide_rc(L);
  b->mtile_rc = c.take<int32_t>(own_rc ? (L->E_loc + 1) * 4 : 0);
  b->tiles_rc = c.take<int4>(own_rc ? (size_t)ffn_max_mtiles(L->E_loc, (int)rows, f32 ? 32 : 256) * sizeof(int4) : 0);
  b->sorted_pair = c.take<int32_t>(P * 4);
  b->pair_pos = c.take<int32_t>(P * 4);
  b->counts = c.take<int32_t>(permute_ws_bytes((int)P, L->E_loc));
  b->G = c.take<float>(rows * h * 4);
  b->U = c.take<float>(rows * h * 4);
  b->dZ = c.take<float>(rows * h * 4);
  b->dGU = c.take<void>(rows * 2 * h * eb);
  b->ZW = c.take<void>(rows * h * eb);
  b->dgate = c.take<float>(P * 4);
  b->dXp = c.take<float>(rows * d * 4);
  b->Gs = c.take<float>(T * hs * 4);
  b->Us = c.take<float>(T * hs * 4);
  b->dZs = c.take<float>(T * hs * 4);
  b->dGUs = c.take<void>(T * 2 * hs * eb);
  b->ZWs = c.take<void>(T * hs * eb);
  b->dXs = c.take<float>(hs ? T * d * 4 : 0);
  b->dL = c.take<float>(T * E * 4);
  b->dLc = c.take<void>(T * Epad * eb);
  b->dXr = c.take<float>(L->w_router ? T * d * 4 : 0);
  b->cnt = c.take<int32_t>(E * 4);
  b->stats = c.take<void>(router_stats_ws_bytes(L->T, L->E));
  size_t part = 0;
  if (L->w_router) part = std::max(part, (size_t)tn_slices(L->T, L->E, L->d) * E * d);
  if (hs) {
    part = std::max(part, (size_t)tn_slices(L->T, L->d, (int)hs) * d * hs);
    part = std::max(part, (size_t)tn_slices(L->T, 2 * (int)hs, L->d) * 2 * hs * d);
  }
  // the routed weight gradients' row chunks (dWd: d x h, dWg and dWu: 2h x d
  // per expert): their virtual groups and partial slots
  size_t vmax = 0, xmax = 0;
  const size_t Ms[2] = {d, 2 * h}, Ns[2] = {h, d};
  for (int i = 0; i < 2; ++i) {
    const int CH = tn_chunk_rows((int)rows, bwd_group_max(L), (int)Ms[i], (int)Ns[i]);
    if (!CH) continue;
    vmax = std::max(vmax, (size_t)L->E_loc + rows / CH);
    xmax = std::max(xmax, rows / CH);
    part = std::max(part, rows / CH * Ms[i] * Ns[i]);
  }
  b->chunks = c.take<int4>(vmax * sizeof(int4));
  b->chunk_ext = c.take<int4>(xmax * sizeof(int4));
  b->part = c.take<float>(part * 4);
  b->colpart = c.take<float>(colsum_ws_floats(L->T, L->E) * 4);
  return c.used;
}

int check_bwd(const moe_layer_desc* L) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (L->w_dtype == MOE_I4G128) return MOE_EUNSUPPORTED;  // packed INT4 experts are not trained
  if ((size_t)layer_rows_max(L) * 2 * L->h * 4 > 0xFFFFFFFFull) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// One single-group weight gradient C = A^T B over all T rows: row slices into
// b->part, then their fixed-order sum (rows m >= M1 of the result to C2).
int tn_single(bool bf, const void* A, int lda, const void* B, int ldb, int T, int M, int N, int M1, float* C1,
              float* C2, int ldc, float* part, hipStream_t s) {
  const int S = tn_slices(T, M, N);
  bwdg::TnArgs t{};
  t.A = A;
  t.lda = lda;
  t.a_div = 1;
  t.B = B;
  t.ldb = ldb;
  t.b_div = 1;
  t.rows = T;
  t.slice = round_up((T + S - 1) / S, 32);
  t.M = M;
  t.N = N;
  t.mtiles = (M + bwdg::kTnTile - 1) / bwdg::kTnTile;
  const int nz = (T + t.slice - 1) / t.slice;
  if (nz <= 1) {
    t.C1 = C1;
    t.C2 = C2;
    t.M1 = M1;
    t.ldc = ldc;
    MOE_HIP(launch_bwd_tn(bf, t, 1, s));
    return MOE_OK;
  }
  t.C1 = t.C2 = part;
  t.M1 = M;
  t.ldc = N;
  t.c_stride = (long long)M * N;
  MOE_HIP(launch_bwd_tn(bf, t, nz, s));
  MOE_HIP(launch_sum_slices(nz, M, N, M1, part, C1, C2, ldc, s));
  return MOE_OK;
}

// Gate/up pre-activations of one expert set, fp32 [rows, h] each.
// g = a Wg^T and u = a Wu^T in fp32, as the forward's gate/up GEMM forms them
// before the activation.  BM 256: both in one launch of the wide kernel (two
// problems); else two launches of the narrow kernel.
int recompute_gu(int wt, bool grouped, const void* x, int T, int k, const int32_t* sorted_pair,
                 const int32_t* offsets, const int32_t* mtile, const int4* tiles, int E_loc, int rows, int d, int h,
                 int BM, const void* wg, const void* wu, float* G, float* U, hipStream_t s) {
  FfnGemmArgs g{};
  g.A = x;
  g.row_index = grouped ? sorted_pair : nullptr;
  g.row_div = grouped ? k : 1;
  g.offsets = grouped ? offsets : nullptr;
  g.mtile_start = grouped ? mtile : nullptr;
  g.tile_tab = grouped ? tiles : nullptr;
  g.E_loc = grouped ? E_loc : 1;
  g.rows_max = rows;
  g.K = d;
  g.N = h;
  g.a_rows = T;
  g.out_f32 = 1;
  if (BM == 256) {
    const int nfw = wide_rc_nf(wt == W_BF16, d, h);
    if (!nfw) return MOE_EUNSUPPORTED;
    FfnGemmArgs u = g;
    g.W0 = wg;
    g.out = G;
    u.W0 = wu;
    u.out = U;
    MOE_HIP(launch_ffn_gemm_wide_pair(g, u, false, nfw, nullptr, nullptr, s));
    return MOE_OK;
  }
  const int NF = (wt == W_BF16 && h % 128 == 0) ? 2 : 1;
  g.W0 = wg;
  g.out = G;
  MOE_HIP(launch_ffn_gemm(g, false, wt, false, BM, NF, s));
  g.W0 = wu;
  g.out = U;
  MOE_HIP(launch_ffn_gemm(g, false, wt, false, BM, NF, s));
  return MOE_OK;
}

// ---------------------------------------------------------------- allocation-free grouping
// Scratch of moe_permute_noalloc (the per-block expert histograms and bases of
// the grouping step): one static device array per GPU, held until the process
// ends.  Its name is a host-side stand-in in host code; the device address of
// each GPU's copy is looked up once per device (hipGetSymbolAddress with that
// device current) and only that address reaches kernels.
constexpr size_t kNoallocScratchBytes = (size_t)MOE_PERMUTE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) int32_t scratch[kNoallocScratchBytes / sizeof(int32_t)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null until looked up)

// Device address of this stream's device's copy of `scratch`.
int scratch_ptr(hipStream_t s, int32_t** out) {
  int dev = 0;
  if (s) MOE_HIP(hipStreamGetDevice(s, &dev));
  else MOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    MOE_HIP(hipGetDevice(&cur));
    if (cur != dev) MOE_HIP(hipSetDevice(dev));
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) return hip_fail(e2);
    }
    if (e != hipSuccess) return hip_fail(e);
    if (!p) return MOE_EHIP;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Argument checks shared by moe_permute and moe_permute_noalloc.
int check_permute(int T, int k, int E, const int32_t* topk_ids, const int32_t* expert_map, int E_loc, int capacity,
                  const int32_t* expert_offsets, const int32_t* sorted_pair, const int32_t* pair_pos, const void* x,
                  int d, int act_dtype, const void* x_perm) {
  int rc = check_route_dims(T, E, k);
  if (rc) return rc;
  if (E_loc <= 0 || E_loc > E || capacity < 0) return MOE_EINVAL;
  if (!expert_map && E_loc != E) return MOE_EINVAL;
  if (!expert_offsets) return MOE_EINVAL;
  if (T > 0 && (!topk_ids || !sorted_pair || !pair_pos)) return MOE_EINVAL;
  if (!all_a4(topk_ids, expert_map, expert_offsets, sorted_pair, pair_pos) || !all_a16(x, x_perm)) return MOE_EINVAL;
  if (x_perm) {
    if (!act_dtype_ok(act_dtype)) return MOE_EUNSUPPORTED;
    if ((rc = check_width(d, act_dtype))) return rc;
    if (!x) return MOE_EINVAL;
  }
  return MOE_OK;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported dtype, activation or shape";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch failed";
    default: return "unknown error";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_route(int T, int d, int E, int k, int act_dtype, const void* x, const void* w_router,
              const float* logits_in, const float* expert_bias, int renorm, int32_t* topk_ids,
              float* topk_w, float* logits_out, void* stream) {
  int rc = check_route_dims(T, E, k);
  if (rc) return rc;
  if (!act_dtype_ok(act_dtype)) return MOE_EUNSUPPORTED;
  if (!logits_in) {
    if ((rc = check_width(d, act_dtype))) return rc;
    if (!x || !w_router) return MOE_EINVAL;
  }
  if (T > 0 && (!topk_ids || !topk_w)) return MOE_EINVAL;
  if (!all_a16(x, w_router) || !all_a4(logits_in, expert_bias, topk_ids, topk_w, logits_out)) return MOE_EINVAL;
  MOE_HIP(launch_route(T, d, E, k, act_dtype == MOE_BF16, x, w_router, logits_in, expert_bias, renorm,
                       topk_ids, topk_w, logits_out, as_stream(stream)));
  return MOE_OK;
}

size_t moe_router_stats_workspace_bytes(int T, int E) {
  if (T < 0 || E <= 0 || E > kMaxE) return 0;
  return router_stats_ws_bytes(T, E);
}

int moe_router_stats(int T, int E, int k, const float* logits, const float* expert_bias, const int32_t* topk_ids,
                     int32_t* expert_counts, float* prob_mean, float* balance_loss, void* ws, size_t ws_bytes,
                     void* stream) {
  int rc = check_route_dims(T, E, k);
  if (rc) return rc;
  if (T > 0 && (!logits || !topk_ids)) return MOE_EINVAL;
  if (!all_a4(logits, expert_bias, topk_ids, expert_counts, prob_mean, balance_loss) || !all_a16(ws))
    return MOE_EINVAL;
  const size_t need = router_stats_ws_bytes(T, E);
  if (ws_bytes < need) return MOE_EWORKSPACE;
  if (need > 0 && !ws) return MOE_EINVAL;
  if (!expert_counts && !prob_mean && !balance_loss) return MOE_OK;
  MOE_HIP(launch_router_stats(T, E, k, logits, expert_bias, topk_ids, expert_counts, prob_mean, balance_loss, ws,
                              as_stream(stream)));
  return MOE_OK;
}

namespace {
int check_tree(int T, int d, int E, int k, int branch, int levels, int act_dtype, TreeShape* sh) {
  if (T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E || branch <= 0 || levels <= 0) return MOE_EINVAL;
  if (!act_dtype_ok(act_dtype) || d % 64 || k > kMaxK || k * branch > 1024) return MOE_EUNSUPPORTED;
  if (!tree_shape(E, branch, levels, sh) || sh->n[levels - 1] > kMaxE) return MOE_EUNSUPPORTED;
  if ((long long)T * k * branch * 16 >= (1LL << 40) || (long long)T * k >= (1LL << 31)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}
}  // namespace

long long moe_tree_gate_rows(int E, int branch, int levels) {
  TreeShape sh;
  if (E <= 0 || branch <= 0 || levels <= 0) return MOE_EINVAL;
  if (!tree_shape(E, branch, levels, &sh)) return MOE_EUNSUPPORTED;
  return sh.rows;
}

size_t moe_route_tree_workspace_bytes(int T, int d, int E, int k, int branch, int levels, int act_dtype) {
  TreeShape sh;
  if (check_tree(T, d, E, k, branch, levels, act_dtype, &sh)) return 0;
  return tree_ws_bytes(T, d, k, branch, levels, act_dtype == MOE_BF16, sh);
}

int moe_route_tree(int T, int d, int E, int k, int branch, int levels, int act_dtype, const void* x,
                   const void* w_tree, int renorm, int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                   void* stream) {
  TreeShape sh;
  const int rc = check_tree(T, d, E, k, branch, levels, act_dtype, &sh);
  if (rc) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !w_tree || !topk_ids || !topk_w || !ws) return MOE_EINVAL;
  if (!all_a16(x, w_tree, ws) || !all_a4(topk_ids, topk_w)) return MOE_EINVAL;
  if (ws_bytes < tree_ws_bytes(T, d, k, branch, levels, act_dtype == MOE_BF16, sh)) return MOE_EWORKSPACE;
  MOE_HIP(launch_route_tree(T, d, E, k, branch, levels, act_dtype == MOE_BF16, x, w_tree, renorm, topk_ids, topk_w,
                            ws, as_stream(stream)));
  return MOE_OK;
}

size_t moe_permute_workspace_bytes(int T, int k, int E_loc) {
  if (T < 0 || k <= 0 || E_loc <= 0) return 0;
  return align_up(permute_ws_bytes(T * k, E_loc));
}

int moe_permute(int T, int k, int E, const int32_t* topk_ids, const int32_t* expert_map, int E_loc,
                int capacity, int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_pos,
                const void* x, int d, int act_dtype, void* x_perm, void* ws, size_t ws_bytes,
                void* stream) {
  const int rc = check_permute(T, k, E, topk_ids, expert_map, E_loc, capacity, expert_offsets, sorted_pair, pair_pos,
                               x, d, act_dtype, x_perm);
  if (rc) return rc;
  if (ws_bytes < moe_permute_workspace_bytes(T, k, E_loc)) return MOE_EWORKSPACE;
  if ((T > 0 && !ws) || !all_a16(ws)) return MOE_EINVAL;
  hipStream_t s = as_stream(stream);
  MOE_HIP(launch_permute(T, k, E, topk_ids, expert_map, E_loc, capacity, 16, expert_offsets, nullptr, nullptr,
                         sorted_pair, pair_pos, static_cast<int32_t*>(ws), s));
  if (x_perm && T > 0)
    MOE_HIP(launch_gather_rows(T * k, d, act_dtype == MOE_BF16, x, sorted_pair, k, expert_offsets + E_loc,
                               x_perm, s));
  return MOE_OK;
}

int moe_permute_noalloc(int T, int k, int E, const int32_t* topk_ids, const int32_t* expert_map, int E_loc,
                        int capacity, int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_pos,
                        const void* x, int d, int act_dtype, void* x_perm, void* stream) {
  int rc = check_permute(T, k, E, topk_ids, expert_map, E_loc, capacity, expert_offsets, sorted_pair, pair_pos, x,
                         d, act_dtype, x_perm);
  if (rc) return rc;
  // every scratch entry the kernels read is written first in the same call
  // (histograms, then bases), so nothing needs clearing between calls
  if (permute_ws_bytes(T * k, E_loc) > kNoallocScratchBytes) return MOE_EUNSUPPORTED;
  hipStream_t s = as_stream(stream);
  int32_t* ws = nullptr;
  if ((rc = scratch_ptr(s, &ws))) return rc;
  MOE_HIP(launch_permute(T, k, E, topk_ids, expert_map, E_loc, capacity, 16, expert_offsets, nullptr, nullptr,
                         sorted_pair, pair_pos, ws, s));
  if (x_perm && T > 0)
    MOE_HIP(launch_gather_rows(T * k, d, act_dtype == MOE_BF16, x, sorted_pair, k, expert_offsets + E_loc,
                               x_perm, s));
  return MOE_OK;
}

size_t moe_dispatch_owners_workspace_bytes(int T, int k, int E) {
  if (T < 0 || k <= 0 || E <= 0 || E > kMaxE) return 0;
  return align_up((size_t)E * 4) + align_up((size_t)(E + 1) * 4) + align_up(permute_ws_bytes(T * k, E));
}

int moe_dispatch_owners(int T, int k, int E, int n_owners, int placement, int capacity, const int32_t* topk_ids,
                        int32_t* owner_offsets, int32_t* recv_offsets, int32_t* expert_offsets,
                        int32_t* sorted_pair, int32_t* pair_pos, const void* x, int d, int act_dtype,
                        void* x_send, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_route_dims(T, E, k);
  if (rc) return rc;
  if (n_owners <= 0 || E % n_owners != 0 || capacity < 0) return MOE_EINVAL;
  if (placement != MOE_PLACE_ROUND_ROBIN && placement != MOE_PLACE_CONTIGUOUS) return MOE_EINVAL;
  if (!owner_offsets) return MOE_EINVAL;
  if (T > 0 && (!topk_ids || !sorted_pair || !pair_pos)) return MOE_EINVAL;
  if (x_send) {
    if (!act_dtype_ok(act_dtype)) return MOE_EUNSUPPORTED;
    if ((rc = check_width(d, act_dtype))) return rc;
    if (!x) return MOE_EINVAL;
  }
  if (ws_bytes < moe_dispatch_owners_workspace_bytes(T, k, E)) return MOE_EWORKSPACE;
  if (!ws) return MOE_EINVAL;
  if (!all_a4(topk_ids, owner_offsets, recv_offsets, expert_offsets, sorted_pair, pair_pos) ||
      !all_a16(x, x_send, ws))
    return MOE_EINVAL;
  Carver c(ws);
  int32_t* map = c.take<int32_t>((size_t)E * 4);
  int32_t* eo_ws = c.take<int32_t>((size_t)(E + 1) * 4);
  int32_t* counts = c.take<int32_t>(permute_ws_bytes(T * k, E));
  int32_t* eo = expert_offsets ? expert_offsets : eo_ws;
  hipStream_t s = as_stream(stream);
  MOE_HIP(launch_owner_dispatch(T, k, E, n_owners, placement, capacity, topk_ids, owner_offsets, recv_offsets, eo,
                                sorted_pair, pair_pos, map, counts, s));
  if (x_send && T > 0)
    MOE_HIP(launch_gather_rows(T * k, d, act_dtype == MOE_BF16, x, sorted_pair, k, eo + E, x_send, s));
  return MOE_OK;
}

size_t moe_expert_ffn_workspace_bytes(int E_loc, int rows_max, int d, int h, int act_dtype) {
  (void)d;
  if (E_loc <= 0 || rows_max < 0 || h <= 0 || !act_dtype_ok(act_dtype)) return 0;
  // z, then two m-tile tables (gate/up, and down when its tile height differs)
  return align_up((size_t)rows_max * h * 4) +
         2 * (align_up((size_t)(E_loc + 1) * 4) + align_up((size_t)ffn_max_mtiles(E_loc, rows_max, 16) * sizeof(int4)));
}

int moe_expert_ffn(int E_loc, int rows_max, int d, int h, int act, int act_dtype, int w_dtype,
                   const void* x_perm, const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                   const void* w_down, const void* s_gate, const void* s_up, const void* s_down,
                   void* y_perm, void* ws, size_t ws_bytes, void* stream) {
  if (E_loc <= 0 || rows_max < 0) return MOE_EINVAL;
  if (E_loc > kMaxE) return MOE_EUNSUPPORTED;
  if (!act_ok(act) || !act_dtype_ok(act_dtype) || !mix_ok(act_dtype, w_dtype)) return MOE_EUNSUPPORTED;
  int rc;
  if ((rc = check_width(d, w_dtype)) || (rc = check_width(h, w_dtype))) return rc;
  if (!expert_offsets && E_loc != 1) return MOE_EINVAL;
  if (!w_gate || !w_up || !w_down) return MOE_EINVAL;
  if (w_dtype == MOE_I4G128 && (!s_gate || !s_up || !s_down)) return MOE_EINVAL;
  if (rows_max > 0 && (!x_perm || !y_perm)) return MOE_EINVAL;
  if (!all_a16(x_perm, w_gate, w_up, w_down, y_perm, ws) || !all_a4(expert_offsets, s_gate, s_up, s_down))
    return MOE_EINVAL;
  // the grouped GEMMs address activation rows with 32-bit byte offsets
  if ((size_t)rows_max * d * 4 > 0xFFFFFFFFull || (size_t)rows_max * h * 4 > 0xFFFFFFFFull) return MOE_EUNSUPPORTED;
  if (ws_bytes < moe_expert_ffn_workspace_bytes(E_loc, rows_max, d, h, act_dtype)) return MOE_EWORKSPACE;
  if (rows_max == 0) return MOE_OK;
  if (!ws) return MOE_EINVAL;
  hipStream_t s = as_stream(stream);
  Carver c(ws);
  void* z = c.take<void>((size_t)rows_max * h * 4);
  int32_t* mtile = c.take<int32_t>((size_t)(E_loc + 1) * 4);
  int4* tab = c.take<int4>((size_t)ffn_max_mtiles(E_loc, rows_max, 16) * sizeof(int4));
  int32_t* mtile_dn = c.take<int32_t>((size_t)(E_loc + 1) * 4);
  int4* tab_dn = c.take<int4>((size_t)ffn_max_mtiles(E_loc, rows_max, 16) * sizeof(int4));
  const int wt = wtype_of(w_dtype);
  const FfnPlan plan = plan_ffn((double)rows_max / E_loc, E_loc, d, h, wt);
  const bool own_dn = plan.BM_down && plan.BM_down != plan.BM;
  if (expert_offsets) MOE_HIP(launch_mtile_prefix(E_loc, plan.BM, expert_offsets, mtile, tab, s));
  if (expert_offsets && own_dn) MOE_HIP(launch_mtile_prefix(E_loc, plan.BM_down, expert_offsets, mtile_dn, tab_dn, s));
  return run_ffn(E_loc, rows_max, d, h, act, w_dtype, x_perm, rows_max, nullptr, 1, expert_offsets,
                 expert_offsets ? mtile : nullptr, expert_offsets ? tab : nullptr, plan.BM, plan, w_gate, w_up,
                 w_down, s_gate, s_up, s_down, z, y_perm, Y_OUT, s, nullptr, nullptr, mtile_dn, tab_dn);
}

int moe_combine(int T, int k, int d, int act_dtype, const void* y_perm, const int32_t* pair_pos,
                const float* topk_w, const void* shared_y, void* out, void* stream) {
  if (T < 0 || k <= 0 || k > kMaxK) return k > kMaxK ? MOE_EUNSUPPORTED : MOE_EINVAL;
  if (!act_dtype_ok(act_dtype)) return MOE_EUNSUPPORTED;
  int rc;
  if ((rc = check_width(d, act_dtype))) return rc;
  if (T > 0 && (!y_perm || !pair_pos || !topk_w || !out)) return MOE_EINVAL;
  if (!all_a16(y_perm, shared_y, out) || !all_a4(pair_pos, topk_w)) return MOE_EINVAL;
  MOE_HIP(launch_combine(T, k, d, act_dtype == MOE_BF16, Y_OUT, y_perm, pair_pos, topk_w,
                         shared_y, out, as_stream(stream)));
  return MOE_OK;
}

size_t moe_layer_workspace_bytes(const moe_layer_desc* L) {
  if (check_layer(L) != MOE_OK) return 0;
  LayerBufs b;
  return carve_layer(L, nullptr, &b);
}

int moe_layer_plan(const moe_layer_desc* L, moe_layer_plan_info* out) {
  if (!out) return MOE_EINVAL;
  const int rc = check_layer(L);
  if (rc) return rc;
  const FfnPlan p = layer_plan(L, layer_rows_max(L));
  const bool wide = p.BM == 256;
  moe_layer_plan_info r{};
  r.tile_m = p.BM;
  r.tile_n_up = wide ? 32 * p.NF_up : 64 * p.NF_up;
  r.tile_n_down = 64 * p.NF_down;
  if (L->h_shared > 0) {
    const FfnPlan sp = shared_plan(L->T, L->d, L->h_shared, wtype_of(L->act_dtype));
    const SharedMode m = shared_mode(L, p, sp);
    r.shared_tile_m = m == SharedMode::kNarrowPair ? p.BM : sp.BM;
    r.shared_in_routed_launches = (m == SharedMode::kWidePair || m == SharedMode::kNarrowPair) ? 1 : 0;
  }
  *out = r;
  return MOE_OK;
}

int moe_layer_fwd(const moe_layer_desc* L, const void* x, const float* logits_in, void* out,
                  const moe_layer_trace* trace, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (!logits_in && !L->w_router) return MOE_EINVAL;
  if (L->T > 0 && (!x || !out)) return MOE_EINVAL;
  if (!all_a16(x, out, ws) || !all_a4(logits_in)) return MOE_EINVAL;
  if (trace && !all_a4(trace->logits, trace->topk_ids, trace->topk_w, trace->expert_offsets, trace->pair_pos,
                       trace->expert_counts, trace->prob_mean, trace->balance_loss))
    return MOE_EINVAL;
  const size_t need = moe_layer_workspace_bytes(L);
  if (ws_bytes < need) return MOE_EWORKSPACE;
  if (L->T == 0) return MOE_OK;
  if (!ws) return MOE_EINVAL;
  hipStream_t s = as_stream(stream);
  LayerBufs b;
  carve_layer(L, ws, &b);
  moe_layer_trace tr{};
  if (trace) tr = *trace;
  int32_t* ids = tr.topk_ids ? tr.topk_ids : b.ids;
  float* tw = tr.topk_w ? tr.topk_w : b.tw;
  int32_t* offsets = tr.expert_offsets ? tr.expert_offsets : b.offsets;
  int32_t* pair_pos = tr.pair_pos ? tr.pair_pos : b.pair_pos;
  const bool bf16 = L->act_dtype == MOE_BF16;
  const int ytype = bf16 ? Y_F16 : Y_F32;  // storage of the expert outputs until the combine
  const int T = L->T, k = L->k;
  auto mark = [&](int i) -> hipError_t {
    return tr.events[i] ? hipEventRecord(static_cast<hipEvent_t>(tr.events[i]), s) : hipSuccess;
  };
  const int rows = layer_rows_max(L);

  MOE_HIP(mark(MOE_EV_START));
  const FfnPlan plan = layer_plan(L, rows);
  const int swt = L->act_dtype;  // shared weights are in the activation dtype
  const FfnPlan sp = L->h_shared > 0 ? shared_plan(T, L->d, L->h_shared, wtype_of(swt)) : FfnPlan{16, 1, 1, false};
  const SharedMode smode = shared_mode(L, plan, sp);

  // 1-2: router logits (GEMM, or the caller's), then softmax + top-k per token
  const float* lsrc = logits_in;
  int nsplit = 1;
  const bool want_stats = tr.expert_counts || tr.prob_mean || tr.balance_loss;
  float* lout = nullptr;
  // by-products from the selection launch: one partial row per workgroup
  const bool fused = !lsrc && router_fused_ok(T, L->d, L->E, k, bf16);
  const int srows = select_stats_rows(T, L->E, k, fused);
  // the same test that sized the workspace (for the larger of the two paths' rows)
  const bool sel_stats = want_stats && sel_stats_bytes(T, L->E, k) > 0;
  StatsPart stp{};
  if (sel_stats) {
    unsigned char* base = static_cast<unsigned char*>(b.stats);
    const size_t n = (size_t)srows * L->E;
    stp.part_p = reinterpret_cast<double*>(base);
    stp.part_c = reinterpret_cast<int32_t*>(base + align_up(n * 8));
    unsigned char* fin = base + align_up(n * 8) + align_up(n * 4);  // the finishing pass's memory
    const size_t m = (size_t)kStatsMaxRowSplits * L->E;
    stp.mid_p = reinterpret_cast<double*>(fin);
    stp.mid_c = reinterpret_cast<int32_t*>(fin + align_up(m * 8));
    stp.counter = reinterpret_cast<unsigned*>(fin + align_up(m * 8) + align_up(m * 4));
  }
  if (fused) {
    // one launch: the biased logits reach memory only when something reads them
    lout = tr.logits ? tr.logits : (want_stats && !sel_stats ? b.logits : nullptr);
    MOE_HIP(launch_router_fused(T, L->d, L->E, k, x, L->w_router, L->expert_bias, L->renorm, ids, tw, lout, s,
                                sel_stats ? &stp : nullptr));
  } else {
    if (!lsrc) {
      nsplit = router_logits_splits(T, L->d, L->E, bf16);
      float* lbuf = (tr.logits && nsplit == 1) ? tr.logits : b.logits;
      MOE_HIP(launch_router_logits(T, L->d, L->E, bf16, x, L->w_router, lbuf, nsplit, s));
      lsrc = lbuf;
    }
    // the summed, biased logits go to the trace buffer, else (partial arrays)
    // over the first partial array when the by-products read them
    lout = tr.logits ? tr.logits : (nsplit > 1 && want_stats && !sel_stats ? b.logits : nullptr);
    MOE_HIP(launch_select(T, L->E, k, lsrc, nsplit, L->expert_bias, L->renorm, ids, tw, lout, s,
                          sel_stats ? &stp : nullptr));
  }
  // router by-products
  if (sel_stats)
    MOE_HIP(launch_stats_finish(T, L->E, srows, stp, tr.expert_counts, tr.prob_mean,
                                tr.balance_loss, s));
  else if (want_stats)
    MOE_HIP(launch_router_stats(T, L->E, k, lout ? lout : lsrc, lout ? nullptr : L->expert_bias, ids,
                                tr.expert_counts, tr.prob_mean, tr.balance_loss, b.stats, s));
  MOE_HIP(mark(MOE_EV_ROUTED));
  // 3: grouping (the m-tile table of the grouped GEMMs comes out of the same scan)
  MOE_HIP(launch_permute(T, k, L->E, ids, L->expert_map, L->E_loc, L->capacity, plan.BM, offsets, b.mtile, b.tiles,
                         b.sorted_pair, pair_pos, b.counts, s));
  if (plan.BM_down && plan.BM_down != plan.BM)
    MOE_HIP(launch_mtile_prefix(L->E_loc, plan.BM_down, offsets, b.mtile_dn, b.tiles_dn, s));
  MOE_HIP(mark(MOE_EV_GROUPED));
  // 4 (+ 5 when paired): routed experts, activations gathered straight from x
  // by pair index; the shared expert as the second problem of the same launches
  void* kev[4] = {tr.gate_up_kernel_events[0], tr.gate_up_kernel_events[1], tr.down_kernel_events[0],
                  tr.down_kernel_events[1]};
  const void* shared_y = nullptr;
  if (smode == SharedMode::kWidePair || smode == SharedMode::kNarrowPair) {
    const bool wide = smode == SharedMode::kWidePair;
    const FfnPlan& shp = wide ? sp : plan;
    FfnGemmArgs rg = gate_up_args(L->E_loc, rows, L->d, L->h, L->act, x, T, b.sorted_pair, k, offsets, b.mtile,
                                  b.tiles, plan, L->w_gate, L->w_up, nullptr, nullptr, b.z);
    const FfnGemmArgs sg = gate_up_args(1, T, L->d, L->h_shared, L->act, x, T, nullptr, 1, nullptr, nullptr,
                                        nullptr, shp, L->ws_gate, L->ws_up, nullptr, nullptr, b.zs);
    if (wide) {
      MOE_HIP(launch_ffn_gemm_wide_pair(rg, sg, true, plan.NF_up, kev[0], kev[1], s));
    } else {
      rg.ev_start = kev[0];
      rg.ev_stop = kev[1];
      MOE_HIP(launch_ffn_gemm_pair(rg, sg, true, wtype_of(L->w_dtype), plan.BM, plan.NF_up, s));
      rg.ev_start = rg.ev_stop = nullptr;
    }
    MOE_HIP(mark(MOE_EV_GATE_UP));
    FfnGemmArgs rd = down_args(rg, L->w_down, nullptr, b.y, ytype);
    const FfnGemmArgs sd = down_args(sg, L->ws_down, nullptr, b.ys, ytype);
    if (wide) {
      // the deeper problem's tiles are dispatched first
      if (L->h_shared > L->h) MOE_HIP(launch_ffn_gemm_wide_pair(sd, rd, false, plan.NF_down, kev[2], kev[3], s));
      else MOE_HIP(launch_ffn_gemm_wide_pair(rd, sd, false, plan.NF_down, kev[2], kev[3], s));
    } else {
      rd.ev_start = kev[2];
      rd.ev_stop = kev[3];
      MOE_HIP(launch_ffn_gemm_pair(rd, sd, false, wtype_of(L->w_dtype), plan.BM, plan.NF_down, s));
    }
    shared_y = b.ys;
    MOE_HIP(mark(MOE_EV_DOWN));
  } else {
    rc = run_ffn(L->E_loc, rows, L->d, L->h, L->act, L->w_dtype, x, T, b.sorted_pair, k, offsets, b.mtile, b.tiles,
                 plan.BM, plan, L->w_gate, L->w_up, L->w_down, L->s_gate, L->s_up, L->s_down, b.z, b.y, ytype, s,
                 tr.events[MOE_EV_GATE_UP], kev, b.mtile_dn, b.tiles_dn);
    if (rc) return rc;
    MOE_HIP(mark(MOE_EV_DOWN));
    // 5: the shared expert on every token, on the same stream
    if (smode == SharedMode::kSerial) {
      rc = run_ffn(1, T, L->d, L->h_shared, L->act, swt, x, T, nullptr, 1, nullptr, nullptr, nullptr, sp.BM, sp,
                   L->ws_gate, L->ws_up, L->ws_down, nullptr, nullptr, nullptr, b.zs, b.ys, ytype, s);
      if (rc) return rc;
      shared_y = b.ys;
    }
  }
  MOE_HIP(mark(MOE_EV_SHARED));
  // 6: the weighted combine
  MOE_HIP(launch_combine(T, k, L->d, bf16, ytype, b.y, pair_pos, tw, shared_y, out, s));
  MOE_HIP(mark(MOE_EV_END));
  return MOE_OK;
}

size_t moe_layer_bwd_workspace_bytes(const moe_layer_desc* L) {
  if (check_bwd(L) != MOE_OK) return 0;
  BwdBufs b;
  return carve_bwd(L, nullptr, &b);
}

int moe_layer_bwd(const moe_layer_desc* L, const void* x, const float* logits_in, const void* dout, float balance,
                  const moe_layer_grads* gr, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_bwd(L);
  if (rc) return rc;
  if (!logits_in && !L->w_router) return MOE_EINVAL;
  if (!gr || !gr->dx) return MOE_EINVAL;
  if (L->T > 0 && (!x || !dout)) return MOE_EINVAL;
  if ((gr->dw_gate == nullptr) != (gr->dw_up == nullptr)) return MOE_EINVAL;
  if ((gr->dws_gate == nullptr) != (gr->dws_up == nullptr)) return MOE_EINVAL;
  if (gr->dw_router && !L->w_router) return MOE_EINVAL;
  if (gr->dbias && !L->expert_bias) return MOE_EINVAL;
  if (!(balance == balance)) return MOE_EINVAL;  // NaN
  if (!all_a16(x, dout, ws, gr->dx, gr->dw_router, gr->dw_gate, gr->dw_up, gr->dw_down, gr->dws_gate, gr->dws_up,
               gr->dws_down) ||
      !all_a4(logits_in, gr->dlogits, gr->dbias, gr->dgates))
    return MOE_EINVAL;
  const size_t need = moe_layer_bwd_workspace_bytes(L);
  if (ws_bytes < need) return MOE_EWORKSPACE;
  if (L->T == 0) return MOE_OK;
  if (!ws) return MOE_EINVAL;
  hipStream_t s = as_stream(stream);
  BwdBufs b;
  carve_bwd(L, ws, &b);
  const bool bf = L->act_dtype == MOE_BF16;
  const int wt = wtype_of(L->w_dtype);
  const int T = L->T, k = L->k, E = L->E, E_loc = L->E_loc, d = L->d, h = L->h, hs = L->h_shared;
  const int rows = layer_rows_max(L);
  const int Epad = round_up(E, 32);
  const int BMb = bwd_bm(L, bf);
  const int grid_m = ffn_max_mtiles(E_loc, rows, BMb);

  // 1. routing, as the forward: logits (GEMM or given) + bias, selection, grouping
  const float* lsrc = logits_in;
  int nsplit = 1;
  if (!lsrc && router_fused_ok(T, d, E, k, bf)) {
    MOE_HIP(launch_router_fused(T, d, E, k, x, L->w_router, L->expert_bias, L->renorm, b.ids, b.tw, b.Lw, s));
  } else {
    if (!lsrc) {
      nsplit = router_logits_splits(T, d, E, bf);
      MOE_HIP(launch_router_logits(T, d, E, bf, x, L->w_router, b.Lraw, nsplit, s));
      lsrc = b.Lraw;
    }
    MOE_HIP(launch_select(T, E, k, lsrc, nsplit, L->expert_bias, L->renorm, b.ids, b.tw, b.Lw, s));
  }
  MOE_HIP(launch_permute(T, k, E, b.ids, L->expert_map, E_loc, L->capacity, BMb, b.offsets, b.mtile, b.tiles,
                         b.sorted_pair, b.pair_pos, b.counts, s));
  // the fp32 grouped GEMM of the forward takes at most 32-row tiles; the wide
  // recompute takes 256-row tiles
  const bool wide_rc = bwd_wide_rc(L);
  const int BMrc = !bf ? 32 : (wide_rc ? 256 : BMb);
  const bool own_rc = !bf || wide_rc;
  if (own_rc) MOE_HIP(launch_mtile_prefix(E_loc, BMrc, b.offsets, b.mtile_rc, b.tiles_rc, s));

  // The routed experts' data gradient GEMMs take the wide 256 x 256 tiles where
  // the forward's gate/up does (its recompute built the 256-row m-tile table);
  // their weight gradient GEMMs take them whenever the shapes fit (bf16): a
  // tile's contraction runs over its expert's rows however few, and the wide
  // tile stores its fp32 gradient as 16-byte row chunks (decode: 1.77 against
  // 1.92 ms per backward).  Else the 128-wide kernels.
  auto run_nn = [&](bwdg::NnArgs a) -> hipError_t {
    if (wide_rc && bwd_nn_wide_ok(a)) {
      a.mtile_start = b.mtile_rc;
      a.tile_tab = b.tiles_rc;
      return launch_bwd_nn_wide(a, s);
    }
    return launch_bwd_nn(bf, a, BMb, grid_m, s);
  };
  auto run_tn = [&](const bwdg::TnArgs& a) -> hipError_t {
    return (bf && bwd_tn_wide_ok(a)) ? launch_bwd_tn_wide(a, E_loc, s) : launch_bwd_tn(bf, a, E_loc, s);
  };
  // A routed weight gradient on the wide kernel whose groups may hold more
  // rows than an even share of the launch: the groups are cut into row
  // chunks (a device-built table), chunks past a group's first write partial
  // slots, and those are added to the group's gradient in chunk order.
  auto run_tn_routed = [&](bwdg::TnArgs a) -> hipError_t {
    const int CH = (bf && bwd_tn_wide_ok(a)) ? tn_chunk_rows(rows, bwd_group_max(L), a.M, a.N) : 0;
    if (!CH) return run_tn(a);
    const int Vmax = E_loc + rows / CH, Xmax = rows / CH;
    hipError_t e = launch_tn_chunk_table(E_loc, b.offsets, CH, Vmax, Xmax, b.chunks, b.chunk_ext, s);
    if (e != hipSuccess) return e;
    a.chunks = b.chunks;
    a.part = b.part;
    if ((e = launch_bwd_tn_wide(a, Vmax, s)) != hipSuccess) return e;
    return launch_tn_chunk_add(Xmax, a.M, a.N, a.M1, a.C1, a.C2, a.ldc, a.c_stride, b.part, b.chunk_ext, s);
  };

  // The shared expert's set-up, here because its fused gate/up launch (below)
  // can ride in the routed one.
  const int swt = wtype_of(L->act_dtype);
  const int BMsr = (hs > 0 && shared_plan(T, d, hs, swt).BM == 256 && wide_rc_nf(bf, d, hs)) ? 256 : (bf ? BMb : 32);
  const FfnPlan wide_plan{256, 4, 4, false, 0};
  const FfnGemmArgs sgu_bwd = gate_up_args(1, T, d, hs, L->act, x, T, nullptr, 1, nullptr, nullptr, nullptr,
                                           wide_plan, L->ws_gate, L->ws_up, nullptr, nullptr, b.ZWs);
  const bool fused_sgb = hs > 0 && BMsr == 256 && gateup_bwd_wide_ok(sgu_bwd);
  const int BMs = (bf && T >= 4096) ? 128 : 64;
  const int gms = (T + BMs - 1) / BMs;
  // the shared expert's rows are one dense group: wide tiles from as many
  // tokens as the forward gives it wide tiles
  auto run_nn_shared = [&](const bwdg::NnArgs& a) -> hipError_t {
    return (bf && T >= kSharedWideMinRows && bwd_nn_wide_ok(a)) ? launch_bwd_nn_wide(a, s)
                                                                : launch_bwd_nn(bf, a, BMs, gms, s);
  };
  // dz's = dout Wsd
  auto shared_dz = [&]() -> hipError_t {
    bwdg::NnArgs m{};
    m.A = dout;
    m.lda = d;
    m.a_div = 1;
    m.B1 = L->ws_down;
    m.K1 = d;
    m.ldb = hs;
    m.K_valid = d;
    m.C = b.dZs;
    m.ldc = hs;
    m.rows = T;
    m.N = hs;
    m.K = d;
    return run_nn_shared(m);
  };
  const GateBwdOut sgbo{b.dZs, nullptr, static_cast<uint16_t*>(b.dGUs), static_cast<uint16_t*>(b.ZWs), b.Gs};

  // 2. routed experts: g, u again; dz' = dout Wd; gate backward; weight and data gradients.
  // Where the forward's gate/up takes the wide tiles, the recompute is that
  // launch again with the gate backward in its epilogue (after dz'): g and u
  // never leave registers, and the gate gradients come out as partial sums
  // per 64 hidden units (in G's memory), added up in a fixed order.
  const FfnGemmArgs gu_bwd = gate_up_args(E_loc, rows, d, h, L->act, x, T, b.sorted_pair, k, b.offsets, b.mtile_rc,
                                          b.tiles_rc, wide_plan, L->w_gate, L->w_up, nullptr, nullptr, b.ZW);
  const bool fused_gb = wide_rc && gateup_bwd_wide_ok(gu_bwd);
  if (!fused_gb &&
      (rc = recompute_gu(wt, true, x, T, k, b.sorted_pair, b.offsets, own_rc ? b.mtile_rc : b.mtile,
                         own_rc ? b.tiles_rc : b.tiles, E_loc, rows, d, h, BMrc, L->w_gate, L->w_up, b.G, b.U, s)))
    return rc;
  bwdg::NnArgs n{};
  n.A = dout;
  n.lda = d;
  n.a_index = b.sorted_pair;
  n.a_div = k;
  n.B1 = L->w_down;
  n.K1 = d;
  n.ldb = h;
  n.b_stride = (long long)d * h;
  n.K_valid = d;
  n.C = b.dZ;
  n.ldc = h;
  n.mtile_start = b.mtile;
  n.tile_tab = b.tiles;
  n.groups = E_loc;
  n.rows = rows;
  n.N = h;
  n.K = d;
  MOE_HIP(run_nn(n));
  if (fused_gb) {
    // the rows' gates in U's memory, the gate-gradient partials in G's
    MOE_HIP(launch_row_gates(rows, b.offsets + E_loc, b.sorted_pair, b.tw, b.U, s));
    const GateBwdOut gbo{b.dZ, b.U, static_cast<uint16_t*>(b.dGU), static_cast<uint16_t*>(b.ZW), b.G};
    if (fused_sgb) {
      // the shared expert's gate/up rides in the same launch as in the forward
      // (its dz' first); its gate-gradient partials go to Gs and stay there
      MOE_HIP(shared_dz());
      const FfnGemmArgs two[2] = {gu_bwd, sgu_bwd};
      const GateBwdOut outs[2] = {gbo, sgbo};
      MOE_HIP(launch_gateup_bwd_wide(two, outs, 2, s));
    } else {
      MOE_HIP(launch_gateup_bwd_wide(&gu_bwd, &gbo, 1, s));
    }
    MOE_HIP(launch_gate_part_sum(rows, h, b.offsets + E_loc, b.G, b.sorted_pair, b.dgate, s));
  } else {
    MOE_HIP(launch_gate_bwd(bf, L->act, rows, h, b.offsets + E_loc, b.G, b.U, b.dZ, b.sorted_pair, b.tw, b.dGU,
                            b.ZW, b.dgate, s));
  }
  if (gr->dw_down) {
    bwdg::TnArgs t{};
    t.A = dout;
    t.lda = d;
    t.a_index = b.sorted_pair;
    t.a_div = k;
    t.B = b.ZW;
    t.ldb = h;
    t.b_div = 1;
    t.offsets = b.offsets;
    t.C1 = t.C2 = gr->dw_down;
    t.M1 = d;
    t.ldc = h;
    t.c_stride = (long long)d * h;
    t.M = d;
    t.N = h;
    t.mtiles = (d + bwdg::kTnTile - 1) / bwdg::kTnTile;
    MOE_HIP(run_tn_routed(t));
  }
  if (gr->dw_gate) {
    bwdg::TnArgs t{};
    t.A = b.dGU;
    t.lda = 2 * h;
    t.a_div = 1;
    t.B = x;
    t.ldb = d;
    t.b_index = b.sorted_pair;
    t.b_div = k;
    t.offsets = b.offsets;
    t.C1 = gr->dw_gate;
    t.C2 = gr->dw_up;
    t.M1 = h;
    t.ldc = d;
    t.c_stride = (long long)h * d;
    t.M = 2 * h;
    t.N = d;
    t.mtiles = (2 * h + bwdg::kTnTile - 1) / bwdg::kTnTile;
    MOE_HIP(run_tn_routed(t));
  }
  n = bwdg::NnArgs{};
  n.A = b.dGU;
  n.lda = 2 * h;
  n.a_div = 1;
  n.B1 = L->w_gate;
  n.B2 = L->w_up;
  n.K1 = h;
  n.ldb = d;
  n.b_stride = (long long)h * d;
  n.K_valid = 2 * h;
  n.C = b.dXp;
  n.ldc = d;
  n.mtile_start = b.mtile;
  n.tile_tab = b.tiles;
  n.groups = E_loc;
  n.rows = rows;
  n.N = d;
  n.K = 2 * h;
  MOE_HIP(run_nn(n));

  // 3. shared expert on every token (gate 1)
  if (hs > 0) {
    // (done in the routed launch when both gate/up launches took the gate backward)
    if (!(fused_gb && fused_sgb)) {
      if (!fused_sgb && (rc = recompute_gu(swt, false, x, T, 1, nullptr, nullptr, nullptr, nullptr, 1, T, d, hs,
                                           BMsr, L->ws_gate, L->ws_up, b.Gs, b.Us, s)))
        return rc;
      MOE_HIP(shared_dz());
      if (fused_sgb)
        MOE_HIP(launch_gateup_bwd_wide(&sgu_bwd, &sgbo, 1, s));
      else
        MOE_HIP(launch_gate_bwd(bf, L->act, T, hs, nullptr, b.Gs, b.Us, b.dZs, nullptr, nullptr, b.dGUs, b.ZWs,
                                nullptr, s));
    }
    if (gr->dws_down && (rc = tn_single(bf, dout, d, b.ZWs, hs, T, d, hs, d, gr->dws_down, gr->dws_down, hs, b.part,
                                        s)))
      return rc;
    if (gr->dws_gate && (rc = tn_single(bf, b.dGUs, 2 * hs, x, d, T, 2 * hs, d, hs, gr->dws_gate, gr->dws_up, d,
                                        b.part, s)))
      return rc;
    n = bwdg::NnArgs{};
    n.A = b.dGUs;
    n.lda = 2 * hs;
    n.a_div = 1;
    n.B1 = L->ws_gate;
    n.B2 = L->ws_up;
    n.K1 = hs;
    n.ldb = d;
    n.K_valid = 2 * hs;
    n.C = b.dXs;
    n.ldc = d;
    n.rows = T;
    n.N = d;
    n.K = 2 * hs;
    MOE_HIP(run_nn_shared(n));
  }

  // 4. gates, softmax and balance loss back to the logits; router GEMMs
  if (balance != 0.f)
    MOE_HIP(launch_router_stats(T, E, k, b.Lw, nullptr, b.ids, b.cnt, nullptr, nullptr, b.stats, s));
  const float bal = (float)((double)balance * E / ((double)T * (double)T));
  float* dLt = (logits_in && gr->dlogits) ? gr->dlogits : b.dL;
  MOE_HIP(launch_router_bwd(bf, T, E, Epad, k, L->renorm, b.Lw, b.ids, b.pair_pos, b.dgate,
                            balance != 0.f ? b.cnt : nullptr, bal, dLt, b.dLc, gr->dgates, s));
  if (!logits_in) {
    n = bwdg::NnArgs{};
    n.A = b.dLc;
    n.lda = Epad;
    n.a_div = 1;
    n.B1 = L->w_router;
    n.K1 = Epad;
    n.ldb = d;
    n.K_valid = E;
    n.C = b.dXr;
    n.ldc = d;
    n.rows = T;
    n.N = d;
    n.K = Epad;
    const int BMr = (bf && T >= 4096) ? 128 : 64;
    MOE_HIP(launch_bwd_nn(bf, n, BMr, (T + BMr - 1) / BMr, s));
    if (gr->dw_router &&
        (rc = tn_single(bf, b.dLc, Epad, x, d, T, E, d, E, gr->dw_router, gr->dw_router, d, b.part, s)))
      return rc;
  }
  if (gr->dbias) MOE_HIP(launch_colsum(T, E, dLt, b.colpart, gr->dbias, s));

  // 5. dx = routed pairs + shared expert + router
  MOE_HIP(launch_dx_assemble(bf, T, k, d, b.dXp, b.pair_pos, hs > 0 ? b.dXs : nullptr, logits_in ? nullptr : b.dXr,
                             gr->dx, s));
  return MOE_OK;
}

int moe_quantize_int4(int rows, int K, const float* w, uint8_t* packed, uint16_t* scales, void* stream) {
  if (rows < 0 || K <= 0) return MOE_EINVAL;
  if (K % kI4Group) return MOE_EUNSUPPORTED;
  if (rows > 0 && (!w || !packed || !scales)) return MOE_EINVAL;
  if (!all_a4(w, packed, scales)) return MOE_EINVAL;
  MOE_HIP(launch_quantize_int4(rows, K, w, packed, scales, as_stream(stream)));
  return MOE_OK;
}

}  // extern "C"
#pragma GCC visibility pop
