/*
 * moe_lds.h - C ABI of the top-k routed Mixture-of-Experts FFN layer forward
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (forward only) runs in five steps, each a call below:
 *   moe_route       router logits GEMM, softmax and top-k selection
 *   moe_router_stats per-expert counts, mean probabilities, balance loss
 *   moe_route_tree  hierarchical routing down an expert tree (a router for
 *                   very large expert pools)
 *   moe_permute     grouping of (token, slot) pairs by expert
 *   moe_dispatch_owners  the same grouping by owner of the expert (sender
 *                   side of expert parallelism)
 *   moe_expert_ffn  grouped gated expert GEMMs (SwiGLU / GeGLU; bf16, fp32 or
 *                   signed INT4 with fp16 group scales)
 *   moe_combine     weighted top-k combine plus the optional shared expert
 *   moe_layer_fwd   all of the above, fused where it pays, on one stream
 *   moe_layer_bwd   gradients of the layer (bf16 and fp32 weights)
 *
 * Sources of the operation (web pages; section named where the page has one):
 *   "Sharding d'experts" (Kvasir wiki), section "Deux roles": the backbone /
 *     worker cut of an MoE layer; the backbone routes once (softmax of the
 *     router logits, top k), a worker runs the three matrix products of each
 *     selected expert, and the backbone adds the gate-weighted partial outputs
 *     and the shared expert's output.
 *   moe_stream.py (MoE-Stream), MoEFFN.forward: bias-free router, optional
 *     per-expert logit bias before the softmax, softmax over all experts, topk,
 *     division of the k gates by their sum, per-expert gather / scatter-add.
 *   MoEEvolve, "Architecture": SwiGLU experts, one always-active shared
 *     expert, capacity-factor static-shape dispatch.
 *   kieve-moe, "Features": top-k GeGLU experts; fractal tiling routing, a
 *     self-similar routing down a branch^levels expert tree for very large
 *     expert pools (one sentence, no formula: moe_route_tree states the
 *     reading it implements).
 *   ExpertMesh README: group-scaled signed INT4 weights with FP16 group
 *     scales in the [expert, output, packed_input] layout, a stable C ABI,
 *     per-expert grouping of activations that keeps each token and top-k
 *     slot, and a reduction of the expert outputs with the top-k weights.
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers unless stated otherwise; the
 *     caller owns every buffer (inputs, outputs, workspace).  The library never
 *     allocates or frees memory, creates no stream or event, keeps no pointer
 *     after returning and has no mutable global state (apart from the
 *     per-thread text of the last HIP error, and the one static scratch array
 *     of moe_permute_noalloc); each call enqueues all of its work on `stream`,
 *     and calls on different streams may run concurrently (except
 *     moe_permute_noalloc calls on one GPU, which share its scratch).
 *   - Arrays are dense and row-major; weight matrices are [out, in].
 *     Activations, weights (packed INT4 codes included), expert and layer
 *     outputs, their gradients and every workspace start at a multiple of 16
 *     bytes; the other arrays (indices, offsets, gates, logits, biases, scales,
 *     counts) at a multiple of 4.  hipMalloc and torch allocations satisfy
 *     both; a call given an array that does not returns MOE_EINVAL (the
 *     arrays a descriptor, trace or gradient struct points to included).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; no call synchronises the device or reads device memory
 *     on the host.
 *   - Every call returns MOE_OK (0) or a negative error code.  Arguments are
 *     validated before anything is enqueued, so an error never leaves a
 *     partial launch behind; MOE_EHIP reports a failed launch (text via
 *     moe_last_error()).
 *   - Inputs must be finite; NaN or Inf inputs give unspecified results.
 *   - bf16 values are passed as their 16-bit patterns (uint16 storage);
 *     fp16 scales likewise.
 *
 * Limits (MOE_EUNSUPPORTED beyond them): 1 <= k <= min(E, 32), E <= 1024,
 * E_loc <= E, d and h multiples of 64 (of 128 for INT4 weights), T*k < 2^31.
 */
#ifndef MOE_LDS_H
#define MOE_LDS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ---------------------------------------------------- */
enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* null required pointer, negative size, k > E, ... */
  MOE_EUNSUPPORTED = -2,  /* dtype/activation mix or shape outside the limits */
  MOE_EWORKSPACE = -3,    /* ws_bytes below the matching *_workspace_bytes()  */
  MOE_EHIP = -4           /* a HIP launch failed                              */
};

/* ---- element types -------------------------------------------------- */
enum moe_dtype {
  MOE_F32 = 0,     /* IEEE float32                                            */
  MOE_BF16 = 1,    /* bfloat16                                                */
  MOE_I4G128 = 2   /* weights only: signed INT4 codes, two per byte (input 2i
                      in the low nibble, 2i+1 in the high nibble, two's
                      complement), packed [.., N, K/2] uint8, plus fp16 scales
                      [.., N, K/128]; weight = scale[n, k/128] * code[n, k]    */
};

/* ---- gate activations ----------------------------------------------- */
enum moe_act {
  MOE_SWIGLU = 0,  /* z = SiLU(g) * u, SiLU(g) = g / (1 + exp(-g))            */
  MOE_GEGLU = 1    /* z = GELU(g) * u, exact erf GELU                         */
};

/*
 * moe_route - router logits, softmax and top-k ("Deux roles" pseudo-code;
 * moe_stream.py MoEFFN.forward).
 *
 *   L[t,e] = sum_i x[t,i] * w_router[e,i] + expert_bias[e]      (fp32 accumulate)
 *            or logits_in[t,e] + expert_bias[e] when logits_in != NULL
 *   topk_ids[t,j]  = the j-th largest L[t,.] (ties: lower expert id first)
 *   topk_w[t,j]    = softmax(L[t,.])[id] over all E experts; with renorm != 0
 *                    divided by the sum over the k selected (no epsilon)
 *
 *   T, d, E, k     tokens, model width, experts, top-k (T = 0 is a no-op)
 *   act_dtype      MOE_F32 or MOE_BF16: dtype of x and w_router
 *   x              [T, d]; w_router [E, d]; both ignored (may be NULL) when
 *                  logits_in != NULL
 *   logits_in      [T, E] fp32 or NULL
 *   expert_bias    [E] fp32 or NULL (added before selection and softmax)
 *   topk_ids       out [T, k] int32;  topk_w  out [T, k] fp32
 *   logits_out     out [T, E] fp32 or NULL: the L used for selection
 */
int moe_route(int T, int d, int E, int k, int act_dtype,
              const void* x, const void* w_router, const float* logits_in,
              const float* expert_bias, int renorm,
              int32_t* topk_ids, float* topk_w, float* logits_out, void* stream);

/*
 * moe_router_stats - router by-products of one batch (moe_stream.py
 * MoEFFN.forward, load-balancing part; the balance loss is the batch-local
 * auxiliary loss that keeps the experts evenly used).
 *
 *   L[t,e]            = logits[t,e] + expert_bias[e]   (bias may be NULL)
 *   expert_counts[e]  = number of tokens t with e among topk_ids[t, 0..k-1]
 *                       (a token counts once per expert; ids outside [0, E)
 *                       match no expert)
 *   prob_mean[e]      = (1/T) sum_t softmax(L[t, .])[e], softmax over all E
 *   balance_loss[0]   = E * sum_e (expert_counts[e] / T) * prob_mean[e]
 *
 *   T, E, k        tokens, experts, top-k; T = 0 writes zero counts, zero
 *                  means and a zero loss
 *   logits         [T, E] fp32 (as moe_route's logits_out, or without bias)
 *   topk_ids       [T, k] int32
 *   expert_counts  out [E] int32 or NULL;  prob_mean out [E] fp32 or NULL;
 *   balance_loss   out [1] fp32 or NULL
 *   ws, ws_bytes   device workspace of at least
 *                  moe_router_stats_workspace_bytes(T, E) bytes (NULL allowed
 *                  when that is 0)
 * Counts are exact; prob_mean and the loss come from fp32 softmax values added
 * in fp64 in a fixed order, so repeated calls give identical bits.
 */
size_t moe_router_stats_workspace_bytes(int T, int E);
int moe_router_stats(int T, int E, int k, const float* logits, const float* expert_bias,
                     const int32_t* topk_ids, int32_t* expert_counts, float* prob_mean,
                     float* balance_loss, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_tree - hierarchical routing down an expert tree (kieve-moe
 * "Features", fractal tiling routing: self-similar routing over a
 * branch^levels expert tree, a cheap router for very large expert pools).
 * The page gives no formula; this is the reading implemented:
 *
 *   tree     the E experts are the leaves of a tree with B = branch children
 *            per node and L = levels levels (E <= B^L); leaf e is reached by
 *            the base-B digits of e, most significant first; node i at depth
 *            l has children i*B + c; depth l holds n_l = ceil(E / B^(L-l))
 *            nodes (those with a leaf below them)
 *   gates    one row of w_tree per non-root node: child j of depth l+1 has
 *            row first_l + j, first_l = B * (n_0 + ... + n_{l-1}); the table
 *            has moe_tree_gate_rows(E, branch, levels) = first_L rows (rows of
 *            children that do not exist are never read)
 *   scores   s(child) = sum_i x[t,i] * w_tree[row(child), i] (fp32 accumulate);
 *            each node's existing children share a softmax, and a leaf's
 *            log-probability is the sum of its path's log-softmax terms
 *   select   beam search of width k: at each depth the kept nodes' children
 *            are ranked by path log-probability (higher first, ties to the
 *            lower node id) and the best min(k, n_{l+1}) kept; topk_ids[t,j]
 *            = the j-th leaf kept at the last depth, topk_w[t,j] = its path
 *            probability, divided by the sum over the k when renorm != 0.
 *            With levels = 1 this is moe_route with w_router = the first E
 *            rows and no bias.
 *
 *   T, d           tokens (T = 0 is a no-op), model width (a multiple of 64)
 *   E, k           experts (leaves), picks: 1 <= k <= min(E, 32), k*branch <= 1024
 *   branch, levels 2 <= branch <= 64, 1 <= levels <= 16, E <= branch^levels,
 *                  and at most 1024 nodes above the leaves (E <= 1024 * branch)
 *   act_dtype      MOE_F32 or MOE_BF16: dtype of x and w_tree
 *   x              [T, d];  w_tree [moe_tree_gate_rows(E, branch, levels), d]
 *   topk_ids       out [T, k] int32;  topk_w out [T, k] fp32
 *   ws, ws_bytes   device workspace of at least
 *                  moe_route_tree_workspace_bytes(T, d, E, k, branch, levels, act_dtype)
 * Deterministic: repeated calls give identical bits.  Errors: MOE_EINVAL for
 * a NULL buffer or k outside [1, E]; MOE_EUNSUPPORTED outside the limits;
 * MOE_EWORKSPACE for a short workspace.
 */
long long moe_tree_gate_rows(int E, int branch, int levels);   /* < 0: error code */
size_t moe_route_tree_workspace_bytes(int T, int d, int E, int k, int branch, int levels, int act_dtype);
int moe_route_tree(int T, int d, int E, int k, int branch, int levels, int act_dtype,
                   const void* x, const void* w_tree, int renorm,
                   int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_permute - group the pairs p = t*k + j by local expert (ExpertMesh:
 * grouping that keeps token and top-k slot identity; MoEEvolve: capacity
 * dispatch).
 *
 *   local(p)        = expert_map ? expert_map[topk_ids[p]] : topk_ids[p]
 *                     (-1 = not local; expert_map == NULL requires E_loc == E;
 *                     ids outside [0, E) and map entries outside [0, E_loc)
 *                     also count as not local)
 *   kept            the first `capacity` pairs of each expert in ascending p
 *                   (capacity 0 = all), local pairs only
 *   expert_offsets  out [E_loc+1]: exclusive prefix sum of kept counts
 *   sorted_pair     out [T*k]: sorted_pair[r] = p of the pair in grouped row r,
 *                   rows in ascending p inside each expert; entries at rows >=
 *                   expert_offsets[E_loc] are unspecified
 *   pair_pos        out [T*k]: the row of pair p, or -1 if dropped / not local
 *   x, d, act_dtype optional row gather: x_perm[r, :] = x[sorted_pair[r] / k, :]
 *                   into x_perm [T*k, d]; pass x_perm = NULL to skip (then x
 *                   and d are ignored)
 *   ws, ws_bytes    device workspace of at least moe_permute_workspace_bytes()
 * Output is deterministic (no dependence on atomic ordering).
 */
size_t moe_permute_workspace_bytes(int T, int k, int E_loc);
int moe_permute(int T, int k, int E, const int32_t* topk_ids,
                const int32_t* expert_map, int E_loc, int capacity,
                int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_pos,
                const void* x, int d, int act_dtype, void* x_perm,
                void* ws, size_t ws_bytes, void* stream);

/*
 * moe_permute_noalloc - moe_permute without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, outputs
 * and errors as moe_permute, minus ws / ws_bytes.
 *
 * Its scratch (the grouping step's per-block expert histograms and bases) is
 * a static device array of MOE_PERMUTE_NOALLOC_SCRATCH_BYTES inside the
 * library, one copy per GPU, held from the first call on that GPU until the
 * process ends; no call allocates or frees anything.  Sizes whose
 * moe_permute_workspace_bytes(T, k, E_loc) exceeds it (1024 * E_loc * 4 bytes
 * per block of 1024 pairs: T*k*E_loc up to about 1e9) return
 * MOE_EUNSUPPORTED.  Every call on one GPU uses that GPU's one array, which
 * keeps the last call's contents: two calls that may overlap on the same GPU
 * (e.g. on two streams without an order between them) race and give
 * undefined results; the caller must order them.
 */
#define MOE_PERMUTE_NOALLOC_SCRATCH_BYTES (4u << 20)
int moe_permute_noalloc(int T, int k, int E, const int32_t* topk_ids,
                        const int32_t* expert_map, int E_loc, int capacity,
                        int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_pos,
                        const void* x, int d, int act_dtype, void* x_perm, void* stream);

/*
 * moe_dispatch_owners - sender side of expert parallelism: every (token, slot)
 * pair grouped by the owner that holds its expert, in one pass (ExpertMesh
 * README: deterministic placement of the expert pool across stationary
 * owners; a dispatcher that groups the routed activations by expert owner and
 * keeps each token and top-k slot).
 *
 *   placement  MOE_PLACE_ROUND_ROBIN: owner(e) = e % n_owners, local(e) = e / n_owners
 *              MOE_PLACE_CONTIGUOUS:  owner(e) = e / per,      local(e) = e % per
 *              with per = E / n_owners (E must be a multiple of n_owners)
 *   rows       ordered by (owner, local expert, p = t*k + j); with capacity > 0
 *              only the first `capacity` pairs of each expert (ascending p)
 *              are kept; ids outside [0, E) are dropped
 *   owner_offsets   out [n_owners+1]: owner o sends rows [owner_offsets[o],
 *                   owner_offsets[o+1])
 *   recv_offsets    out [n_owners, per+1] or NULL: owner o's expert offsets
 *                   counted from its first row (offsets[0] = 0), as the
 *                   receiving owner passes them to moe_expert_ffn
 *   expert_offsets  out [E+1] or NULL: the same offsets over the whole buffer,
 *                   expert (o, l) at index o*per + l
 *   sorted_pair, pair_pos   as moe_permute, over the whole buffer
 *   x, d, act_dtype, x_send optional row gather x_send[r, :] = x[sorted_pair[r] / k, :]
 *                   into x_send [T*k, d] (NULL = no gather)
 *   ws, ws_bytes    device workspace of at least moe_dispatch_owners_workspace_bytes()
 * Output is deterministic.
 */
enum moe_placement {
  MOE_PLACE_ROUND_ROBIN = 0,
  MOE_PLACE_CONTIGUOUS = 1
};
size_t moe_dispatch_owners_workspace_bytes(int T, int k, int E);
int moe_dispatch_owners(int T, int k, int E, int n_owners, int placement, int capacity,
                        const int32_t* topk_ids, int32_t* owner_offsets, int32_t* recv_offsets,
                        int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_pos,
                        const void* x, int d, int act_dtype, void* x_send,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn - grouped gated expert FFN ("Deux roles": the three matrix
 * products a worker runs per expert; ExpertMesh: SwiGLU experts on INT4 weights).  For each local
 * expert e and each row r in [expert_offsets[e], expert_offsets[e+1]):
 *
 *   g = W_gate[e] a,  u = W_up[e] a,  z = act(g) * u,  y_perm[r] = W_down[e] z
 *   with a = x_perm[r].  Accumulation in fp32; z is rounded to act_dtype, or
 *   to fp16 with INT4 weights (beyond fp16's range, 65504, it becomes infinite).
 *
 *   E_loc, d, h     local experts, model width, expert hidden width
 *   rows_max        rows of x_perm / y_perm (>= expert_offsets[E_loc]); the
 *                   offsets are read on the device only
 *   act_dtype       MOE_F32 (requires w_dtype MOE_F32) or MOE_BF16 (w_dtype
 *                   MOE_BF16 or MOE_I4G128)
 *   x_perm          [rows_max, d] act_dtype;   y_perm out [rows_max, d] act_dtype
 *   expert_offsets  [E_loc+1] int32, non-decreasing, offsets[0] = 0;
 *                   NULL = one group of rows_max rows (E_loc must be 1)
 *   w_gate, w_up    [E_loc, h, d]  (MOE_I4G128: uint8 [E_loc, h, d/2])
 *   w_down          [E_loc, d, h]  (MOE_I4G128: uint8 [E_loc, d, h/2])
 *   s_gate, s_up    MOE_I4G128 only: fp16 [E_loc, h, d/128]; s_down [E_loc, d, h/128];
 *                   NULL otherwise
 *   ws, ws_bytes    at least moe_expert_ffn_workspace_bytes()
 * Rows of y_perm outside the groups are left untouched.
 */
size_t moe_expert_ffn_workspace_bytes(int E_loc, int rows_max, int d, int h, int act_dtype);
int moe_expert_ffn(int E_loc, int rows_max, int d, int h, int act, int act_dtype, int w_dtype,
                   const void* x_perm, const int32_t* expert_offsets,
                   const void* w_gate, const void* w_up, const void* w_down,
                   const void* s_gate, const void* s_up, const void* s_down,
                   void* y_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine - weighted top-k combine ("Deux roles": gate-weighted sum of the
 * partial outputs plus the shared expert; ExpertMesh data-flow figure: the
 * expert outputs reduced with the top-k weights).
 *
 *   out[t] = sum_{j ascending, pair_pos[t*k+j] >= 0} topk_w[t,j] * y_perm[pair_pos[t*k+j]]
 *            + shared_y[t]                         (fp32 sum, one final rounding)
 *
 *   y_perm     [rows, d] act_dtype;  pair_pos [T*k] int32;  topk_w [T*k] fp32
 *   shared_y   [T, d] act_dtype or NULL;  out  out [T, d] act_dtype
 * Tokens with no kept pair and no shared expert get zeros.
 */
int moe_combine(int T, int k, int d, int act_dtype, const void* y_perm,
                const int32_t* pair_pos, const float* topk_w, const void* shared_y,
                void* out, void* stream);

/*
 * moe_layer_fwd - the whole layer forward on one stream.
 */
struct moe_layer_desc {
  int T, d, E, k, h;          /* tokens, model width, global experts, top-k, hidden */
  int act;                    /* enum moe_act (routed and shared experts)           */
  int act_dtype;              /* MOE_F32 or MOE_BF16: x, out, w_router, shared weights */
  int w_dtype;                /* routed expert weights: MOE_F32, MOE_BF16, MOE_I4G128 */
  int renorm;                 /* 1: gates divided by their top-k sum                 */
  int capacity;               /* per-expert pair limit, 0 = unlimited                */
  int E_loc;                  /* resident experts (== E without expert_map)          */
  const int32_t* expert_map;  /* [E] global -> local id or -1, or NULL (identity)    */
  const void* w_router;       /* [E, d]; NULL when routing comes as logits_in        */
  const float* expert_bias;   /* [E] or NULL                                         */
  const void* w_gate;         /* routed expert weights and scales, as moe_expert_ffn */
  const void* w_up;
  const void* w_down;
  const void* s_gate;
  const void* s_up;
  const void* s_down;
  int h_shared;               /* 0 = no shared expert                                */
  const void* ws_gate;        /* shared expert [h_shared, d], act_dtype              */
  const void* ws_up;          /* [h_shared, d]                                       */
  const void* ws_down;        /* [d, h_shared]                                       */
  /* Tile hints for the grouped GEMMs, 0 = automatic.  tile_m: rows per tile
   * (16, 32, 64, 128; INT4 weights at most 64; fp32 at most 32; 256 selects
   * the wide bf16 kernel and needs h % 128 == 0 and d % 256 == 0); tile_n_up /
   * tile_n_down: output columns per workgroup of the gate/up and down GEMMs
   * (64 or 128, 128 requiring h resp. d to be a multiple of 128; with
   * tile_m 256: gate/up 64 or 128, down 128 or 256).  Other values give
   * MOE_EUNSUPPORTED. */
  int tile_m, tile_n_up, tile_n_down;
};

/* Optional device outputs of the intermediate results, and optional timing
 * events (any field may be NULL). */
enum {
  MOE_EV_START = 0,           /* before the router                         */
  MOE_EV_ROUTED = 1,          /* after routing (logits, softmax, top-k)     */
  MOE_EV_GROUPED = 2,         /* after the grouping of pairs by expert      */
  MOE_EV_GATE_UP = 3,         /* after the routed gate/up GEMM              */
  MOE_EV_DOWN = 4,            /* after the routed down GEMM                 */
  MOE_EV_SHARED = 5,          /* after the shared expert (if any)           */
  MOE_EV_END = 6,             /* after the combine                          */
  MOE_NUM_EVENTS = 7
};
struct moe_layer_trace {
  float* logits;              /* [T, E] fp32 logits used for selection (router GEMM path) */
  int32_t* topk_ids;          /* [T, k]   */
  float* topk_w;              /* [T, k]   */
  int32_t* expert_offsets;    /* [E_loc+1] */
  int32_t* pair_pos;          /* [T*k]    */
  void* events[MOE_NUM_EVENTS]; /* hipEvent_t handles owned by the caller, each
                                   recorded on `stream` at its step boundary */
  /* router by-products (written when T > 0), as moe_router_stats over the layer's L and topk_ids
   * (all E experts and all T tokens, whatever expert_map keeps local): */
  int32_t* expert_counts;     /* [E]      */
  float* prob_mean;           /* [E]      */
  float* balance_loss;        /* [1]      */
  /* hipEvent_t start/stop pairs (timing-enabled, caller-owned) attached to the
   * launches of the routed gate/up and down GEMMs themselves
   * (hipExtLaunchKernel): they time exactly those kernels and, unlike the
   * step events above, put no extra packet on the stream */
  void* gate_up_kernel_events[2];
  void* down_kernel_events[2];
};

/*
 * moe_layer_plan - how moe_layer_fwd runs the expert GEMMs of layer L (host
 * only; reads the descriptor's sizes and types, no device memory): the tile
 * shapes it picks and whether the shared expert's gate/up and down GEMMs run
 * inside the routed GEMMs' own launches (then the kernel events of
 * moe_layer_trace time those combined launches, and MOE_EV_GATE_UP and
 * MOE_EV_DOWN fall after the shared expert's GEMMs too).  Returns what
 * moe_layer_workspace_bytes would reject L with, else MOE_OK.
 */
struct moe_layer_plan_info {
  int tile_m;                     /* rows per tile of the routed GEMMs (256: wide kernel) */
  int tile_n_up;                  /* output columns per tile of the routed gate/up GEMM   */
  int tile_n_down;                /* output columns per tile of the routed down GEMM      */
  int shared_tile_m;              /* rows per tile of the shared expert's GEMMs, 0 if none */
  int shared_in_routed_launches;  /* 1: the shared expert shares the routed launches;
                                     0: it runs after them, on the same stream          */
};
int moe_layer_plan(const struct moe_layer_desc* L, struct moe_layer_plan_info* out);

/*
 *   x          [T, d] act_dtype (always read: the experts run on it)
 *   logits_in  [T, E] fp32 routing logits (a share that receives its routing
 *              from upstream), or NULL to run the router GEMM on w_router
 *   out        out [T, d] act_dtype
 *   trace      NULL or a struct of optional outputs
 *   ws         at least moe_layer_workspace_bytes(desc)
 * Precision: logits, gates and every sum are fp32.  The gated activations z
 * are rounded to bf16 (bf16 weights) or to fp16 (INT4 weights); the expert
 * and shared-expert outputs are kept in fp16 in bf16 layers (in fp32 in fp32
 * layers) until the combine, which sums in fp32 and rounds once to
 * act_dtype.  An INT4 layer's z or an expert output beyond fp16's range
 * (65504 in magnitude) becomes infinite.
 */
size_t moe_layer_workspace_bytes(const struct moe_layer_desc* L);
int moe_layer_fwd(const struct moe_layer_desc* L, const void* x, const float* logits_in,
                  void* out, const struct moe_layer_trace* trace,
                  void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_bwd - gradients of moe_layer_fwd (the trainers among the sources,
 * MoEEvolve, kieve-moe and moe_stream.py, train this layer; moe_stream.py
 * returns a batch balance loss next to the output).  The routing, the
 * grouping and the gate/up products are recomputed from x as the forward
 * computes them (bit-identical), so only x, the weights and dout are needed.
 * Selection and capacity drops are held fixed (they carry no gradient).
 *
 *   loss = <dout, out> + balance * E * sum_e (count[e] / T) * prob_mean[e]
 *   per kept pair p (token t, slot j, expert e, gate w): the expert's output
 *   gradient is w * dout[t]; d(loss)/d(w) = <dout[t], y_p>; the gates pass it to
 *   the softmax as in moe_route (renorm: w_j = pi_j / sum_sel pi), the softmax
 *   to L, and L = x Wr^T + bias to x, Wr and the bias.
 *
 *   L, x, logits_in  as moe_layer_fwd; w_dtype MOE_I4G128 is not supported
 *   dout       [T, d] act_dtype, upstream gradient of the output
 *   balance    coefficient of the balance loss (0 = none); with expert_map it
 *              belongs to one share only, the loss being per layer
 *   g          output buffers (device, fp32 unless stated; NULL = not wanted):
 *     dx        [T, d] act_dtype, required
 *     dlogits   [T, E]: d(loss)/d(logits_in) (only with logits_in)
 *     dw_router [E, d] (needs w_router);  dbias [E] (needs expert_bias)
 *     dw_gate, dw_up [E_loc, h, d], dw_down [E_loc, d, h]  (gate and up both or neither)
 *     dws_gate, dws_up [h_shared, d], dws_down [d, h_shared] (gate and up both or neither)
 *     dgates    [T, k]: d(loss)/d(topk_w), 0 for pairs not kept
 *   ws         at least moe_layer_bwd_workspace_bytes(L)
 * Gradients are accumulated in fp32 in a fixed order: repeated calls give
 * identical bits.  Expert weight gradients of experts without rows are zero.
 */
struct moe_layer_grads {
  void* dx;
  float* dlogits;
  float* dw_router;
  float* dbias;
  float* dw_gate;
  float* dw_up;
  float* dw_down;
  float* dws_gate;
  float* dws_up;
  float* dws_down;
  float* dgates;
};
size_t moe_layer_bwd_workspace_bytes(const struct moe_layer_desc* L);
int moe_layer_bwd(const struct moe_layer_desc* L, const void* x, const float* logits_in, const void* dout,
                  float balance, const struct moe_layer_grads* g, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_quantize_int4 - weight preparation for MOE_I4G128 (ExpertMesh: bit-exact
 * quantiser of group-scaled signed INT4 weights with FP16 scales).  For each of
 * `rows` rows of K inputs and each 128-input group:
 *   scale = fp16_rne(fp32(max |w|) / 7);  code = clip(rint_even(w / fp32(scale)), -8, 7)
 *   (code 0 when the scale is 0)
 *   w       [rows, K] fp32;  packed out [rows, K/2] uint8;  scales out [rows, K/128] fp16
 * K must be a multiple of 128.
 */
int moe_quantize_int4(int rows, int K, const float* w, uint8_t* packed, uint16_t* scales,
                      void* stream);

/* Static text of an error code; and the text of the last HIP error seen by
 * this thread (empty if none). */
const char* moe_strerror(int code);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LDS_H */
