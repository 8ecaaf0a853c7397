"""Plain float64 oracle of the top-k routed MoE FFN layer forward.

TEST INFRASTRUCTURE: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this module.  It shares no code
with the HIP library.

What the layer computes, and where it is stated:

* Router logits and top-k routing.  "Sharding d'experts" (Kvasir wiki),
  section "Deux rôles", backbone/worker pseudo-code: the backbone multiplies
  the normed activations by the router matrix, applies a softmax, keeps the 8
  most probable experts, and that choice is final.  moe_stream.py,
  ``MoEFFN.forward``: the router is a linear layer without bias, an optional
  per-expert bias is added to the logits before the softmax, the softmax runs
  over all experts, the k largest are kept and their weights are divided by
  their sum.
* Grouping of (token, slot) pairs by expert.  ExpertMesh README, feature list:
  the activations are grouped per expert while each token's identity and
  top-k slot are kept.  MoEEvolve "Architecture": capacity-factor dispatch
  with static shapes, so pairs beyond an expert's capacity are dropped.
* Expert FFN.  kieve-moe "Features": top-k GeGLU experts; MoEEvolve
  "Architecture": SwiGLU experts and one shared expert that is always active;
  ExpertMesh runtime list: SwiGLU experts with INT4 weights.  The gated form
  is ``down(act(gate x) * (up x))`` with no biases.
* Owner-grouped dispatch (sender side of expert parallelism).  ExpertMesh
  README, feature list and data-flow figure: deterministic placement of the
  expert pool across stationary owners, and a dispatcher that groups the
  routed activations by expert owner.
* Backward pass.  The trainers among the pages (MoEEvolve, kieve-moe,
  moe_stream.py) differentiate the layer; the gradients here are the chain
  rule of the forward definition, with the selection held fixed.
* Router by-products.  moe_stream.py ``MoEFFN.forward``: per-expert counts of
  the tokens that chose each expert, the mean softmax probability per expert,
  and the batch-local balance loss built from both.
* Combine.  "Sharding d'experts", "Deux rôles": the backbone adds to the
  residual the gate-weighted sum of the workers' partial outputs and the shared
  expert's output; ExpertMesh data-flow figure: the expert outputs are reduced
  with the top-k weights; moe_stream.py ``MoEFFN.forward``: each expert's
  output is scaled by its gate and scattered back into the rows it came from.
* INT4 weights.  ExpertMesh README: group-scaled signed INT4 weights with FP16
  group scales, laid out ``[expert, output, packed_input]``, plus a bit-exact
  NumPy quantiser and dequantiser.
* Hierarchical (fractal) router.  kieve-moe "Features": a cheap router for very
  large expert pools that routes self-similarly down an expert tree of
  ``branch`` children per node and ``levels`` levels.  The page gives that one
  sentence and no formula: ``tree_route`` is this repository's reading of it
  (below), and its parity is UNPINNED against the page; the pins hold it to the
  reading only.

Readings taken where the pages are silent (each is listed in the design notes
of the repository):

* selection is done on the logits (softmax is strictly increasing, so the
  chosen set is the same as on the probabilities) and ties go to the lower
  expert id; slot j holds the j-th largest logit;
* the gate renormalisation has no epsilon;
* capacity keeps, per expert, the first ``capacity`` pairs in ascending
  flattened pair index p = t*k + j; dropped pairs contribute nothing and the
  surviving gates are not renormalised;
* GeGLU's GELU is the exact erf form; SiLU(g) = g / (1 + exp(-g));
* the shared expert is added with weight 1 on every token;
* placement of experts on owners is round-robin (owner = e mod n, local id
  e div n) unless stated otherwise; a contiguous rule is also provided;
* INT4: per (output row, 128-input group) the scale is
  ``fp16(fp32(max|w|) / 7)`` (both roundings to nearest-even), the code is
  ``clip(rint(w / fp32(scale)), -8, 7)`` with the division in float32 and
  ties to even, an all-zero group (or a scale that rounds to zero) gets code
  0; byte i of a packed row holds input 2i in its low nibble and 2i+1 in its
  high nibble, two's complement; the weight is ``float(scale) * code``;
* hierarchical router: the E experts are the leaves of a tree with ``branch``
  children per node and ``levels`` levels (E <= branch**levels); leaf e is
  reached by the base-``branch`` digits of e, most significant first; node i at
  depth l has children i*branch + c, and a node exists when a leaf below it
  does, so depth l holds ``ceil(E / branch**(levels - l))`` nodes.  Every
  internal node scores its existing children with its own bias-free linear gate
  (one weight row per non-root node) and takes the softmax over them; a leaf's
  probability is the product of the child probabilities on its path.
  Selection is a beam search of width k: at each depth the kept nodes' children
  are ranked by path log-probability (higher first, ties to the lower node id)
  and the best ``min(k, nodes at that depth)`` are kept; the k leaves kept at
  the last depth are the selected experts, slot j the j-th best, and a gate is
  the leaf's path probability, divided by the sum over the k when ``renorm``.

Parity pins: every function here is checked by ``tests/test_oracle_pins.py``
against closed forms, library routines, brute force and invariants.
``tree_route`` and ``tree_path_logprob`` are parity unpinned against the page
(one sentence, no formula): their pins check the reading above.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

INT4_GROUP = 128


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------
def router_logits(x, w_router, bias=None) -> np.ndarray:
    """``L[t, e] = sum_i x[t, i] * Wr[e, i] + b[e]`` in float64.

    "Sharding d'experts", "Deux rôles": activations times the router matrix; moe_stream.py
    ``MoEFFN.forward``: bias-free ``gate`` linear layer plus the optional
    per-expert bias added before the softmax.
    """
    L = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        L = L + np.asarray(bias, np.float64)[None, :]
    return L


def select_topk(L, k: int) -> np.ndarray:
    """The k largest logits of each row, largest first, ties to the lower id.

    moe_stream.py ``MoEFFN.forward`` (``torch.topk`` of the softmax, which is
    sorted); the page leaves ties open, they go to the lower id here.  Done as k rounds of
    "take the first position of the row maximum, then strike it out".
    """
    L = np.asarray(L, np.float64)
    T, E = L.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    work = L.copy()
    ids = np.empty((T, k), np.int64)
    rows = np.arange(T)
    for j in range(k):
        e = np.argmax(work, axis=1)  # first occurrence of the maximum
        ids[:, j] = e
        work[rows, e] = -np.inf
    return ids


def gates(L, ids, renorm: bool) -> np.ndarray:
    """Gate of each selected slot.

    ``pi = softmax(L)`` over all experts (max-subtracted); the gate is
    ``pi[t, ids[t, j]]``, divided by the sum over the k selected when
    ``renorm`` (moe_stream.py ``MoEFFN.forward``), or used as is (the ``p`` of
    the "Deux rôles" pseudo-code).
    """
    L = np.asarray(L, np.float64)
    m = L.max(axis=1, keepdims=True)
    ex = np.exp(L - m)
    pi = ex / ex.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(pi, np.asarray(ids), axis=1)
    if renorm:
        sel = sel / sel.sum(axis=1, keepdims=True)
    return sel


def route(k: int, renorm: bool, x=None, w_router=None, bias=None, logits=None):
    """Router step: returns (L, ids, w).  ``logits`` replaces the GEMM when given
    (a share that receives its routing from upstream, as in the ExpertMesh
    data-flow figure where the router sits before the dispatcher).  A bias is
    added to given logits too."""
    if logits is not None:
        L = np.asarray(logits, np.float64)
        if bias is not None:
            L = L + np.asarray(bias, np.float64)[None, :]
    else:
        L = router_logits(x, w_router, bias)
    ids = select_topk(L, k)
    return L, ids, gates(L, ids, renorm)


def router_stats(L, ids):
    """Router by-products of one batch: per-expert token counts, mean router
    probabilities and the batch-local load-balancing loss.

    moe_stream.py ``MoEFFN.forward``: over the S = T tokens of the batch,
    ``count[e]`` is the number of tokens whose top-k choice contains e (a token
    counts once per expert), ``f[e] = count[e] / T``, ``P[e]`` is the mean over
    tokens of the softmax over all experts (bias included, i.e. of ``L``), and
    the loss is ``E * sum_e f[e] P[e]``.  Ids outside ``[0, E)`` match no
    expert.  T = 0 gives zero counts, zero P and a zero loss (the page divides
    by S and says nothing of an empty batch).  Returns
    ``(count int64 [E], P float64 [E], loss float)``.
    """
    L = np.asarray(L, np.float64)
    T, E = L.shape
    ids = np.asarray(ids)
    ids = ids.reshape(T, ids.shape[-1] if ids.ndim > 1 else -1)
    count = np.array([np.count_nonzero((ids == e).any(axis=1)) for e in range(E)], np.int64)
    if T == 0:
        return count, np.zeros(E), 0.0
    m = L.max(axis=1, keepdims=True)
    ex = np.exp(L - m)
    pi = ex / ex.sum(axis=1, keepdims=True)
    f = count / T
    P = pi.sum(axis=0) / T
    return count, P, float(E * np.sum(f * P))


# --------------------------------------------------------------------------
# Grouping of (token, slot) pairs by expert
# --------------------------------------------------------------------------
def permute(ids, expert_map=None, E_loc: Optional[int] = None, capacity: int = 0):
    """Group the flattened pairs p = t*k + j by (local) expert.

    Returns ``offsets [E_loc+1]``, ``sorted_pair [n_kept]`` (the pair index of
    each grouped row) and ``pair_pos [T*k]`` (row of each pair, -1 when the pair
    is dropped or its expert is not local).  Inside an expert, rows follow
    ascending p; with ``capacity > 0`` only the first ``capacity`` of them are
    kept (ExpertMesh feature list: grouping that keeps token and slot identity;
    MoEEvolve "Architecture": capacity-factor dispatch).
    """
    ids = np.asarray(ids)
    flat = ids.reshape(-1).astype(np.int64)
    if expert_map is not None:
        emap = np.asarray(expert_map, np.int64)
        loc = emap[flat]
        if E_loc is None:
            E_loc = int(emap.max()) + 1
    else:
        loc = flat
        if E_loc is None:
            raise ValueError("E_loc is required without an expert map")
    if capacity < 0:
        raise ValueError("capacity must be >= 0")
    P = flat.size
    pair_pos = np.full(P, -1, np.int64)
    offsets = np.zeros(E_loc + 1, np.int64)
    groups = []
    for e in range(E_loc):
        members = np.nonzero(loc == e)[0]  # ascending p
        if capacity > 0:
            members = members[:capacity]
        groups.append(members)
        offsets[e + 1] = offsets[e] + members.size
    sorted_pair = np.concatenate(groups) if groups else np.zeros(0, np.int64)
    for e in range(E_loc):
        pair_pos[groups[e]] = offsets[e] + np.arange(groups[e].size)
    return offsets, sorted_pair.astype(np.int64), pair_pos


def placement(E: int, n_owners: int, rule: str = "round_robin"):
    """Owner and local id of every expert.

    ExpertMesh README, feature list: the expert pool is placed
    deterministically across stationary owners (896 experts on 32 owners), but
    the rule is not given.  "round_robin": ``owner = e mod n``,
    ``local = e div n``; "contiguous": ``owner = e div (E/n)``,
    ``local = e mod (E/n)``.  E must be a multiple of n.  Returns
    ``(owner int64 [E], local int64 [E])``.
    """
    if n_owners <= 0 or E % n_owners:
        raise ValueError("E must be a positive multiple of n_owners")
    e = np.arange(E)
    per = E // n_owners
    if rule == "round_robin":
        return e % n_owners, e // n_owners
    if rule == "contiguous":
        return e // per, e % per
    raise ValueError(rule)


def owner_dispatch(ids, E: int, n_owners: int, rule: str = "round_robin", capacity: int = 0):
    """Sender side of expert parallelism: every (token, slot) pair grouped by the
    owner of its expert, inside an owner by local expert, inside an expert by
    ascending pair index p = t*k + j; with ``capacity > 0`` only the first
    ``capacity`` pairs of each expert are kept.

    ExpertMesh README: the dispatcher groups the routed activations by expert
    owner (feature list and data-flow figure) and keeps each token's id and
    top-k slot; MoEEvolve "Architecture": capacity-factor dispatch.  Done as one
    stable sort on the key (owner, local, p).  Returns a dict with
    ``sorted_pair``, ``pair_pos`` (-1 for dropped pairs and ids outside
    [0, E)), ``expert_offsets [E+1]`` in (owner, local) order,
    ``owner_offsets [n+1]`` and ``recv_offsets [n, E/n + 1]`` (each owner's
    expert offsets counted from its first row).
    """
    owner, local = placement(E, n_owners, rule)
    per = E // n_owners
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    P = flat.size
    valid = (flat >= 0) & (flat < E)
    p = np.nonzero(valid)[0]
    o, l = owner[flat[p]], local[flat[p]]
    order = np.lexsort((p, l, o))  # last key is the primary one
    p, o, l = p[order], o[order], l[order]
    slot = o * per + l  # position of the expert in owner-major order
    # rank of each pair inside its expert (pairs of one expert are adjacent)
    start = np.searchsorted(slot, slot, side="left")
    keep = np.ones(p.size, bool) if capacity <= 0 else (np.arange(p.size) - start) < capacity
    p, slot = p[keep], slot[keep]
    counts = np.bincount(slot, minlength=E)
    expert_offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    pair_pos = np.full(P, -1, np.int64)
    pair_pos[p] = np.arange(p.size)
    owner_offsets = expert_offsets[::per].copy()
    recv = np.stack([expert_offsets[i * per:(i + 1) * per + 1] - expert_offsets[i * per]
                     for i in range(n_owners)])
    return {"sorted_pair": p.astype(np.int64), "pair_pos": pair_pos, "expert_offsets": expert_offsets,
            "owner_offsets": owner_offsets, "recv_offsets": recv}


# --------------------------------------------------------------------------
# Expert FFN
# --------------------------------------------------------------------------
def silu(g):
    """SiLU(g) = g / (1 + exp(-g)) (the SwiGLU gate of MoEEvolve's experts)."""
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def gelu_erf(g):
    """Exact GELU, g * Phi(g) = 0.5 g (1 + erf(g / sqrt 2)) (kieve-moe's GeGLU;
    moe_stream.py's experts use the default, exact form of ``nn.GELU``)."""
    g = np.asarray(g, np.float64)
    return 0.5 * g * (1.0 + _erf(g / np.sqrt(2.0)))


_ACTS = {"swiglu": silu, "geglu": gelu_erf}


def gated_ffn(a, wg, wu, wd, act: str) -> np.ndarray:
    """``y = Wd (act(Wg a) * (Wu a))`` for each row a; weights ``[out, in]``.

    Three matrices per expert (the kieve-moe "Parametric sizing" flagship,
    15 layers x 32 experts of H=768, I=4096, is 4.5B parameters only with three
    matrices per expert)."""
    a = np.asarray(a, np.float64)
    g = a @ np.asarray(wg, np.float64).T
    u = a @ np.asarray(wu, np.float64).T
    z = _ACTS[act](g) * u
    return z @ np.asarray(wd, np.float64).T


def act_grad(g, act: str) -> np.ndarray:
    """Derivative of the gate activation: SiLU' = s (1 + g (1 - s)) with s the
    logistic sigmoid; GELU' = Phi(g) + g phi(g) (standard normal cdf and pdf)."""
    g = np.asarray(g, np.float64)
    if act == "swiglu":
        with np.errstate(over="ignore"):
            sg = 1.0 / (1.0 + np.exp(-g))
        return sg * (1.0 + g * (1.0 - sg))
    if act == "geglu":
        return 0.5 * (1.0 + _erf(g / np.sqrt(2.0))) + g * np.exp(-0.5 * g * g) / np.sqrt(2.0 * np.pi)
    raise ValueError(act)


def gated_ffn_bwd(a, wg, wu, wd, act: str, dy):
    """Chain rule through ``y = Wd (act(Wg a) * (Wu a))`` for rows ``a`` with
    upstream ``dy``: ``dz = dy Wd``, ``dWd = dy^T z``, ``dg = dz * u * act'(g)``,
    ``du = dz * act(g)``, ``da = dg Wg + du Wu``, ``dWg = dg^T a``,
    ``dWu = du^T a``.  Returns ``(da, dWg, dWu, dWd)``."""
    a = np.asarray(a, np.float64)
    wg, wu, wd = (np.asarray(m, np.float64) for m in (wg, wu, wd))
    dy = np.asarray(dy, np.float64)
    g = a @ wg.T
    u = a @ wu.T
    ag = _ACTS[act](g)
    z = ag * u
    dz = dy @ wd
    dg = dz * u * act_grad(g, act)
    du = dz * ag
    return dg @ wg + du @ wu, dg.T @ a, du.T @ a, dy.T @ z


def moe_layer_bwd(x, weights: LayerWeights, k: int, renorm: bool, act: str, dout, *,
                  w_router=None, logits=None, bias=None, expert_map=None, capacity: int = 0,
                  shared: Optional[Sequence] = None, balance: float = 0.0, ids=None):
    """Gradients of the layer forward (float64) for an upstream gradient ``dout``
    of its output, plus ``balance`` times the gradient of the batch balance
    loss (the trainers of moe_stream.py, MoEEvolve and kieve-moe train the
    layer; moe_stream.py ``MoEFFN.forward`` returns the balance loss next to the
    output and the model adds it with a small coefficient).

    The selection (top-k ids, capacity drops) and the expert counts of the
    balance loss are piecewise constant and carry no gradient.  Per kept pair p
    of token t, slot j, expert e: ``dw[t, j] = <dout[t], y_p>`` and the expert
    receives ``dy_p = w[t, j] dout[t]``.  Gates: with ``renorm``,
    ``w_j = pi_j / S`` over the k selected, so ``dpi_i = dw_i / S -
    sum_j dw_j pi_j / S^2``; without, ``dpi_i = dw_i``.  Balance loss
    ``E / T^2 sum_e count_e sum_t pi[t, e]``: ``dpi[t, e] += balance * E *
    count_e / T^2``.  Softmax: ``dL = pi * (dpi - <dpi, pi>)``.  Router:
    ``dx += dL Wr``, ``dWr = dL^T x``, ``dbias = sum_t dL``; with given logits
    ``dlogits = dL``.  ``ids`` overrides the selection as in ``moe_layer``.
    Returns a dict of the gradients (weights of local experts only; None
    where the input does not exist).
    """
    x = np.asarray(x, np.float64)
    dout = np.asarray(dout, np.float64)
    T, d = x.shape
    L, ids_o, w = route(k, renorm, x=x, w_router=w_router, bias=bias, logits=logits)
    if ids is not None:
        ids_o = np.asarray(ids, np.int64)
        w = gates(L, ids_o, renorm)
    ids = ids_o
    E = L.shape[1]
    E_loc = weights.E_loc
    offsets, sorted_pair, pair_pos = permute(ids, expert_map, E_loc, capacity)
    dx = np.zeros((T, d))
    dw = np.zeros((T, k))
    wg0, wu0, wd0 = weights.expert(0)
    dWg = np.zeros((E_loc,) + wg0.shape)
    dWu = np.zeros((E_loc,) + wu0.shape)
    dWd = np.zeros((E_loc,) + wd0.shape)
    for e in range(E_loc):
        rows = sorted_pair[offsets[e]:offsets[e + 1]]
        if rows.size == 0:
            continue
        t, j = rows // k, rows % k
        wg, wu, wd = weights.expert(e)
        y = gated_ffn(x[t], wg, wu, wd, act)
        dw[t, j] = np.sum(dout[t] * y, axis=1)
        da, dWg[e], dWu[e], dWd[e] = gated_ffn_bwd(x[t], wg, wu, wd, act, w[t, j][:, None] * dout[t])
        np.add.at(dx, t, da)
    dshared = None
    if shared is not None:
        da, gsg, gsu, gsd = gated_ffn_bwd(x, shared[0], shared[1], shared[2], act, dout)
        dx += da
        dshared = (gsg, gsu, gsd)
    m = L.max(axis=1, keepdims=True)
    ex = np.exp(L - m)
    pi = ex / ex.sum(axis=1, keepdims=True)
    dpi = np.zeros((T, E))
    rows = np.arange(T)[:, None]
    if renorm:
        psel = np.take_along_axis(pi, ids, axis=1)
        S = psel.sum(axis=1, keepdims=True)
        dsel = dw / S - np.sum(dw * psel, axis=1, keepdims=True) / S ** 2
    else:
        dsel = dw
    np.add.at(dpi, (np.broadcast_to(rows, ids.shape), ids), dsel)
    if balance:
        count = router_stats(L, ids)[0]
        dpi += balance * E * count[None, :] / float(T * T)
    dL = pi * (dpi - np.sum(dpi * pi, axis=1, keepdims=True))
    out = {"dx": dx, "dw_gate": dWg, "dw_up": dWu, "dw_down": dWd, "dshared": dshared,
           "dw_router": None, "dlogits": None, "dbias": None, "dgates": dw, "dL": dL}
    if logits is None:
        Wr = np.asarray(w_router, np.float64)
        out["dx"] = dx + dL @ Wr
        out["dw_router"] = dL.T @ x
    else:
        out["dlogits"] = dL
    if bias is not None:
        out["dbias"] = dL.sum(axis=0)
    return out


# --------------------------------------------------------------------------
# Signed INT4 with fp16 group scales
# --------------------------------------------------------------------------
def pack_int4(q) -> np.ndarray:
    """int codes [N, K] in [-8, 7] -> bytes [N, K/2]; input 2i in the low nibble."""
    q = np.asarray(q)
    if q.shape[-1] % 2:
        raise ValueError("K must be even")
    if q.min(initial=0) < -8 or q.max(initial=0) > 7:
        raise ValueError("codes out of the signed 4-bit range")
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed) -> np.ndarray:
    """bytes [N, K/2] -> int8 codes [N, K] (two's complement nibbles)."""
    b = np.asarray(packed, np.uint8)
    lo = (b & 0xF).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def quantize_int4(w):
    """float32 weights [..., N, K] -> (packed uint8 [..., N, K/2], scales float16 [..., N, K/128]).

    Per output row and 128-input group: ``s = fp16(fp32(max|w|) / 7)``,
    ``q = clip(rint(w / fp32(s)), -8, 7)`` (float32 division, ties to even);
    a zero scale gives code 0."""
    w32 = np.asarray(w, np.float32)
    K = w32.shape[-1]
    if K % INT4_GROUP:
        raise ValueError("K must be a multiple of 128")
    grp = w32.reshape(w32.shape[:-1] + (K // INT4_GROUP, INT4_GROUP))
    amax = np.abs(grp).max(axis=-1)                     # exact in float32
    s16 = (amax / np.float32(7.0)).astype(np.float16)   # float32 divide, then RNE to fp16
    sf = s16.astype(np.float32)[..., None]
    safe = np.where(sf > 0, sf, np.float32(1.0))
    q = np.where(sf > 0, np.rint(grp / safe), np.float32(0.0))  # float32 divide, rint = ties-to-even
    q = np.clip(q, -8, 7).astype(np.int8).reshape(w32.shape)
    return pack_int4(q), s16


def dequantize_int4(packed, scales) -> np.ndarray:
    """(packed [..., N, K/2], fp16 scales [..., N, K/128]) -> float64 ``scale * code``."""
    q = unpack_int4(packed).astype(np.float64)
    s = np.asarray(scales, np.float16).astype(np.float64)
    K = q.shape[-1]
    return (q.reshape(q.shape[:-1] + (K // INT4_GROUP, INT4_GROUP)) * s[..., None]).reshape(q.shape)


# --------------------------------------------------------------------------
# Output rounding
# --------------------------------------------------------------------------
def round_to_dtype(v, dt: str) -> np.ndarray:
    """Round float64 values once, to nearest-even, to ``dt`` ("f32" | "bf16"),
    returned as float64."""
    v = np.asarray(v, np.float64)
    if dt == "f64":
        return v.copy()
    if dt == "f32":
        return v.astype(np.float32).astype(np.float64)
    if dt == "bf16":
        _, e = np.frexp(v)
        e = np.maximum(e, -125)           # below bf16's normal range the spacing stays 2**-133
        return np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)
    raise ValueError(dt)


# --------------------------------------------------------------------------
# The layer
# --------------------------------------------------------------------------
@dataclasses.dataclass
class LayerWeights:
    """Local expert weights in float64, or INT4 packed codes and fp16 scales."""
    wg: Optional[np.ndarray] = None       # [E_loc, h, d]
    wu: Optional[np.ndarray] = None
    wd: Optional[np.ndarray] = None       # [E_loc, d, h]
    qg: Optional[tuple] = None            # (packed [E_loc, h, d/2], scales [E_loc, h, d/128])
    qu: Optional[tuple] = None
    qd: Optional[tuple] = None            # (packed [E_loc, d, h/2], scales [E_loc, d, h/128])

    @property
    def E_loc(self) -> int:
        return (self.wg if self.wg is not None else self.qg[0]).shape[0]

    def expert(self, e: int):
        if self.wg is not None:
            return self.wg[e], self.wu[e], self.wd[e]
        return (dequantize_int4(self.qg[0][e], self.qg[1][e]),
                dequantize_int4(self.qu[0][e], self.qu[1][e]),
                dequantize_int4(self.qd[0][e], self.qd[1][e]))


def moe_layer(x, weights: LayerWeights, k: int, renorm: bool, act: str, *,
              w_router=None, logits=None, bias=None, expert_map=None, capacity: int = 0,
              shared: Optional[Sequence] = None, tokens=None, ids=None):
    """Forward pass of the layer (float64, not rounded).

    ``out[t] = sum_{j: pair kept} w[t, j] * y[t*k + j] + shared(x[t])``, the
    sum taken in ascending slot order, ``y`` being the pair's expert FFN of
    ``x[t]`` (the combine of the "Deux rôles" pseudo-code).  ``tokens``
    restricts the output to those rows (routing and capacity still look at all
    tokens).  ``ids`` overrides the selection (gates are then taken from the
    oracle's own logits at those ids).
    Returns a dict with ``out`` and the routing intermediates.
    """
    x = np.asarray(x, np.float64)
    T, d = x.shape
    L, ids_o, w = route(k, renorm, x=x, w_router=w_router, bias=bias, logits=logits)
    if ids is not None:
        ids_o = np.asarray(ids, np.int64)
        w = gates(L, ids_o, renorm)
    E_loc = weights.E_loc
    offsets, sorted_pair, pair_pos = permute(ids_o, expert_map, E_loc, capacity)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    want = np.zeros(T, bool)
    want[toks] = True
    Y = np.zeros((T, k, d), np.float64)
    for e in range(E_loc):
        rows = sorted_pair[offsets[e]:offsets[e + 1]]
        rows = rows[want[rows // k]]
        if rows.size == 0:
            continue
        wg, wu, wd = weights.expert(e)
        Y[rows // k, rows % k] = gated_ffn(x[rows // k], wg, wu, wd, act)
    shared_y = None
    if shared is not None:
        shared_y = gated_ffn(x[toks], shared[0], shared[1], shared[2], act)
    out = combine(Y[toks], pair_pos.reshape(T, k)[toks], w[toks], shared_y)
    return {"out": out, "L": L, "ids": ids_o, "w": w, "offsets": offsets,
            "sorted_pair": sorted_pair, "pair_pos": pair_pos, "tokens": toks}


def combine(y_slots, pair_pos, w, shared_y=None) -> np.ndarray:
    """Weighted top-k combine of one token row at a time.

    ``y_slots [T, k, d]`` holds each slot's expert output, ``pair_pos [T, k]``
    marks kept slots (>= 0), ``w [T, k]`` the gates:
    ``out[t] = sum_{j ascending, kept} w[t, j] y[t, j] (+ shared_y[t])`` ("Deux
    rôles": gate-weighted partial outputs plus the shared expert; ExpertMesh:
    expert outputs reduced with the top-k weights; moe_stream.py: each expert's
    output scaled by its gate and added back into its token's row)."""
    y_slots = np.asarray(y_slots, np.float64)
    T, k, d = y_slots.shape
    kept = np.asarray(pair_pos) >= 0
    out = np.zeros((T, d), np.float64)
    for j in range(k):
        out += np.where(kept[:, j], np.asarray(w, np.float64)[:, j], 0.0)[:, None] * y_slots[:, j]
    if shared_y is not None:
        out += np.asarray(shared_y, np.float64)
    return out


# --------------------------------------------------------------------------
# Hierarchical (fractal) router: reading of kieve-moe "Features"; parity
# unpinned against the page
# --------------------------------------------------------------------------
def tree_nodes(E: int, branch: int, levels: int):
    """Existing nodes per depth, ``n[l] = ceil(E / branch**(levels - l))`` for
    l = 0..levels (n[0] = 1 root, n[levels] = E leaves), and the first gate row
    of each depth's children: ``first[l] = branch * (n[0] + ... + n[l-1])``.
    The child j of depth l+1 (j < branch * n[l]) has gate row ``first[l] + j``;
    the table has ``first[levels]`` rows."""
    if branch < 2 or levels < 1 or not (1 <= E <= branch ** levels):
        raise ValueError("need branch >= 2, levels >= 1, 1 <= E <= branch**levels")
    n = [-(-E // branch ** (levels - l)) for l in range(levels + 1)]
    first = [branch * sum(n[:l]) for l in range(levels + 1)]
    return n, first


def _children_logprob(xt, W, first_l, node, branch, n_next):
    """log-softmax of one node's existing children: (child ids, log p)."""
    kids = np.arange(node * branch, min(node * branch + branch, n_next))
    z = W[first_l + kids] @ xt
    m = z.max()
    return kids, z - (m + np.log(np.sum(np.exp(z - m))))


def tree_route(k: int, renorm: bool, x, w_tree, branch: int, levels: int, E: int):
    """Beam-search routing down the expert tree, one token at a time.

    Returns ``(ids [T, k] int64, w [T, k] float64, margin [T] float64)``;
    ``margin[t]`` is the smallest log-probability gap on which the token's
    result depends: at every depth between the last kept and the first dropped
    candidate, and at the last depth also between consecutive kept ones
    (+inf when nothing is dropped and k = 1)."""
    x = np.asarray(x, np.float64)
    W = np.asarray(w_tree, np.float64)
    n, first = tree_nodes(E, branch, levels)
    if W.shape != (first[levels], x.shape[1]):
        raise ValueError("w_tree must be [%d, d]" % first[levels])
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    T = x.shape[0]
    ids = np.empty((T, k), np.int64)
    w = np.empty((T, k), np.float64)
    margin = np.full(T, np.inf)
    for t in range(T):
        beam = [(0.0, 0)]  # (path log-probability, node id) at depth 0
        for l in range(levels):
            cand = []
            for score, node in beam:
                kids, lp = _children_logprob(x[t], W, first[l], node, branch, n[l + 1])
                cand += [(score + v, int(c)) for c, v in zip(kids, lp)]
            cand.sort(key=lambda sv: (-sv[0], sv[1]))
            keep = min(k, n[l + 1])
            if len(cand) > keep:
                margin[t] = min(margin[t], cand[keep - 1][0] - cand[keep][0])
            if l == levels - 1:
                for a, b in zip(cand[:keep - 1], cand[1:keep]):
                    margin[t] = min(margin[t], a[0] - b[0])
            beam = cand[:keep]
        ids[t] = [node for _, node in beam]
        p = np.exp([score for score, _ in beam])
        w[t] = p / p.sum() if renorm else p
    return ids, w, margin


def tree_path_logprob(x, w_tree, branch: int, levels: int, E: int, ids):
    """Path log-probability of given leaves: ``lp[t, j] = log P(ids[t, j] | x[t])``,
    the sum over the path's depths of the child's log-softmax within its
    parent (the same definition as ``tree_route``'s scores, for any leaf)."""
    x = np.asarray(x, np.float64)
    W = np.asarray(w_tree, np.float64)
    n, first = tree_nodes(E, branch, levels)
    ids = np.asarray(ids)
    lp = np.zeros(ids.shape, np.float64)
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            for l in range(levels):
                node = e // branch ** (levels - l)
                child = e // branch ** (levels - l - 1)
                kids, v = _children_logprob(x[t], W, first[l], node, branch, n[l + 1])
                lp[t, j] += v[child - kids[0]]
    return lp
