"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against a hand-worked fixture, a closed
form, a library routine, brute force on tiny inputs, or an invariant of the
method, chosen so that a dropped term, a wrong sign or index, or a transposed
operand fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as orc
from golden_io import activation_points, int4_case, route_cases, tree_route_cases

RNG = np.random.default_rng(1234)


def _rand_layer(T, d, E, k, h, *, E_loc=None, dtype=np.float64, shared_h=0, seed=0):
    rng = np.random.default_rng(seed)
    E_loc = E if E_loc is None else E_loc
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) / np.sqrt(d)
    W = orc.LayerWeights(wg=rng.standard_normal((E_loc, h, d)) / np.sqrt(d),
                         wu=rng.standard_normal((E_loc, h, d)) / np.sqrt(d),
                         wd=rng.standard_normal((E_loc, d, h)) / np.sqrt(h))
    shared = None
    if shared_h:
        shared = (rng.standard_normal((shared_h, d)) / np.sqrt(d),
                  rng.standard_normal((shared_h, d)) / np.sqrt(d),
                  rng.standard_normal((d, shared_h)) / np.sqrt(shared_h))
    return x, wr, W, shared


# ---------------------------------------------------------------- routing
@pytest.mark.parametrize("case", route_cases())
def test_route_worked_examples(case):
    L = np.array([case["logits"]])
    ids = orc.select_topk(L, case["k"])
    assert ids[0].tolist() == case["ids"]
    np.testing.assert_allclose(orc.gates(L, ids, True)[0], case["w_renorm"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(orc.gates(L, ids, False)[0], case["w_raw"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("E,k", [(8, 2), (32, 2), (192, 4), (128, 8), (896, 16), (5, 5)])
def test_selection_equals_stable_sort(E, k):
    # integer-valued logits from a small range: many exact ties
    L = RNG.integers(-3, 4, size=(300, E)).astype(np.float64)
    ref = np.argsort(-L, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(orc.select_topk(L, k), ref)
    L2 = RNG.standard_normal((200, E))
    np.testing.assert_array_equal(orc.select_topk(L2, k),
                                  np.argsort(-L2, axis=1, kind="stable")[:, :k])


@pytest.mark.parametrize("E", [1, 2, 3, 4, 5, 6])
def test_selection_brute_force_over_subsets(E):
    for k in range(1, E + 1):
        for _ in range(40):
            row = RNG.integers(0, 3, size=E).astype(np.float64)

            def beats(a, b):
                return row[a] > row[b] or (row[a] == row[b] and a < b)
            winners = [S for S in itertools.combinations(range(E), k)
                       if all(beats(s, o) for s in S for o in range(E) if o not in S)]
            assert len(winners) == 1
            S = sorted(winners[0], key=lambda e: (-row[e], e))
            assert orc.select_topk(row[None, :], k)[0].tolist() == S


def test_gates_closed_forms_and_invariants():
    for E, k in [(8, 2), (192, 4), (128, 8), (896, 16)]:
        L = RNG.standard_normal((100, E)) * 3
        ids = orc.select_topk(L, k)
        sel = np.take_along_axis(L, ids, axis=1)
        w_r = orc.gates(L, ids, True)
        w_n = orc.gates(L, ids, False)
        # renormalised gates = softmax over the selected logits only (library softmax)
        np.testing.assert_allclose(w_r, scipy.special.softmax(sel, axis=1), rtol=1e-14, atol=1e-16)
        # raw gates = the selected entries of the full softmax (library softmax)
        np.testing.assert_allclose(w_n, np.take_along_axis(scipy.special.softmax(L, axis=1), ids, 1),
                                   rtol=1e-14, atol=1e-18)
        np.testing.assert_allclose(w_r.sum(1), 1.0, rtol=0, atol=1e-14)
        assert np.all(np.diff(w_r, axis=1) <= 0) and np.all(np.diff(w_n, axis=1) <= 0)
        assert np.all(w_n.sum(1) <= 1 + 1e-14)
    # k = E: raw gates are the whole softmax and sum to one
    L = RNG.standard_normal((50, 7))
    assert np.allclose(orc.gates(L, orc.select_topk(L, 7), False).sum(1), 1.0, atol=1e-14)


def test_bias_shifts_logits_before_selection():
    x = RNG.standard_normal((20, 16))
    wr = RNG.standard_normal((6, 16))
    b = np.array([0, 0, 100.0, 0, 0, 0])
    L, ids, w = orc.route(2, True, x=x, w_router=wr, bias=b)
    assert np.all(ids[:, 0] == 2)  # a huge bias wins every token
    np.testing.assert_allclose(L, x @ wr.T + b, rtol=1e-14, atol=1e-12)


def test_zero_input_special_case():
    T, d, E, k, h = 16, 32, 8, 3, 16
    _, wr, W, shared = _rand_layer(T, d, E, k, h, shared_h=8)
    x = np.zeros((T, d))
    for renorm, g in [(True, 1 / k), (False, 1 / E)]:
        r = orc.moe_layer(x, W, k, renorm, "swiglu", w_router=wr, shared=shared)
        assert np.all(r["ids"] == np.arange(k))
        np.testing.assert_allclose(r["w"], g, rtol=1e-15)
        assert np.all(r["out"] == 0.0)


# ---------------------------------------------------------------- router by-products
def test_router_stats_uniform_logits_give_loss_k():
    """Equal logits: P = 1/E (to rounding), so the loss is the mean number of distinct
    experts per token, k for distinct ids.  Dividing f by T*k, dropping the
    factor E, or using the top-k gates for P all miss this."""
    T, E, k = 37, 9, 3
    L = np.full((T, E), 0.25)
    ids = orc.select_topk(L, k)
    cnt, P, loss = orc.router_stats(L, ids)
    np.testing.assert_allclose(P, np.full(E, 1.0 / E), rtol=1e-14)
    assert cnt.sum() == T * k
    assert loss == pytest.approx(k, rel=1e-14)


@pytest.mark.parametrize("E", [4, 8, 64])
def test_router_stats_one_hot_extremes(E):
    """k = 1 with a margin of 60 nats: all tokens on one expert gives loss E;
    tokens spread evenly over the experts gives loss 1 (the two bounds of the
    loss for one-hot routing); the closed-form P of a two-level row
    ``e^a / (e^a + E - 1)`` is checked on the way."""
    T, a = 4 * E, 60.0
    L = np.zeros((T, E))
    L[:, 2] = a
    cnt, P, loss = orc.router_stats(L, orc.select_topk(L, 1))
    assert cnt[2] == T and cnt.sum() == T
    top = math.exp(a) / (math.exp(a) + E - 1)
    assert P[2] == pytest.approx(top, rel=1e-15)
    assert loss == pytest.approx(E * top, rel=1e-14)
    L = np.zeros((T, E))
    L[np.arange(T), np.arange(T) % E] = a
    cnt, P, loss = orc.router_stats(L, orc.select_topk(L, 1))
    np.testing.assert_array_equal(cnt, np.full(E, T // E))
    assert loss == pytest.approx(top, rel=1e-14)


def test_router_stats_brute_force_with_duplicate_and_foreign_ids():
    """Per-token sets and math.fsum on a tiny batch; ids repeat inside a row
    (the token counts once) and some lie outside [0, E) (they match nothing)."""
    rng = np.random.default_rng(3)
    T, E, k = 11, 5, 3
    L = rng.standard_normal((T, E)) * 2
    ids = rng.integers(-2, E + 2, size=(T, k))
    ids[0] = [1, 1, 1]
    cnt, P, loss = orc.router_stats(L, ids)
    bc = [0] * E
    cols = [[] for _ in range(E)]
    for t in range(T):
        for e in set(int(v) for v in ids[t]):
            if 0 <= e < E:
                bc[e] += 1
        row = [math.exp(v) for v in L[t]]
        z = math.fsum(row)
        for e in range(E):
            cols[e].append(row[e] / z)
    Pb = [math.fsum(c) / T for c in cols]
    lb = E * math.fsum(bc[e] / T * Pb[e] for e in range(E))
    np.testing.assert_array_equal(cnt, bc)
    np.testing.assert_allclose(P, Pb, rtol=1e-13)
    assert loss == pytest.approx(lb, rel=1e-13)


def test_router_stats_invariants():
    """P sums to 1; counts equal the expert histogram of the grouping step (no
    capacity, distinct ids); relabelling the experts permutes counts and P and
    keeps the loss; shuffling tokens changes nothing; T = 0 gives zeros."""
    rng = np.random.default_rng(5)
    T, E, k = 200, 16, 4
    L = rng.standard_normal((T, E)) + np.log(np.arange(1, E + 1))[None, :]
    ids = orc.select_topk(L, k)
    cnt, P, loss = orc.router_stats(L, ids)
    assert P.sum() == pytest.approx(1.0, rel=1e-14)
    offsets = orc.permute(ids, E_loc=E)[0]
    np.testing.assert_array_equal(cnt, np.diff(offsets))
    perm = rng.permutation(E)
    inv = np.argsort(perm)
    cnt2, P2, loss2 = orc.router_stats(L[:, perm], inv[ids])
    np.testing.assert_array_equal(cnt2, cnt[perm])
    np.testing.assert_allclose(P2, P[perm], rtol=1e-14)
    assert loss2 == pytest.approx(loss, rel=1e-14)
    tp = rng.permutation(T)
    cnt3, P3, loss3 = orc.router_stats(L[tp], ids[tp])
    np.testing.assert_array_equal(cnt3, cnt)
    np.testing.assert_allclose(P3, P, rtol=1e-13)
    cnt0, P0, loss0 = orc.router_stats(np.zeros((0, E)), np.zeros((0, k), np.int64))
    assert cnt0.sum() == 0 and not P0.any() and loss0 == 0.0


def test_router_stats_p_matches_torch_softmax_column_mean():
    """P against torch's float64 softmax, with a per-expert bias added."""
    rng = np.random.default_rng(9)
    L = rng.standard_normal((64, 12)) * 3
    b = rng.standard_normal(12)
    _, P, _ = orc.router_stats(L + b, orc.select_topk(L + b, 2))
    ref = torch.softmax(torch.from_numpy(L + b), dim=-1).mean(0).numpy()
    np.testing.assert_allclose(P, ref, rtol=1e-13)


# ---------------------------------------------------------------- permutation
@pytest.mark.parametrize("T,k,E,owners", [(64, 2, 8, 1), (333, 4, 192, 1), (512, 16, 896, 32),
                                          (100, 8, 128, 4)])
def test_permutation_equals_stable_sort(T, k, E, owners):
    L = RNG.standard_normal((T, E))
    ids = orc.select_topk(L, k)
    emap = np.full(E, -1)
    mine = np.arange(0, E, owners)
    emap[mine] = np.arange(mine.size)
    E_loc = mine.size
    offsets, sp, pos = orc.permute(ids, emap if owners > 1 else None, E_loc)
    loc = emap[ids.reshape(-1)]
    order = np.argsort(np.where(loc < 0, E_loc, loc), kind="stable")  # library stable sort
    n_kept = int((loc >= 0).sum())
    np.testing.assert_array_equal(sp, order[:n_kept])
    np.testing.assert_array_equal(np.diff(offsets), np.bincount(loc[loc >= 0], minlength=E_loc))
    assert offsets[-1] == n_kept
    np.testing.assert_array_equal(pos[sp], np.arange(n_kept))
    assert np.all(pos[loc < 0] == -1)


def test_permutation_capacity_invariants():
    T, k, E, cap = 500, 4, 16, 97
    ids = orc.select_topk(RNG.standard_normal((T, E)) + np.linspace(2, 0, E), k)
    offsets, sp, pos = orc.permute(ids, None, E, cap)
    cnt = np.bincount(ids.reshape(-1), minlength=E)
    np.testing.assert_array_equal(np.diff(offsets), np.minimum(cnt, cap))
    assert np.all(np.diff(offsets) >= 0)
    for e in range(E):
        rows = sp[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(rows) > 0)                    # ascending p inside an expert
        assert np.all(ids.reshape(-1)[rows] == e)
    np.testing.assert_array_equal(pos[sp], np.arange(sp.size))
    assert (pos >= 0).sum() == sp.size


def test_capacity_brute_force_sequential_dispatch():
    # exhaustive over tiny cases: a sequential per-expert counter that admits
    # a pair while its expert has room (static-capacity dispatch in token order)
    E, k = 3, 2
    choices = list(itertools.permutations(range(E), k))
    for T in (1, 2, 3):
        for combo in itertools.product(choices, repeat=T):
            ids = np.array(combo)
            for cap in (0, 1, 2, 3):
                counter = [0] * E
                expect = []
                for p, e in enumerate(ids.reshape(-1)):
                    if cap == 0 or counter[e] < cap:
                        counter[e] += 1
                        expect.append(True)
                    else:
                        expect.append(False)
                _, _, pos = orc.permute(ids, None, E, cap)
                assert (pos >= 0).tolist() == expect


# ---------------------------------------------------------------- owner-grouped dispatch
@pytest.mark.parametrize("rule", ["round_robin", "contiguous"])
@pytest.mark.parametrize("cap", [0, 2])
def test_owner_dispatch_brute_force(rule, cap):
    """Python's sorted() on (owner, local, p) tuples with a per-expert counter,
    ids outside [0, E) included; capacity keeps the first pairs of each expert."""
    rng = np.random.default_rng(4)
    T, k, E, n = 13, 3, 12, 4
    ids = rng.integers(-1, E + 1, size=(T, k))
    per = E // n
    own = (lambda e: e % n) if rule == "round_robin" else (lambda e: e // per)
    loc = (lambda e: e // n) if rule == "round_robin" else (lambda e: e % per)
    keys = sorted((own(int(e)), loc(int(e)), p) for p, e in enumerate(ids.reshape(-1)) if 0 <= e < E)
    seen = {}
    rows = []
    for o, l, p in keys:
        seen[(o, l)] = seen.get((o, l), 0) + 1
        if cap == 0 or seen[(o, l)] <= cap:
            rows.append((o, l, p))
    r = orc.owner_dispatch(ids, E, n, rule, capacity=cap)
    np.testing.assert_array_equal(r["sorted_pair"], [p for _, _, p in rows])
    pos = [-1] * (T * k)
    for i, (_, _, p) in enumerate(rows):
        pos[p] = i
    np.testing.assert_array_equal(r["pair_pos"], pos)
    for o in range(n):
        mine = [i for i, row in enumerate(rows) if row[0] == o]
        assert r["owner_offsets"][o + 1] - r["owner_offsets"][o] == len(mine)
        for l in range(per):
            cnt = sum(1 for row in rows if row[0] == o and row[1] == l)
            assert r["recv_offsets"][o, l + 1] - r["recv_offsets"][o, l] == cnt
    assert r["owner_offsets"][-1] == len(rows) == r["expert_offsets"][-1]


def test_owner_dispatch_special_cases():
    """One owner is the plain grouping by expert; one expert per owner makes
    owner offsets equal expert offsets; the composed map (owner * E/n + local)
    handed to the grouping step gives the same rows."""
    rng = np.random.default_rng(8)
    T, k, E = 50, 4, 16
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    off, sp, pos = orc.permute(ids, E_loc=E)
    r = orc.owner_dispatch(ids, E, 1)
    np.testing.assert_array_equal(r["sorted_pair"], sp)
    np.testing.assert_array_equal(r["pair_pos"], pos)
    np.testing.assert_array_equal(r["recv_offsets"][0], off)
    r = orc.owner_dispatch(ids, E, E, "contiguous")
    np.testing.assert_array_equal(r["owner_offsets"], off)
    for n, rule, cap in [(4, "round_robin", 0), (8, "contiguous", 5), (2, "round_robin", 3)]:
        owner, local = orc.placement(E, n, rule)
        off, sp, pos = orc.permute(ids, expert_map=owner * (E // n) + local, E_loc=E, capacity=cap)
        r = orc.owner_dispatch(ids, E, n, rule, capacity=cap)
        np.testing.assert_array_equal(r["expert_offsets"], off)
        np.testing.assert_array_equal(r["sorted_pair"], sp)
        np.testing.assert_array_equal(r["pair_pos"], pos)


def test_round_robin_share_of_owner_zero():
    """896 experts on 32 owners: owner 0 holds 0, 32, ..., 864 with local ids
    0..27, the share of the INT4 workload recipe."""
    from moe_synth import CONFIGS
    owner, local = orc.placement(896, 32)
    mine = np.nonzero(owner == 0)[0]
    np.testing.assert_array_equal(mine, np.arange(0, 896, 32))
    np.testing.assert_array_equal(local[mine], np.arange(28))
    assert mine.tolist() == CONFIGS["int4_share"].local_experts()
    assert np.bincount(owner).tolist() == [28] * 32


# ---------------------------------------------------------------- expert FFN
@pytest.mark.parametrize("name,g,v", activation_points())
def test_activation_textbook_points(name, g, v):
    f = orc.silu if name == "silu" else orc.gelu_erf
    assert abs(float(f(g)) - v) <= 2e-16 * max(1.0, abs(v))


def test_activations_equal_torch_float64():
    g = np.linspace(-30, 30, 10001)
    tg = torch.from_numpy(g)
    np.testing.assert_allclose(orc.silu(g), torch.nn.functional.silu(tg).numpy(), rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(orc.gelu_erf(g), torch.nn.functional.gelu(tg).numpy(), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("act", ["swiglu", "geglu"])
def test_single_expert_is_a_dense_gated_mlp(act):
    # E = 1, k = 1: every token goes to the one expert with gate 1
    T, d, h = 40, 24, 48
    x, wr, W, _ = _rand_layer(T, d, 1, 1, h)
    r = orc.moe_layer(x, W, 1, True, act, w_router=wr)
    tx = torch.from_numpy(x)
    a = torch.nn.functional.silu if act == "swiglu" else torch.nn.functional.gelu
    ref = torch.nn.functional.linear(
        a(torch.nn.functional.linear(tx, torch.from_numpy(W.wg[0])))
        * torch.nn.functional.linear(tx, torch.from_numpy(W.wu[0])), torch.from_numpy(W.wd[0]))
    np.testing.assert_allclose(r["out"], ref.numpy(), rtol=1e-12, atol=1e-13)


def test_k_equals_E_is_the_full_softmax_mixture():
    T, d, E, h = 30, 16, 5, 12
    x, wr, W, _ = _rand_layer(T, d, E, E, h)
    r = orc.moe_layer(x, W, E, True, "swiglu", w_router=wr)
    pi = scipy.special.softmax(x @ wr.T, axis=1)
    ys = np.stack([orc.gated_ffn(x, W.wg[e], W.wu[e], W.wd[e], "swiglu") for e in range(E)], 1)
    np.testing.assert_allclose(r["out"], (pi[:, :, None] * ys).sum(1), rtol=1e-11, atol=1e-12)


def _dense_masked(x, wr, W, k, renorm, act, bias=None, shared=None, keep=None):
    """All experts on all tokens, times a [T, E] gate matrix that is zero off the top-k."""
    L = x @ wr.T + (0 if bias is None else bias)
    E = L.shape[1]
    ids = np.argsort(-L, axis=1, kind="stable")[:, :k]
    pi = scipy.special.softmax(L, axis=1)
    G = np.zeros_like(L)
    np.put_along_axis(G, ids, np.take_along_axis(pi, ids, 1), 1)
    if renorm:
        G = G / G.sum(1, keepdims=True)
    if keep is not None:
        G = G * keep
    out = np.zeros_like(x)
    for e in range(E):
        out += G[:, e:e + 1] * orc.gated_ffn(x, W.wg[e], W.wu[e], W.wd[e], act)
    if shared is not None:
        out += orc.gated_ffn(x, *shared, act)
    return out


@pytest.mark.parametrize("renorm,act", [(True, "swiglu"), (False, "swiglu"), (True, "geglu")])
def test_sparse_equals_dense_masked(renorm, act):
    T, d, E, k, h = 256, 64, 8, 2, 128
    x, wr, W, shared = _rand_layer(T, d, E, k, h, shared_h=32)
    bias = -1.1 * np.log1p(np.arange(E))
    r = orc.moe_layer(x, W, k, renorm, act, w_router=wr, bias=bias, shared=shared)
    ref = _dense_masked(x, wr, W, k, renorm, act, bias=bias, shared=shared)
    assert np.abs(r["out"] - ref).max() <= 1e-12 * np.sqrt((ref ** 2).mean())


def test_sparse_equals_dense_masked_with_capacity():
    T, d, E, k, h, cap = 120, 16, 6, 2, 8, 30
    x, wr, W, _ = _rand_layer(T, d, E, k, h)
    r = orc.moe_layer(x, W, k, True, "swiglu", w_router=wr, capacity=cap)
    # keep mask from a sequential per-expert counter in token order
    ids = np.argsort(-(x @ wr.T), axis=1, kind="stable")[:, :k]
    keep = np.zeros((T, E))
    cnt = np.zeros(E, int)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            if cnt[e] < cap:
                keep[t, e] = 1
                cnt[e] += 1
    ref = _dense_masked(x, wr, W, k, True, "swiglu", keep=keep)
    assert np.abs(r["out"] - ref).max() <= 1e-12 * np.sqrt((ref ** 2).mean())


def test_sum_over_owner_shares_equals_full_layer():
    T, d, E, k, h, owners = 64, 32, 64, 8, 16, 32
    x, wr, W, _ = _rand_layer(T, d, E, k, h)
    full = orc.moe_layer(x, W, k, True, "swiglu", w_router=wr)["out"]
    acc = np.zeros_like(full)
    for o in range(owners):
        mine = np.arange(o, E, owners)
        emap = np.full(E, -1)
        emap[mine] = np.arange(mine.size)
        Wo = orc.LayerWeights(wg=W.wg[mine], wu=W.wu[mine], wd=W.wd[mine])
        acc += orc.moe_layer(x, Wo, k, True, "swiglu", w_router=wr, expert_map=emap)["out"]
    assert np.abs(acc - full).max() <= 1e-12 * np.sqrt((full ** 2).mean())


def test_token_subset_matches_full_rows():
    T, d, E, k, h = 90, 16, 6, 2, 8
    x, wr, W, shared = _rand_layer(T, d, E, k, h, shared_h=8)
    full = orc.moe_layer(x, W, k, True, "swiglu", w_router=wr, capacity=25, shared=shared)["out"]
    sub = [0, 7, 33, 89]
    part = orc.moe_layer(x, W, k, True, "swiglu", w_router=wr, capacity=25, shared=shared,
                         tokens=sub)["out"]
    np.testing.assert_allclose(part, full[sub], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- brute force
def _brute_force_layer(x, wr, W, k, renorm, act, capacity, shared):
    """Pure-Python loops, following moe_stream.py's per-expert mask / gather /
    scatter-add formulation of MoEFFN.forward."""
    T, d = len(x), len(x[0])
    E = len(wr)

    def dot(a, b):
        return sum(ai * bi for ai, bi in zip(a, b))

    def actf(g):
        return g / (1 + math.exp(-g)) if act == "swiglu" else 0.5 * g * (1 + math.erf(g / math.sqrt(2)))

    def ffn(a, wg, wu, wd):
        z = [actf(dot(wg[n], a)) * dot(wu[n], a) for n in range(len(wg))]
        return [dot(wd[i], z) for i in range(len(wd))]

    top_idx, top_w = [], []
    for t in range(T):
        L = [dot(x[t], wr[e]) for e in range(E)]
        m = max(L)
        ex = [math.exp(v - m) for v in L]
        s = sum(ex)
        p = [v / s for v in ex]
        chosen = []
        for _ in range(k):
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or L[e] > L[best]:
                    best = e
            chosen.append(best)
        w = [p[e] for e in chosen]
        if renorm:
            sw = sum(w)
            w = [v / sw for v in w]
        top_idx.append(chosen)
        top_w.append(w)
    kept = [[True] * k for _ in range(T)]
    if capacity:
        cnt = [0] * E
        for t in range(T):
            for j in range(k):
                e = top_idx[t][j]
                kept[t][j] = cnt[e] < capacity
                cnt[e] += kept[t][j]
    out = [[0.0] * d for _ in range(T)]
    for i in range(E):
        for t in range(T):
            w = sum(top_w[t][j] for j in range(k) if top_idx[t][j] == i and kept[t][j])
            if any(top_idx[t][j] == i and kept[t][j] for j in range(k)):
                y = ffn(x[t], W.wg[i].tolist(), W.wu[i].tolist(), W.wd[i].tolist())
                for c in range(d):
                    out[t][c] += w * y[c]
    if shared is not None:
        for t in range(T):
            y = ffn(x[t], *(m.tolist() for m in shared))
            for c in range(d):
                out[t][c] += y[c]
    return np.array(out)


@pytest.mark.parametrize("renorm,act,cap,sh", [(True, "swiglu", 0, 0), (False, "geglu", 0, 4),
                                               (True, "swiglu", 3, 4)])
def test_vectorised_oracle_equals_pure_python_loops(renorm, act, cap, sh):
    T, d, E, k, h = 12, 6, 5, 2, 4
    x, wr, W, shared = _rand_layer(T, d, E, k, h, shared_h=sh, seed=7)
    r = orc.moe_layer(x, W, k, renorm, act, w_router=wr, capacity=cap, shared=shared)
    ref = _brute_force_layer(x.tolist(), wr.tolist(), W, k, renorm, act, cap, shared)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- backward
def _bwd_case(seed, T=7, d=8, E=5, k=2, h=6, shared_h=0, given_logits=False, biased=False):
    x, wr, W, shared = _rand_layer(T, d, E, k, h, shared_h=shared_h, seed=seed)
    rng = np.random.default_rng(seed + 100)
    logits = rng.standard_normal((T, E)) * 1.5 if given_logits else None
    bias = rng.standard_normal(E) * 0.3 if biased else None
    R = rng.standard_normal((T, d))
    return x, (None if given_logits else wr), W, shared, logits, bias, R


def _objective(x, wr, W, shared, logits, bias, R, k, renorm, act, cap, balance, ids_ref):
    r = orc.moe_layer(x, W, k, renorm, act, w_router=wr, logits=logits, bias=bias, capacity=cap, shared=shared)
    assert np.array_equal(r["ids"], ids_ref), "selection moved under the perturbation"
    f = float(np.sum(r["out"] * R))
    if balance:
        f += balance * orc.router_stats(r["L"], r["ids"])[2]
    return f


@pytest.mark.parametrize("act,renorm,cap,sh,given,balance", [
    ("swiglu", True, 0, 0, False, 0.0), ("geglu", False, 0, 4, False, 0.0), ("swiglu", True, 2, 4, False, 0.3),
    ("geglu", True, 0, 0, True, 0.5), ("swiglu", False, 3, 0, True, 0.0)])
def test_backward_central_differences(act, renorm, cap, sh, given, balance):
    """Every gradient output against central differences of
    F = sum(out * R) + balance * balance_loss (step 1e-5, float64)."""
    x, wr, W, shared, logits, bias, R = _bwd_case(11, shared_h=sh, given_logits=given, biased=True)
    k = 2
    g = orc.moe_layer_bwd(x, W, k, renorm, act, R, w_router=wr, logits=logits, bias=bias, capacity=cap,
                          shared=shared, balance=balance)
    ids_ref = orc.moe_layer(x, W, k, renorm, act, w_router=wr, logits=logits, bias=bias, capacity=cap)["ids"]
    eps = 1e-5
    rng = np.random.default_rng(0)

    def fd(arr, idx, rebuild):
        old = arr[idx]
        arr[idx] = old + eps
        fp = _objective(*rebuild(), R, k, renorm, act, cap, balance, ids_ref)
        arr[idx] = old - eps
        fm = _objective(*rebuild(), R, k, renorm, act, cap, balance, ids_ref)
        arr[idx] = old
        return (fp - fm) / (2 * eps)

    def rebuild():
        return x, wr, W, shared, logits, bias

    checks = [(x, g["dx"])]
    checks += [(W.wg, g["dw_gate"]), (W.wu, g["dw_up"]), (W.wd, g["dw_down"])]
    if shared is not None:
        checks += list(zip(shared, g["dshared"]))
    if wr is not None:
        checks.append((wr, g["dw_router"]))
    if logits is not None:
        checks.append((logits, g["dlogits"]))
    checks.append((bias, g["dbias"]))
    for arr, grad in checks:
        assert grad.shape == arr.shape
        flat = [tuple(int(v) for v in np.unravel_index(i, arr.shape))
                for i in rng.choice(arr.size, size=min(arr.size, 12), replace=False)]
        for idx in flat:
            num = fd(arr, idx, rebuild)
            assert abs(num - grad[idx]) <= 1e-6 * max(1.0, abs(num)), (idx, num, grad[idx])


@pytest.mark.parametrize("act,renorm,cap", [("swiglu", True, 0), ("geglu", False, 2), ("geglu", True, 3)])
def test_backward_matches_torch_autograd(act, renorm, cap):
    """An independent forward in torch float64 (the oracle's selection and
    capacity mask held fixed as constants) differentiated by autograd."""
    T, d, E, k, h, sh = 9, 8, 6, 3, 5, 4
    x, wr, W, shared, _, bias, R = _bwd_case(5, T, d, E, k, h, shared_h=sh, biased=True)
    fwd = orc.moe_layer(x, W, k, renorm, act, w_router=wr, bias=bias, capacity=cap, shared=shared)
    ids = torch.from_numpy(fwd["ids"])
    kept = torch.from_numpy((fwd["pair_pos"].reshape(T, k) >= 0).astype(np.float64))
    tt = {n: torch.tensor(v, dtype=torch.float64, requires_grad=True)
          for n, v in [("x", x), ("wr", wr), ("b", bias), ("wg", W.wg), ("wu", W.wu), ("wd", W.wd),
                       ("sg", shared[0]), ("su", shared[1]), ("sd", shared[2])]}
    a = torch.nn.functional.silu if act == "swiglu" else torch.nn.functional.gelu
    L = tt["x"] @ tt["wr"].T + tt["b"]
    pi = torch.softmax(L, dim=-1)
    psel = torch.gather(pi, 1, ids)
    wgt = psel / psel.sum(-1, keepdim=True) if renorm else psel
    out = torch.zeros(T, d, dtype=torch.float64)
    for j in range(k):
        for t in range(T):
            e = int(ids[t, j])
            xt = tt["x"][t]
            y = tt["wd"][e] @ (a(tt["wg"][e] @ xt) * (tt["wu"][e] @ xt))
            out[t] = out[t] + kept[t, j] * wgt[t, j] * y
    out = out + (a(tt["x"] @ tt["sg"].T) * (tt["x"] @ tt["su"].T)) @ tt["sd"].T
    (out * torch.from_numpy(R)).sum().backward()
    g = orc.moe_layer_bwd(x, W, k, renorm, act, R, w_router=wr, bias=bias, capacity=cap, shared=shared)
    pairs = [("x", g["dx"]), ("wr", g["dw_router"]), ("b", g["dbias"]), ("wg", g["dw_gate"]),
             ("wu", g["dw_up"]), ("wd", g["dw_down"]), ("sg", g["dshared"][0]), ("su", g["dshared"][1]),
             ("sd", g["dshared"][2])]
    for n, ours in pairs:
        np.testing.assert_allclose(ours, tt[n].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=n)


def test_backward_special_cases():
    """One expert (k = E = 1): the softmax is constant 1, so the router gets no
    gradient and the rest is the dense gated MLP's; the activation derivatives
    at 0 are 1/2; the sum of the owners' gradients is the full layer's."""
    x, wr, W, _, _, _, R = _bwd_case(3, T=6, d=8, E=1, k=1, h=4)
    g = orc.moe_layer_bwd(x, W, 1, True, "swiglu", R, w_router=wr)
    assert np.abs(g["dw_router"]).max() == 0.0
    da, dwg, dwu, dwd = orc.gated_ffn_bwd(x, W.wg[0], W.wu[0], W.wd[0], "swiglu", R)
    np.testing.assert_allclose(g["dx"], da, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(g["dw_down"][0], dwd, rtol=1e-13, atol=1e-14)
    assert orc.act_grad(0.0, "swiglu") == 0.5 and orc.act_grad(0.0, "geglu") == 0.5
    # the sum over owner shares of their gradients is the whole layer's gradient
    T, d, E, k, h, owners = 10, 8, 8, 3, 4, 4
    x, wr, W, _, _, _, R = _bwd_case(9, T, d, E, k, h)
    full = orc.moe_layer_bwd(x, W, k, True, "geglu", R, w_router=wr)
    dx = np.zeros_like(full["dx"])
    dwr = np.zeros_like(full["dw_router"])
    for o in range(owners):
        mine = np.arange(o, E, owners)
        emap = np.full(E, -1)
        emap[mine] = np.arange(mine.size)
        Wo = orc.LayerWeights(wg=W.wg[mine], wu=W.wu[mine], wd=W.wd[mine])
        go = orc.moe_layer_bwd(x, Wo, k, True, "geglu", R, w_router=wr, expert_map=emap)
        dx += go["dx"]
        dwr += go["dw_router"]
        np.testing.assert_allclose(go["dw_gate"], full["dw_gate"][mine], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dx, full["dx"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dwr, full["dw_router"], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- INT4
def test_int4_worked_example():
    c = int4_case()
    w = np.zeros((1, 384), np.float32)
    for g in range(3):
        vals = c[f"group{g}_w"]
        w[0, 128 * g:128 * g + len(vals)] = vals
    packed, scales = orc.quantize_int4(w)
    codes = orc.unpack_int4(packed)[0]
    for g in range(3):
        assert int(scales[0, g].view(np.uint16)) == c[f"group{g}_scale_bits"]
        n = len(c[f"group{g}_codes"])
        assert codes[128 * g:128 * g + n].tolist() == c[f"group{g}_codes"]
        assert np.all(codes[128 * g + n:128 * (g + 1)] == 0)
        nb = len(c[f"group{g}_bytes"])
        assert packed[0, 64 * g:64 * g + nb].tolist() == c[f"group{g}_bytes"]
        assert np.all(packed[0, 64 * g + nb:64 * (g + 1)] == 0)
    deq = orc.dequantize_int4(packed, scales)
    assert deq[0, 0] == 0.875 and deq[0, 1] == 0.25 and deq[0, 5] == -0.875
    assert deq[0, 256] == 7 * 0.142822265625


def test_int4_pack_unpack_all_bytes():
    b = np.arange(256, dtype=np.uint8)[None, :]
    q = orc.unpack_int4(b)
    assert q.min() == -8 and q.max() == 7
    np.testing.assert_array_equal(orc.pack_int4(q), b)
    # byte 0x8f: low nibble 0xf = -1, high nibble 0x8 = -8
    assert orc.unpack_int4(np.array([[0x8F]], np.uint8)).tolist() == [[-1, -8]]


def test_int4_quantise_dequantise_round_trip_is_bit_exact():
    w = (np.random.default_rng(5).standard_normal((256, 7168)) / np.sqrt(7168)).astype(np.float32)
    p1, s1 = orc.quantize_int4(w)
    deq = orc.dequantize_int4(p1, s1)
    # dequantised weights are exact in float32 (11-bit significand times |q| <= 8)
    assert np.array_equal(deq.astype(np.float32).astype(np.float64), deq)
    p2, s2 = orc.quantize_int4(deq.astype(np.float32))
    assert np.array_equal(p1, p2) and np.array_equal(s1.view(np.uint16), s2.view(np.uint16))
    q = orc.unpack_int4(p1).reshape(256, 56, 128)
    assert np.all(np.abs(q).max(-1) == 7) and q.min() > -8
    # the scale is the float32 max|w|/7 rounded once to fp16: within half an fp16 ulp
    amax = np.abs(w.reshape(256, 56, 128)).max(-1).astype(np.float64)
    s = s1.astype(np.float64)
    ulp = np.spacing(s.astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(s - amax / 7) <= 0.5 * ulp + 1e-12 * s)


def test_int4_zero_and_tiny_groups():
    w = np.zeros((2, 256), np.float32)
    w[1, :128] = 1e-9      # max/7 underflows fp16 to zero: codes must be 0
    p, s = orc.quantize_int4(w)
    assert np.all(p == 0) and np.all(s == 0)


# ---------------------------------------------------------------- rounding
def test_round_bf16_matches_torch_on_float32_values():
    v = RNG.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** RNG.integers(-30, 30, 100000)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.round_to_dtype(v.astype(np.float64), "bf16"), ref)


def test_round_bf16_ties_and_single_rounding():
    r = orc.round_to_dtype(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -40, -(1 + 2 ** -8)]), "bf16")
    # ties go to even; a float64 value just above a tie rounds up (no detour via float32)
    assert r.tolist() == [1.0, 1 + 2 ** -6, 1 + 2 ** -7, -1.0]



# ---------------------------------------------------------------- hierarchical router
# The page (kieve-moe "Features") gives one sentence and no formula, so these
# pins hold tree_route to the reading written in the oracle's header, not to
# the page: parity unpinned against the page.
def _tree_case(B, L, E, d, T, seed):
    rng = np.random.default_rng(seed)
    n, first = orc.tree_nodes(E, B, L)
    return rng.standard_normal((T, d)), rng.standard_normal((first[L], d)) / np.sqrt(d)


def _leaf_probs_brute_force(xt, W, B, L, E):
    """Probability of every leaf by enumerating the whole tree: a node at depth
    l exists when its first leaf (id * B**(L - l)) is below E; each node's
    children share a softmax of x . row over the existing ones."""
    first = 0
    probs = {(): 1.0}  # digit prefix -> probability
    for l in range(L):
        nxt = {}
        row_base = first
        for prefix, p in probs.items():
            node = sum(dg * B ** (len(prefix) - 1 - i) for i, dg in enumerate(prefix))
            kids = [c for c in range(B) if (node * B + c) * B ** (L - l - 1) < E]
            z = [math.fsum(xt[i] * W[row_base + node * B + c, i] for i in range(len(xt))) for c in kids]
            m = max(z)
            den = math.fsum(math.exp(v - m) for v in z)
            for c, v in zip(kids, z):
                nxt[prefix + (c,)] = p * math.exp(v - m) / den
        first += B * len({sum(dg * B ** (len(pr) - 1 - i) for i, dg in enumerate(pr)) for pr in probs})
        probs = nxt
    out = np.zeros(E)
    for prefix, p in probs.items():
        out[sum(dg * B ** (L - 1 - i) for i, dg in enumerate(prefix))] = p
    return out


@pytest.mark.parametrize("case", tree_route_cases(), ids=lambda c: "B%d_L%d_E%d" % (c["branch"], c["levels"], c["E"]))
def test_tree_route_worked_examples(case):
    x = np.array([case["x"]])
    W = np.array(case["rows"])
    for sub in case["subs"]:
        for renorm, key in ((False, "w_raw"), (True, "w_renorm")):
            ids, w, margin = orc.tree_route(sub["k"], renorm, x, W, case["branch"], case["levels"], case["E"])
            assert ids[0].tolist() == sub["ids"], (sub["k"], ids)
            np.testing.assert_allclose(w[0], sub[key], rtol=0, atol=1e-14)
            if sub["margin"] is not None:
                assert abs(margin[0] - sub["margin"]) < 1e-14
        lp = orc.tree_path_logprob(x, W, case["branch"], case["levels"], case["E"], np.array([sub["ids"]]))
        np.testing.assert_allclose(np.exp(lp[0]), sub["w_raw"], rtol=0, atol=1e-14)


def test_tree_layout_sizes():
    # a full tree has B + B^2 + ... + B^L gate rows; a trimmed one drops the
    # nodes with no leaf below them
    assert orc.tree_nodes(16, 2, 4) == ([1, 2, 4, 8, 16], [0, 2, 6, 14, 30])
    assert orc.tree_nodes(896, 32, 2) == ([1, 28, 896], [0, 32, 928])
    assert orc.tree_nodes(20, 3, 3) == ([1, 3, 7, 20], [0, 3, 12, 33])
    for bad in ((5, 2, 2), (4, 1, 2), (4, 2, 0), (0, 2, 2)):
        with pytest.raises(ValueError):
            orc.tree_nodes(*bad)


@pytest.mark.parametrize("E,B,renorm", [(5, 8, True), (8, 8, False), (3, 4, True)])
def test_tree_route_one_level_is_the_flat_router(E, B, renorm):
    # one level: the root's softmax over its E children is the flat router's
    # softmax over E experts, and a beam of width k is plain top-k
    x, W = _tree_case(B, 1, E, 16, 60, seed=E)
    for k in range(1, E + 1):
        ids, w, _ = orc.tree_route(k, renorm, x, W, B, 1, E)
        _, ids_f, w_f = orc.route(k, renorm, x=x, w_router=W[:E])
        assert np.array_equal(ids, ids_f)
        np.testing.assert_allclose(w, w_f, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("B,L,E", [(3, 3, 20), (2, 4, 16), (4, 2, 13), (2, 3, 5)])
def test_tree_route_wide_beam_equals_exhaustive_top_k(B, L, E):
    # a beam as wide as the widest inner depth keeps every node, so the result
    # is the exact top-k of the whole leaf distribution
    n, _ = orc.tree_nodes(E, B, L)
    x, W = _tree_case(B, L, E, 8, 25, seed=B * 100 + E)
    for k in sorted({n[L - 1], E}):
        ids, w, _ = orc.tree_route(k, False, x, W, B, L, E)
        for t in range(x.shape[0]):
            p = _leaf_probs_brute_force(x[t], W, B, L, E)
            assert abs(p.sum() - 1) < 1e-12  # the hierarchical softmax is a distribution
            order = sorted(range(E), key=lambda e: (-p[e], e))[:k]
            assert ids[t].tolist() == order
            np.testing.assert_allclose(w[t], p[order], rtol=1e-12, atol=1e-15)
        if k == E:
            np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_tree_route_narrow_beam_is_greedy_per_depth():
    # width 1 follows the most probable child at every depth (the first one on
    # ties); checked against the brute-force leaf probabilities
    B, L, E = 3, 3, 27
    x, W = _tree_case(B, L, E, 8, 40, seed=7)
    ids, w, _ = orc.tree_route(1, False, x, W, B, L, E)
    _, first = orc.tree_nodes(E, B, L)
    for t in range(x.shape[0]):
        node = 0
        for l in range(L):
            z = W[first[l] + node * B: first[l] + node * B + B] @ x[t]
            node = node * B + int(np.argmax(z))
        assert ids[t, 0] == node
        assert abs(w[t, 0] - _leaf_probs_brute_force(x[t], W, B, L, E)[node]) < 1e-12


def test_tree_route_subtree_relabelling():
    # swapping the root's children 0 and 2 (their gate rows and the blocks of
    # rows that score their children) swaps the leading digit of every leaf
    B, L, E = 3, 2, 9
    x, W = _tree_case(B, L, E, 12, 50, seed=3)
    W2 = W.copy()
    W2[[0, 2]] = W[[2, 0]]
    W2[3:6], W2[9:12] = W[9:12], W[3:6]
    for k in (1, 2, 4, 9):
        ids, w, _ = orc.tree_route(k, True, x, W, B, L, E)
        ids2, w2, _ = orc.tree_route(k, True, x, W2, B, L, E)
        swap = np.array([(2 - e // 3) * 3 + e % 3 if e // 3 != 1 else e for e in range(9)])
        assert np.array_equal(swap[ids2], ids)
        np.testing.assert_allclose(w2, w, rtol=1e-12)


def test_tree_route_gates_and_margins():
    B, L, E = 4, 3, 50
    x, W = _tree_case(B, L, E, 16, 30, seed=11)
    ids, w, margin = orc.tree_route(6, False, x, W, B, L, E)
    lp = orc.tree_path_logprob(x, W, B, L, E, ids)
    np.testing.assert_allclose(w, np.exp(lp), rtol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0) and np.all(margin >= 0)
    assert all(len(set(r)) == 6 for r in ids.tolist()) and ids.min() >= 0 and ids.max() < E
    ids_n, w_n, _ = orc.tree_route(6, True, x, W, B, L, E)
    assert np.array_equal(ids_n, ids)
    np.testing.assert_allclose(w_n, w / w.sum(axis=1, keepdims=True), rtol=1e-12)
