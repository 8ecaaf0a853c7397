"""GPU parity of hierarchical routing down an expert tree (moe_route_tree)
against the float64 oracle (``oracle.tree_route``).

The operation is this repository's reading of one sentence of kieve-moe
"Features" (fractal tiling routing over a branch^levels expert tree); its
parity against the page is unpinned, and these tests hold the HIP path to the
oracle of that reading.

Selection is an integer result decided in floating point: the GPU ranks fp32
path log-probabilities, the oracle float64 ones, from the same inputs.  Tokens
whose oracle margin (the smallest gap the result depends on, at any depth) is
above MARGIN must pick the same leaves in the same slots, bit for bit.  For the
others, the GPU's picks must be valid (distinct existing leaves) and the j-th
pick's exact log-probability must be within MARGIN of the oracle's j-th.
Gates are compared, for every token, with the exact path probabilities of the
GPU's own picks (renormalised over them when asked): relative error <= GATE_TOL.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from golden_io import tree_route_cases
from moe_synth import TREE_CONFIGS, TreeRouteConfig, make_tree_inputs
from moe_synth.generate import as_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
MARGIN = 1e-4
GATE_TOL = 1e-5


def _moe():
    import sparse_mixture_experts_lds_amd as moe
    moe.load()  # fail loudly if the library is missing
    return moe


def _check(x64, w64, B, L, E, k, renorm, ids_gpu, tw_gpu, report=None):
    ids_o, w_o, margin = orc.tree_route(k, renorm, x64, w64, B, L, E)
    ids_g = ids_gpu.cpu().numpy().astype(np.int64)
    tw_g = tw_gpu.cpu().numpy().astype(np.float64)
    T = x64.shape[0]
    safe = margin > MARGIN
    # bit-exact ids where the oracle's decision is not a near-tie
    bad = np.nonzero(safe & np.any(ids_g != ids_o, axis=1))[0]
    assert bad.size == 0, "tokens %s: gpu %s oracle %s" % (bad[:4], ids_g[bad[:2]], ids_o[bad[:2]])
    # every token: valid picks, near-optimal in every slot, gates exact for them
    assert ids_g.min() >= 0 and ids_g.max() < E
    assert all(len(set(r)) == k for r in ids_g.tolist())
    lp_g = orc.tree_path_logprob(x64, w64, B, L, E, ids_g)
    lp_o = np.log(w_o) if not renorm else orc.tree_path_logprob(x64, w64, B, L, E, ids_o)
    assert np.max(np.abs(lp_g - lp_o)) <= MARGIN
    ref = np.exp(lp_g)
    if renorm:
        ref = ref / ref.sum(axis=1, keepdims=True)
    err = np.max(np.abs(tw_g - ref) / ref)
    assert err <= GATE_TOL, err
    if report is not None:
        report.update(tokens=T, near_ties=int((~safe).sum()), flipped=int(np.any(ids_g != ids_o, axis=1).sum()),
                      gate_relerr=float(err))


def _run(cfg, moe):
    rows = moe.tree_gate_rows(cfg.E, cfg.branch, cfg.levels)
    assert rows == orc.tree_nodes(cfg.E, cfg.branch, cfg.levels)[1][cfg.levels]
    x, w = make_tree_inputs(cfg, rows)
    xd, wd = x.to(DEV), w.to(DEV)
    ids, tw = moe.route_tree(xd, wd, cfg.E, cfg.k, cfg.branch, cfg.levels, cfg.renorm)
    torch.cuda.synchronize()
    return x, w, xd, wd, ids, tw


def _cfg(name, T, d, E, k, B, L, dt, renorm=True, seed=0):
    return TreeRouteConfig(name, T=T, d=d, E=E, k=k, branch=B, levels=L, dtype=dt, renorm=renorm, seed=seed)


# Depths where the beam holds at least a quarter of the nodes (and at most
# 1024 children) are scored by one dense GEMM, the others per node on grouped
# pairs; the cases below cover both, in bf16 and fp32, with 1 to 4 16-column
# fragments per node and a width split.
SMALL = [
    # the INT4 share's 896-expert pool (28 x 32), narrow width, ragged token count (dense depths)
    _cfg("pool896_small", 300, 64, 896, 16, 32, 2, "bf16"),
    # grouped fp32 (two fragments) and grouped bf16 with 40 children (three)
    _cfg("f32_grouped", 190, 128, 1024, 2, 32, 2, "f32"),
    _cfg("branch40", 260, 128, 1600, 4, 40, 2, "bf16"),
    # trimmed three-level tree in fp32, d of three 64-wide pieces
    _cfg("trimmed_f32", 257, 192, 20, 4, 3, 3, "f32"),
    # one level: the flat router
    _cfg("one_level_f32", 130, 128, 8, 2, 8, 1, "f32", renorm=False),
    # 4096 experts as 16^3, eight picks, no renormalisation
    _cfg("three_level_bf16", 200, 64, 4096, 8, 16, 3, "bf16", renorm=False),
    # k = E: every leaf picked, gates sum to one
    _cfg("k_equals_E", 64, 64, 13, 13, 4, 2, "f32", renorm=False),
    # widest candidate set (k * branch = 1024), partly missing last node
    _cfg("branch64", 150, 64, 4000, 16, 64, 2, "bf16"),
    # deep binary tree
    _cfg("binary_deep", 100, 64, 32, 3, 2, 5, "f32"),
    # one token; 17 tokens (a ragged tile)
    _cfg("one_token", 1, 64, 896, 16, 32, 2, "bf16"),
    _cfg("ragged17", 17, 256, 1000, 5, 10, 3, "bf16"),
    # long rows and few tokens: the grouped scores are split over the width
    _cfg("split_width", 40, 4096, 4096, 4, 16, 3, "bf16"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_route_tree_small(cfg):
    moe = _moe()
    x, w, _, _, ids, tw = _run(cfg, moe)
    rep = {}
    _check(as_f64(x), as_f64(w), cfg.branch, cfg.levels, cfg.E, cfg.k, cfg.renorm, ids, tw, report=rep)
    if cfg.k == cfg.E and not cfg.renorm:
        np.testing.assert_allclose(tw.sum(dim=1).cpu().numpy(), 1.0, rtol=0, atol=1e-5)
    print(cfg.name, rep)


def test_route_tree_one_level_matches_flat_router():
    # with one level the tree router is moe_route on the first E rows, no bias
    moe = _moe()
    cfg = _cfg("flat", 300, 256, 64, 4, 64, 1, "bf16")
    x, w, xd, wd, ids, tw = _run(cfg, moe)
    ids_f, tw_f, _ = moe.route(xd, wd[:cfg.E].contiguous(), cfg.k, True)
    _, _, margin = orc.tree_route(cfg.k, True, as_f64(x), as_f64(w), cfg.branch, 1, cfg.E)
    safe = torch.from_numpy(margin > MARGIN).to(DEV)
    assert torch.equal(ids[safe], ids_f[safe])
    assert torch.allclose(tw[safe], tw_f[safe], rtol=2e-5, atol=0)


@pytest.mark.parametrize("case", tree_route_cases(), ids=lambda c: "B%d_L%d_E%d" % (c["branch"], c["levels"], c["E"]))
def test_route_tree_worked_examples(case):
    # the hand-worked trees, padded to a width of 64 with zeros (fp32)
    moe = _moe()
    d = 64
    x = torch.zeros((1, d), dtype=torch.float32)
    x[0, :2] = torch.tensor(case["x"])
    W = torch.zeros((len(case["rows"]), d), dtype=torch.float32)
    W[:, :2] = torch.tensor(case["rows"])
    assert moe.tree_gate_rows(case["E"], case["branch"], case["levels"]) == W.shape[0]
    for sub in case["subs"]:
        for renorm, key in ((False, "w_raw"), (True, "w_renorm")):
            ids, tw = moe.route_tree(x.to(DEV), W.to(DEV), case["E"], sub["k"], case["branch"], case["levels"], renorm)
            assert ids[0].tolist() == sub["ids"], (sub["k"], renorm)
            np.testing.assert_allclose(tw[0].cpu().numpy(), sub[key], rtol=2e-6, atol=0)


def test_route_tree_deterministic_and_workspace_reuse():
    moe = _moe()
    cfg = _cfg("det", 700, 512, 896, 16, 32, 2, "bf16")
    _, _, xd, wd, ids, tw = _run(cfg, moe)
    nb = moe.route_tree_workspace_bytes(cfg.T, cfg.d, cfg.E, cfg.k, cfg.branch, cfg.levels, xd.dtype)
    ws = torch.full((nb,), 0xA5, dtype=torch.uint8, device=DEV)  # stale contents must not matter
    for _ in range(3):
        ids2, tw2 = moe.route_tree(xd, wd, cfg.E, cfg.k, cfg.branch, cfg.levels, cfg.renorm, ws=ws)
        assert torch.equal(ids, ids2) and torch.equal(tw.view(torch.int32), tw2.view(torch.int32))


@pytest.mark.parametrize("name", list(TREE_CONFIGS))
def test_route_tree_full_size(name):
    # the bench's workloads, every token compared
    moe = _moe()
    cfg = TREE_CONFIGS[name]
    x, w, _, _, ids, tw = _run(cfg, moe)
    rep = {}
    _check(as_f64(x), as_f64(w), cfg.branch, cfg.levels, cfg.E, cfg.k, cfg.renorm, ids, tw, report=rep)
    print(name, rep)


def _random_tree(seed):
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(2, 65))
    Lmax = 1
    while Lmax < 4 and B ** (Lmax + 1) <= 32768:
        Lmax += 1
    L = int(rng.integers(1, Lmax + 1))
    E = int(rng.integers(2, min(B ** L, 4096) + 1))
    k = int(rng.integers(1, min(E, 32, 1024 // B) + 1))
    T = int(rng.choice([1, int(rng.integers(2, 64)), int(rng.integers(64, 700))]))
    d = int(64 * rng.integers(1, 9))
    dt = str(rng.choice(["bf16", "f32"]))
    return _cfg("random_tree_%d" % seed, T, d, E, k, B, L, dt, renorm=bool(rng.random() < 0.5), seed=seed)


# seeded random trees: branching 2..64, one to four levels, trimmed last
# nodes, beams from 1 to the widest candidate set, both dtypes
@pytest.mark.parametrize("seed", range(32))
def test_route_tree_random(seed):
    moe = _moe()
    cfg = _random_tree(seed)
    print(cfg, flush=True)
    x, w, _, _, ids, tw = _run(cfg, moe)
    rep = {}
    _check(as_f64(x), as_f64(w), cfg.branch, cfg.levels, cfg.E, cfg.k, cfg.renorm, ids, tw, report=rep)
    print(seed, rep)
