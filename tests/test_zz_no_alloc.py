"""moe_permute_noalloc (the grouping step on the library's static scratch)
against moe_permute on the same ids: bit-exact offsets, sorted pairs, pair
positions and gathered rows, over two calls in a row (the second smaller, so
the scratch holds the first call's larger contents when it starts)."""
import numpy as np
import pytest
import torch

from moe_synth import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _moe():
    import sparse_mixture_experts_lds_amd as moe
    moe.load()
    return moe


def _ids(rng, T, k, E):
    # distinct ids per token, with a skew so some experts get many pairs
    L = rng.standard_normal((T, E)) - 0.7 * np.log1p(np.arange(E))[None, :]
    return np.argsort(-L, axis=1, kind="stable")[:, :k].astype(np.int32)


def _check(moe, ids, E, E_loc=None, emap=None, capacity=0, x=None):
    t = torch.from_numpy(ids).to(DEV)
    em = torch.from_numpy(emap).to(DEV) if emap is not None else None
    xd = x.to(DEV) if x is not None else None
    ref = moe.permute(t, E, E_loc, em, capacity, xd)
    got = moe.permute_noalloc(t, E, E_loc, em, capacity, xd)
    torch.cuda.synchronize()
    n = int(ref[0][-1])
    assert torch.equal(got[0], ref[0])
    assert torch.equal(got[1][:n], ref[1][:n])
    assert torch.equal(got[2], ref[2])
    if x is not None:
        assert torch.equal(got[3][:n], ref[3][:n])


@pytest.mark.parametrize("order", ["large_then_small", "granular_then_tiny"])
def test_noalloc_permute_matches_permute_twice(order):
    moe = _moe()
    rng = np.random.default_rng(11)
    if order == "large_then_small":
        # 40 blocks of 1024 pairs over 256 experts, then 3 blocks over 48
        _check(moe, _ids(rng, 10000, 4, 256), 256, capacity=180,
               x=torch.from_numpy(rng.standard_normal((10000, 128)).astype(np.float32)).to(torch.bfloat16))
        _check(moe, _ids(rng, 700, 4, 48), 48,
               x=torch.from_numpy(rng.standard_normal((700, 64)).astype(np.float32)))
    else:
        cfg = CONFIGS["granular_bf16"]
        inp = make_inputs(cfg)
        import oracle as orc
        from moe_synth.generate import as_f64
        ids = orc.select_topk(as_f64(inp.x) @ as_f64(inp.w_router).T, cfg.k).astype(np.int32)
        _check(moe, ids, cfg.E, capacity=inp.capacity, x=inp.x)
        # then a smaller share with an expert map: 896 experts over 32 owners
        emap = np.full(896, -1, np.int32)
        emap[0::32] = np.arange(28, dtype=np.int32)
        _check(moe, _ids(rng, 300, 16, 896), 896, E_loc=28, emap=emap)
