"""GPU parity of the owner-grouped dispatch (sender side of expert parallelism).

The grouping is integer work and must match the oracle bit for bit, the
gathered send rows byte for byte.  At the full size of the INT4 share workload
(512 tokens, top-16 over 896 experts, 32 owners of 28 experts, d 7168, h 2048)
the owners' results must add up to the whole layer: the layer of all 896
experts, dispatched by owner and run share by share, gives the same output as
the layer run at once (the "sharded equals monolithic" property of the float64
oracle, checked here on the GPU's own results).
"""
import numpy as np
import pytest
import torch

import oracle as orc
from moe_synth import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _moe():
    import sparse_mixture_experts_lds_amd as moe
    moe.load()
    return moe


@pytest.mark.parametrize("T,k,E,n,rule,cap", [
    (512, 16, 896, 32, "round_robin", 0),     # the INT4 share workload's routing, all owners
    (512, 16, 896, 32, "contiguous", 0),
    (8192, 4, 192, 8, "round_robin", 214),    # capacity drops
    (3001, 8, 128, 4, "contiguous", 40),
    (1, 2, 8, 2, "round_robin", 0),
    (700, 32, 1024, 64, "round_robin", 0),
    (64, 4, 12, 12, "contiguous", 0),         # one expert per owner
])
def test_dispatch_owners_bit_exact(T, k, E, n, rule, cap):
    moe = _moe()
    rng = np.random.default_rng(T + E + n)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    d = 256
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    r = moe.dispatch_owners(torch.from_numpy(ids).to(DEV), E, n, rule, cap, x=x.to(DEV))
    torch.cuda.synchronize()
    o = orc.owner_dispatch(ids, E, n, rule, capacity=cap)
    rows = int(o["expert_offsets"][-1])
    np.testing.assert_array_equal(r["owner_offsets"].cpu().numpy(), o["owner_offsets"])
    np.testing.assert_array_equal(r["recv_offsets"].cpu().numpy(), o["recv_offsets"])
    np.testing.assert_array_equal(r["expert_offsets"].cpu().numpy(), o["expert_offsets"])
    np.testing.assert_array_equal(r["sorted_pair"].cpu().numpy()[:rows], o["sorted_pair"])
    np.testing.assert_array_equal(r["pair_pos"].cpu().numpy()[:T * k], o["pair_pos"])
    xs = r["x_send"][:rows].cpu().view(torch.int16).numpy()
    ref = x.view(torch.int16).numpy()[o["sorted_pair"] // k]
    np.testing.assert_array_equal(xs, ref)


def test_dispatch_owners_foreign_ids_and_empty_batch():
    moe = _moe()
    rng = np.random.default_rng(2)
    T, k, E, n = 300, 5, 40, 8
    ids = rng.integers(-4, E + 4, size=(T, k)).astype(np.int32)
    r = moe.dispatch_owners(torch.from_numpy(ids).to(DEV), E, n, "round_robin")
    o = orc.owner_dispatch(ids, E, n, "round_robin")
    rows = int(o["expert_offsets"][-1])
    np.testing.assert_array_equal(r["expert_offsets"].cpu().numpy(), o["expert_offsets"])
    np.testing.assert_array_equal(r["sorted_pair"].cpu().numpy()[:rows], o["sorted_pair"])
    np.testing.assert_array_equal(r["pair_pos"].cpu().numpy(), o["pair_pos"])
    r = moe.dispatch_owners(torch.zeros((0, k), dtype=torch.int32, device=DEV), E, n, "contiguous")
    torch.cuda.synchronize()
    assert not r["owner_offsets"].any() and not r["recv_offsets"].any()


def _half_ulp_bf16(v):
    """Half the bf16 spacing at |v| (0 at 0: an exact zero carries no rounding)."""
    v = np.asarray(v, np.float64)
    _, e = np.frexp(np.abs(v))
    return np.where(v == 0, 0.0, np.ldexp(1.0, e - 9))


def test_owner_shares_sum_to_full_layer_full_scale():
    """896 INT4 experts (round-robin on 32 owners), the INT4 share workload's
    tokens and routing.  (1) dispatch by owner, each owner's grouped FFN on its
    rows with its receive offsets, one weighted combine; (2) each owner's share
    of the layer (its 28 experts through expert_map), partial outputs summed;
    both against the layer of all 896 experts at once."""
    moe = _moe()
    cfg = CONFIGS["int4_share"]
    T, d, E, k, h, n = cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, cfg.owners
    per = E // n
    inp = make_inputs(cfg, fast_weights=True, device=DEV)
    inp.wg = inp.wu = inp.wd = None  # owner 0 only; all owners are drawn below
    torch.cuda.empty_cache()
    x = inp.x.to(DEV)
    logits = inp.logits.to(DEV)
    # owner-major INT4 weights: slot o*per + l holds global expert l*n + o
    qg = torch.empty((E, h, d // 2), dtype=torch.uint8, device=DEV)
    qu = torch.empty((E, h, d // 2), dtype=torch.uint8, device=DEV)
    qd = torch.empty((E, d, h // 2), dtype=torch.uint8, device=DEV)
    sg = torch.empty((E, h, d // 128), dtype=torch.float16, device=DEV)
    su = torch.empty((E, h, d // 128), dtype=torch.float16, device=DEV)
    sd = torch.empty((E, d, h // 128), dtype=torch.float16, device=DEV)
    g = torch.Generator(device=DEV)
    for o in range(n):
        g.manual_seed(5000 + o)
        sl = slice(o * per, (o + 1) * per)
        for (q, s), shape, fan in [((qg, sg), (per, h, d), d), ((qu, su), (per, h, d), d),
                                   ((qd, sd), (per, d, h), h)]:
            w = torch.randn(shape, generator=g, device=DEV, dtype=torch.float32) / np.sqrt(fan)
            q[sl], s[sl] = moe.quantize_int4(w)
            del w
    torch.cuda.synchronize()
    owner, local = orc.placement(E, n)
    slot = torch.from_numpy((owner * per + local).astype(np.int32)).to(DEV)

    # the whole layer: every expert local, global id -> owner-major slot
    W_all = moe.LayerWeights(E=E, k=k, act=cfg.act, renorm=cfg.renorm, wg=qg, wu=qu, wd=qd, sg=sg, su=su,
                             sd=sd, expert_map=slot)
    out_all, tr = moe.layer_fwd(x, W_all, logits=logits, trace=True)
    ids, tw = tr["topk_ids"], tr["topk_w"]

    # (1) dispatch by owner, per-owner grouped FFN, one combine
    r = moe.dispatch_owners(ids, E, n, "round_robin", x=x)
    oo = r["owner_offsets"].cpu().numpy()
    y_send = torch.zeros((T * k, d), dtype=x.dtype, device=DEV)
    for o in range(n):
        a, b = int(oo[o]), int(oo[o + 1])
        if b == a:
            continue
        sl = slice(o * per, (o + 1) * per)
        y_send[a:b] = moe.expert_ffn(r["x_send"][a:b], r["recv_offsets"][o].contiguous(), qg[sl], qu[sl], qd[sl],
                                     cfg.act, sg[sl], su[sl], sd[sl])
    out_disp = moe.combine(y_send, r["pair_pos"], tw)

    # (2) the 32 shares through the layer, partial outputs summed in fp32
    acc = torch.zeros((T, d), dtype=torch.float64, device=DEV)
    halfulp = np.zeros((T, d))
    for o in range(n):
        emap = torch.from_numpy(np.where(owner == o, local, -1).astype(np.int32)).to(DEV)
        sl = slice(o * per, (o + 1) * per)
        W_o = moe.LayerWeights(E=E, k=k, act=cfg.act, renorm=cfg.renorm, wg=qg[sl], wu=qu[sl], wd=qd[sl],
                               sg=sg[sl], su=su[sl], sd=sd[sl], expert_map=emap)
        part = moe.layer_fwd(x, W_o, logits=logits).double()
        acc += part
        halfulp += _half_ulp_bf16(part.cpu().numpy())
    torch.cuda.synchronize()

    full = out_all.double().cpu().numpy()
    rms = np.sqrt(np.mean(full ** 2))
    # same rows, same kernels up to tiling: within fp32 reassociation and one bf16 rounding
    # (the send path also rounds each expert output to bf16 before the combine:
    # at most sum_j w_j * half_ulp(y_j) per element)
    dd = np.abs(out_disp.double().cpu().numpy() - full)
    pp = r["pair_pos"].cpu().numpy().reshape(T, k)
    hu_y = _half_ulp_bf16(y_send.float().cpu().numpy())
    w64 = tw.double().cpu().numpy()
    y_round = np.zeros((T, d))
    for j in range(k):
        y_round += w64[:, j:j + 1] * hu_y[pp[:, j]]
    print("dispatch vs whole layer: max |d| / rms = %.3g, identical = %s" % (dd.max() / rms, bool((dd == 0).all())))
    assert np.all(dd <= y_round + 2 * _half_ulp_bf16(full) + 1e-3 * rms)
    # partials rounded to bf16 one by one, then added: bounded by their half ulps
    ds = np.abs(acc.cpu().numpy() - full)
    print("sum of shares vs whole layer: max |d| / rms = %.3g" % (ds.max() / rms))
    assert np.all(ds <= halfulp + _half_ulp_bf16(full) + 1e-3 * rms)
    # every pair of the batch was dispatched once
    assert int(oo[-1]) == T * k


# seeded random groupings: token counts from 1 up, 1..32 slots, 2..1024
# experts on 1..64 owners (both rules), with and without capacity, ids with
# repeats within a token, some ids foreign (outside [0, E))
@pytest.mark.parametrize("seed", range(24))
def test_dispatch_owners_random(seed):
    moe = _moe()
    rng = np.random.default_rng(7000 + seed)
    E = int(rng.integers(2, 1025))
    n = int(rng.choice([d for d in range(1, min(E, 64) + 1) if E % d == 0]))
    k = int(rng.integers(1, 33))
    T = int(rng.choice([1, int(rng.integers(2, 100)), int(rng.integers(100, 5000))]))
    rule = str(rng.choice(["round_robin", "contiguous"]))
    cap = int(rng.integers(1, 64)) if rng.random() < 0.3 else 0
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if rng.random() < 0.3:
        ids[rng.random((T, k)) < 0.05] = int(rng.choice([-1, E]))
    d = 64 * int(rng.integers(1, 5))
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    print(dict(T=T, k=k, E=E, n=n, rule=rule, cap=cap, d=d), flush=True)
    r = moe.dispatch_owners(torch.from_numpy(ids).to(DEV), E, n, rule, cap, x=x.to(DEV))
    torch.cuda.synchronize()
    o = orc.owner_dispatch(ids, E, n, rule, capacity=cap)
    rows = int(o["expert_offsets"][-1])
    np.testing.assert_array_equal(r["owner_offsets"].cpu().numpy(), o["owner_offsets"])
    np.testing.assert_array_equal(r["recv_offsets"].cpu().numpy(), o["recv_offsets"])
    np.testing.assert_array_equal(r["expert_offsets"].cpu().numpy(), o["expert_offsets"])
    np.testing.assert_array_equal(r["sorted_pair"].cpu().numpy()[:rows], o["sorted_pair"])
    np.testing.assert_array_equal(r["pair_pos"].cpu().numpy()[:T * k], o["pair_pos"])
    xs = r["x_send"][:rows].cpu().view(torch.int16).numpy()
    np.testing.assert_array_equal(xs, x.view(torch.int16).numpy()[o["sorted_pair"] // k])
