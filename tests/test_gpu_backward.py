"""GPU parity of the layer backward (moe_layer_bwd through the C ABI) against
the float64 oracle's chain rule on the same inputs.

The selection is piecewise constant, so both sides use the GPU's own top-k
(taken from a traced forward; the backward recomputes the same routing): a
near-tie that rounds differently in bf16 would otherwise move a whole expert's
gradient.  Tolerances: fp32, max |gpu - ref| / RMS(ref) <= 1e-5 per gradient.
bf16: the path feeds its MFMA GEMMs bf16 operands (z as in the forward, w z,
dg, du, dL), so a gradient element that sums many products is off by up to
n 2^-8 times the sum of the products' magnitudes; weight gradients are heavy
tailed and cancel, so max error / RMS is no measure for them.  Each element
is held to the first-order bound of moe_testutil.bwd_error_bounds, plus 5% of
it (a rounded value comes out of an fp32 sum with its own relative error
eps, which adds eps / 2^-8 to the ratio) and 1e-6 RMS(ref); dx keeps the
forward's metric (net of its final rounding) at 2e-2.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from moe_synth import CONFIGS, make_inputs, scaled
from moe_synth.generate import as_f64
from moe_testutil import TOL, bwd_error_bounds, device_weights, oracle_weights, out_err, relerr, shared_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"

BWD = {
    "tiny_fp32": CONFIGS["tiny_fp32"],
    "granular_small": scaled("granular_bf16", T=512, d=256, E=48, h=128, h_shared=256),
    "wide_geglu_small": scaled("wide_geglu_bf16", T=1024, d=256, E=8, h=512),
    "decode_small": scaled("decode_bf16", T=136, d=512, E=32, h=256, h_shared=256),
    "given_logits": scaled("decode_bf16", T=200, d=256, E=64, k=4, h=128, h_shared=0, logits_input=1.0,
                           renorm=True),
    "share_of_4": scaled("granular_bf16", T=300, d=256, E=32, k=4, h=128, h_shared=0, capacity_factor=None,
                         owners=4),
    "fp32_geglu_bias": scaled("tiny_fp32", T=100, E=12, k=3, act="geglu", zipf_bias=0.7, h_shared=64,
                              renorm=False),
    # routed and shared g, u recomputed, and the data and weight gradient GEMMs
    # run, on the wide 256 x 256 tiles
    "wide_recompute": scaled("granular_bf16", T=4096, d=256, E=64, h=512, h_shared=256),
    # the same tiles with skewed routing: experts from several 256-row tiles to
    # none (their weight gradients are zero)
    "wide_skewed": scaled("granular_bf16", T=4096, d=256, E=64, h=512, h_shared=0, capacity_factor=None,
                          zipf_bias=1.5),
    # GeGLU on the wide tiles: the routed and shared gate/up recomputes with
    # the gate backward in their epilogue, in one launch (Zipf-skewed experts
    # of one to several 256-row tiles)
    "wide_geglu_recompute": scaled("wide_geglu_bf16", T=4096, d=256, E=8, h=1024, h_shared=512),
}


def _moe():
    import sparse_mixture_experts_lds_amd as moe
    moe.load()
    return moe


def _dout(inp, seed=0):
    rng = np.random.default_rng(seed + 77)
    t = torch.from_numpy(rng.standard_normal((inp.cfg.T, inp.cfg.d)).astype(np.float32))
    return t if inp.cfg.dtype == "f32" else t.to(torch.bfloat16)


def check_backward(inp, balance=0.0, report=None):
    moe = _moe()
    cfg = inp.cfg
    W = device_weights(inp)
    x = inp.x.to(DEV)
    logits = inp.logits.to(DEV) if inp.logits is not None else None
    dout = _dout(inp)
    _, tr = moe.layer_fwd(x, W, logits=logits, trace=True)
    g = moe.layer_bwd(x, W, dout.to(DEV), logits=logits, balance=balance)
    torch.cuda.synchronize()
    ids = tr["topk_ids"].cpu().numpy().astype(np.int64)
    ref = orc.moe_layer_bwd(as_f64(inp.x), oracle_weights(inp), cfg.k, cfg.renorm, cfg.act, as_f64(dout),
                            w_router=as_f64(inp.w_router), logits=as_f64(inp.logits), bias=as_f64(inp.bias),
                            expert_map=inp.expert_map, capacity=inp.capacity, shared=shared_f64(inp),
                            balance=balance, ids=ids)
    tol = TOL["f32"] if cfg.dtype == "f32" else TOL["bf16"]
    errs = {"dx": out_err(g["dx"].float().cpu().numpy(), ref["dx"], cfg.dtype)}
    pairs = [("dw_gate", ref["dw_gate"]), ("dw_up", ref["dw_up"]), ("dw_down", ref["dw_down"]),
             ("dgates", np.where(tr["pair_pos"].cpu().numpy().reshape(cfg.T, cfg.k) >= 0, ref["dgates"], 0.0))]
    if ref["dshared"] is not None:
        pairs += [("dws_gate", ref["dshared"][0]), ("dws_up", ref["dshared"][1]), ("dws_down", ref["dshared"][2])]
    if ref["dw_router"] is not None:
        pairs.append(("dw_router", ref["dw_router"]))
    if ref["dlogits"] is not None:
        pairs.append(("dlogits", ref["dlogits"]))
    if ref["dbias"] is not None:
        pairs.append(("dbias", ref["dbias"]))
    bounds = bwd_error_bounds(inp, dout, ids, balance) if cfg.dtype != "f32" else None
    over = {}
    for n, r in pairs:
        got = g[n].cpu().numpy().astype(np.float64)
        errs[n] = relerr(got, r)
        if bounds is not None:
            # largest ratio of the error to its element's bound (<= 1 passes)
            bnd = 1.05 * bounds[n] + 1e-6 * np.sqrt(np.mean(r ** 2))
            ratio = float(np.max(np.abs(got - r) / np.maximum(bnd, 1e-300), initial=0.0))
            errs[n + "/bound"] = ratio
            if ratio > 1.0:
                over[n] = ratio
        elif errs[n] > tol:
            over[n] = errs[n]
    if report is not None:
        report.update(errs)
    if errs["dx"] > tol:
        over["dx"] = errs["dx"]
    assert not over, "gradients above tolerance: %s" % over
    return g


# the cases meant for the wide tiles (and their shared expert in the routed launches)
WIDE_BWD = {"wide_recompute", "wide_skewed", "wide_geglu_recompute"}


@pytest.mark.parametrize("name", list(BWD))
def test_backward_scaled(name):
    rep = {}
    inp = make_inputs(BWD[name])
    if name in WIDE_BWD:
        moe = _moe()
        plan = moe.layer_plan(device_weights(inp), inp.cfg.T, inp.cfg.d, 1)
        assert plan["tile_m"] == 256, plan
        if inp.cfg.h_shared:
            assert plan["shared_in_routed_launches"] == 1, plan
    check_backward(inp, report=rep)
    print(name, {k: "%.2e" % v for k, v in rep.items()})


@pytest.mark.parametrize("name", ["granular_small", "given_logits", "fp32_geglu_bias"])
def test_backward_with_balance_loss(name):
    rep = {}
    check_backward(make_inputs(BWD[name]), balance=0.25, report=rep)
    print(name, {k: "%.2e" % v for k, v in rep.items()})


@pytest.mark.parametrize("name", ["tiny_fp32", "granular_bf16", "decode_bf16"])
def test_backward_full_size(name):
    rep = {}
    check_backward(make_inputs(CONFIGS[name]), balance=0.01, report=rep)
    print(name, {k: "%.2e" % v for k, v in rep.items()})


def test_backward_is_deterministic():
    moe = _moe()
    inp = make_inputs(BWD["granular_small"])
    W = device_weights(inp)
    x = inp.x.to(DEV)
    dout = _dout(inp).to(DEV)
    a = moe.layer_bwd(x, W, dout, balance=0.1)
    b = moe.layer_bwd(x, W, dout, balance=0.1)
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_backward_rejects_int4_weights():
    moe = _moe()
    inp = make_inputs(scaled("int4_share", T=16, d=256, E=64, h=128, owners=8))
    from moe_testutil import quantize_inputs
    W = device_weights(inp, quantize_inputs(inp))
    with pytest.raises(moe.MoEError):
        moe.layer_bwd(inp.x.to(DEV), W, _dout(inp).to(DEV), logits=inp.logits.to(DEV))
