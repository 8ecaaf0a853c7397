"""Shared helpers of the GPU parity tests: device copies of the seeded inputs,
oracle-side weights, and the comparison protocol."""
import numpy as np
import torch

import oracle as orc
from moe_synth import make_inputs
from moe_synth.generate import as_f64

TOL = {"f32": 1e-5, "bf16": 2e-2, "i4g128": 2e-2}


def relerr(got, ref) -> float:
    """max |got - ref| / RMS(ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    if rms == 0:
        return float(np.abs(got - ref).max(initial=0.0))
    return float(np.abs(got - ref).max(initial=0.0) / rms)


_MANT = {"bf16": 8, "f32": 24}


def out_err(got, ref, out_dt: str) -> float:
    """Error of a result delivered in ``out_dt`` against the exact (float64)
    value, relative to RMS(ref), net of the one final rounding to ``out_dt``
    that the definition of the output includes:
    max_i (|got_i - ref_i| - ulp_i / 2) / RMS(ref), ulp taken at the larger of
    |got_i|, |ref_i| (0 when the result is at most half an ulp off)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    _, e = np.frexp(np.maximum(np.abs(got), np.abs(ref)))
    half_ulp = np.ldexp(1.0, e - _MANT[out_dt] - 1)
    ex = np.maximum(np.abs(got - ref) - half_ulp, 0.0).max(initial=0.0)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(ex / rms) if rms > 0 else float(ex)


def quantize_inputs(inp):
    """INT4 codes and scales of the expert weights, from the oracle's quantiser."""
    return {n: orc.quantize_int4(getattr(inp, n).numpy()) for n in ("wg", "wu", "wd")}


def oracle_weights(inp, q=None):
    if inp.cfg.w_dtype == "i4g128":
        q = q or quantize_inputs(inp)
        return orc.LayerWeights(qg=q["wg"], qu=q["wu"], qd=q["wd"])
    return orc.LayerWeights(wg=as_f64(inp.wg), wu=as_f64(inp.wu), wd=as_f64(inp.wd))


def device_weights(inp, q=None, dev="cuda"):
    import sparse_mixture_experts_lds_amd as moe
    cfg = inp.cfg

    def d(t):
        return None if t is None else t.to(dev).contiguous()
    if cfg.w_dtype == "i4g128":
        q = q or quantize_inputs(inp)
        wg, sg = (torch.from_numpy(q["wg"][0]).to(dev), torch.from_numpy(q["wg"][1]).to(dev))
        wu, su = (torch.from_numpy(q["wu"][0]).to(dev), torch.from_numpy(q["wu"][1]).to(dev))
        wd, sd = (torch.from_numpy(q["wd"][0]).to(dev), torch.from_numpy(q["wd"][1]).to(dev))
    else:
        wg, wu, wd = d(inp.wg), d(inp.wu), d(inp.wd)
        sg = su = sd = None
    emap = torch.from_numpy(inp.expert_map).to(dev) if inp.expert_map is not None else None
    return moe.LayerWeights(E=cfg.E, k=cfg.k, act=cfg.act, renorm=cfg.renorm, wg=wg, wu=wu, wd=wd,
                            sg=sg, su=su, sd=sd, w_router=d(inp.w_router), bias=d(inp.bias),
                            expert_map=emap, capacity=inp.capacity, wsg=d(inp.wsg), wsu=d(inp.wsu),
                            wsd=d(inp.wsd))


def sample_tokens(T, n, seed=0):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed + 17)
    s = set(rng.choice(T, size=n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s))


def shared_f64(inp):
    if inp.wsg is None:
        return None
    return (as_f64(inp.wsg), as_f64(inp.wsu), as_f64(inp.wsd))


# fp32 softmax values (a few ulp each) added in fp64, then one rounding to fp32
STATS_RTOL = 2e-6


def check_router_stats(L, ids, counts, prob_mean, loss):
    """Counts bit-exact; mean probabilities and loss within STATS_RTOL of the
    oracle's float64 values on the same logits and ids."""
    c_o, P_o, l_o = orc.router_stats(L, ids)
    np.testing.assert_array_equal(counts.cpu().numpy(), c_o)
    P_g = prob_mean.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(P_g - P_o) <= STATS_RTOL * P_o + 1e-30), float(np.abs(P_g - P_o).max())
    l_g = float(loss.cpu().numpy()[0])
    assert abs(l_g - l_o) <= STATS_RTOL * abs(l_o), (l_g, l_o)


def check_layer(inp, q=None, tokens=None, wdev=None, report=None, tol=None):
    """Run the GPU layer and check it against the oracle with the comparison
    protocol: selection bit-exact on the GPU's own fp32 logits, grouping
    bit-exact on the GPU's ids, outputs within the dtype tolerance of the
    oracle (run with the GPU's ids only where a near-tie legitimately flipped)."""
    import sparse_mixture_experts_lds_amd as moe
    cfg = inp.cfg
    dev = "cuda"
    wdev = wdev or device_weights(inp, q, dev)
    x = inp.x.to(dev)
    logits_dev = inp.logits.to(dev) if inp.logits is not None else None
    out, tr = moe.layer_fwd(x, wdev, logits=logits_dev, trace=True, stats=True)
    torch.cuda.synchronize()
    ids_g = tr["topk_ids"].cpu().numpy().astype(np.int64)
    tw_g = tr["topk_w"].cpu().numpy().astype(np.float64)
    if "logits" in tr:
        Lg = tr["logits"].cpu().numpy().astype(np.float64)
    else:
        Lg = as_f64(inp.logits) + (as_f64(inp.bias)[None, :] if inp.bias is not None else 0.0)
    # (a) selection and gates on the GPU's own logits
    ids_a = orc.select_topk(Lg, cfg.k)
    np.testing.assert_array_equal(ids_g, ids_a)
    w_a = orc.gates(Lg, ids_a, cfg.renorm)
    assert np.abs(w_a - tw_g).max() <= 1e-6
    # (a') router by-products of the GPU's own logits and ids
    check_router_stats(Lg, ids_g, tr["expert_counts"], tr["prob_mean"], tr["balance_loss"])
    # (c) grouping of the GPU's ids, bit-exact
    offs, sp, pos = orc.permute(ids_g, inp.expert_map, cfg.E_loc, inp.capacity)
    np.testing.assert_array_equal(tr["expert_offsets"].cpu().numpy(), offs)
    np.testing.assert_array_equal(tr["pair_pos"].cpu().numpy(), pos)
    # (b) end to end against the independent oracle
    Wo = oracle_weights(inp, q)
    x64 = as_f64(inp.x)
    kw = dict(w_router=as_f64(inp.w_router), logits=as_f64(inp.logits), bias=as_f64(inp.bias),
              expert_map=inp.expert_map, capacity=inp.capacity, shared=shared_f64(inp),
              tokens=tokens)
    r = orc.moe_layer(x64, Wo, cfg.k, cfg.renorm, cfg.act, **kw)
    flipped = 0
    if not np.array_equal(r["ids"], ids_g):
        L = r["L"]
        srt = -np.sort(-L, axis=1)
        margin = srt[:, cfg.k - 1] - srt[:, cfg.k] if cfg.k < L.shape[1] else np.full(L.shape[0], np.inf)
        bad = np.nonzero((r["ids"] != ids_g).any(1))[0]
        tau = 1e-4 * np.sqrt(np.mean(L ** 2))
        assert np.all(margin[bad] < tau), "top-k mismatch outside near-ties"
        flipped = bad.size
        r = orc.moe_layer(x64, Wo, cfg.k, cfg.renorm, cfg.act, ids=ids_g, **kw)
    got = out.float().cpu().numpy()[r["tokens"]]
    err = out_err(got, r["out"], cfg.dtype)
    raw = relerr(got, r["out"])
    if report is not None:
        # floor: the raw figure of the exact result itself, rounded once to the
        # output dtype (what the output format alone costs)
        floor = relerr(orc.round_to_dtype(r["out"], cfg.dtype), r["out"])
        report.update(err=err, raw=raw, floor=floor, flipped=flipped, tokens=len(r["tokens"]))
    bar = TOL[cfg.w_dtype if cfg.w_dtype != "bf16" else "bf16"] if tol is None else tol
    assert err <= bar, "relative error %.3g above tolerance %.3g (flipped %d)" % (err, bar, flipped)
    return out, tr, err


BF16_U = 2.0 ** -8  # unit roundoff of bf16: 8 significand bits, round to nearest even


def bwd_error_bounds(inp, dout, ids, balance=0.0):
    """First-order bounds on the error of the bf16 backward, element by element.

    The bf16 path feeds its GEMMs bf16 operands: z (as the forward does), w*z,
    dg, du and dL are rounded once (w*z twice) and all sums are in fp32.  A sum
    of products whose operand carries a relative error of at most n U (U =
    2^-8) is off by at most n U sum |a||b|, so each bound below is that
    absolute-term sum, taken from float64 values; the gate gradients' errors
    are carried through the gate normalisation and the softmax to the router
    gradients.  Returns name -> bound array, for the gradients present.
    """
    cfg = inp.cfg
    U = BF16_U
    k = cfg.k
    x = as_f64(inp.x)
    dout = as_f64(dout)
    W = oracle_weights(inp)
    L = orc.route(k, cfg.renorm, x=x, w_router=as_f64(inp.w_router), bias=as_f64(inp.bias),
                  logits=as_f64(inp.logits))[0]
    ids = np.asarray(ids, np.int64)
    w = orc.gates(L, ids, cfg.renorm)
    offsets, sp, pos = orc.permute(ids, inp.expert_map, cfg.E_loc, inp.capacity)
    act = {"swiglu": orc.silu, "geglu": orc.gelu_erf}[cfg.act]
    T, E = L.shape
    b = {"dw_gate": np.zeros((cfg.E_loc, cfg.h, cfg.d)), "dw_up": np.zeros((cfg.E_loc, cfg.h, cfg.d)),
         "dw_down": np.zeros((cfg.E_loc, cfg.d, cfg.h)), "dgates": np.zeros((T, k))}
    a_gate = np.zeros((T, k))  # sum_c |dz'_c| |z_c| per kept pair
    for e in range(cfg.E_loc):
        rows = sp[offsets[e]:offsets[e + 1]]
        if rows.size == 0:
            continue
        t, j = rows // k, rows % k
        wg, wu, wd = W.expert(e)
        a = x[t]
        g, u = a @ wg.T, a @ wu.T
        A = act(g)
        z = A * u
        dzp = dout[t] @ wd
        ww = w[t, j][:, None]
        dz = ww * dzp
        dg = dz * u * orc.act_grad(g, cfg.act)
        du = dz * A
        a_gate[t, j] = np.sum(np.abs(dzp) * np.abs(z), axis=1)
        b["dw_down"][e] = 2 * U * np.abs(dout[t]).T @ np.abs(ww * z)
        b["dw_gate"][e] = U * np.abs(dg).T @ np.abs(a)
        b["dw_up"][e] = U * np.abs(du).T @ np.abs(a)
    b["dgates"] = U * a_gate
    if inp.wsg is not None:
        sg, su, sd = (as_f64(m) for m in (inp.wsg, inp.wsu, inp.wsd))
        g, u = x @ sg.T, x @ su.T
        A = act(g)
        dz = dout @ sd
        b["dws_down"] = 2 * U * np.abs(dout).T @ np.abs(A * u)
        b["dws_gate"] = U * np.abs(dz * u * orc.act_grad(g, cfg.act)).T @ np.abs(x)
        b["dws_up"] = U * np.abs(dz * A).T @ np.abs(x)
    # router: gate errors through the normalisation and the softmax
    m = L.max(axis=1, keepdims=True)
    pi = np.exp(L - m)
    pi /= pi.sum(axis=1, keepdims=True)
    delta = b["dgates"] * (pos.reshape(T, k) >= 0)
    psel = np.take_along_axis(pi, ids, axis=1)
    if cfg.renorm:
        S = psel.sum(axis=1, keepdims=True)
        ddsel = delta / S + np.sum(delta * psel, axis=1, keepdims=True) / S ** 2
    else:
        ddsel = delta
    ddpi = np.zeros((T, E))
    np.add.at(ddpi, (np.broadcast_to(np.arange(T)[:, None], ids.shape), ids), ddsel)
    dL = orc.moe_layer_bwd(x, W, k, cfg.renorm, cfg.act, dout, w_router=as_f64(inp.w_router),
                           logits=as_f64(inp.logits), bias=as_f64(inp.bias), expert_map=inp.expert_map,
                           capacity=inp.capacity, balance=balance, ids=ids)["dL"]
    ddL = pi * (ddpi + np.sum(ddpi * pi, axis=1, keepdims=True))
    if inp.logits is not None:
        b["dlogits"] = ddL
    else:
        b["dw_router"] = (ddL + U * np.abs(dL)).T @ np.abs(x)
    if inp.bias is not None:
        b["dbias"] = ddL.sum(axis=0)
    return b
