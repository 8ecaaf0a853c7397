"""GPU parity of the whole layer on seeded random shapes, against the float64
oracle (the same protocol as test_gpu_parity.check_layer: selection and
grouping bit-exact on the GPU's own logits and ids, outputs within the dtype
tolerance of the oracle).

Each case draws, from its seed: a base workload (its dtype, weights and
activation), token count, widths, expert count, top-k, shared expert,
capacity, router bias skew, owner share (INT4) and a tile hint, so that the
kernels' edge paths (ragged tiles, empty experts, capacity drops, one-token
batches, every tile shape) are crossed with each other.  Sizes stay small
enough for the oracle to finish in a second or two per case.
"""
import dataclasses

import numpy as np
import pytest

from moe_synth import make_inputs, scaled
from moe_testutil import check_layer, device_weights

pytestmark = pytest.mark.gpu
N_CASES = 64


def random_case(seed):
    rng = np.random.default_rng(9000 + seed)
    base = str(rng.choice(["granular_bf16", "wide_geglu_bf16", "decode_bf16", "int4_share", "tiny_fp32"]))
    i4, f32 = base == "int4_share", base == "tiny_fp32"
    unit = 128 if i4 else 64
    d = int(unit * rng.integers(1, 9 if unit == 64 else 5))
    h = int(unit * rng.integers(1, 9))
    # a quarter of the bf16 cases on the wide 256-row tiles (d % 256, h % 128)
    wide = not (i4 or f32) and rng.random() < 0.25
    if wide:
        d, h = int(256 * rng.integers(1, 3)), int(128 * rng.integers(1, 5))
    E = int(rng.integers(2, 97))
    k = int(rng.integers(1, min(E, 8) + 1))
    r = rng.random()
    T = 1 if r < 0.1 else int(rng.integers(2, 64)) if r < 0.4 else int(rng.integers(64, 3000))
    # keep the oracle's float64 GEMMs to a second or two
    T = max(1, min(T, int(4e8 // (6 * k * d * h))))
    kw = dict(T=T, d=d, E=E, k=k, h=h, act=str(rng.choice(["swiglu", "geglu"])))
    kw["h_shared"] = int(64 * rng.integers(1, 9)) if (not f32 and rng.random() < 0.4) else 0
    kw["capacity_factor"] = float(rng.choice([0.5, 1.0, 2.0])) if rng.random() < 0.3 else None
    kw["zipf_bias"] = float(rng.choice([0.5, 1.1, 1.5])) if rng.random() < 0.4 else None
    if i4:
        kw["owners"] = int(rng.choice([1, 2, 4]))
    cfg = dataclasses.replace(scaled(base, seed=seed, **kw), name="random_%d" % seed)
    # a tile hint the shapes allow (0 = the automatic plan)
    if f32:
        choices = [0, 16, 32]
    elif i4:
        choices = [0, 16, 32, 64]
    else:
        choices = [0, 16, 32, 64, 128] + ([256] if (h % 128 == 0 and d % 256 == 0) else [])
    tile_m = 256 if wide else int(rng.choice(choices))
    return cfg, tile_m


@pytest.mark.parametrize("seed", range(N_CASES))
def test_layer_random_shapes(seed):
    import sparse_mixture_experts_lds_amd as moe
    moe.load()
    cfg, tile_m = random_case(seed)
    print(cfg, "tile_m", tile_m, flush=True)
    inp = make_inputs(cfg)
    w = device_weights(inp)
    w.tiles = (tile_m, 0, 0)
    rep = {}
    check_layer(inp, wdev=w, report=rep)
    print(seed, rep)
