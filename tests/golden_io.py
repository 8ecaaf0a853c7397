"""Readers for the hand-worked fixtures under tests/golden/."""
import math
import os
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


def _logit(tok):
    neg = tok.startswith("-")
    t = tok[1:] if neg else tok
    v = math.log(float(t[3:-1])) if t.startswith("ln(") else float(t)
    return -v if neg else v


def route_cases():
    cases, cur = [], {}
    for ln in _lines("route_worked_example.txt"):
        key, _, val = ln.partition(":")
        toks = val.split()
        if key == "logits":
            cur = {"logits": [_logit(t) for t in toks]}
            cases.append(cur)
        elif key == "k":
            cur["k"] = int(toks[0])
        elif key == "ids":
            cur["ids"] = [int(t) for t in toks]
        else:
            cur[key] = [float(Fraction(t)) for t in toks]
    return cases


def int4_case():
    out = {}
    for ln in _lines("int4_worked_example.txt"):
        key, _, val = ln.partition(":")
        toks = val.split()
        if key.endswith("_w"):
            out[key] = [float(t) for t in toks]
        elif key.endswith("_scale_bits"):
            out[key] = int(toks[0], 16)
        elif key.endswith("_codes"):
            out[key] = [int(t) for t in toks]
        elif key.endswith("_bytes"):
            out[key] = [int(t, 16) for t in toks]
    return out


def activation_points():
    pts = []
    for ln in _lines("activations.txt"):
        name, g, v = ln.split()
        pts.append((name, float(g), float(v)))
    return pts


def tree_route_cases():
    """Cases of tree_route_worked_example.txt: dicts with branch, levels, E, x,
    rows and a list of (k, ids, w_raw, w_renorm, margin or None)."""
    cases, cur, sub = [], None, None
    for ln in _lines("tree_route_worked_example.txt"):
        key, _, val = ln.partition(":")
        toks = val.split()
        if key == "branch":
            cur = {"branch": int(toks[0]), "rows": [], "subs": []}
            cases.append(cur)
        elif key in ("levels", "E"):
            cur[key] = int(toks[0])
        elif key == "x":
            cur["x"] = [_logit(t) for t in toks]
        elif key == "row":
            cur["rows"].append([_logit(t) for t in toks])
        elif key == "k":
            sub = {"k": int(toks[0]), "margin": None}
            cur["subs"].append(sub)
        elif key == "ids":
            sub["ids"] = [int(t) for t in toks]
        elif key == "margin":
            sub["margin"] = float(toks[0])
        else:
            sub[key] = [float(Fraction(t)) for t in toks]
    return cases
