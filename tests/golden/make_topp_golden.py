"""Writes topp_golden.json: hand-derived top-k / top-p selections for small score rows.

The expected selections come from the definition of the hybrid rule (SpargeAttention2
page, section 2(1): keep the union of the top-k% entries and of the smallest set whose
cumulative probability reaches p), evaluated here in exact-enough decimal arithmetic
(60 digits) from the softmax of the given scores. Nothing here imports the oracle.
p values are chosen halfway between consecutive cumulative probabilities, so no fp32
rounding inside a correct implementation can move the boundary.

Run: python tests/golden/make_topp_golden.py
"""
import json
import math
import os
from decimal import Decimal, getcontext

getcontext().prec = 60


def softmax_cum(scores):
    order = sorted(range(len(scores)), key=lambda j: (-scores[j], j))
    m = max(scores)
    e = [Decimal(s - m).exp() for s in scores]
    z = sum(e)
    cum, acc = [], Decimal(0)
    for j in order:
        acc += e[j]
        cum.append(acc / z)
    return order, cum


def m_k(k, n):
    return min(n, max(1, math.ceil(k * n - 1e-9)))


def case(name, scores, k, cite, p_list=None):
    order, cum = softmax_cum(scores)
    n = len(scores)
    out = []
    if p_list is None:
        # midpoints between consecutive cumulative probabilities, plus the extremes
        p_list = [float(cum[0] / 2)] + [float((cum[i] + cum[i + 1]) / 2) for i in range(n - 1)]
    for p in p_list:
        if p >= 1.0:
            mp = n
        else:
            mp = next((r + 1 for r in range(n) if cum[r] >= Decimal(p)), n)
        keep = max(m_k(k, n), mp)
        out.append({"p": p, "m_p": mp, "kept": sorted(order[:keep])})
    return {"name": name, "scores": scores, "k": k, "cite": cite, "m_k": m_k(k, n), "cases": out}


def main():
    fixtures = [
        case("geometric_8", [3.0, 2.0, 1.0, 0.0, -1.0, -2.0, -3.0, -4.0], 0.25,
             "SpargeAttention2 page, section 2(1): top-p = smallest set reaching p"),
        case("permuted_geometric_8", [0.0, -4.0, 3.0, -1.0, 1.0, -3.0, 2.0, -2.0], 0.25,
             "SpargeAttention2 page, section 2(1): selection follows scores, not positions"),
        case("two_level_12", [1.5] * 3 + [0.0] * 9, 0.1,
             "SpargeAttention2 page, section 2(1): union of the two rules"),
        case("p_one_keeps_all", [2.0, 0.5, -1.0, 0.25], 0.0,
             "SpargeAttention2 page, section 2(1): p = 1 needs every entry", [1.0]),
    ]
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "topp_golden.json"), "w") as f:
        json.dump(fixtures, f, indent=1)


if __name__ == "__main__":
    main()
