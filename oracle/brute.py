"""Brute-force layer for tiny inputs, in pure Python scalar loops.

TEST INFRASTRUCTURE ONLY.  It shares nothing with ``moe_oracle`` (no NumPy
arithmetic, no sorting routine): every expert is evaluated for every token and
the output is sum_e G[t, e] * FFN_e(x_t) with a dense gate matrix G that is
zero for unselected experts.  The selection is an explicit scan for the
largest score, repeated k times; the permutation is built by appending each
assignment to its expert's bucket in order.  It exists to pin the oracle.
"""

from __future__ import annotations

import math


def _rows(a):
    return [list(map(float, r)) for r in a]


def brute_forward(hidden, gain, w_router, bias, w_gate, w_up, w_down, k: int, eps: float):
    H = _rows(hidden)
    g = [float(v) for v in gain]
    Wr = _rows(w_router)
    b = [float(v) for v in bias]
    E = len(Wr)
    d = len(g)
    F = len(w_gate[0])
    out, sel_all, gate_all = [], [], []
    for h in H:
        ss = 0.0
        for v in h:
            ss += v * v
        r = math.sqrt(ss / d + eps)
        x = [g[i] * (h[i] / r) for i in range(d)]
        z = []
        for e in range(E):
            acc = 0.0
            for i in range(d):
                acc += float(Wr[e][i]) * x[i]
            z.append(acc)
        s = [z[e] + b[e] for e in range(E)]
        chosen = []
        for _ in range(k):
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or s[e] > s[best]:
                    best = e
            chosen.append(best)
        if k == 1:
            den = sum(math.exp(z[e]) for e in range(E))
            gts = [math.exp(z[chosen[0]]) / den]
        else:
            den = sum(math.exp(z[e]) for e in chosen)
            gts = [math.exp(z[e]) / den for e in chosen]
        G = [0.0] * E
        for e, gt in zip(chosen, gts):
            G[e] = gt
        o = [0.0] * d
        for e in range(E):
            # every expert, every token; unselected ones carry G = 0
            a = []
            for f in range(F):
                gg = 0.0
                uu = 0.0
                for i in range(d):
                    gg += float(w_gate[e][f][i]) * x[i]
                    uu += float(w_up[e][f][i]) * x[i]
                a.append(gg / (1.0 + math.exp(-gg)) * uu)
            for m in range(d):
                acc = 0.0
                for f in range(F):
                    acc += float(w_down[e][m][f]) * a[f]
                o[m] += G[e] * acc
        out.append(o)
        sel_all.append(chosen)
        gate_all.append(gts)
    # bucket permutation
    buckets = [[] for _ in range(E)]
    for t, ch in enumerate(sel_all):
        for j, e in enumerate(ch):
            buckets[e].append(t * k + j)
    counts = [len(bk) for bk in buckets]
    gather, scatter = [], [0] * (len(H) * k)
    for e in range(E):
        for a in buckets[e]:
            scatter[a] = len(gather)
            gather.append(a // k)
    return {"out": out, "sel": sel_all, "gate": gate_all, "counts": counts,
            "gather": gather, "scatter": scatter}
