"""Pure-Python brute-force restatement of the LSA path for tiny inputs.

TEST INFRASTRUCTURE ONLY.  Written independently of ``lsa_oracle`` (no shared
helpers) and with different formulations where one exists, so that the two can
check each other:
  * selection by rank counting: a candidate is taken when fewer than m other
    candidates beat it (higher score, or equal score and lower position), instead
    of sorting;
  * softmax without the max shift (inputs are tiny, no overflow);
  * block means and scores by explicit sums.
Same readings as the numpy oracle (R1-R11, R15, R16).
"""
from __future__ import annotations

import math


def relu(x):
    return x if x > 0.0 else 0.0


def score(q, w, k):
    """sum_h w[h] * ReLU(sum_d q[h][d] * k[d])  (R1)."""
    tot = 0.0
    for h in range(len(q)):
        dot = 0.0
        for d in range(len(k)):
            dot += q[h][d] * k[d]
        tot += w[h] * relu(dot)
    return tot


def coarse(q, w, kb):
    """max_h w[h] * ReLU(q[h] . kb)  (R10)."""
    best = None
    for h in range(len(q)):
        dot = 0.0
        for d in range(len(kb)):
            dot += q[h][d] * kb[d]
        v = w[h] * relu(dot)
        best = v if best is None or v > best else best
    return best


def forced(p, S, W):
    """Sink [0,S) and window [p-W+1, p] inside [0, p]  (R4, R5)."""
    return {s for s in range(p + 1) if s < S or s > p - W}


def beats(a, b, sc):
    return sc[a] > sc[b] or (sc[a] == sc[b] and a < b)


def rank_select(cands, sc, m):
    """Candidates beaten by fewer than m others (R6): the top m by (score desc, pos asc)."""
    out = []
    for s in cands:
        n_better = sum(1 for c in cands if c != s and beats(c, s, sc))
        if n_better < m:
            out.append(s)
    return out


def select(scores_by_pos, p, K, S, W, cands=None):
    F = forced(p, S, W)
    if cands is None:
        cands = [s for s in range(p + 1) if s not in F]
    fill = rank_select(cands, scores_by_pos, K - len(F))
    sel = sorted(set(F) | set(fill))
    return sel + [-1] * (K - len(sel))


def means(keys, Bs, nb):
    out = []
    for j in range(nb):
        acc = [0.0] * len(keys[0])
        for s in range(j * Bs, j * Bs + Bs):
            for d in range(len(acc)):
                acc[d] += keys[s][d]
        out.append([a / Bs for a in acc])
    return out


def hi_select(q, w, keys, p, K, S, W, Bs, n_keep):
    """Coarse block top-n_keep (eligible blocks only, R9), then fine select inside."""
    F = forced(p, S, W)
    nb = len(keys) // Bs
    kb = means(keys, Bs, nb)
    elig = [j for j in range(nb)
            if j * Bs + Bs - 1 <= p and any(s not in F for s in range(j * Bs, j * Bs + Bs))]
    csc = {j: coarse(q, w, kb[j]) for j in elig}
    kept = sorted(rank_select(elig, csc, n_keep))
    cands = set()
    for j in kept:
        cands |= {s for s in range(j * Bs, j * Bs + Bs) if s <= p and s not in F}
    tail_lo = ((p + 1) // Bs) * Bs
    cands |= {s for s in range(tail_lo, p + 1) if s not in F}
    cands = sorted(cands)
    sc = {s: score(q, w, keys[s]) for s in cands}
    return select(sc, p, K, S, W, cands), kept + [-1] * (n_keep - len(kept))


def attend(q, k_rows, v_rows, idx, tau, Hkv):
    """Softmax over the selected rows, written as exp(z)/sum exp(z) (no shift)."""
    Hq = len(q)
    g = Hq // Hkv
    sel = [s for s in idx if s >= 0]
    outs, lses = [], []
    for hq in range(Hq):
        kvh = hq // g
        ez = []
        for s in sel:
            z = 0.0
            for d in range(len(q[hq])):
                z += q[hq][d] * k_rows[s][kvh][d]
            ez.append(math.exp(tau * z))
        den = sum(ez)
        dv = len(v_rows[0][kvh])
        o = [sum(ez[i] * v_rows[s][kvh][c] for i, s in enumerate(sel)) / den for c in range(dv)]
        outs.append(o)
        lses.append(math.log(den))
    return outs, lses
