"""Float64 brute-force rollout for tiny inputs (pins the oracle; test-only).

Written independently of the oracle: plain Python loops over scalars in
double precision, ``math.exp`` / ``math.tanh``, and the candidate pool built
by the union walk (visit every (row, id) entry of the block's base logits in
order of value descending then id ascending, collecting distinct ids) rather
than by ranking a per-id maximum.  Only usable for vocabularies of a few
dozen ids and widths of a handful.
"""
import math


def _dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += float(x) * float(y)
    return s


def _sig(x):
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


def _cell(x, h, w_ih, w_hh):
    g = len(h)
    out = []
    for j in range(g):
        ar = _dot(w_ih[j], x)
        az = _dot(w_ih[g + j], x)
        an = _dot(w_ih[2 * g + j], x)
        cr = _dot(w_hh[j], h)
        cz = _dot(w_hh[g + j], h)
        cn = _dot(w_hh[2 * g + j], h)
        r = _sig(ar + cr)
        z = _sig(az + cz)
        n = math.tanh(an + r * cn)
        out.append((1.0 - z) * n + z * h[j])
    return out


def _best(cands, val):
    """(winner, top, margin) with the lowest candidate id winning ties."""
    best_id, best = None, None
    for c in sorted(cands):
        if best is None or val[c] > best:
            best_id, best = c, val[c]
    second = None
    for c in cands:
        if c != best_id and (second is None or val[c] > second):
            second = val[c]
    return best_id, best, (math.inf if second is None else best - second)


def union_walk_pool(base_rows, K):
    """Pool of K ids from the block's rows by the union walk."""
    V = len(base_rows[0])
    entries = [(-base_rows[t][v], v) for t in range(len(base_rows)) for v in range(V)]
    entries.sort()
    seen, pool = set(), []
    for _, v in entries:
        if v not in seen:
            seen.add(v)
            pool.append(v)
            if len(pool) == K:
                break
    return sorted(pool)


def brute_rollout(w, hidden, step_s, verified, K, forced=None):
    """w: dict of nested lists / arrays (float), hidden [B][T][H], step_s [B][S][r]."""
    lm, E = w["lm_head"], w["embed"]
    w_ih, w_hh, F1, F2, b2 = w["gru_w_ih"], w["gru_w_hh"], w["fc1_w"], w["fc2_w"], w["fc2_b"]
    V = len(lm)
    B, T = len(hidden), len(hidden[0])
    g = len(w_hh[0])
    res = {"tokens": [], "top1": [], "margin": [], "pools": []}
    for b in range(B):
        rows = [[_dot(hidden[b][t], lm[v]) for v in range(V)] for t in range(T)]
        full = list(range(V))
        cands = full if (K == 0 or K >= V) else union_walk_pool(rows, K)
        res["pools"].append(None if cands is full else cands)
        toks, tops, mars = [], [], []
        p1, top, mar = _best(full, rows[0])
        toks.append(p1)
        tops.append(top)
        mars.append(mar)
        feed = (lambda j: toks[j]) if forced is None else (lambda j: int(forced[b][j]))
        h = [0.0] * g
        h = _cell(E[int(verified[b])], h, w_ih, w_hh)
        h = _cell(E[feed(0)], h, w_ih, w_hh)
        for k in range(1, T):
            u = []
            for i in range(len(F1)):
                a = _dot(F1[i], h) + float(step_s[b][k - 1][i])
                u.append(a * _sig(a))
            val = {c: rows[k][c] + (_dot(F2[c], u) + float(b2[c])) for c in cands}
            tok, top, mar = _best(cands, val)
            toks.append(tok)
            tops.append(top)
            mars.append(mar)
            if k < T - 1:
                h = _cell(E[feed(k)], h, w_ih, w_hh)
        res["tokens"].append(toks)
        res["top1"].append(tops)
        res["margin"].append(mars)
    return res
