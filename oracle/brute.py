"""Brute-force decode attention in 50-digit decimal arithmetic.

TEST INFRASTRUCTURE ONLY. A second implementation of the definition (page
"MoA-Structured Decode Attention", §2: Step I scores s = scale * (K q),
Step II softmax with the max subtracted, Step III out = a V; §6: query head h
reads KV head h // (h_q // h_kv)), written independently of ``oracle.c`` in
pure-Python loops over ``decimal.Decimal``. It is meant for tiny inputs only
(a few rows, a few dimensions) and pins the fp64 oracle there: with 50
significant digits its own rounding is far below fp64's.
"""
from __future__ import annotations

from decimal import Decimal, localcontext


def attend_one(q, K, V, scale) -> list[Decimal]:
    """One head: q length d_k, K n x d_k, V n x d_v (nested lists of numbers)."""
    with localcontext() as ctx:
        ctx.prec = 50
        sc = Decimal(float(scale))
        qd = [Decimal(float(x)) for x in q]
        s = [sc * sum(qd[j] * Decimal(float(row[j])) for j in range(len(qd))) for row in K]
        m = max(s)
        e = [(x - m).exp() for x in s]
        Z = sum(e)
        a = [x / Z for x in e]
        d_v = len(V[0])
        return [sum(a[l] * Decimal(float(V[l][d])) for l in range(len(V))) for d in range(d_v)]


def decode(q, k_cache, v_cache, lens, scale):
    """Batched GQA decode: q [B][h_q][d_k], caches [B][h_kv][cap][d], lens [B]."""
    out = []
    for b in range(len(q)):
        h_q, h_kv = len(q[b]), len(k_cache[b])
        g = h_q // h_kv
        n = int(lens[b])
        rows = []
        for h in range(h_q):
            kvh = h // g
            rows.append(attend_one(q[b][h], k_cache[b][kvh][:n], v_cache[b][kvh][:n], scale))
        out.append(rows)
    return out


def decode_multi(q, k_cache, v_cache, lens, scale):
    """Multi-query causal decode as masked attention over the whole cache (the forward form
    with a mask, page "Phase 3, Section 6: StoryLM-0 head-parallel attention", §3: softmax of
    scale * scores + mask over the key axis): q [B][T][h_q][d_k], caches [B][h_kv][cap][d],
    lens [B]. Query t of sequence b sits at position lens[b] - T + t; the mask is 0 for key
    rows at or before that position and minus infinity after it (up to lens[b])."""
    out = []
    with localcontext() as ctx:
        ctx.prec = 50
        sc = Decimal(float(scale))
        minus_inf = Decimal("-Infinity")
        for b in range(len(q)):
            T, h_q, h_kv = len(q[b]), len(q[b][0]), len(k_cache[b])
            g = h_q // h_kv
            L = int(lens[b])
            per_t = []
            for t in range(T):
                pos = L - T + t
                rows = []
                for h in range(h_q):
                    K, V = k_cache[b][h // g][:L], v_cache[b][h // g][:L]
                    qd = [Decimal(float(x)) for x in q[b][t][h]]
                    s = [sc * sum(qd[j] * Decimal(float(K[l][j])) for j in range(len(qd)))
                         + (Decimal(0) if l <= pos else minus_inf) for l in range(L)]
                    m = max(s)
                    e = [(x - m).exp() for x in s]
                    Z = sum(e)
                    rows.append([sum(e[l] / Z * Decimal(float(V[l][d])) for l in range(L))
                                 for d in range(len(V[0]))])
                per_t.append(rows)
            out.append(per_t)
    return out


def decode_lse(q, k_cache, v_cache, lens, scale):
    """Attention over one shard of the rows with each head's log-sum-exp ln sum_l exp(s[l]),
    computed from the definition (the logarithm of the summed exponentials of the scores):
    q [B][h_q][d_k], caches [B][h_kv][cap][d], lens [B] (0: no rows; out 0, lse -Infinity).
    Returns (out [B][h_q][d_v], lse [B][h_q]) as Decimals."""
    outs, lses = [], []
    with localcontext() as ctx:
        ctx.prec = 50
        sc = Decimal(float(scale))
        for b in range(len(q)):
            h_q, h_kv = len(q[b]), len(k_cache[b])
            g = h_q // h_kv
            n = int(lens[b])
            rows, ls = [], []
            for h in range(h_q):
                K, V = k_cache[b][h // g][:n], v_cache[b][h // g][:n]
                d_v = len(v_cache[b][h // g][0])
                if n == 0:
                    rows.append([Decimal(0)] * d_v)
                    ls.append(Decimal("-Infinity"))
                    continue
                qd = [Decimal(float(x)) for x in q[b][h]]
                s = [sc * sum(qd[j] * Decimal(float(row[j])) for j in range(len(qd))) for row in K]
                e = [x.exp() for x in s]
                Z = sum(e)
                rows.append([sum(e[l] / Z * Decimal(float(V[l][d])) for l in range(n)) for d in range(d_v)])
                ls.append(Z.ln())
            outs.append(rows)
            lses.append(ls)
    return outs, lses
