"""Brute-force masked attention with exact pure-Python sums (oracle; test infrastructure only).

Builds the full visibility matrix explicitly -- query row i (owned by chunk
c(i)) sees logical key j iff kv_begin[c(i)] <= j < kv_end[c(i)] -- and
evaluates softmax attention over all j with that mask, summing with
``math.fsum``.  Only for tiny inputs (a few hundred rows/keys).  It pins the
slicing and chunk bookkeeping of ``attention.chunk_attention`` against an
independently written formulation of the same definition (Wave Forcing
abstract: chunk-wise causal attention; keys of earlier chunks plus the
chunk's own tokens).
"""
import math


def brute_force_attention(q, k, v, q_off, kv_begin, kv_end, scale=None):
    """q [Nq][H][D], k/v [L][H][D] as nested sequences or arrays (key j = logical position j).

    Returns (O as nested lists [Nq][H][D], LSE as nested lists [H][Nq]).
    """
    nq = len(q)
    nh = len(q[0])
    d = len(q[0][0])
    nkeys = len(k)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    owner = [None] * nq
    for c in range(len(q_off) - 1):
        for i in range(int(q_off[c]), int(q_off[c + 1])):
            owner[i] = c
    if any(x is None for x in owner):
        raise ValueError("query offsets must cover every query row")
    mask = [[int(kv_begin[owner[i]]) <= j < int(kv_end[owner[i]]) for j in range(nkeys)]
            for i in range(nq)]
    o = [[[0.0] * d for _ in range(nh)] for _ in range(nq)]
    lse = [[0.0] * nq for _ in range(nh)]
    for i in range(nq):
        for h in range(nh):
            scores = {}
            for j in range(nkeys):
                if mask[i][j]:
                    scores[j] = scale * math.fsum(float(q[i][h][t]) * float(k[j][h][t]) for t in range(d))
            if not scores:
                raise ValueError("row %d sees no key" % i)
            m = max(scores.values())
            w = {j: math.exp(s - m) for j, s in scores.items()}
            l = math.fsum(w.values())
            for t in range(d):
                o[i][h][t] = math.fsum(w[j] * float(v[j][h][t]) for j in w) / l
            lse[h][i] = m + math.log(l)
    return o, lse
