"""Pure-Python brute-force attention for tiny inputs (pins the numpy oracle).

TEST INFRASTRUCTURE ONLY (see oracle.attention).  Works on *unpaged* logical
tensors given as float64 numpy arrays, uses only Python floats, math.exp and
math.fsum, and shares nothing with oracle.attention: no gather, no numpy
reductions, no masking by -inf.  Each output element is the softmax-weighted
sum written out term by term.
"""
from __future__ import annotations

import math
from typing import Optional


def _attend(q_vec, keys, vals, scale):
    """q_vec: list of floats; keys/vals: list of (list of floats).
    Returns (out list, lse float)."""
    if not keys:
        return [0.0] * (len(vals[0]) if vals else 0), -math.inf
    scores = [scale * math.fsum(a * b for a, b in zip(q_vec, kv)) for kv in keys]
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    den = math.fsum(w)
    dv = len(vals[0])
    out = [math.fsum(w[t] * vals[t][d] for t in range(len(vals))) / den for d in range(dv)]
    return out, m + math.log(den)


def decode(q, K, V, seq_lens, scale, Hk):
    """q [B, Hq, D]; K, V: logical per-sequence keys, K[b] of shape [Hk, L_b, D].
    Query head h uses KV head h * Hk // Hq (contiguous groups)."""
    B, Hq, D = q.shape
    out = [[None] * Hq for _ in range(B)]
    lse = [[None] * Hq for _ in range(B)]
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hq):
            g = (h * Hk) // Hq
            keys = [[float(x) for x in K[b][g][t]] for t in range(L)]
            vals = [[float(x) for x in V[b][g][t]] for t in range(L)]
            if L == 0:
                out[b][h], lse[b][h] = [0.0] * D, -math.inf
            else:
                out[b][h], lse[b][h] = _attend([float(x) for x in q[b, h]], keys, vals, scale)
    return out, lse


def prefill(q, k, v, seq_lens, scale, *, k_rope=None, block_mask: Optional[object] = None):
    """Per-sequence lists: q[b] [L, Hq, Dqk], k[b] [L, Hk, Dn], v[b] [L, Hk, Dv],
    k_rope[b] [L, Dr] or None.  Causal with query i seeing key j <= i; with a
    block mask, also mask[b][i // 64][j // 64] must be nonzero.  The rope part
    of each query head is paired with the one shared rope key row."""
    outs, lses = [], []
    for b, L in enumerate(seq_lens):
        qb, kb, vb = q[b], k[b], v[b]
        Hq, Hk = qb.shape[1], kb.shape[1]
        Dn = kb.shape[2]
        ob = [[None] * Hq for _ in range(L)]
        lb = [[None] * Hq for _ in range(L)]
        for i in range(L):
            for h in range(Hq):
                g = (h * Hk) // Hq
                keys, vals = [], []
                for j in range(L):
                    if j > i:
                        continue
                    if block_mask is not None and not block_mask[b][i // 64][j // 64]:
                        continue
                    key = [float(x) for x in kb[j, g]]
                    if k_rope is not None:
                        key = key + [float(x) for x in k_rope[b][j]]
                    keys.append(key)
                    vals.append([float(x) for x in vb[j, g]])
                qv = [float(x) for x in qb[i, h, :Dn + (len(k_rope[b][0]) if k_rope is not None else 0)]]
                if not keys:
                    ob[i][h], lb[i][h] = [0.0] * vb.shape[2], -math.inf
                else:
                    ob[i][h], lb[i][h] = _attend(qv, keys, vals, scale)
        outs.append(ob)
        lses.append(lb)
    return outs, lses


def chunk_prefill(q, k, v, offsets, scale, k_rope=None):
    """Per-sequence lists: q[b] [n_b, Hq, Dn + Dr] (the chunk's queries), k[b]
    [Lk_b, Hk, Dn], v[b] [Lk_b, Hk, Dv] (every logical key of the sequence),
    offsets[b] = Lk_b - n_b, k_rope[b] [Lk_b, Dr] or None.  Query i sees key j
    iff j < Lk_b and j <= offsets[b] + i; the rope part of the query pairs with
    the one shared rope key row."""
    outs, lses = [], []
    for b in range(len(q)):
        qb, kb, vb = q[b], k[b], v[b]
        n, Hq = qb.shape[0], qb.shape[1]
        Lk, Hk = kb.shape[0], kb.shape[1]
        ob = [[None] * Hq for _ in range(n)]
        lb = [[None] * Hq for _ in range(n)]
        for i in range(n):
            for h in range(Hq):
                g = (h * Hk) // Hq
                keys, vals = [], []
                for jj in range(Lk):
                    if jj <= offsets[b] + i:
                        key = [float(x) for x in kb[jj, g]]
                        if k_rope is not None:
                            key = key + [float(x) for x in k_rope[b][jj]]
                        keys.append(key)
                        vals.append([float(x) for x in vb[jj, g]])
                if not keys:
                    ob[i][h], lb[i][h] = [0.0] * vb.shape[2], -math.inf
                else:
                    ob[i][h], lb[i][h] = _attend([float(x) for x in qb[i, h]], keys, vals, scale)
        outs.append(ob)
        lses.append(lb)
    return outs, lses
