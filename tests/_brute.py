"""Brute-force routed attention in pure Python floats, for tiny inputs only.

Written independently of the oracle, straight from the method's description:
posting lists are simulated as streaming ring buffers (a block enters its
address's buffer at the first token of the query block that may first see it,
and the oldest entry is evicted when the buffer exceeds its capacity), probes
scan every product address, and every top-k is a selection loop.  Attention is
an explicit loop over the visible keys with math.exp.
"""

from __future__ import annotations

import math
from collections import deque


def _dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def brute_routed_attention(q, k, v, codebook, bias, w, force=None):
    """q, k, v: lists [S][D] of floats; codebook [G][C][D]; bias [G][C] or None.

    Returns dict(addr, overflow, sel (list of lists), out (list [S][D])) and the raw scores behind every
    decision: logits [nb][G][C] of the block summaries, probe_scores [S][A] of every product address,
    cand_scores [S] (the rerank score of each candidate, in candidate order).
    """
    S, D = len(q), len(q[0])
    blk, L, R, P, cap, M = w.block, w.local, w.remote, w.probes, w.capacity, w.cand_limit
    G, C = len(codebook), len(codebook[0])
    A = C ** G
    nb = S // blk

    def logit(x, g, c):
        return _dot(codebook[g][c], x) + (bias[g][c] if bias is not None else 0.0)

    ksum = []
    for i in range(nb):
        ksum.append([sum(k[i * blk + r][d] for r in range(blk)) / blk for d in range(D)])

    logits = [[[logit(ksum[i], g, c) for c in range(C)] for g in range(G)] for i in range(nb)]
    addr = []
    for i in range(nb):
        a = 0
        for g in range(G):
            best, bv = 0, logit(ksum[i], g, 0)
            for c in range(1, C):
                lv = logit(ksum[i], g, c)
                if lv > bv:
                    best, bv = c, lv
            a = a * C + best
        addr.append(a)

    rings = [deque() for _ in range(A)]
    evicted = 0
    sels, outs, probe_scores, cand_scores = [], [], [], []
    for t in range(S):
        j = t // blk
        if t % blk == 0 and j - L >= 0:
            i = j - L
            ring = rings[addr[i]]
            ring.append(i)
            if len(ring) > cap:
                ring.popleft()
                evicted += 1
        mu = [[logit(q[t], g, c) for c in range(C)] for g in range(G)]
        score = []
        for a in range(A):
            digits, x = [], a
            for _ in range(G):
                digits.append(x % C)
                x //= C
            digits.reverse()
            s = 0.0
            for g in range(G):
                s += mu[g][digits[g]]
            score.append(s)
        chosen, remaining = [], list(range(A))
        for _ in range(min(P, A)):
            best = remaining[0]
            for a in remaining[1:]:
                if score[a] > score[best]:
                    best = a
            chosen.append(best)
            remaining.remove(best)
        cands = []
        for a in chosen:
            cands.extend(reversed(rings[a]))
        cands = cands[:M]
        rho = {i: _dot(q[t], ksum[i]) for i in cands}
        probe_scores.append(score)
        cand_scores.append([rho[i] for i in cands])
        sel, pool = [], list(cands)
        for _ in range(min(R, len(pool))):
            best = pool[0]
            for i in pool[1:]:
                if rho[i] > rho[best] or (rho[i] == rho[best] and i < best):
                    best = i
            sel.append(best)
            pool.remove(best)
        if force is not None and force[t] >= 0 and R > 0:
            f = force[t]
            if f <= j - L and f not in sel:
                if len(sel) < R:
                    sel.append(f)
                else:
                    sel[-1] = f
        keys = [s for i in sel for s in range(i * blk, (i + 1) * blk)]
        keys += list(range(max(0, (j - L + 1) * blk), t + 1))
        sc = [_dot(q[t], k[s]) / math.sqrt(D) for s in keys]
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        z = sum(e)
        outs.append([sum(e[n] * v[s][d] for n, s in enumerate(keys)) / z for d in range(D)])
        sels.append(sel)
    return dict(addr=addr, overflow=evicted, sel=sels, out=outs, logits=logits, probe_scores=probe_scores,
                cand_scores=cand_scores)


def _largest_first(values):
    """The values sorted largest first, by insertion."""
    out = []
    for x in values:
        out.append(x)
        n = len(out) - 1
        while n > 0 and out[n - 1] < x:
            out[n] = out[n - 1]
            n -= 1
        out[n] = x
    return out


def top_gap(values, keep):
    """Smallest difference between neighbours among the `keep` largest values (inf with fewer than two):
    how close a ranking of the top `keep - 1` values, and its boundary with the next, comes to a tie."""
    s = _largest_first(values)[:keep]
    gaps = [s[n] - s[n + 1] for n in range(len(s) - 1)]
    return min(gaps) if gaps else math.inf


def brute_margins(bf, w):
    """The decision margins of one brute-force routing run, each from a full sort of the scores it ranks:
      addr_margin [nb][G]   best minus second-best logit of each subspace (inf with one code)
      second_gap  [nb][G]   second minus third-best logit (inf with fewer than three codes)
      probe_margin [S]      smallest neighbour gap among the min(P + 1, A) best address scores
      sel_margin [S]        smallest neighbour gap among the min(R + 1, n) best candidate scores
                            (inf without candidates or with R = 0)
      alt_gap [nb]          with G > 1, the second-smallest subspace margin minus the smallest (which
                            subspace the alternate address changes); inf with one subspace"""
    G = w.subspaces
    A = w.codes ** G
    addr_margin, second_gap, alt_gap = [], [], []
    for lg in bf["logits"]:
        am = [top_gap(lg[g], 2) if len(lg[g]) > 1 else math.inf for g in range(G)]
        addr_margin.append(am)
        sg = []
        for g in range(G):
            s = _largest_first(lg[g])
            sg.append(s[1] - s[2] if len(s) > 2 else math.inf)
        second_gap.append(sg)
        if G > 1 and w.codes > 1:
            srt = _largest_first([-m for m in am])
            alt_gap.append(srt[0] - srt[1])
        else:
            alt_gap.append(math.inf)
    probe_margin = [top_gap(sc, min(w.probes + 1, A)) for sc in bf["probe_scores"]]
    sel_margin = [top_gap(cs, min(w.remote + 1, len(cs))) if cs and w.remote > 0 else math.inf
                  for cs in bf["cand_scores"]]
    return dict(addr_margin=addr_margin, second_gap=second_gap, probe_margin=probe_margin, sel_margin=sel_margin,
                alt_gap=alt_gap)


def brute_posting_csr(addr, n_addr, local):
    """CSR of the posting lists by counting: off[a] = number of filed blocks (i < nb - L) with an address
    below a; the entries of address a are its filed blocks in ascending order."""
    filed = range(max(0, len(addr) - local))
    off = [sum(1 for i in filed if addr[i] < a) for a in range(n_addr + 1)]
    idx = [i for a in range(n_addr) for i in filed if addr[i] == a]
    return off, idx


def brute_rope(x, base):
    """RoPE as complex multiplication: pair (i, i + D/2) is z = x_i + 1j x_{i+D/2}, times exp(1j pos theta_i)."""
    S, D = len(x), len(x[0])
    half = D // 2
    out = []
    for pos in range(S):
        row = [0.0] * D
        for i in range(half):
            z = complex(x[pos][i], x[pos][i + half]) * complex(math.cos(pos * base ** (-2.0 * i / D)),
                                                                math.sin(pos * base ** (-2.0 * i / D)))
            row[i], row[i + half] = z.real, z.imag
        out.append(row)
    return out
