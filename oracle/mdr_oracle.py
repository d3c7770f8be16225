"""CPU oracle for the forward pass of Monodratic routed sparse causal attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and never imports it.

What it computes, step by step, for one (batch, head) at a time:

  1. block key summaries: the mean of each block's post-RoPE key rows;
  2. a product address per block: one codebook argmax per subspace, combined
     as a mixed-radix number;
  3. causal posting lists: the blocks filed under each address, a query block
     j seeing only blocks i <= j - L and at most ``capacity`` of them (the most
     recent), with overflow counted;
  4. per query token: probe scores over the product address space, the top-P
     addresses, the concatenated candidate blocks (at most M), a rerank by the
     dot product with the block key summaries, the top-R remote blocks (plus an
     optional forced target block under the same budget);
  5. exact causal softmax attention over the tokens of the selected remote
     blocks and the L local blocks, computed densely under the selected mask.

Sources (the pages are web write-ups of the method; cited by title and section):
  * aitechinspire.com write-up of Monodratic, "Snapshot: key facts from the
    report" and "What's the core idea?": RoPE before addressing; source blocks
    assigned to bounded causal posting lists; each query probes product
    addresses, reranks candidates, keeps a fixed number of remote blocks, adds
    guaranteed local blocks and runs exact causal softmax over those tokens;
    a stateless [batch, sequence, width] -> attention-delta mixer.
  * remio.ai, "Monodratic claims learned routing can make sparse causal
    attention more selective", section "Monodratic turns sparse attention into
    a retrieval decision": a product address combines the decisions of several
    learned code components and points to a bounded posting list; a source
    block may never become available to a query placed before it; capacity
    bounds every returned list and overflow may drop blocks.
  * same article, section "Why learned product-hash routing matters now":
    index assignment is the coarse filter, query probes generate candidates,
    reranking makes the finer choice, exact attention aggregates; forcing the
    labelled block keeps the same maximum second-stage budget.

Readings where the pages leave a step open (each is also listed in the design
notes): routing is per query token; the block summary is the mean key; an
address is the per-subspace argmax of codebook logits over the whole summary,
subspace 0 most significant, ties to the smaller code; probes are the P
addresses with the largest summed per-subspace query logits, ties to the
smaller address; a block is eligible for query block j when i <= j - L; a
posting view holds the newest ``capacity`` eligible entries, newest first;
candidates are concatenated in probe rank order and cut at M; the rerank score
is the unscaled dot product with the summary, ties to the smaller block; a
forced target fills a free slot or replaces the last one; local blocks are the
L most recent including the current one; softmax scale 1/sqrt(D); RoPE pairs
(i, i + D/2) with theta_i = base^(-2i/D).

Precision: every routing decision (argmax, top-P, top-R) is taken in
``rdtype`` -- float32 by default, the precision of the GPU kernels -- and the
oracle records the score margin of each decision so that callers can tell
near-ties apart.  Attention is computed in float64.
"""

from __future__ import annotations

import math

import numpy as np

INF = float("inf")


# ---------------------------------------------------------------- 1. summaries

def block_summaries(k: np.ndarray, block: int, rdtype=np.float32) -> np.ndarray:
    """Mean of each block's key rows.  k [S, D] -> [nb, D] in ``rdtype``."""
    S, D = k.shape
    nb = S // block
    kb = np.asarray(k[: nb * block], dtype=rdtype).reshape(nb, block, D)
    return (kb.sum(axis=1, dtype=rdtype) / rdtype(block)).astype(rdtype)


# ---------------------------------------------------------------- 2. addresses

def code_logits(x: np.ndarray, codebook: np.ndarray, bias, rdtype=np.float32) -> np.ndarray:
    """Per-subspace code logits <codebook[g, c], x> + bias[g, c].  x [n, D] -> [n, G, C]."""
    G, C, D = codebook.shape
    w = np.asarray(codebook, dtype=rdtype).reshape(G * C, D)
    lg = (np.asarray(x, dtype=rdtype).reshape(-1, D) @ w.T).reshape(-1, G, C)
    if bias is not None:
        lg = lg + np.asarray(bias, dtype=rdtype)[None]
    return lg.astype(rdtype)


def address_of_codes(codes: np.ndarray, n_codes: int) -> np.ndarray:
    """Mixed-radix product address, subspace 0 most significant.  codes [..., G] -> [...]."""
    G = codes.shape[-1]
    addr = np.zeros(codes.shape[:-1], dtype=np.int64)
    for g in range(G):
        addr = addr * n_codes + codes[..., g]
    return addr


def block_addresses(ksum: np.ndarray, codebook: np.ndarray, bias, rdtype=np.float32):
    """Per-block codes [nb, G], product address [nb] and per-subspace argmax margin [nb, G].

    The argmax takes the first (smallest) code among equal logits.  The margin is
    top1 - top2 of the logits (inf when C == 1).
    """
    G, C, _ = codebook.shape
    lg = code_logits(ksum, codebook, bias, rdtype)
    codes = lg.argmax(axis=2)
    if C > 1:
        srt = np.sort(lg, axis=2)
        margin = srt[..., -1].astype(np.float64) - srt[..., -2].astype(np.float64)
    else:
        margin = np.full(codes.shape, INF)
    return codes.astype(np.int64), address_of_codes(codes, C), margin


# ---------------------------------------------------------------- 3. posting lists

def posting_lists(addr: np.ndarray, n_addr: int, local: int) -> list:
    """Blocks filed under each address, in ascending block order.

    Only blocks that some query block can see are filed: block i becomes
    eligible at query block i + L, so the last L blocks are never filed.
    """
    nb = len(addr)
    lists = [[] for _ in range(n_addr)]
    for i in range(max(0, nb - local)):
        lists[int(addr[i])].append(i)
    return lists


def posting_csr(lists: list):
    """(offsets [A+1], block indices) of the posting lists."""
    off = np.zeros(len(lists) + 1, dtype=np.int64)
    for a, lst in enumerate(lists):
        off[a + 1] = off[a] + len(lst)
    idx = np.array([i for lst in lists for i in lst], dtype=np.int64)
    return off, idx


def posting_overflow(lists: list, capacity: int) -> int:
    """Blocks that a list of ``capacity`` entries had to drop: sum_a max(0, n_a - capacity)."""
    return int(sum(max(0, len(lst) - capacity) for lst in lists))


def posting_view(lists: list, a: int, j: int, local: int, capacity: int) -> list:
    """What query block j reads from address a: the newest ``capacity`` blocks i <= j - L, newest first."""
    cutoff = j - local
    if cutoff < 0:
        return []
    elig = [i for i in lists[a] if i <= cutoff]
    return elig[::-1][:capacity]


# ---------------------------------------------------------------- 3b. overflow redirect
#
# The pages name two ways to handle a full posting list -- drop the block or redirect it -- and warn
# that either may hide relevant blocks (remio.ai, section "Monodratic turns sparse attention into a
# retrieval decision"); they ask overflow stress tests to report dropped candidates and fallback
# behaviour (same article, "What sparse attention researchers should watch next").  They fix no
# redirect rule.  The reading taken here keeps the drop policy's views unchanged and only reuses
# spare capacity:
#   * a block's alternate address is its own address with one digit changed: in the subspace whose
#     top two code logits are closest (smallest top1 - top2, ties to the smaller subspace), the
#     runner-up code (second by logit desc, code asc) replaces the top code.  No alternate when C = 1.
#   * a filed block leaves its primary view when the capacity-th newer block of the same address
#     becomes eligible, at query block (that block) + L; at that moment it is filed, in time order,
#     into its alternate address's redirect list.
#   * the view of address a at query block j is the drop-policy view (newest `capacity` eligible
#     primaries, newest first) followed, while slots remain, by the newest redirected blocks whose
#     redirect time is <= j, newest first.

def runner_up_codes(ksum: np.ndarray, codebook: np.ndarray, bias, rdtype=np.float32):
    """Per block and subspace: the runner-up code (second by logit desc, code asc) [nb, G] (-1 when
    C == 1) and the margin top1 - top2 evaluated in ``rdtype`` [nb, G] (inf when C == 1)."""
    G, C, _ = codebook.shape
    lg = code_logits(ksum, codebook, bias, rdtype)
    nb = lg.shape[0]
    second = np.full((nb, G), -1, dtype=np.int64)
    margin = np.full((nb, G), INF)
    if C == 1:
        return second, margin
    for i in range(nb):
        for g in range(G):
            order = sorted(range(C), key=lambda c: (-float(lg[i, g, c]), c))
            second[i, g] = order[1]
            margin[i, g] = float(rdtype(lg[i, g, order[0]]) - rdtype(lg[i, g, order[1]]))
    return second, margin


def runner_up_gap(ksum: np.ndarray, codebook: np.ndarray, bias, rdtype=np.float32) -> np.ndarray:
    """Per block and subspace, second - third largest logit [nb, G] (inf when C < 3): how close the
    runner-up choice itself is to a tie."""
    G, C, _ = codebook.shape
    lg = code_logits(ksum, codebook, bias, rdtype)
    if C < 3:
        return np.full(lg.shape[:2], INF)
    srt = np.sort(lg.astype(np.float64), axis=2)
    return srt[..., -2] - srt[..., -3]


def alternate_addresses(codes: np.ndarray, second: np.ndarray, margin: np.ndarray, n_codes: int):
    """Alternate address of each block [nb] (-1 when C == 1) and the gap between the smallest and the
    next smallest subspace margin (the decision's own margin; inf with one subspace)."""
    nb, G = codes.shape
    alt = np.full(nb, -1, dtype=np.int64)
    gap = np.full(nb, INF)
    if n_codes == 1:
        return alt, gap
    for i in range(nb):
        g_star = min(range(G), key=lambda g: (margin[i, g], g))
        digits = list(codes[i])
        digits[g_star] = int(second[i, g_star])
        a = 0
        for d in digits:
            a = a * n_codes + d
        alt[i] = a
        if G > 1:
            rest = sorted(margin[i, g] for g in range(G) if g != g_star)
            gap[i] = rest[0] - margin[i, g_star]
    return alt, gap


def redirect_lists(lists: list, alt: np.ndarray, capacity: int, local: int) -> list:
    """Per address, the blocks redirected into it as (time, block) in time order.  The block at
    position k of list a leaves the primary view when the block at position k + capacity becomes
    eligible, i.e. at query block lists[a][k + capacity] + L."""
    rd = [[] for _ in range(len(lists))]
    for lst in lists:
        for k in range(len(lst) - capacity):
            x = lst[k]
            if alt[x] >= 0:
                rd[int(alt[x])].append((lst[k + capacity] + local, x))
    for r in rd:
        r.sort()
    return rd


def posting_view_redirect(lists: list, rd: list, a: int, j: int, local: int, capacity: int) -> list:
    """The drop-policy view of address a at query block j, then the newest redirected blocks with
    time <= j (newest first) while slots remain."""
    view = posting_view(lists, a, j, local, capacity)
    room = capacity - len(view)
    if room > 0:
        arrived = [x for (tm, x) in rd[a] if tm <= j]
        view = view + arrived[::-1][:room]
    return view


def redirect_overflow(lists: list, rd: list, capacity: int) -> int:
    """Blocks no final view returns: the drop-policy overflow minus the redirected blocks that fill
    spare slots at the last query block (every redirect happens by then)."""
    shown = sum(min(max(0, capacity - len(lists[a])), len(rd[a])) for a in range(len(lists)))
    return posting_overflow(lists, capacity) - shown


def view_dropped(lists: list, rd, alt, a: int, j: int, local: int, capacity: int) -> int:
    """Eligible blocks held by address a at query block j that its view does not return:
    max(0, held - capacity).  Under drop, a holds its eligible primaries; under redirect, those
    not yet redirected away (a block left behind without an alternate stays held and dropped),
    plus the redirected blocks that have arrived."""
    cutoff = j - local
    elig = [i for i in lists[a] if i <= cutoff]
    held = len(elig)
    if rd is not None:
        away = sum(1 for i in elig[:max(0, len(elig) - capacity)] if alt[i] >= 0)
        held += sum(1 for (tm, _) in rd[a] if tm <= j) - away
    return max(0, held - capacity)


# ---------------------------------------------------------------- 4. probe, candidates, rerank

def address_scores(mu: np.ndarray, n_codes: int) -> np.ndarray:
    """sigma[a] = sum over subspaces g (in order) of mu[g, digit_g(a)].  mu [..., G, C] -> [..., A]."""
    G = mu.shape[-2]
    a = np.arange(n_codes ** G)
    sigma = None
    for g in range(G):
        digit = (a // n_codes ** (G - 1 - g)) % n_codes
        term = mu[..., g, digit]
        sigma = term if sigma is None else sigma + term
    return sigma


def top_probes(sigma: np.ndarray, probes: int):
    """Top-P addresses by score, ties to the smaller address.

    Also returns the decision margin: the smallest gap between consecutive scores
    among the best min(P + 1, A) (rank order matters downstream, not only the
    boundary between the P-th and the (P+1)-th address)."""
    order = np.argsort(-sigma, axis=-1, kind="stable")
    top = order[..., :probes]
    A = sigma.shape[-1]
    n = min(probes + 1, A)
    if n >= 2:
        s = np.take_along_axis(sigma, order[..., :n], axis=-1).astype(np.float64)
        margin = (s[..., :-1] - s[..., 1:]).min(axis=-1)
    else:
        margin = np.full(sigma.shape[:-1], INF)
    return top, margin


def rerank(q_t: np.ndarray, ksum: np.ndarray, cands: list, remote: int, rdtype=np.float32):
    """Top-R candidates by <q_t, summary>, ties to the smaller block; (selected, margin).

    The margin is the smallest gap between consecutive scores among the best
    min(R + 1, n) candidates (the selection is stored in rank order)."""
    if not cands or remote == 0:
        return [], INF
    rho = np.asarray(ksum[cands], dtype=rdtype) @ np.asarray(q_t, dtype=rdtype)
    order = sorted(range(len(cands)), key=lambda n: (-float(rho[n]), cands[n]))
    sel = [cands[n] for n in order[:remote]]
    top = [float(rho[n]) for n in order[:remote + 1]]
    margin = min((a - b for a, b in zip(top[:-1], top[1:])), default=INF)
    return sel, margin


def apply_force(sel: list, f: int, j: int, local: int, remote: int):
    """Force block f into the selection without growing it past ``remote``.

    f must be eligible (0 <= f <= j - L); it fills a free slot, or replaces the
    lowest-ranked selected block when all R slots are taken.  Returns (sel, ignored).
    """
    if f < 0:
        return sel, False
    if f > j - local or remote == 0:
        return sel, True
    if f in sel:
        return sel, False
    sel = list(sel)
    if len(sel) < remote:
        sel.append(f)
    else:
        sel[remote - 1] = f
    return sel, False


def route_head(q: np.ndarray, k: np.ndarray, codebook: np.ndarray, bias, w, force=None,
               tokens=None, rdtype=np.float32, policy: str = "drop", addr=None, alt=None) -> dict:
    """Routing for one (batch, head).  q, k [S, D] post-RoPE; codebook [G, C, D]; bias [G, C] or None.

    ``w`` carries the sizes (block, codes, capacity, probes, cand_limit, remote,
    local).  ``tokens`` restricts the per-token steps to a subset (all by default).
    Returns the summaries, codes, addresses, posting lists, overflow, and per
    token the probes, candidates, selection, capacity-dropped candidates and
    decision margins.  ``policy`` is "drop" or "redirect" (section 3b).  ``addr`` [nb], when given,
    replaces the computed block addresses (so the posting lists, probes and rerank can be checked on
    another implementation's addresses); the summaries, codes and margins are still this oracle's.
    ``alt`` [nb] likewise replaces the alternate addresses of the redirect policy.
    """
    S, D = q.shape
    blk, L, R, P = w.block, w.local, w.remote, w.probes
    G, C, _ = codebook.shape
    A = C ** G
    M = w.cand_limit
    ksum = block_summaries(k, blk, rdtype)
    codes, own_addr, addr_margin = block_addresses(ksum, codebook, bias, rdtype)
    addr = own_addr if addr is None else np.asarray(addr, dtype=np.int64)
    lists = posting_lists(addr, A, L)
    off, idx = posting_csr(lists)
    alt = alt_gap = rd = None
    if policy == "redirect":
        second, margin32 = runner_up_codes(ksum, codebook, bias, rdtype)
        own_alt, alt_gap = alternate_addresses(codes, second, margin32, C)
        alt = own_alt if alt is None else np.asarray(alt, dtype=np.int64)
        rd = redirect_lists(lists, alt, w.capacity, L)
        overflow = redirect_overflow(lists, rd, w.capacity)
    elif policy == "drop":
        overflow = posting_overflow(lists, w.capacity)
    else:
        raise ValueError(f"unknown overflow policy {policy!r}")

    toks = np.arange(S) if tokens is None else np.asarray(tokens, dtype=np.int64)
    mu = code_logits(q[toks], codebook, bias, rdtype)             # [n, G, C]
    sigma = address_scores(mu, C)                                  # [n, A]
    probes, probe_margin = top_probes(sigma, min(P, A))
    n = len(toks)
    sel = np.full((n, R), -1, dtype=np.int64)
    sel_margin = np.full(n, INF)
    n_cand = np.zeros(n, dtype=np.int64)
    n_drop = np.zeros(n, dtype=np.int64)
    cands_all = []
    force_ignored = 0
    for row, t in enumerate(toks):
        j = int(t) // blk
        cands = []
        for a in probes[row]:
            if rd is None:
                cands += posting_view(lists, int(a), j, L, w.capacity)
            else:
                cands += posting_view_redirect(lists, rd, int(a), j, L, w.capacity)
            if j - L >= 0:
                n_drop[row] += view_dropped(lists, rd, alt, int(a), j, L, w.capacity)
        cands = cands[:M]
        chosen, margin = rerank(q[t], ksum, cands, R, rdtype)
        if force is not None:
            chosen, ignored = apply_force(chosen, int(force[t]), j, L, R)
            force_ignored += int(ignored)
        sel[row, :len(chosen)] = chosen
        sel_margin[row] = margin
        n_cand[row] = len(cands)
        cands_all.append(cands)
    return dict(ksum=ksum, codes=codes, addr=addr, addr_margin=addr_margin, lists=lists, off=off,
                idx=idx, overflow=overflow, tokens=toks, probes=probes, probe_margin=probe_margin,
                cands=cands_all, n_cand=n_cand, n_drop=n_drop, sel=sel, sel_margin=sel_margin,
                force_ignored=force_ignored, alt=alt, alt_gap=alt_gap, rd=rd)


# ---------------------------------------------------------------- 5. attention

def selected_mask(sel_rows: np.ndarray, tokens: np.ndarray, S: int, block: int, local: int) -> np.ndarray:
    """Boolean mask [n, S]: key s is visible to token t iff its block is selected for t,
    or s lies in the L local blocks and s <= t."""
    n = len(tokens)
    m = np.zeros((n, S), dtype=bool)
    s = np.arange(S)
    for row, t in enumerate(tokens):
        j = int(t) // block
        lo = max(0, (j - local + 1) * block)
        m[row] = (s >= lo) & (s <= t)
        for i in sel_rows[row]:
            if i >= 0:
                m[row, i * block:(i + 1) * block] = True
    return m


def attention_dense(q, k, v, sel_rows, block, local, tokens=None, scale=None) -> np.ndarray:
    """softmax(q k^T * scale, masked to the selected set) v, densely in float64.

    q, k, v [S, D]; sel_rows [n, R] (the selection of each token in ``tokens``).
    Returns [n, D] float64.
    """
    S, D = q.shape
    toks = np.arange(S) if tokens is None else np.asarray(tokens, dtype=np.int64)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q64 = np.asarray(q, dtype=np.float64)[toks]
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    mask = selected_mask(np.asarray(sel_rows), toks, S, block, local)
    scores = (q64 @ k64.T) * scale
    scores = np.where(mask, scores, -np.inf)
    mx = scores.max(axis=1, keepdims=True)
    p = np.exp(scores - mx)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v64


def attention_packed(q, k, v, sel_rows, block, local, tokens=None, scale=None, dtype=np.float64):
    """The same sum computed by gathering only the selected tokens (no dense mask)."""
    S, D = q.shape
    toks = np.arange(S) if tokens is None else np.asarray(tokens, dtype=np.int64)
    scale = dtype(1.0 / math.sqrt(D) if scale is None else scale)
    out = np.zeros((len(toks), D), dtype=dtype)
    for row, t in enumerate(toks):
        j = int(t) // block
        lo = max(0, (j - local + 1) * block)
        idx = [np.arange(i * block, (i + 1) * block) for i in sel_rows[row] if i >= 0]
        idx.append(np.arange(lo, t + 1))
        idx = np.concatenate(idx)
        s = (np.asarray(k[idx], dtype=dtype) @ np.asarray(q[t], dtype=dtype)) * scale
        p = np.exp(s - s.max())
        out[row] = (p @ np.asarray(v[idx], dtype=dtype)) / p.sum()
    return out


def attention_lse2(q, k, sel_rows, block, local, tokens=None, scale=None) -> np.ndarray:
    """Per token, log2 of sum_s 2^(scale * log2(e) * q_t . k_s) over its selected keys (float64): the
    softmax normaliser in base 2 that the backward pass uses to recompute the weights."""
    S, D = q.shape
    toks = np.arange(S) if tokens is None else np.asarray(tokens, dtype=np.int64)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    mask = selected_mask(np.asarray(sel_rows), toks, S, block, local)
    scores = (np.asarray(q, dtype=np.float64)[toks] @ np.asarray(k, dtype=np.float64).T) * scale
    scores = np.where(mask, scores, -np.inf)
    mx = scores.max(axis=1)
    return (mx + np.log(np.exp(scores - mx[:, None]).sum(axis=1))) / math.log(2.0)


def attention_backward_dense(q, k, v, sel_rows, block, local, d_out, scale=None):
    """Gradients of attention_dense over all tokens (the routing held fixed) for the upstream
    gradient d_out, densely in float64.  With P the masked softmax of scale * q k^T and O = P v:
    dV = P^T dO; dP = dO v^T; dS = P * (dP - rowsum(dO * O)); dQ = scale * dS k; dK = scale * dS^T q.
    q, k, v, d_out [S, D]; sel_rows [S, R].  Returns (dq, dk, dv) [S, D] float64."""
    S, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q64, k64, v64, do64 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, d_out))
    mask = selected_mask(np.asarray(sel_rows), np.arange(S), S, block, local)
    scores = np.where(mask, (q64 @ k64.T) * scale, -np.inf)
    p = np.exp(scores - scores.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o = p @ v64
    dv = p.T @ do64
    dp = do64 @ v64.T
    ds = p * (dp - (do64 * o).sum(axis=1, keepdims=True))
    return scale * ds @ k64, scale * ds.T @ q64, dv


def attention_backward_packed(q, k, v, sel_rows, block, local, d_out, scale=None):
    """The gradients of attention_backward_dense, token by token over gathered keys only, so that it
    runs at lengths where an S x S matrix does not fit.  Entry r of token t's row counts when
    0 <= sel <= j - L and it repeats no earlier entry (the visible set is a set of blocks); the
    local window is blocks j - L + 1 .. j up to t.  Per token: p = softmax over its keys, o = p v,
    D = dO . o, ds = p (v dO - D); dq_t = scale ds k; dk += scale ds q_t; dv += p dO_t.
    q, k, v, d_out [S, D]; sel_rows [S, R].  Returns (dq, dk, dv) [S, D] float64."""
    S, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q64, k64, v64, do64 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, d_out))
    dq = np.zeros((S, D))
    dk = np.zeros((S, D))
    dv = np.zeros((S, D))
    for t in range(S):
        j = t // block
        blocks = []
        for i in sel_rows[t]:
            i = int(i)
            if 0 <= i <= j - local and i not in blocks:
                blocks.append(i)
        idx = [np.arange(i * block, (i + 1) * block) for i in blocks]
        idx.append(np.arange(max(0, (j - local + 1) * block), t + 1))
        idx = np.concatenate(idx)
        s = (k64[idx] @ q64[t]) * scale
        p = np.exp(s - s.max())
        p /= p.sum()
        o = p @ v64[idx]
        ds = p * (v64[idx] @ do64[t] - do64[t] @ o)
        dq[t] = scale * (ds @ k64[idx])
        dk[idx] += scale * ds[:, None] * q64[t][None, :]
        dv[idx] += p[:, None] * do64[t][None, :]
    return dq, dk, dv


# ---------------------------------------------------------------- core + mixer

def routed_attention(q, k, v, codebook, bias, w, force=None, rdtype=np.float32):
    """Route and attend every (batch, head).  q, k, v [B, H, S, D]; codebook [H, G, C, D].

    Returns (out [B, H, S, D] float64, routes[b][h]).
    """
    B, H, S, D = q.shape
    out = np.zeros((B, H, S, D))
    routes = []
    for b in range(B):
        rb = []
        for h in range(H):
            f = None if force is None else force[b, h]
            r = route_head(q[b, h], k[b, h], codebook[h], None if bias is None else bias[h], w, f,
                           rdtype=rdtype)
            out[b, h] = attention_dense(q[b, h], k[b, h], v[b, h], r["sel"], w.block, w.local)
            rb.append(r)
        routes.append(rb)
    return out, routes


def rope(x: np.ndarray, base: float) -> np.ndarray:
    """Rotary position embedding on the last axis, positions 0..S-1 along axis -2.

    Pairs (i, i + D/2) rotate by angle pos * base^(-2i/D)."""
    S, D = x.shape[-2], x.shape[-1]
    half = D // 2
    theta = base ** (-2.0 * np.arange(half) / D)
    ang = np.arange(S)[:, None] * theta[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def mixer_qkv(x, wq, wk, wv, w):
    """Q = RoPE(x wq), K = RoPE(x wk), V = x wv as [B, H, S, D] float64 (no biases, no norms)."""
    B, S, _ = x.shape
    H, D = w.heads, w.head_dim
    x64 = np.asarray(x, dtype=np.float64)

    def heads(y):
        return y.reshape(B, S, H, D).transpose(0, 2, 1, 3)

    q = rope(heads(x64 @ np.asarray(wq, np.float64)), w.rope_base)
    k = rope(heads(x64 @ np.asarray(wk, np.float64)), w.rope_base)
    v = heads(x64 @ np.asarray(wv, np.float64))
    return q, k, v


def round_to_bf16(a) -> np.ndarray:
    """Each value rounded to the nearest bfloat16 (8 significand bits; ties to even), returned as
    float64: keep the top 16 bits of the float32 pattern after adding half an ulp of the kept part
    (0x7FFF plus the lowest kept bit).  Finite inputs only."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def mixer_forward(x, wq, wk, wv, wo, codebook, bias, w, sel_override=None, rdtype=np.float32, io_dtype="f32",
                  policy="drop"):
    """Stateless [B, S, W] -> attention delta [B, S, W] (float64), plus the routes.

    Q, K, V are held in the io dtype between the projections and the core (the core's own inputs):
    with ``io_dtype`` "bf16" they are rounded to bfloat16 first.  Routing reads Q and K rounded to
    ``rdtype``; attention uses them in float64.  ``sel_override`` [B, H, S, R] replaces the oracle's
    own selection (so the attention and output projection can be checked on another router's choice).
    """
    B, S, _ = x.shape
    H, D = w.heads, w.head_dim
    q, k, v = mixer_qkv(x, wq, wk, wv, w)
    if io_dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    o = np.zeros((B, H, S, D))
    routes = []
    for b in range(B):
        rb = []
        for h in range(H):
            r = route_head(q[b, h].astype(rdtype), k[b, h].astype(rdtype), codebook[h],
                           None if bias is None else bias[h], w, rdtype=rdtype, policy=policy)
            sel = r["sel"] if sel_override is None else np.asarray(sel_override[b, h])
            o[b, h] = attention_dense(q[b, h], k[b, h], v[b, h], sel, w.block, w.local)
            rb.append(r)
        routes.append(rb)
    concat = o.transpose(0, 2, 1, 3).reshape(B, S, H * D)
    return concat @ np.asarray(wo, np.float64), routes
