"""Shared helpers of the GPU parity tests: moving seeded inputs to the device,
calling the library, and comparing with the oracle under the near-tie rule.

Near-tie rule: a routing decision (argmax code, probe ranking, selection
ranking) whose oracle score margin is at most NEAR may legitimately come out
either way in fp32 with a different summation order; those cases are counted,
and every other decision must match exactly.
"""

import numpy as np
import torch

import oracle
import synth

NEAR = 1e-4
TOL = {"f32": 1e-5, "bf16": 2e-2}


def cfg_of(mdr, w, policy="drop"):
    return mdr.config(batch=w.batch, seq=w.seq, heads=w.heads, head_dim=w.head_dim, width=w.width, block=w.block,
                      subspaces=w.subspaces, codes=w.codes, capacity=w.capacity, probes=w.probes,
                      max_cand=w.max_cand, remote=w.remote, local=w.local, dtype=w.dtype, rope_base=w.rope_base,
                      overflow_policy=policy)


def io_dtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    elif t.dtype in (torch.int64, torch.int32):
        t = t.to(torch.int32)
    return t.cuda()


def host(t):
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def run_core(mdr, w, inp, force=None, policy="drop", diag=True):
    """mdr_routed_attention with every routing output requested (with ``diag`` also the routing
    diagnostics: probes, scores, margins); returns host arrays."""
    cfg = cfg_of(mdr, w, policy)
    dt = io_dtype(w)
    q, k, v = (dev(inp[n], dt) for n in ("q", "k", "v"))
    cb = dev(inp["codebook"], torch.float32)
    bias = None if inp["bias"] is None else dev(inp["bias"], torch.float32)
    f = None if force is None else dev(force)
    out = torch.empty_like(q)
    rt = mdr.routing_buffers(cfg, diag=diag)
    ws = mdr.workspace(cfg)
    mdr.mdr_routed_attention(cfg, q, k, v, cb, bias, f, out, rt, ws)
    torch.cuda.synchronize()
    res = {n: host(t) for n, t in rt.items()}
    res["out"] = host(out)
    return res


def _bias(inp, h):
    return None if inp["bias"] is None else inp["bias"][h]


def compare_addresses(w, inp, addr_gpu, b, h):
    """GPU addresses vs the oracle's: equal wherever every subspace's argmax margin exceeds NEAR; at a
    near-tie each GPU code must still be a best code up to NEAR (its logit within NEAR of the subspace's
    largest).  Returns the number of near-tie blocks."""
    ks = oracle.block_summaries(inp["k"][b, h], w.block)
    lg = oracle.code_logits(ks, inp["codebook"][h], _bias(inp, h))
    _, addr, margin = oracle.block_addresses(ks, inp["codebook"][h], _bias(inp, h))
    sure = margin.min(axis=1) > NEAR
    assert np.array_equal(addr_gpu[sure], addr[sure]), (b, h)
    G, C = w.subspaces, w.codes
    for i in np.nonzero(~sure)[0]:
        a = int(addr_gpu[i])
        assert 0 <= a < C ** G, (b, h, i, a)
        for g in range(G):
            c = (a // C ** (G - 1 - g)) % C
            assert lg[i, g, c] >= lg[i, g].max() - NEAR, (b, h, i, g, c)
    return int((~sure).sum())


def compare_alternates(w, inp, alt_gpu, addr_gpu, b, h):
    """GPU alternate addresses (redirect policy) vs the oracle's: equal wherever the block's address, the
    choice of subspace (smallest top1 - top2 margin) and that subspace's runner-up code are decided by
    more than NEAR; elsewhere the GPU's alternate must be the GPU's own address with one digit changed,
    in a subspace whose margin is within NEAR of the smallest, to a code whose logit is within NEAR of
    that subspace's second best.  Returns the number of near-tie blocks."""
    ks = oracle.block_summaries(inp["k"][b, h], w.block)
    cb, bias = inp["codebook"][h], _bias(inp, h)
    lg = oracle.code_logits(ks, cb, bias).astype(np.float64)
    codes, addr, margin = oracle.block_addresses(ks, cb, bias)
    second, m32 = oracle.runner_up_codes(ks, cb, bias)
    alt, gap = oracle.alternate_addresses(codes, second, m32, w.codes)
    gap2 = oracle.runner_up_gap(ks, cb, bias)
    G, C = w.subspaces, w.codes
    g_star = np.array([min(range(G), key=lambda g: (m32[i, g], g)) for i in range(w.nblocks)])
    sure = (margin.min(axis=1) > NEAR) & (gap > NEAR) & (gap2[np.arange(w.nblocks), g_star] > NEAR)
    assert np.array_equal(alt_gpu[sure], alt[sure]), (b, h)
    if C == 1:
        return 0
    for i in np.nonzero(~sure)[0]:
        a, x = int(addr_gpu[i]), int(alt_gpu[i])
        da = [(a // C ** (G - 1 - g)) % C for g in range(G)]
        dx = [(x // C ** (G - 1 - g)) % C for g in range(G)]
        diff = [g for g in range(G) if da[g] != dx[g]]
        assert len(diff) == 1, (b, h, i, a, x)
        g = diff[0]
        srt = np.sort(lg[i], axis=1)
        tops = srt[:, -1] - srt[:, -2]
        assert tops[g] <= tops.min() + NEAR, (b, h, i, g)
        assert lg[i, g, dx[g]] >= srt[g, -2] - NEAR, (b, h, i, g)
    return int((~sure).sum())


def route_for(w, inp, b, h, addr=None, force=None, policy="drop", tokens=None, alt=None):
    """The oracle's routing of head (b, h); with ``addr`` (and ``alt``) the blocks are filed under those
    addresses (the GPU's, for heads whose addresses hold near-ties) so the downstream stages are compared
    on the same lists."""
    f = None if force is None else force[b, h]
    return oracle.route_head(inp["q"][b, h], inp["k"][b, h], inp["codebook"][h], _bias(inp, h), w, f,
                             policy=policy, addr=addr, tokens=tokens, alt=alt)


def check_head_routing(w, inp, res, b, h, force=None, policy="drop", tokens=None):
    """One head of a full routing run on the GPU against the oracle: the addresses (near-ties allowed, each
    GPU code then a best code up to NEAR); the posting CSR, overflow and selection against the oracle
    routed on the GPU's own addresses whenever any address is a near-tie (so no head is skipped); the
    selection exact wherever its margins exceed NEAR and otherwise valid (check_near_tie_token).  Returns
    (address near-ties, selection near-ties)."""
    na = compare_addresses(w, inp, res["addr"][b, h], b, h)
    nalt = compare_alternates(w, inp, res["alt"][b, h], res["addr"][b, h], b, h) if policy == "redirect" else 0
    own = na == 0 and nalt == 0
    r = route_for(w, inp, b, h, addr=None if own else res["addr"][b, h], force=force, policy=policy,
                  tokens=tokens, alt=None if own or policy != "redirect" else res["alt"][b, h])
    if policy == "redirect":
        A = w.addresses
        ro, ri, rt = res["redir_off"][b, h], res["redir_idx"][b, h], res["redir_time"][b, h]
        n = 0
        for a in range(A):
            got = [(int(rt[k]), int(ri[k])) for k in range(ro[a], ro[a + 1])]
            assert got == r["rd"][a], (b, h, a)
            n += len(got)
        assert ro[A] == n and np.all(ri[n:] == -1) and np.all(rt[n:] == -1)
    assert res["overflow"][b, h] == r["overflow"], (b, h)
    assert np.array_equal(res["post_off"][b, h], r["off"]), (b, h)
    n_filed = len(r["idx"])
    assert np.array_equal(res["post_idx"][b, h][:n_filed], r["idx"]), (b, h)
    assert np.all(res["post_idx"][b, h][n_filed:] == -1), (b, h)
    probes = res["probes"][b, h] if "probes" in res else None
    f = None if force is None else force[b, h]
    ns = compare_selection(r, res["sel"][b, h], rows=tokens, w=w, inp=inp, b=b, h=h, probes_gpu=probes, force=f,
                           policy=policy)
    sure_p = r["probe_margin"] > NEAR
    rows = slice(None) if tokens is None else tokens
    for n in ("n_cand", "n_drop"):
        if n in res:
            assert np.array_equal(res[n][b, h][rows][sure_p], r[n][sure_p]), (n, b, h)
    return na + nalt, ns


def _view(route, a, j, w, policy):
    if policy == "redirect":
        return oracle.posting_view_redirect(route["lists"], route["rd"], a, j, w.local, w.capacity)
    return oracle.posting_view(route["lists"], a, j, w.local, w.capacity)


def check_near_tie_token(route, row, sel_row, w, inp, b, h, probes_row=None, force_t=-1, policy="drop"):
    """A token whose probe or rerank decision is a near-tie may come out either way, but the GPU's
    selection must still be one a correct router could make:
      * entries are -1 padded at the end, distinct, eligible (0 <= i <= j - L), at most R;
      * with the GPU's probes: they are distinct and each scores within NEAR of the P-th best address;
        the candidates are then those probes' views in order, cut at M, and every selected block is a
        candidate whose rerank score is within NEAR of the R-th best candidate's, in rank order up to NEAR;
      * without them: every selected block lies in the view of some address scoring within NEAR of the
        P-th best, and when the probe decision itself is sure the score checks above apply to the oracle's
        own candidates.
    A forced target (0 <= f <= j - L) must be present; the other entries are checked as above."""
    t = int(route["tokens"][row])
    j = t // w.block
    cutoff = j - w.local
    R, P, C, G = w.remote, w.probes, w.codes, w.subspaces
    A = C ** G
    n = int(np.sum(sel_row >= 0))
    assert np.all(sel_row[:n] >= 0) and np.all(sel_row[n:] == -1), (t, sel_row)
    ent = [int(i) for i in sel_row[:n]]
    assert len(set(ent)) == n and n <= R and all(0 <= i <= cutoff for i in ent), (t, ent)
    q = inp["q"][b, h]
    mu = oracle.code_logits(q[t:t + 1], inp["codebook"][h], _bias(inp, h))
    sigma = oracle.address_scores(mu, C)[0].astype(np.float64)
    thr = np.sort(sigma)[-min(P, A)] - NEAR
    if probes_row is not None:
        pr = [int(a) for a in probes_row[:min(P, A)]]
        assert len(set(pr)) == len(pr) and all(0 <= a < A and sigma[a] >= thr for a in pr), (t, pr)
        for x, y in zip(pr[:-1], pr[1:]):
            assert sigma[x] >= sigma[y] - NEAR, (t, pr)
        cands = []
        for a in pr:
            cands += _view(route, a, j, w, policy) if cutoff >= 0 else []
        cands = cands[:w.cand_limit]
        exact = True
    elif route["probe_margin"][row] > NEAR:
        cands, exact = list(route["cands"][row]), True
    else:
        cands = []
        for a in np.nonzero(sigma >= thr)[0]:
            cands += _view(route, int(a), j, w, policy) if cutoff >= 0 else []
        exact = False
    forced = force_t if 0 <= force_t <= cutoff and R > 0 else None
    if forced is not None:
        assert forced in ent, (t, forced, ent)
    rest = [i for i in ent if i != forced]
    assert all(i in cands for i in rest), (t, rest, cands)
    if exact and cands:
        rho = (np.asarray(route["ksum"][cands], np.float32) @ np.asarray(q[t], np.float32)).astype(np.float64)
        score = dict(zip(cands, rho))
        kth = np.sort(rho)[::-1][min(R, len(cands)) - 1]
        assert all(score[i] >= kth - NEAR for i in rest), (t, rest)
        for x, y in zip(rest[:-1], rest[1:]):
            assert score[x] >= score[y] - NEAR, (t, rest)
        if forced is None:
            assert n == min(R, len(cands)), (t, n, len(cands))


def compare_selection(route, sel_gpu, rows=None, w=None, inp=None, b=None, h=None, probes_gpu=None, force=None,
                      policy="drop"):
    """sel rows vs the oracle route (same token order): equal wherever the probe and rerank margins both
    exceed NEAR; every other token is checked for validity (check_near_tie_token) when the inputs are
    given.  Returns the number of near-tie tokens."""
    sel_o = route["sel"]
    sure = (route["probe_margin"] > NEAR) & (route["sel_margin"] > NEAR)
    g = sel_gpu if rows is None else sel_gpu[rows]
    bad = np.nonzero(sure & np.any(g != sel_o, axis=1))[0]
    assert len(bad) == 0, f"selection mismatch at rows {bad[:8]}: gpu {g[bad[:4]]} oracle {sel_o[bad[:4]]}"
    if w is not None:
        pg = None if probes_gpu is None else (probes_gpu if rows is None else probes_gpu[rows])
        for row in np.nonzero(~sure)[0]:
            t = int(route["tokens"][row])
            ft = -1 if force is None else int(force[t])
            check_near_tie_token(route, row, g[row], w, inp, b, h, None if pg is None else pg[row], ft, policy)
    return int((~sure).sum())


def attention_rows(w, inp, sel_rows, b, h, tokens, dense=False):
    q, k, v = (inp[n][b, h] for n in ("q", "k", "v"))
    if dense:
        return oracle.attention_dense(q, k, v, sel_rows, w.block, w.local, tokens=tokens)
    return oracle.attention_packed(q, k, v, sel_rows, w.block, w.local, tokens=tokens)


def small(name, **over):
    """Test-size versions of the five workloads (the oracle finishes each in seconds)."""
    sizes = {
        "tiny": {},
        "recall": dict(batch=4),
        "sweep": dict(seq=4096),
        "long": dict(heads=2, seq=8192),
        "skew": dict(batch=2, heads=4, seq=4096),
    }
    kw = dict(sizes[name])
    kw.update(over)
    return synth.workload(name, **kw)


def integer_inputs(w, seed):
    """Core inputs rounded to small integers: every code logit, summary and rerank score is then exact
    on both sides, so ties are frequent and decided by the index rules alone."""
    inp = dict(synth.make_core_inputs(w, seed))
    for n in ("q", "k"):
        inp[n] = np.clip(np.rint(inp[n]), -2, 2).astype(inp[n].dtype)
    cb = inp["codebook"]
    inp["codebook"] = np.clip(np.rint(cb / np.abs(cb).max() * 2), -2, 2).astype(cb.dtype)
    if inp["bias"] is not None:
        inp["bias"] = np.rint(inp["bias"]).astype(inp["bias"].dtype)
    return inp
