"""Pins of the CPU oracle against things other than itself (CPU only).

* an independent pure-Python brute force on tiny dyadic inputs, where every
  routing score is exact in float32 and float64 so ties are frequent and the
  tie rules must agree exactly;
* a hand-derived golden case (tests/golden/hand_routing.json);
* reductions to textbook attention: a full routing budget is dense causal
  attention, R = 0 is block-banded causal attention (the pages' local-only
  control), both checked against torch's scaled_dot_product_attention in
  float64;
* invariants: causality of routing and attention, forced target under the same
  budget, linearity in V, overflow equal to the closed form of a planted
  address histogram, zero overflow of the balanced generator;
* the pages' level of agreement between sparse gathering and a dense
  selected-mask computation.
"""

import dataclasses
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._brute import brute_rope, brute_routed_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dyadic_inputs(w, seed, bias=False):
    """Values on a coarse dyadic grid: every routing sum is exact in float32."""
    rng = np.random.default_rng(seed)
    S, D, G, C = w.seq, w.head_dim, w.subspaces, w.codes
    q = rng.integers(-2, 3, size=(S, D)) / 2.0
    k = rng.integers(-2, 3, size=(S, D)) / 2.0
    v = rng.standard_normal((S, D))
    cb = rng.integers(-2, 3, size=(G, C, D)) / 4.0
    b = rng.integers(-2, 3, size=(G, C)) / 8.0 if bias else None
    return q, k, v, cb, b


SMALL = [
    dict(seq=64, head_dim=4, block=4, subspaces=2, codes=3, capacity=2, probes=2, max_cand=0, remote=2, local=2),
    dict(seq=48, head_dim=4, block=4, subspaces=1, codes=4, capacity=1, probes=3, max_cand=2, remote=1, local=1),
    dict(seq=64, head_dim=2, block=8, subspaces=3, codes=2, capacity=3, probes=5, max_cand=0, remote=3, local=1),
    dict(seq=96, head_dim=4, block=4, subspaces=2, codes=2, capacity=4, probes=4, max_cand=6, remote=4, local=3),
    dict(seq=32, head_dim=4, block=2, subspaces=2, codes=2, capacity=2, probes=1, max_cand=0, remote=0, local=2),
]


def _w(**kw):
    base = synth.workload("tiny")
    return dataclasses.replace(base, **kw)


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("rdtype", [np.float32, np.float64])
def test_oracle_equals_brute_force_on_dyadic_inputs(case, seed, rdtype):
    w = _w(**SMALL[case])
    q, k, v, cb, b = _dyadic_inputs(w, seed, bias=(seed == 1))
    r = oracle.route_head(q, k, cb, b, w, rdtype=rdtype)
    out = oracle.attention_dense(q, k, v, r["sel"], w.block, w.local)
    bf = brute_routed_attention(q.tolist(), k.tolist(), v.tolist(), cb.tolist(),
                                None if b is None else b.tolist(), w)
    assert r["addr"].tolist() == bf["addr"]
    assert r["overflow"] == bf["overflow"]
    for t in range(w.seq):
        assert [i for i in r["sel"][t] if i >= 0] == bf["sel"][t], t
    np.testing.assert_allclose(out, np.array(bf["out"]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 3])
def test_forced_target_matches_brute_force(seed):
    w = _w(**SMALL[0])
    q, k, v, cb, b = _dyadic_inputs(w, seed)
    rng = np.random.default_rng(100 + seed)
    force = rng.integers(-1, w.seq // w.block, size=w.seq)
    r = oracle.route_head(q, k, cb, b, w, force=force, rdtype=np.float32)
    bf = brute_routed_attention(q.tolist(), k.tolist(), v.tolist(), cb.tolist(), None, w, force=force.tolist())
    for t in range(w.seq):
        assert [i for i in r["sel"][t] if i >= 0] == bf["sel"][t], t
    out = oracle.attention_dense(q, k, v, r["sel"], w.block, w.local)
    np.testing.assert_allclose(out, np.array(bf["out"]), rtol=0, atol=1e-12)


def test_hand_derived_golden_case():
    g = json.load(open(os.path.join(GOLDEN, "hand_routing.json")))
    c = g["config"]
    w = _w(seq=len(g["k"]), head_dim=2, block=c["block"], subspaces=c["subspaces"], codes=c["codes"],
           capacity=c["capacity"], probes=c["probes"], max_cand=c["max_cand"], remote=c["remote"],
           local=c["local"])
    q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    cb = np.array(g["codebook"], dtype=np.float64)
    r = oracle.route_head(q, k, cb, None, w)
    assert r["addr"].tolist() == g["addr"]
    assert r["overflow"] == g["overflow"]
    assert [[i for i in row if i >= 0] for row in r["sel"]] == g["sel"]
    out = oracle.attention_dense(q, k, v, r["sel"], w.block, w.local)
    for t, vis in g["visible_dots"].items():
        t = int(t)
        wts = np.array([math.exp(d / math.sqrt(2.0)) for _, d in vis])
        expect = (wts[:, None] * v[[s for s, _ in vis]]).sum(0) / wts.sum()
        np.testing.assert_allclose(out[t], expect, rtol=0, atol=1e-14)


def _sdpa(q, k, v, mask=None, causal=False):
    t = [torch.from_numpy(np.asarray(a, dtype=np.float64))[None, None] for a in (q, k, v)]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=m, is_causal=causal)[0, 0].numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_full_budget_is_dense_causal_attention(seed):
    """P = A, capacity >= nb, M = P*capacity and R >= nb select every eligible block."""
    nb, blk = 8, 8
    w = _w(seq=nb * blk, head_dim=16, block=blk, subspaces=2, codes=3, capacity=nb, probes=9,
           max_cand=0, remote=nb, local=2)
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((w.seq, w.head_dim)) for _ in range(3))
    cb = rng.standard_normal((2, 3, 16)) / 4
    r = oracle.route_head(q, k, cb, None, w)
    out = oracle.attention_dense(q, k, v, r["sel"], w.block, w.local)
    np.testing.assert_allclose(out, _sdpa(q, k, v, causal=True), rtol=0, atol=1e-12)


@pytest.mark.parametrize("local", [1, 2, 3])
def test_local_only_is_block_banded_causal_attention(local):
    nb, blk, D = 10, 4, 8
    w = _w(seq=nb * blk, head_dim=D, block=blk, remote=0, local=local)
    rng = np.random.default_rng(local)
    q, k, v = (rng.standard_normal((w.seq, D)) for _ in range(3))
    cb = rng.standard_normal((2, 4, D))
    r = oracle.route_head(q, k, cb, None, w)
    assert (r["sel"].size == 0) or np.all(r["sel"] < 0)
    t = np.arange(w.seq)
    band = (t[None, :] <= t[:, None]) & (t[None, :] // blk >= t[:, None] // blk - local + 1)
    out = oracle.attention_dense(q, k, v, r["sel"], blk, local)
    np.testing.assert_allclose(out, _sdpa(q, k, v, mask=band), rtol=0, atol=1e-12)
    # a window wider than the sequence is plain causal attention
    r2 = oracle.route_head(q, k, cb, None, dataclasses.replace(w, local=nb))
    out2 = oracle.attention_dense(q, k, v, r2["sel"], blk, nb)
    np.testing.assert_allclose(out2, _sdpa(q, k, v, causal=True), rtol=0, atol=1e-12)


@pytest.mark.parametrize("t0", [70, 127, 200])
def test_routing_and_attention_are_causal(t0):
    """Changing tokens after t0 leaves every selection and output up to t0 bit-identical."""
    w = synth.workload("recall", batch=1, heads=1, seq=256, block=16)
    inp = synth.make_core_inputs(w, 5)
    q, k, v = (inp[n][0, 0].copy() for n in ("q", "k", "v"))
    cb = inp["codebook"][0]
    r1 = oracle.route_head(q, k, cb, None, w)
    o1 = oracle.attention_dense(q, k, v, r1["sel"], w.block, w.local)
    rng = np.random.default_rng(9)
    for a in (q, k, v):
        a[t0 + 1:] = rng.standard_normal(a[t0 + 1:].shape).astype(np.float32) * 3
    r2 = oracle.route_head(q, k, cb, None, w)
    o2 = oracle.attention_dense(q, k, v, r2["sel"], w.block, w.local)
    assert np.array_equal(r1["sel"][:t0 + 1], r2["sel"][:t0 + 1])
    assert np.array_equal(o1[:t0 + 1], o2[:t0 + 1])
    assert not np.array_equal(o1[t0 + 1:], o2[t0 + 1:])


def test_forced_target_keeps_budget_and_recovers_recall():
    """Forcing the planted block puts it in every last-block selection, never exceeding R."""
    w = synth.workload("recall", batch=4, heads=2)
    inp = synth.make_core_inputs(w, 1)
    last = np.arange((w.nblocks - 1) * w.block, w.seq)
    for b in range(w.batch):
        for h in range(w.heads):
            args = (inp["q"][b, h], inp["k"][b, h], inp["codebook"][h], None, w)
            free = oracle.route_head(*args, tokens=last)
            forced = oracle.route_head(*args, force=inp["force"][b, h], tokens=last)
            p = int(inp["planted"][b])
            assert forced["force_ignored"] == 0
            for row in range(len(last)):
                s = [i for i in forced["sel"][row] if i >= 0]
                assert p in s and len(s) <= w.remote and len(set(s)) == len(s)
                s0 = [i for i in free["sel"][row] if i >= 0]
                if p in s0:
                    assert s == s0
                elif len(s0) == w.remote:
                    assert s[:-1] == s0[:-1]
            out = oracle.attention_dense(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], forced["sel"],
                                         w.block, w.local, tokens=last)
            pk = oracle.attention_packed(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], forced["sel"],
                                         w.block, w.local, tokens=last)
            np.testing.assert_allclose(out, pk, rtol=0, atol=1e-12)


def test_attention_is_linear_in_v():
    w = synth.workload("recall", batch=1, heads=1, seq=512)
    inp = synth.make_core_inputs(w, 2)
    q, k = inp["q"][0, 0], inp["k"][0, 0]
    r = oracle.route_head(q, k, inp["codebook"][0], None, w)
    rng = np.random.default_rng(3)
    v1, v2 = rng.standard_normal((2, w.seq, w.head_dim))
    a, b = 0.75, -2.5
    lhs = oracle.attention_dense(q, k, a * v1 + b * v2, r["sel"], w.block, w.local)
    rhs = a * oracle.attention_dense(q, k, v1, r["sel"], w.block, w.local) + \
        b * oracle.attention_dense(q, k, v2, r["sel"], w.block, w.local)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)


def _planted_keys(target, w, rng, gain):
    """Keys whose block summaries sit on codebook rows chosen by ``target`` (digits most significant first)."""
    G, C, D, blk = w.subspaces, w.codes, w.head_dim, w.block
    cb = rng.standard_normal((G, C, D)) / math.sqrt(D)
    unit = cb / np.linalg.norm(cb, axis=-1, keepdims=True)
    k = rng.standard_normal((w.seq, D)) * 0.2
    for i, a in enumerate(target):
        push = sum(unit[g, (a // C ** (G - 1 - g)) % C] for g in range(G))
        k[i * blk:(i + 1) * blk] += gain * push
    return k, cb


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_overflow_equals_closed_form_of_planted_histogram(seed):
    w = _w(seq=64 * 16, head_dim=32, block=16, subspaces=2, codes=4, capacity=3, local=2)
    rng = np.random.default_rng(seed)
    nb, A = w.nblocks, w.addresses
    # a skewed assignment: address a drawn with probability ~ 1/(a+1)
    p = 1.0 / np.arange(1, A + 1)
    target = rng.choice(A, size=nb, p=p / p.sum())
    k, cb = _planted_keys(target, w, rng, gain=6.0)
    q = rng.standard_normal((w.seq, w.head_dim))
    r = oracle.route_head(q, k, cb, None, w, tokens=[0])
    assert r["addr"].tolist() == target.tolist()
    hist = np.bincount(target[: nb - w.local], minlength=A)
    assert r["overflow"] == int(np.maximum(hist - w.capacity, 0).sum())
    assert r["overflow"] > 0


@pytest.mark.parametrize("seq", [4096, 8192])
def test_balanced_generator_has_zero_overflow(seq):
    """The pages report zero posting overflow in their balanced scaling runs."""
    w = synth.workload("sweep", seq=seq)
    inp = synth.make_core_inputs(w, 0)
    for h in range(w.heads):
        ks = oracle.block_summaries(inp["k"][0, h], w.block)
        _, addr, margin = oracle.block_addresses(ks, inp["codebook"][h], None)
        assert np.array_equal(addr, inp["target_addr"][h])
        assert margin.min() > 1e-2
        assert oracle.posting_overflow(oracle.posting_lists(addr, w.addresses, w.local), w.capacity) == 0


def test_tie_rules():
    """Equal summaries tie in the rerank (smaller block wins); equal codebook rows tie in the argmax."""
    w = _w(seq=8 * 4, head_dim=4, block=4, subspaces=1, codes=3, capacity=8, probes=1, max_cand=0,
           remote=1, local=1)
    rng = np.random.default_rng(0)
    k = rng.standard_normal((w.seq, 4))
    cb = np.zeros((1, 3, 4))
    cb[0, 0] = cb[0, 1] = [1.0, 0.0, 0.0, 0.0]   # codes 0 and 1 identical
    cb[0, 2] = [-5.0, 0.0, 0.0, 0.0]
    k[:, 0] = np.abs(k[:, 0]) + 0.1              # keep code 2 out of the way
    k[4:8] = k[0:4]                              # blocks 0 and 1 identical -> identical summaries
    k[0:8, 0] += 10.0                            # and they lead the rerank
    q = np.tile([1.0, 0.0, 0.0, 0.0], (w.seq, 1))
    r = oracle.route_head(q, k, cb, None, w)
    assert set(r["codes"][:, 0].tolist()) == {0}
    t = w.seq - 1
    assert r["sel"][t][0] == 0  # block 0 and 1 tie; the smaller index wins


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_sparse_gather_matches_dense_selected_mask(dtype):
    """The pages report the sparse selected-set attention within 1.43e-6 of a dense selected-mask
    oracle; the oracle's two attention codes agree to rounding (float64) and within the fp32
    parity tolerance of 1e-5 when the gather runs in float32."""
    w = synth.workload("recall", batch=1, heads=1, seq=1024)
    inp = synth.make_core_inputs(w, 0)
    q, k, v = (inp[n][0, 0] for n in ("q", "k", "v"))
    r = oracle.route_head(q, k, inp["codebook"][0], None, w)
    dense = oracle.attention_dense(q, k, v, r["sel"], w.block, w.local)
    packed = oracle.attention_packed(q, k, v, r["sel"], w.block, w.local, dtype=dtype)
    tol = 1e-12 if dtype == np.float64 else 1e-5
    assert np.abs(dense - packed).max() <= tol


def test_rope_is_complex_rotation_and_relative():
    rng = np.random.default_rng(0)
    S, D = 12, 8
    x = rng.standard_normal((S, D))
    got = oracle.rope(x, 10000.0)
    np.testing.assert_allclose(got, np.array(brute_rope(x.tolist(), 10000.0)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(got[0], x[0], rtol=0, atol=0)
    # <rope(q)_m, rope(k)_n> depends only on m - n
    qv, kv = rng.standard_normal((2, D))
    qq = oracle.rope(np.tile(qv, (S, 1)), 10000.0)
    kk = oracle.rope(np.tile(kv, (S, 1)), 10000.0)
    assert abs(qq[7] @ kk[4] - qq[5] @ kk[2]) < 1e-12
    assert abs(qq[3] @ kk[3] - qv @ kv) < 1e-12


def test_mixer_matches_brute_force():
    """delta = concat_h(attention) Wo with Q = RoPE(x Wq), K = RoPE(x Wk), V = x Wv (no biases)."""
    w = synth.workload("tiny", seq=64, width=16, heads=2, head_dim=8, block=8, codes=2, capacity=2,
                       probes=2, remote=1, local=1)
    inp = synth.make_mixer_inputs(w, 0)
    delta, routes = oracle.mixer_forward(inp["x"], inp["wq"], inp["wk"], inp["wv"], inp["wo"],
                                         inp["codebook"], None, w, rdtype=np.float64)
    x = inp["x"][0].astype(np.float64)
    H, D = w.heads, w.head_dim
    o = np.zeros((w.seq, H * D))
    for h in range(H):
        cols = slice(h * D, (h + 1) * D)
        proj = [[[sum(x[s, c] * inp[m][c, h * D + d] for c in range(w.width)) for d in range(D)]
                 for s in range(w.seq)] for m in ("wq", "wk", "wv")]
        qh, kh = brute_rope(proj[0], w.rope_base), brute_rope(proj[1], w.rope_base)
        r = routes[0][h]
        for name, m in (("probe_margin", 1e-9), ("sel_margin", 1e-9)):
            assert np.all(r[name] > m)
        assert r["addr_margin"].min() > 1e-9
        bf = brute_routed_attention(qh, kh, proj[2], inp["codebook"][h].tolist(), None, w)
        assert [[i for i in row if i >= 0] for row in r["sel"]] == bf["sel"]
        o[:, cols] = np.array(bf["out"])
    np.testing.assert_allclose(delta[0], o @ inp["wo"].astype(np.float64), rtol=0, atol=1e-11)


def _routed_case(seed, seq=256):
    w = synth.workload("tiny", seq=seq)
    inp = synth.make_core_inputs(w, seed)
    q, k, v = (inp[n][0, 0].astype(np.float64) for n in ("q", "k", "v"))
    r = oracle.route_head(inp["q"][0, 0], inp["k"][0, 0], inp["codebook"][0], None, w)
    return w, q, k, v, r["sel"]


@pytest.mark.parametrize("seed", [0, 1])
def test_attention_backward_matches_autograd(seed):
    """The closed-form gradients against torch autograd through a dense masked softmax (float64)."""
    w, q, k, v, sel = _routed_case(seed)
    rng = np.random.default_rng(100 + seed)
    d_out = rng.standard_normal(q.shape)
    dq, dk, dv = oracle.attention_backward_dense(q, k, v, sel, w.block, w.local, d_out)
    S, D = q.shape
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = torch.from_numpy(oracle.selected_mask(sel, np.arange(S), S, w.block, w.local))
    scores = (tq @ tk.T) / math.sqrt(D)
    out = torch.softmax(scores.masked_fill(~mask, float("-inf")), dim=-1) @ tv
    out.backward(torch.from_numpy(d_out))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_attention_backward_matches_finite_differences():
    """Directional derivatives of <d_out, attention_dense> by central differences."""
    w, q, k, v, sel = _routed_case(2, seq=128)
    rng = np.random.default_rng(7)
    d_out = rng.standard_normal(q.shape)
    dq, dk, dv = oracle.attention_backward_dense(q, k, v, sel, w.block, w.local, d_out)
    f = lambda q_, k_, v_: float((oracle.attention_dense(q_, k_, v_, sel, w.block, w.local) * d_out).sum())
    h = 1e-6
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        u = rng.standard_normal(q.shape)
        args_p = [q, k, v]
        args_m = [q, k, v]
        args_p[which] = args_p[which] + h * u
        args_m[which] = args_m[which] - h * u
        fd = (f(*args_p) - f(*args_m)) / (2 * h)
        assert abs(fd - float((grad * u).sum())) <= 1e-6 * max(1.0, abs(fd))


def test_attention_lse2_is_the_softmax_normaliser():
    w, q, k, v, sel = _routed_case(3)
    S, D = q.shape
    lse2 = oracle.attention_lse2(q, k, sel, w.block, w.local)
    mask = oracle.selected_mask(sel, np.arange(S), S, w.block, w.local)
    direct = np.log2(np.where(mask, np.exp((q @ k.T) / math.sqrt(D)), 0.0).sum(axis=1))
    np.testing.assert_allclose(lse2, direct, rtol=1e-12, atol=1e-12)


def _random_selection(rng, S, block, local, R, p_none=0.2, p_repeat=0.2):
    """Entries in [-1, j - L] with some -1 and some repeated blocks (the shapes a selection can take)."""
    sel = np.full((S, R), -1, dtype=np.int64)
    for t in range(S):
        hi = t // block - local
        for r in range(R):
            u = rng.random()
            if hi < 0 or u < p_none:
                continue
            if r > 0 and u < p_none + p_repeat:
                sel[t, r] = sel[t, rng.integers(0, r)]
            else:
                sel[t, r] = rng.integers(0, hi + 1)
    return sel


@pytest.mark.parametrize("seed", [0, 1])
def test_attention_backward_packed_matches_dense(seed):
    """The token-by-token gradients against the dense closed form, on a routed selection and on a
    random one with empty and repeated entries."""
    w, q, k, v, sel = _routed_case(seed)
    rng = np.random.default_rng(200 + seed)
    d_out = rng.standard_normal(q.shape)
    for rows in (sel, _random_selection(rng, q.shape[0], w.block, w.local, 3)):
        dense = oracle.attention_backward_dense(q, k, v, rows, w.block, w.local, d_out)
        packed = oracle.attention_backward_packed(q, k, v, rows, w.block, w.local, d_out)
        for a, b in zip(packed, dense):
            np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- overflow redirect

def _simulate_rings(addr, alt, A, capacity, local):
    """Step-by-step filing with a primary ring and a redirect ring per address (the streaming
    formulation): at query block j the block j - L is filed; a full primary ring evicts its oldest
    block into the redirect ring of that block's alternate address (or drops it).  Returns the
    views {(a, j): list} under both policies and each block's eviction time."""
    nb = len(addr)
    prim = [[] for _ in range(A)]
    redir = [[] for _ in range(A)]
    evicted_at = {}
    views_drop, views_redirect = {}, {}
    for j in range(nb):
        b = j - local
        if b >= 0:
            ring = prim[int(addr[b])]
            ring.append(b)
            if len(ring) > capacity:
                x = ring.pop(0)
                evicted_at[x] = j
                if alt[x] >= 0:
                    redir[int(alt[x])].append(x)
        for a in range(A):
            pv = prim[a][::-1]
            views_drop[(a, j)] = pv
            views_redirect[(a, j)] = pv + redir[a][::-1][:capacity - len(pv)]
    return views_drop, views_redirect, evicted_at


@pytest.mark.parametrize("seed,capacity,local", [(0, 1, 1), (1, 2, 2), (2, 3, 1), (3, 1, 3)])
def test_redirect_views_match_the_ring_simulation(seed, capacity, local):
    rng = np.random.default_rng(seed)
    A, nb = 6, 40
    addr = rng.integers(0, A, size=nb) if seed % 2 else np.minimum(rng.geometric(0.45, size=nb) - 1, A - 1)
    alt = (addr + rng.integers(1, A, size=nb)) % A  # any address but the block's own
    alt[rng.random(nb) < 0.15] = -1                  # some blocks without an alternate
    lists = oracle.posting_lists(addr, A, local)
    rd = oracle.redirect_lists(lists, alt, capacity, local)
    vd, vr, ev = _simulate_rings(addr, alt, A, capacity, local)
    for a in range(A):
        for j in range(nb):
            assert oracle.posting_view(lists, a, j, local, capacity) == vd[(a, j)], (a, j)
            assert oracle.posting_view_redirect(lists, rd, a, j, local, capacity) == vr[(a, j)], (a, j)
            # held blocks, from the simulation's eviction times
            held = 0
            for x in range(max(0, j - local + 1)):
                gone = x in ev and ev[x] <= j
                if addr[x] == a and not (gone and alt[x] >= 0):
                    held += 1
                if gone and alt[x] == a:
                    held += 1
            assert oracle.view_dropped(lists, rd, alt, a, j, local, capacity) == max(0, held - capacity)
            assert oracle.view_dropped(lists, None, alt, a, j, local, capacity) == \
                max(0, sum(1 for x in range(max(0, j - local + 1)) if addr[x] == a) - capacity)
    final = set()
    for a in range(A):
        final |= set(vr[(a, nb - 1)])
    assert oracle.redirect_overflow(lists, rd, capacity) == (nb - local) - len(final)
    assert oracle.posting_overflow(lists, capacity) == (nb - local) - len({x for a in range(A) for x in vd[(a, nb - 1)]})


def test_redirect_equals_drop_without_overflow():
    rng = np.random.default_rng(9)
    A, nb, cap, L = 8, 30, 8, 2
    addr = rng.integers(0, A, size=nb)
    addr[:] = np.arange(nb) % A  # at most 4 per address: nothing overflows
    alt = (addr + 1) % A
    lists = oracle.posting_lists(addr, A, L)
    rd = oracle.redirect_lists(lists, alt, cap, L)
    assert all(len(r) == 0 for r in rd)
    for a in range(A):
        for j in range(nb):
            assert oracle.posting_view_redirect(lists, rd, a, j, L, cap) == oracle.posting_view(lists, a, j, L, cap)
    assert oracle.redirect_overflow(lists, rd, cap) == 0


def test_alternate_address_worked_example():
    """Hand-computed logits (one-hot summary picks the codebook's first coordinate)."""
    D = 4
    cb = np.zeros((2, 3, D), dtype=np.float32)
    cb[0, :, 0] = [3.0, 2.5, 1.0]  # subspace 0: top 0, runner-up 1, margin 0.5
    cb[1, :, 0] = [0.25, 1.0, 0.875]  # subspace 1: top 1, runner-up 2, margin 0.125
    ks = np.zeros((3, D), dtype=np.float32)
    ks[0, 0] = 1.0
    ks[1, 0] = 2.0            # margins scale: 1.0 and 0.25 -> still subspace 1
    ks[2, 0] = -1.0           # logits negate: subspace 0 top 2 (-1.0), runner-up 1 (-2.5), margin 1.5;
    #                           subspace 1 top 0 (-0.25), runner-up 2 (-0.875), margin 0.625
    codes, addr, _ = oracle.block_addresses(ks, cb, None)
    second, margin = oracle.runner_up_codes(ks, cb, None)
    alt, gap = oracle.alternate_addresses(codes, second, margin, 3)
    assert codes.tolist() == [[0, 1], [0, 1], [2, 0]]
    assert second.tolist() == [[1, 2], [1, 2], [1, 2]]
    np.testing.assert_allclose(margin, [[0.5, 0.125], [1.0, 0.25], [1.5, 0.625]])
    assert addr.tolist() == [1, 1, 6]
    assert alt.tolist() == [0 * 3 + 2, 0 * 3 + 2, 2 * 3 + 2]  # the low-margin subspace 1 changes
    np.testing.assert_allclose(gap, [0.375, 0.75, 0.875])


def test_alternate_address_ties():
    """Equal top logits: margin 0, runner-up the larger tied code; equal margins: the smaller subspace."""
    D = 2
    cb = np.zeros((2, 3, D), dtype=np.float32)
    cb[0, :, 0] = [1.0, 2.0, 2.0]   # top 1 (smaller of the tie), runner-up 2, margin 0
    cb[1, :, 0] = [5.0, 5.0, 1.0]   # top 0, runner-up 1, margin 0
    ks = np.array([[1.0, 0.0]], dtype=np.float32)
    codes, addr, _ = oracle.block_addresses(ks, cb, None)
    second, margin = oracle.runner_up_codes(ks, cb, None)
    alt, _ = oracle.alternate_addresses(codes, second, margin, 3)
    assert codes.tolist() == [[1, 0]] and second.tolist() == [[2, 1]]
    assert alt.tolist() == [2 * 3 + 0]  # both margins 0: subspace 0 changes
    one = np.zeros((1, 1, D), dtype=np.float32)
    s1, m1 = oracle.runner_up_codes(ks, one, None)
    a1, _ = oracle.alternate_addresses(np.zeros((1, 1), dtype=np.int64), s1, m1, 1)
    assert a1.tolist() == [-1]


def test_route_head_redirect_recovers_overflowed_blocks():
    """Under skew with a small capacity, redirect drops fewer blocks than drop and returns at least
    as many candidates overall; every view stays within capacity and holds eligible blocks only."""
    w = synth.workload("skew", batch=1, heads=1, seq=4096, capacity=1)
    inp = synth.make_core_inputs(w, 0)
    args = (inp["q"][0, 0], inp["k"][0, 0], inp["codebook"][0], inp["bias"][0], w)
    rdrop = oracle.route_head(*args, policy="drop")
    rred = oracle.route_head(*args, policy="redirect")
    assert rdrop["overflow"] > 0
    assert rred["overflow"] < rdrop["overflow"]
    assert rred["n_cand"].sum() >= rdrop["n_cand"].sum()
    for row, t in enumerate(rred["tokens"]):
        j = int(t) // w.block
        c = rred["cands"][row]
        assert all(0 <= i <= j - w.local for i in c)
    for a in range(w.addresses):
        for j in range(0, w.nblocks, 5):
            v = oracle.posting_view_redirect(rred["lists"], rred["rd"], a, j, w.local, w.capacity)
            assert len(v) <= w.capacity and len(set(v)) == len(v)


def test_round_to_bf16_matches_torch():
    """The oracle's bfloat16 rounding against torch's conversion (round to nearest even), including
    exact ties, values at the bf16 grid and negative numbers."""
    rng = np.random.default_rng(11)
    a = rng.standard_normal(4096).astype(np.float32) * np.float32(3.0)
    grid = torch.tensor(a).to(torch.bfloat16).float().numpy()
    _, e = np.frexp(grid)                                       # |grid| = m 2^e, 0.5 <= m < 1
    ulp = np.ldexp(np.float32(1.0), e - 8).astype(np.float32)  # bf16 spacing at grid
    ties = (grid + np.sign(grid) * ulp * np.float32(0.5)).astype(np.float32)  # exactly half way
    assert np.all(np.abs(ties - grid) == ulp / 2)
    for x in (a, grid, ties, -ties):
        ref = torch.tensor(x).to(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(oracle.round_to_bf16(x), ref)


# ---------------------------------------------------------------- decision margins
#
# The margins decide which GPU decisions the parity tests compare exactly (a decision whose margin is at
# most 1e-4 may legitimately come out either way in fp32).  They are pinned here against margins taken
# from a full sort of the raw scores the brute force computes, on dyadic inputs where every score is exact.

def margin_mismatches(w, q, k, cb, b, rdtype=np.float32):
    """Every disagreement between the oracle's margins, posting CSR and runner-up gaps and the brute force's."""
    from tests._brute import brute_margins, brute_posting_csr

    bad = []
    r = oracle.route_head(q, k, cb, b, w, rdtype=rdtype)
    bf = brute_routed_attention(q.tolist(), k.tolist(), np.zeros_like(q).tolist(), cb.tolist(),
                                None if b is None else b.tolist(), w)
    bm = brute_margins(bf, w)
    if r["addr_margin"].tolist() != bm["addr_margin"]:
        bad.append("addr_margin")
    if r["probe_margin"].tolist() != bm["probe_margin"]:
        bad.append("probe_margin")
    if r["sel_margin"].tolist() != bm["sel_margin"]:
        bad.append("sel_margin")
    gap = oracle.runner_up_gap(r["ksum"], cb, b, rdtype)
    if gap.tolist() != bm["second_gap"]:
        bad.append("runner_up_gap")
    second, m32 = oracle.runner_up_codes(r["ksum"], cb, b, rdtype)
    _, alt_gap = oracle.alternate_addresses(r["codes"], second, m32, w.codes)
    if alt_gap.tolist() != bm["alt_gap"]:
        bad.append("alt_gap")
    off, idx = brute_posting_csr(bf["addr"], w.addresses, w.local)
    if r["off"].tolist() != off or r["idx"].tolist() != idx:
        bad.append("posting_csr")
    return bad


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("rdtype", [np.float32, np.float64])
def test_margins_match_brute_force_sorts(case, seed, rdtype):
    w = _w(**SMALL[case])
    q, k, v, cb, b = _dyadic_inputs(w, seed, bias=(seed == 1))
    assert margin_mismatches(w, q, k, cb, b, rdtype) == []


def test_margins_count_inner_rank_gaps():
    """Hand cases whose closest gap lies inside the kept ranks, not at the boundary with the first one
    left out: the probe margin over address scores 10, 9.75, 5, 1 with P = 2 is 0.25 (between the first
    and second probe), not 4.75; the rerank margin over candidate scores 8, 7.5, 7.375, 0 with R = 2 is
    0.125; with R = 3 it is still 0.125 (ranks 2-3), not 7.375 (the boundary)."""
    top, m = oracle.top_probes(np.array([[1.0, 10.0, 5.0, 9.75]]), 2)
    assert top.tolist() == [[1, 3]] and m.tolist() == [0.25]
    top, m = oracle.top_probes(np.array([[4.0, 3.0, 2.5, 0.0]]), 3)  # boundary 2.5 | 0 is 2.5, inner 0.5
    assert top.tolist() == [[0, 1, 2]] and m.tolist() == [0.5]
    D = 4
    ks = np.zeros((4, D), dtype=np.float32)
    ks[:, 0] = [8.0, 7.5, 7.375, 0.0]
    q = np.array([1.0, 0.0, 0.0, 0.0], dtype=np.float32)
    sel, m = oracle.rerank(q, ks, [3, 2, 1, 0], 2)
    assert sel == [0, 1] and m == 0.125
    sel, m = oracle.rerank(q, ks, [3, 2, 1, 0], 3)
    assert sel == [0, 1, 2] and m == 0.125
    sel, m = oracle.rerank(q, ks, [3, 0], 2)  # fewer candidates than R + 1: the gap between the two
    assert sel == [0, 3] and m == 8.0
    # block addresses: logits 3, 2.875, 1 in subspace 0 -> margin 0.125; runner-up gap 1.875
    cb = np.zeros((1, 3, D), dtype=np.float32)
    cb[0, :, 0] = [2.875, 3.0, 1.0]
    one = np.zeros((1, D), dtype=np.float32)
    one[0, 0] = 1.0
    codes, addr, margin = oracle.block_addresses(one, cb, None)
    assert codes.tolist() == [[1]] and margin.tolist() == [[0.125]]
    assert oracle.runner_up_gap(one, cb, None).tolist() == [[1.875]]


# Seeded mistakes, each a plausible slip in one margin function, planted in the oracle on the CPU: the pin
# above must catch every one of them.
def _probe_boundary_only(sigma, probes):
    order = np.argsort(-sigma, axis=-1, kind="stable")
    s = np.take_along_axis(sigma, order, axis=-1).astype(np.float64)
    n = min(probes, sigma.shape[-1] - 1)
    return order[..., :probes], s[..., n - 1] - s[..., n]


def _probe_inner_only(sigma, probes):
    order = np.argsort(-sigma, axis=-1, kind="stable")
    s = np.take_along_axis(sigma, order[..., :probes], axis=-1).astype(np.float64)
    m = (s[..., :-1] - s[..., 1:]).min(axis=-1) if probes > 1 else np.full(sigma.shape[:-1], oracle.INF)
    return order[..., :probes], m


def _rerank_boundary_only(q_t, ksum, cands, remote, rdtype=np.float32):
    if not cands or remote == 0:
        return [], oracle.INF
    rho = np.asarray(ksum[cands], dtype=rdtype) @ np.asarray(q_t, dtype=rdtype)
    order = sorted(range(len(cands)), key=lambda n: (-float(rho[n]), cands[n]))
    top = [float(rho[n]) for n in order[:remote + 1]]
    return [cands[n] for n in order[:remote]], (top[-2] - top[-1]) if len(top) > 1 else oracle.INF


def _addresses_wrong_margin(ksum, codebook, bias, rdtype=np.float32):
    codes, addr, margin = _ORIG["block_addresses"](ksum, codebook, bias, rdtype)
    lg = oracle.code_logits(ksum, codebook, bias, rdtype)
    srt = np.sort(lg, axis=2).astype(np.float64)
    return codes, addr, srt[..., -1] - srt[..., 0]  # best minus worst instead of best minus second


def _alternates_wrong_gap(codes, second, margin, n_codes):
    alt, gap = _ORIG["alternate_addresses"](codes, second, margin, n_codes)
    return alt, np.where(np.isfinite(gap), margin.max(axis=1) - margin.min(axis=1), gap)  # largest, not next


def _csr_descending(lists):
    off, idx = _ORIG["posting_csr"](lists)
    return off, np.concatenate([idx[off[a]:off[a + 1]][::-1] for a in range(len(lists))]).astype(np.int64)


def _runner_up_gap_wrong(ksum, codebook, bias, rdtype=np.float32):
    lg = oracle.code_logits(ksum, codebook, bias, rdtype)
    srt = np.sort(lg.astype(np.float64), axis=2)
    return srt[..., -1] - srt[..., -2]  # first minus second instead of second minus third


_ORIG = {n: getattr(oracle.mdr_oracle, n) for n in ("block_addresses", "posting_csr", "alternate_addresses")}


@pytest.mark.parametrize("name,fn,field", [
    ("top_probes", _probe_boundary_only, "probe_margin"),
    ("top_probes", _probe_inner_only, "probe_margin"),
    ("rerank", _rerank_boundary_only, "sel_margin"),
    ("block_addresses", _addresses_wrong_margin, "addr_margin"),
    ("posting_csr", _csr_descending, "posting_csr"),
    ("runner_up_gap", _runner_up_gap_wrong, "runner_up_gap"),
    ("alternate_addresses", _alternates_wrong_gap, "alt_gap"),
])
def test_margin_pins_catch_planted_mistakes(monkeypatch, name, fn, field):
    monkeypatch.setattr(oracle.mdr_oracle, name, fn)
    monkeypatch.setattr(oracle, name, fn)
    found = set()
    for case in range(len(SMALL)):
        w = _w(**SMALL[case])
        for seed in (0, 1, 2):
            q, k, v, cb, b = _dyadic_inputs(w, seed, bias=(seed == 1))
            found.update(margin_mismatches(w, q, k, cb, b))
    assert field in found
