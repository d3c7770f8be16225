"""Pins of the packed C oracle (oracle/mdr_packed.c), the CPU baseline's timed implementation (CPU only).

It is checked against things other than itself:
* the independent pure-Python brute force (tests/_brute.py) on tiny dyadic inputs, where every
  routing score is exact in float32 so ties are frequent and the tie rules must agree exactly;
* the hand-derived golden case (tests/golden/hand_routing.json);
* a full routing budget, which reduces to dense causal attention (torch's
  scaled_dot_product_attention in float64);
* the NumPy oracle on the workload shapes: selections equal wherever the NumPy oracle's probe and
  rerank margins exceed the near-tie bound (the two take the same fp32 decisions but add in different
  orders), attention equal to its packed and dense forms on the C oracle's own selection.
A mistake planted in the C file (a dropped term, a wrong sign, a flipped tie rule) fails the brute
force or the golden case.
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
from oracle import packed
from tests._brute import brute_routed_attention
from tests.test_oracle_pins import SMALL, _dyadic_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NEAR = 1e-4


def _w(**kw):
    return dataclasses.replace(synth.workload("tiny"), **kw)


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_packed_equals_brute_force_on_dyadic_inputs(case, seed):
    w = _w(**SMALL[case])
    q, k, v, cb, b = _dyadic_inputs(w, seed, bias=(seed == 1))
    sel, out = packed.packed_forward(q, k, v, cb, b, w)
    bf = brute_routed_attention(q.tolist(), k.tolist(), v.tolist(), cb.tolist(),
                                None if b is None else b.tolist(), w)
    for t in range(w.seq):
        assert [i for i in sel[t] if i >= 0] == bf["sel"][t], t
    # q, k, v pass through float32 (the dyadic q and k exactly; v is rounded)
    np.testing.assert_allclose(out, np.array(bf["out"]), rtol=0, atol=1e-6)
    v32 = v.astype(np.float32).astype(np.float64)
    ref = oracle.attention_dense(q, k, v32, sel, w.block, w.local)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_packed_hand_derived_golden_case():
    g = json.load(open(os.path.join(GOLDEN, "hand_routing.json")))
    c = g["config"]
    w = _w(seq=len(g["k"]), head_dim=2, block=c["block"], subspaces=c["subspaces"], codes=c["codes"],
           capacity=c["capacity"], probes=c["probes"], max_cand=c["max_cand"], remote=c["remote"],
           local=c["local"])
    q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    cb = np.array(g["codebook"], dtype=np.float64)
    sel, out = packed.packed_forward(q, k, v, cb, None, w)
    assert [[i for i in row if i >= 0] for row in sel] == g["sel"]
    for t, vis in g["visible_dots"].items():
        t = int(t)
        wts = np.array([math.exp(d / math.sqrt(2.0)) for _, d in vis])
        expect = (wts[:, None] * v[[s for s, _ in vis]]).sum(0) / wts.sum()
        np.testing.assert_allclose(out[t], expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_packed_full_budget_is_dense_causal_attention(seed):
    nb, blk = 8, 8
    w = _w(seq=nb * blk, head_dim=16, block=blk, subspaces=2, codes=3, capacity=nb, probes=9,
           max_cand=0, remote=nb, local=2)
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((w.seq, w.head_dim)).astype(np.float32).astype(np.float64) for _ in range(3))
    cb = rng.standard_normal((2, 3, 16)) / 4
    _, out = packed.packed_forward(q, k, v, cb, None, w)
    t = [torch.from_numpy(a)[None, None] for a in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True)[0, 0].numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name,over,seed", [
    ("recall", dict(batch=1), 1), ("sweep", dict(seq=4096, heads=2), 2), ("skew", dict(batch=1, heads=2, seq=2048), 3),
    ("long", dict(heads=1, seq=4096), 4)])
def test_packed_agrees_with_numpy_oracle(name, over, seed):
    w = synth.workload(name, **over)
    inp = synth.make_core_inputs(w, seed)
    near = 0
    for h in range(w.heads):
        bias = None if inp["bias"] is None else inp["bias"][h]
        q, k, v = (inp[n][0, h] for n in ("q", "k", "v"))
        r = oracle.route_head(q, k, inp["codebook"][h], bias, w)
        t0 = w.seq // 3  # a token range that starts inside the sequence
        sel, out = packed.packed_forward(q, k, v, inp["codebook"][h], bias, w, t0=t0)
        sure = (r["probe_margin"][t0:] > NEAR) & (r["sel_margin"][t0:] > NEAR)
        assert r["addr_margin"].min() > NEAR  # no address near-tie in these heads
        bad = np.nonzero(sure & np.any(sel != r["sel"][t0:], axis=1))[0]
        assert len(bad) == 0, (h, bad[:8])
        near += int((~sure).sum())
        ref = oracle.attention_packed(q, k, v, sel, w.block, w.local, tokens=np.arange(t0, w.seq))
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
        toks = np.arange(t0, w.seq, 97)
        dense = oracle.attention_dense(q, k, v, sel[toks - t0], w.block, w.local, tokens=toks)
        np.testing.assert_allclose(out[toks - t0], dense, rtol=0, atol=1e-12)
    print(f"{name}: near-ties {near}")


def test_packed_rejects_invalid_sizes():
    w = _w(seq=64, head_dim=4, block=8, subspaces=2, codes=3, capacity=2, probes=2, max_cand=0, remote=2, local=2)
    q = np.zeros((60, 4))  # not a whole number of blocks
    with pytest.raises(ValueError):
        packed.packed_forward(q, q, q, np.zeros((2, 3, 4)), None, w)
