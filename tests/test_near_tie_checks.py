"""The near-tie validity check of the GPU parity tests, exercised on the CPU: the oracle's own selection
passes it on every token, and selections a correct router could not make fail it."""

import numpy as np
import pytest

import oracle
import synth
from tests._gpu import check_near_tie_token, compare_addresses, route_for


@pytest.mark.parametrize("name,over", [("recall", dict(batch=1, heads=1, seq=1024)),
                                       ("skew", dict(batch=1, heads=1, seq=2048)),
                                       ("tiny", {})])
def test_oracle_selection_passes_on_every_token(name, over):
    w = synth.workload(name, **over)
    inp = synth.make_core_inputs(w, 0)
    r = route_for(w, inp, 0, 0)
    for row in range(0, w.seq, 7):
        check_near_tie_token(r, row, r["sel"][row], w, inp, 0, 0)
        check_near_tie_token(r, row, r["sel"][row], w, inp, 0, 0, probes_row=r["probes"][row])


def _late_token(w, r):
    """A token with at least R + 1 candidates (so a non-selected candidate exists)."""
    for row in range(w.seq - 1, 0, -1):
        if len(r["cands"][row]) > w.remote and np.all(r["sel"][row] >= 0):
            return row
    raise AssertionError("no token with spare candidates")


def test_invalid_selections_fail():
    w = synth.workload("recall", batch=1, heads=1)
    inp = synth.make_core_inputs(w, 0)
    r = route_for(w, inp, 0, 0)
    row = _late_token(w, r)
    t = int(r["tokens"][row])
    good = r["sel"][row].copy()
    cutoff = t // w.block - w.local

    def fails(sel, probes=None):
        with pytest.raises(AssertionError):
            check_near_tie_token(r, row, np.asarray(sel), w, inp, 0, 0, probes_row=probes)

    dup = good.copy()
    dup[1] = dup[0]
    fails(dup)                                   # a repeated block
    inel = good.copy()
    inel[0] = cutoff + 1
    fails(inel)                                  # a block inside the local window
    gap = good.copy()
    gap[0] = -1
    fails(gap)                                   # -1 before a real entry
    outside = good.copy()
    outside[-1] = next(i for i in range(cutoff + 1) if i not in r["cands"][row])
    fails(outside)                               # not a candidate of any plausible probe
    # the lowest-scoring candidate in place of the last selected one (not a near-tie here)
    rho = np.asarray(r["ksum"][r["cands"][row]], np.float32) @ np.asarray(inp["q"][0, 0][t], np.float32)
    worst = r["cands"][row][int(np.argmin(rho))]
    low = good.copy()
    low[-1] = worst
    fails(low)
    fails(good, probes=r["probes"][row][::-1])   # probes out of rank order
    swapped = good.copy()
    swapped[0], swapped[1] = good[1], good[0]
    if r["sel_margin"][row] > 1e-4:
        fails(swapped)                           # selection out of rank order


def test_address_check_accepts_near_ties_and_rejects_wrong_codes():
    w = synth.workload("tiny")
    inp = synth.make_core_inputs(w, 0)
    ks = oracle.block_summaries(inp["k"][0, 0], w.block)
    _, addr, margin = oracle.block_addresses(ks, inp["codebook"][0], None)
    assert compare_addresses(w, inp, addr.copy(), 0, 0) == int((margin.min(axis=1) <= 1e-4).sum())
    bad = addr.copy()
    i = int(np.argmax(margin.min(axis=1)))
    bad[i] = (bad[i] + 1) % w.addresses
    with pytest.raises(AssertionError):
        compare_addresses(w, inp, bad, 0, 0)
