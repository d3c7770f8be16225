"""Overflow policies on the GPU: the redirect policy's alternates, redirect lists, views, overflow
count and the per-token dropped-candidate count, against the oracle (through the C ABI).

Integer results must match exactly wherever every floating-point decision behind them has an
oracle margin above 1e-4 (the near-tie rule of the other parity tests): an alternate address is
sure when the block's address is sure, the smallest subspace margin is clear of the next one and
the runner-up code is clear of the third code.  Redirect lists, overflow and views depend on the
addresses and alternates of a whole (b, h), so they are compared when all of them are sure; the
staged tests feed the oracle's own upstream to each stage, so nothing upstream can be a tie.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import (NEAR, TOL, attention_rows, cfg_of, check_head_routing, compare_selection, dev, host, io_dtype,
                        run_core, small)

pytestmark = pytest.mark.gpu

# (workload, overrides): each overflows its lists under the given capacity
CASES = [
    ("tiny", dict(capacity=1)),                               # fp32, 16 addresses, generic probe shape
    ("skew", dict(batch=1, heads=2, seq=4096, capacity=1)),   # bf16, zipf-biased codes, fixed probe
    ("skew", dict(batch=1, heads=2, seq=8192, capacity=2)),
    ("recall", dict(batch=2, capacity=1)),                    # fp32, P16 M5
    ("sweep", dict(heads=2, seq=4096, capacity=1, plant="none")),  # bf16, the bench shape, unplanted codes
]
# end-to-end seeds with at least one (b, h) free of alternate near-ties (checked on the oracle alone)
E2E_SEED = [0, 1, 0, 0, 0]


def oracle_routes(w, inp, policy):
    return [[oracle.route_head(inp["q"][b, h], inp["k"][b, h], inp["codebook"][h],
                               None if inp["bias"] is None else inp["bias"][h], w, policy=policy)
             for h in range(w.heads)] for b in range(w.batch)]


def alt_sure(w, inp, r, b, h):
    bias = None if inp["bias"] is None else inp["bias"][h]
    gap2 = oracle.runner_up_gap(r["ksum"], inp["codebook"][h], bias)
    second, margin = oracle.runner_up_codes(r["ksum"], inp["codebook"][h], bias)
    g_star = np.array([min(range(w.subspaces), key=lambda g: (margin[i, g], g)) for i in range(w.nblocks)])
    return ((r["addr_margin"].min(axis=1) > NEAR) & (r["alt_gap"] > NEAR) &
            (gap2[np.arange(w.nblocks), g_star] > NEAR))


@pytest.mark.parametrize("name,over,seed", [c + (sd,) for c, sd in zip(CASES, E2E_SEED)])
def test_redirect_end_to_end(gpu_lib, name, over, seed):
    mdr = gpu_lib
    w = small(name, **over)
    inp = synth.make_core_inputs(w, seed)
    res = run_core(mdr, w, inp, policy="redirect")
    near_up = near_sel = 0
    over_total = 0
    for b in range(w.batch):
        for h in range(w.heads):
            nu, ns = check_head_routing(w, inp, res, b, h, policy="redirect")
            near_up += nu
            near_sel += ns
            over_total += int(res["overflow"][b, h])
    assert over_total > 0 or name == "recall"
    print(f"{name} {over}: every head compared (on the GPU's addresses and alternates where they hold "
          f"near-ties: {near_up}), selection near-ties {near_sel} (validated), overflow {over_total}")


@pytest.mark.parametrize("name,over", CASES[:3])
def test_drop_policy_dropped_candidates(gpu_lib, name, over):
    """n_drop under the drop policy (the default path, fused lists where specialised)."""
    mdr = gpu_lib
    w = small(name, **over)
    inp = synth.make_core_inputs(w, 1)
    res = run_core(mdr, w, inp)
    total = 0
    for b in range(w.batch):
        for h in range(w.heads):
            check_head_routing(w, inp, res, b, h)  # n_drop on every probe-sure token, every head
            total += int(res["n_drop"][b, h].sum())
    assert total > 0
    print(f"{name} {over}: dropped candidates {total}")


@pytest.mark.parametrize("name,over", CASES)
def test_staged_redirect_on_oracle_upstream(gpu_lib, name, over):
    """mdr_stage_address (alternates), mdr_stage_post (redirect lists) on the oracle's addresses and
    alternates, and mdr_stage_probe_rerank on the oracle's lists: no upstream near-tie can leak."""
    mdr = gpu_lib
    w = small(name, **over)
    inp = synth.make_core_inputs(w, 2)
    cfg = cfg_of(mdr, w, "redirect")
    B, H, S, nb, A = w.batch, w.heads, w.seq, w.nblocks, w.addresses
    routes = oracle_routes(w, inp, "redirect")
    i32 = dict(dtype=torch.int32, device="cuda")
    bias = None if inp["bias"] is None else dev(inp["bias"], torch.float32)
    cb = dev(inp["codebook"], torch.float32)
    # addresses and alternates
    ksum = torch.empty(B, H, nb, w.head_dim, dtype=torch.float32, device="cuda")
    addr = torch.empty(B, H, nb, **i32)
    alt = torch.empty(B, H, nb, **i32)
    mdr.mdr_stage_address(cfg, dev(inp["k"], io_dtype(w)), cb, bias, ksum, addr, alt)
    torch.cuda.synchronize()
    alt_g = host(alt)
    for b in range(B):
        for h in range(H):
            sure = alt_sure(w, inp, routes[b][h], b, h)
            assert np.array_equal(alt_g[b, h][sure], routes[b][h]["alt"][sure])
    # lists from the oracle's addresses and alternates
    o_addr = np.stack([np.stack([r["addr"] for r in rb]) for rb in routes]).astype(np.int32)
    o_alt = np.stack([np.stack([r["alt"] for r in rb]) for rb in routes]).astype(np.int32)
    off = torch.empty(B, H, A + 1, **i32)
    idx = torch.empty(B, H, nb, **i32)
    roff = torch.empty(B, H, A + 1, **i32)
    ridx = torch.empty(B, H, nb, **i32)
    rtime = torch.empty(B, H, nb, **i32)
    ovf = torch.empty(B, H, **i32)
    mdr.mdr_stage_post(cfg, dev(o_addr), off, idx, ovf, alt=dev(o_alt), redir_off=roff, redir_idx=ridx,
                       redir_time=rtime)
    torch.cuda.synchronize()
    roff_h, ridx_h, rtime_h, ovf_h = host(roff), host(ridx), host(rtime), host(ovf)
    for b in range(B):
        for h in range(H):
            r = routes[b][h]
            assert ovf_h[b, h] == r["overflow"]
            for a in range(A):
                got = [(int(rtime_h[b, h, k]), int(ridx_h[b, h, k])) for k in range(roff_h[b, h, a], roff_h[b, h, a + 1])]
                assert got == r["rd"][a], (b, h, a)
    # probe + rerank on the oracle's summaries and lists (primary and redirect)
    o_ksum = np.stack([np.stack([r["ksum"] for r in rb]) for rb in routes]).astype(np.float32)
    o_off = np.stack([np.stack([r["off"] for r in rb]) for rb in routes]).astype(np.int32)
    o_idx = np.full((B, H, nb), -1, dtype=np.int32)
    o_roff = np.zeros((B, H, A + 1), dtype=np.int32)
    o_ridx = np.full((B, H, nb), -1, dtype=np.int32)
    o_rtime = np.full((B, H, nb), -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            r = routes[b][h]
            o_idx[b, h, :len(r["idx"])] = r["idx"]
            k = 0
            for a in range(A):
                o_roff[b, h, a] = k
                for tm, x in r["rd"][a]:
                    o_ridx[b, h, k], o_rtime[b, h, k] = x, tm
                    k += 1
            o_roff[b, h, A] = k
    sel = torch.empty(B, H, S, w.remote, **i32)
    ncand = torch.empty(B, H, S, **i32)
    ndrop = torch.empty(B, H, S, **i32)
    mdr.mdr_stage_probe_rerank(cfg, dev(inp["q"], io_dtype(w)), cb, bias, dev(o_ksum), dev(o_off), dev(o_idx),
                               None, sel, ncand, redir_off=dev(o_roff), redir_idx=dev(o_ridx),
                               redir_time=dev(o_rtime), n_drop=ndrop)
    torch.cuda.synchronize()
    sel, ncand, ndrop = host(sel), host(ncand), host(ndrop)
    near = 0
    for b in range(B):
        for h in range(H):
            r = routes[b][h]
            near += compare_selection(r, sel[b, h], w=w, inp=inp, b=b, h=h, policy="redirect")
            sure = r["probe_margin"] > NEAR
            assert np.array_equal(ncand[b, h][sure], r["n_cand"][sure])
            assert np.array_equal(ndrop[b, h][sure], r["n_drop"][sure])
    print(f"{name} {over}: staged redirect, probe near-ties {near}")


def test_redirect_without_overflow_equals_drop(gpu_lib):
    """With room in every list nothing is redirected: the two policies give identical results."""
    mdr = gpu_lib
    w = small("sweep", heads=2, seq=4096)  # balanced addresses, capacity twice the mean list length
    inp = synth.make_core_inputs(w, 3)
    a = run_core(mdr, w, inp, policy="drop")
    b = run_core(mdr, w, inp, policy="redirect")
    assert int(b["redir_off"][..., -1].sum()) == 0 or int(a["overflow"].sum()) > 0
    if int(a["overflow"].sum()) == 0:
        for n in ("sel", "n_cand", "n_drop", "overflow", "addr"):
            assert np.array_equal(a[n], b[n]), n
        np.testing.assert_array_equal(a["out"], b["out"])


@pytest.mark.parametrize("policy", ["drop", "redirect"])
def test_stress_full_size_sampled(gpu_lib, policy):
    """The benchmark's overflow-stress shape at full size and its strongest skew (B2 H8 S16384 D128, 3x8
    codes, capacity 8, P6, R8, code bias -ln(c + 1)): every head's addresses, posting lists, overflow
    (and redirect lists) against the oracle, the routing of sampled tokens under the near-tie rule, and
    their attention rows with the GPU's selection."""
    mdr = gpu_lib
    w = small("skew", batch=2, heads=8, seq=16384, zipf_kappa=1.0)
    inp = synth.make_core_inputs(w, 0)
    res = run_core(mdr, w, inp, policy=policy)
    rng = np.random.default_rng(5)
    toks = np.unique(np.concatenate([rng.choice(w.seq, 64, replace=False), [0, w.block - 1, w.seq - 1]]))
    near_up = near_sel = 0
    err = 0.0
    for b in range(w.batch):
        for h in range(w.heads):
            nu, ns = check_head_routing(w, inp, res, b, h, policy=policy, tokens=toks)
            near_up += nu
            near_sel += ns
            ref = attention_rows(w, inp, res["sel"][b, h][toks], b, h, toks)
            err = max(err, float(np.abs(res["out"][b, h][toks] - ref).max()))
    print(f"stress {policy}: overflow {int(res['overflow'].sum())}, upstream near-ties {near_up}, sampled "
          f"selection near-ties {near_sel}, sampled max abs err {err:.3g}")
    assert int(res["overflow"].sum()) > 0
    assert err <= TOL[w.dtype]
