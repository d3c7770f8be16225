"""Parity of the HIP path with the CPU oracle on the GPU (through the C ABI).

Routing indices must match exactly wherever the oracle's decision margin
exceeds 1e-4 (near-ties are counted); attention must match within 1e-5
absolute in fp32 and 2e-2 in bf16.  Each stage is also run on the oracle's
own upstream output, so a near-tie upstream cannot cascade into a failure.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import (NEAR, TOL, attention_rows, cfg_of, check_head_routing, compare_addresses, compare_selection,
                        dev, host, integer_inputs, io_dtype, route_for, run_core, small)

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "recall", "sweep", "long", "skew"]


@pytest.mark.parametrize("name", NAMES)
def test_stage_address(gpu_lib, name):
    mdr = gpu_lib
    w = small(name)
    inp = synth.make_core_inputs(w, 0)
    cfg = cfg_of(mdr, w)
    k = dev(inp["k"], io_dtype(w))
    ksum = torch.empty(w.batch, w.heads, w.nblocks, w.head_dim, dtype=torch.float32, device="cuda")
    addr = torch.empty(w.batch, w.heads, w.nblocks, dtype=torch.int32, device="cuda")
    bias = None if inp["bias"] is None else dev(inp["bias"], torch.float32)
    mdr.mdr_stage_address(cfg, k, dev(inp["codebook"], torch.float32), bias, ksum, addr)
    torch.cuda.synchronize()
    ksum, addr = host(ksum), host(addr)
    near = 0
    for b in range(w.batch):
        for h in range(w.heads):
            ks = oracle.block_summaries(inp["k"][b, h], w.block)
            np.testing.assert_allclose(ksum[b, h], ks, rtol=1e-5, atol=1e-6)
            near += compare_addresses(w, inp, addr[b, h], b, h)
    print(f"{name}: address near-ties {near}")


@pytest.mark.parametrize("nb,G,C,L,cap,skew", [(16, 2, 4, 2, 8, 0.0), (512, 2, 16, 2, 4, 0.0),
                                               (64, 3, 8, 2, 8, 2.0), (1024, 2, 32, 2, 16, 1.5),
                                               (3, 2, 4, 2, 1, 0.0), (2, 1, 4, 2, 1, 0.0), (100, 1, 7, 1, 3, 1.0),
                                               (8192, 3, 16, 3, 2, 0.5)])
def test_stage_post(gpu_lib, nb, G, C, L, cap, skew):
    """CSR and overflow from arbitrary address arrays must equal the oracle's exactly."""
    mdr = gpu_lib
    A = C ** G
    rng = np.random.default_rng(nb + A)
    BH = 3
    p = 1.0 / np.arange(1, A + 1) ** skew
    addr = rng.choice(A, size=(1, BH, nb), p=p / p.sum()).astype(np.int32)
    cfg = mdr.config(batch=1, seq=nb * 32, heads=BH, head_dim=32, block=32, subspaces=G, codes=C, capacity=cap,
                     probes=1, remote=1, local=L, dtype="f32")
    assert mdr.mdr_check_config(cfg) == 0
    off = torch.empty(1, BH, A + 1, dtype=torch.int32, device="cuda")
    idx = torch.empty(1, BH, nb, dtype=torch.int32, device="cuda")
    ovf = torch.empty(1, BH, dtype=torch.int32, device="cuda")
    mdr.mdr_stage_post(cfg, dev(addr), off, idx, ovf)
    torch.cuda.synchronize()
    off, idx, ovf = host(off), host(idx), host(ovf)
    for h in range(BH):
        lists = oracle.posting_lists(addr[0, h], A, L)
        o_off, o_idx = oracle.posting_csr(lists)
        assert np.array_equal(off[0, h], o_off)
        assert np.array_equal(idx[0, h, :len(o_idx)], o_idx)
        assert np.all(idx[0, h, len(o_idx):] == -1)
        assert ovf[0, h] == oracle.posting_overflow(lists, cap)


@pytest.mark.parametrize("name", NAMES)
def test_stage_probe_rerank_on_oracle_index(gpu_lib, name):
    mdr = gpu_lib
    w = small(name)
    inp = synth.make_core_inputs(w, 1)
    force = inp.get("force")
    cfg = cfg_of(mdr, w)
    B, H, S, nb = w.batch, w.heads, w.seq, w.nblocks
    routes = [[oracle.route_head(inp["q"][b, h], inp["k"][b, h], inp["codebook"][h],
                                 None if inp["bias"] is None else inp["bias"][h], w,
                                 None if force is None else force[b, h]) for h in range(H)] for b in range(B)]
    ksum = np.stack([np.stack([r["ksum"] for r in rb]) for rb in routes]).astype(np.float32)
    off = np.stack([np.stack([r["off"] for r in rb]) for rb in routes]).astype(np.int32)
    idx = np.full((B, H, nb), -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            idx[b, h, :len(routes[b][h]["idx"])] = routes[b][h]["idx"]
    sel = torch.empty(B, H, S, w.remote, dtype=torch.int32, device="cuda")
    ncand = torch.empty(B, H, S, dtype=torch.int32, device="cuda")
    bias = None if inp["bias"] is None else dev(inp["bias"], torch.float32)
    mdr.mdr_stage_probe_rerank(cfg, dev(inp["q"], io_dtype(w)), dev(inp["codebook"], torch.float32), bias,
                               dev(ksum), dev(off), dev(idx), None if force is None else dev(force), sel, ncand)
    torch.cuda.synchronize()
    sel, ncand = host(sel), host(ncand)
    near = 0
    for b in range(B):
        for h in range(H):
            r = routes[b][h]
            near += compare_selection(r, sel[b, h], w=w, inp=inp, b=b, h=h,
                                      force=None if force is None else force[b, h])
            sure = r["probe_margin"] > NEAR
            assert np.array_equal(ncand[b, h][sure], r["n_cand"][sure])
    print(f"{name}: probe/rerank near-tie tokens {near} of {B * H * S}")


@pytest.mark.parametrize("name,policy,cap", [(n, "drop", None) for n in NAMES] +
                         [(n, "redirect", 1) for n in ("tiny", "recall", "skew")])
def test_integer_scores_route_exactly(gpu_lib, name, policy, cap):
    """With exact scores the routing must equal the oracle's on every token, ties included (no
    near-tie allowance): the code, address and candidate rankings break ties by the lower index.
    Capacity 1 under the redirect policy makes lists overflow and redirect."""
    mdr = gpu_lib
    w = small(name) if cap is None else small(name, capacity=cap)
    inp = integer_inputs(w, 4)
    res = run_core(mdr, w, inp, force=inp.get("force"), policy=policy)
    ties = 0
    for b in range(w.batch):
        for h in range(w.heads):
            f = None if inp.get("force") is None else inp["force"][b, h]
            r = oracle.route_head(inp["q"][b, h], inp["k"][b, h], inp["codebook"][h],
                                  None if inp["bias"] is None else inp["bias"][h], w, f, policy=policy)
            ks = oracle.block_summaries(inp["k"][b, h], w.block)
            _, addr, _ = oracle.block_addresses(ks, inp["codebook"][h], None if inp["bias"] is None else inp["bias"][h])
            assert np.array_equal(res["addr"][b, h], addr), (b, h)
            assert res["overflow"][b, h] == r["overflow"]
            assert np.array_equal(res["sel"][b, h], r["sel"]), (b, h)
            ties += int(((r["probe_margin"] <= NEAR) | (r["sel_margin"] <= NEAR)).sum())
    print(f"{name} {policy}: tokens with tied rankings {ties}, overflow {int(res['overflow'].sum())}, all matched")


@pytest.mark.parametrize("name", NAMES)
def test_stage_attend_on_oracle_selection(gpu_lib, name):
    mdr = gpu_lib
    w = small(name)
    inp = synth.make_core_inputs(w, 2)
    B, H = w.batch, w.heads
    sel = np.stack([np.stack([oracle.route_head(inp["q"][b, h], inp["k"][b, h], inp["codebook"][h],
                                                None if inp["bias"] is None else inp["bias"][h], w)["sel"]
                              for h in range(H)]) for b in range(B)]).astype(np.int32)
    cfg = cfg_of(mdr, w)
    dt = io_dtype(w)
    q, k, v = (dev(inp[n], dt) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    mdr.mdr_stage_attend(cfg, q, k, v, dev(sel), out, mdr.workspace(cfg))
    torch.cuda.synchronize()
    out = host(out)
    err = 0.0
    for b in range(B):
        for h in range(H):
            ref = attention_rows(w, inp, sel[b, h], b, h, None, dense=w.seq <= 4096)
            err = max(err, float(np.abs(out[b, h] - ref).max()))
    print(f"{name}: max abs err {err:.3g}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("name", NAMES)
def test_routed_attention_end_to_end(gpu_lib, name):
    mdr = gpu_lib
    w = small(name)
    inp = synth.make_core_inputs(w, 0)
    res = run_core(mdr, w, inp, force=inp.get("force"))
    near_a = near_s = 0
    err = 0.0
    for b in range(w.batch):
        for h in range(w.heads):
            na, ns = check_head_routing(w, inp, res, b, h, force=inp.get("force"))
            near_a += na
            near_s += ns
            ref = attention_rows(w, inp, res["sel"][b, h], b, h, None, dense=w.seq <= 4096)
            err = max(err, float(np.abs(res["out"][b, h] - ref).max()))
    print(f"{name}: address near-ties {near_a}, selection near-ties {near_s} (each checked for validity), "
          f"max abs err {err:.3g}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("name,over", [(n, {}) for n in NAMES] + [("sweep", dict(seq=8192)),
                                                                   ("long", dict(heads=8)),
                                                                   ("skew", dict(batch=8, heads=8))])
def test_diagnostics_leave_routing_unchanged(gpu_lib, name, over):
    """Asking for the routing diagnostics runs the probe with one more address and candidate ranked, in
    256-token work-groups, every candidate's score kept in LDS; without them the rerank keeps only each
    token's top-R, and small grids take 64-token (the test sizes) or 128-token (sweep at 8K) work-groups,
    the long shape 128-token ones (its LDS holds more of them; 8 heads at 8K) and the skew shape at 8 x 8
    heads 256-token ones.  Every other output must be bit-identical between the two runs."""
    mdr = gpu_lib
    w = small(name, **over)
    inp = synth.make_core_inputs(w, 5)
    a = run_core(mdr, w, inp, force=inp.get("force"), diag=False)
    b = run_core(mdr, w, inp, force=inp.get("force"), diag=True)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("name", NAMES)
def test_diagnostics_match_the_oracle(gpu_lib, name):
    """The GPU's probes equal the oracle's wherever the probe margin exceeds NEAR; its selection scores,
    probe, rerank and address margins equal the oracle's up to fp32 summation order (where the oracle's
    routing is the GPU's: no address near-tie in the head)."""
    mdr = gpu_lib
    w = small(name)
    inp = synth.make_core_inputs(w, 6)
    res = run_core(mdr, w, inp)
    checked = 0
    for b in range(w.batch):
        for h in range(w.heads):
            na = compare_addresses(w, inp, res["addr"][b, h], b, h)
            r = route_for(w, inp, b, h, addr=res["addr"][b, h] if na else None)
            am = res["addr_margin"][b, h]
            np.testing.assert_allclose(am, r["addr_margin"].min(axis=1), rtol=1e-4, atol=1e-4)
            sure = r["probe_margin"] > NEAR
            assert np.array_equal(res["probes"][b, h][sure], r["probes"][sure])
            pm, om = res["probe_margin"][b, h], r["probe_margin"]
            fin = np.isfinite(om)
            assert np.array_equal(np.isfinite(pm), fin)
            np.testing.assert_allclose(pm[fin], om[fin], rtol=1e-4, atol=1e-4)
            sure &= r["sel_margin"] > NEAR
            sm, osm = res["sel_margin"][b, h], r["sel_margin"]
            fin = np.isfinite(osm) & sure
            np.testing.assert_allclose(sm[fin], osm[fin], rtol=1e-4, atol=1e-4)
            q = inp["q"][b, h].astype(np.float32)
            for t in np.nonzero(sure)[0]:
                sel = r["sel"][t]
                for k in range(w.remote):
                    if sel[k] < 0:
                        assert res["sel_score"][b, h, t, k] == -np.inf
                    else:
                        ref = float(np.asarray(r["ksum"][sel[k]], np.float32) @ q[t])
                        assert abs(res["sel_score"][b, h, t, k] - ref) <= 1e-4 * max(1.0, abs(ref)), (t, k)
                checked += 1
    print(f"{name}: diagnostics checked on {checked} tokens")
    assert checked > 0


def test_recall_forced_target_full_batch(gpu_lib):
    """All 16 sequences of the recall workload; forcing the planted block puts it into every selection of
    the last query block under the same budget R."""
    mdr = gpu_lib
    w = synth.workload("recall")
    inp = synth.make_core_inputs(w, 0)
    free = run_core(mdr, w, inp)
    forced = run_core(mdr, w, inp, force=inp["force"])
    last = slice((w.nblocks - 1) * w.block, w.seq)
    hits_free = hits_forced = 0
    for b in range(w.batch):
        p = inp["planted"][b]
        for h in range(w.heads):
            hits_free += int(np.sum(np.any(free["sel"][b, h, last] == p, axis=1)))
            s = forced["sel"][b, h, last]
            hits_forced += int(np.sum(np.any(s == p, axis=1)))
            assert np.all((s >= 0).sum(axis=1) <= w.remote)
            ref = attention_rows(w, inp, forced["sel"][b, h], b, h, None, dense=True)
            assert np.abs(forced["out"][b, h] - ref).max() <= TOL[w.dtype]
    total = w.batch * w.heads * w.block
    print(f"planted-block recall: untrained router {hits_free}/{total}, forced {hits_forced}/{total}")
    assert hits_forced == total


def test_deterministic(gpu_lib):
    mdr = gpu_lib
    w = small("skew")
    inp = synth.make_core_inputs(w, 3)
    a = run_core(mdr, w, inp)
    b = run_core(mdr, w, inp)
    for n in ("out", "sel", "addr", "post_idx", "overflow", "ksum"):
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("name,t0", [("recall", 1000), ("sweep", 2047), ("skew", 3000)])
def test_causal_on_gpu(gpu_lib, name, t0):
    """Perturbing tokens after t0 leaves every selection and output up to t0 bit-identical."""
    mdr = gpu_lib
    w = small(name)
    inp = synth.make_core_inputs(w, 4)
    a = run_core(mdr, w, inp)
    rng = np.random.default_rng(5)
    for n in ("q", "k", "v"):
        x = inp[n].copy()
        x[:, :, t0 + 1:] = synth.bf16_round(rng.standard_normal(x[:, :, t0 + 1:].shape).astype(np.float32) * 2)
        inp[n] = x
    b = run_core(mdr, w, inp)
    assert np.array_equal(a["sel"][:, :, :t0 + 1], b["sel"][:, :, :t0 + 1])
    assert np.array_equal(a["out"][:, :, :t0 + 1], b["out"][:, :, :t0 + 1])
    assert not np.array_equal(a["out"][:, :, t0 + 1:], b["out"][:, :, t0 + 1:])


@pytest.mark.parametrize("over", [
    dict(remote=0),                      # local-only control
    dict(seq=64, local=2),               # nb == L: nothing is ever eligible
    dict(seq=128, local=1),
    dict(local=1, capacity=1, probes=1),
    dict(local=3, remote=5, probes=3),
    dict(seq=1024 + 64),                 # blocks not a multiple of the 64-token waves
])
def test_edge_cases(gpu_lib, over):
    mdr = gpu_lib
    w = small("recall", batch=2, **over)
    inp = synth.make_core_inputs(dataclass_replace_plant(w), 6)
    res = run_core(mdr, w, inp)
    for b in range(w.batch):
        for h in range(w.heads):
            check_head_routing(w, inp, res, b, h)
            ref = attention_rows(w, inp, res["sel"][b, h], b, h, None, dense=True)
            assert np.abs(res["out"][b, h] - ref).max() <= TOL[w.dtype]


def dataclass_replace_plant(w):
    import dataclasses

    return dataclasses.replace(w, plant="none")


def test_mixer_forward(gpu_lib):
    """[batch, seq, width] -> attention delta on the tiny workload (fp32, 1e-5)."""
    mdr = gpu_lib
    w = synth.workload("tiny")
    inp = synth.make_mixer_inputs(w, 0)
    cfg = cfg_of(mdr, w)
    t = {n: dev(inp[n], torch.float32) for n in ("x", "wq", "wk", "wv", "wo", "codebook")}
    delta = torch.empty_like(t["x"])
    rt = mdr.routing_buffers(cfg)
    mdr.mdr_mixer_forward(cfg, t["x"], t["wq"], t["wk"], t["wv"], t["wo"], t["codebook"], None, delta, rt,
                          mdr.workspace(cfg))
    torch.cuda.synchronize()
    sel = host(rt["sel"])
    ref, routes = oracle.mixer_forward(inp["x"], inp["wq"], inp["wk"], inp["wv"], inp["wo"], inp["codebook"], None,
                                       w, sel_override=sel)
    for h in range(w.heads):
        compare_selection(routes[0][h], sel[0, h])
    err = float(np.abs(host(delta) - ref).max())
    print(f"mixer max abs err {err:.3g}")
    assert err <= TOL["f32"]


FULL = {
    "sweep": dict(),
    "long": dict(),
    "skew": dict(),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled(gpu_lib, name):
    """The largest workloads at full size in the benchmark's launch configuration, checked on sampled
    tokens (routing with the near-tie rule, overflow of every head, attention rows with the GPU's
    selection)."""
    mdr = gpu_lib
    w = synth.workload(name, **FULL[name])
    inp = synth.make_core_inputs(w, 0)
    res = run_core(mdr, w, inp)
    rng = np.random.default_rng(7)
    heads = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    near_a = {}
    for b, h in heads:
        near_a[b, h] = compare_addresses(w, inp, res["addr"][b, h], b, h)
        lists = oracle.posting_lists(res["addr"][b, h], w.addresses, w.local)  # on the GPU's addresses
        assert res["overflow"][b, h] == oracle.posting_overflow(lists, w.capacity)
    picks = [heads[i] for i in rng.choice(len(heads), size=min(4, len(heads)), replace=False)]
    err = 0.0
    near = 0
    for b, h in picks:
        toks = np.unique(np.concatenate([rng.choice(w.seq, 96, replace=False), [0, w.block - 1, w.seq - 1]]))
        _, ns = check_head_routing(w, inp, res, b, h, tokens=toks)
        near += ns
        ref = attention_rows(w, inp, res["sel"][b, h][toks], b, h, toks)
        err = max(err, float(np.abs(res["out"][b, h][toks] - ref).max()))
    print(f"{name} full size: overflow total {int(res['overflow'].sum())}, address near-ties "
          f"{sum(near_a.values())}, sampled selection near-ties {near}, "
          f"R_eff {float((res['sel'] >= 0).sum(-1).mean()):.3f}, sampled max abs err {err:.3g}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("name,over", [
    ("long", dict(heads=2, seq=4096, remote=2)),                  # bf16, D 128, blocks of 128
    ("skew", dict(batch=1, heads=4, seq=4096, remote=2)),         # bf16, D 128, blocks of 64
    ("long", dict(heads=1, seq=2048, block=64, remote=1, dtype="f32")),  # fp32, D 128, blocks of 64, R = 1
    ("recall", dict(batch=2, seq=8192, remote=2)),                # the longest sequence the scan takes
])
def test_short_sequence_remote_scan(gpu_lib, name, over):
    """Up to 8,192 tokens with R <= 2 the remote kernel finds each block's pairs in the selection itself
    (no binning kernel): head dims, block sizes and dtypes beyond the sweep's, against the oracle."""
    mdr = gpu_lib
    w = small(name, **over)
    inp = synth.make_core_inputs(dataclass_replace_plant(w) if w.plant == "recall" else w, 10)
    res = run_core(mdr, w, inp)
    near = 0
    err = 0.0
    for b in range(w.batch):
        for h in range(w.heads):
            near += check_head_routing(w, inp, res, b, h)[1]
            ref = attention_rows(w, inp, res["sel"][b, h], b, h, None, dense=w.seq <= 4096)
            err = max(err, float(np.abs(res["out"][b, h] - ref).max()))
    print(f"{name} {over}: selection near-ties {near}, max abs err {err:.3g}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("name,over", [("sweep", dict(probes=3)), ("long", dict(remote=3)),
                                       ("skew", dict(probes=5, remote=7)), ("recall", dict(codes=6, probes=11)),
                                       ("tiny", dict(subspaces=1, codes=8, probes=3))])
def test_generic_probe_kernel(gpu_lib, name, over):
    """Routing sizes outside the compile-time specialisations run the generic probe kernel."""
    mdr = gpu_lib
    w = small(name, **over)
    inp = synth.make_core_inputs(dataclass_replace_plant(w) if w.plant == "recall" else w, 8)
    res = run_core(mdr, w, inp)
    near = 0
    for b in range(w.batch):
        for h in range(w.heads):
            near += check_head_routing(w, inp, res, b, h)[1]
            ref = attention_rows(w, inp, res["sel"][b, h], b, h, None, dense=w.seq <= 4096)
            assert np.abs(res["out"][b, h] - ref).max() <= TOL[w.dtype]
    print(f"{name} {over}: selection near-ties {near}")


def hot_block_selection(w, seed):
    """Every eligible token selects block 0 in slot 0; each other slot holds a seeded random eligible
    block (blocks 1 .. j - L, none twice for one token, as the router selects) or nothing."""
    rng = np.random.default_rng(seed)
    B, H, S, R = w.batch, w.heads, w.seq, w.remote
    j = np.arange(S) // w.block
    sel = np.full((B, H, S, R), -1, dtype=np.int32)
    sel[:, :, j >= w.local, 0] = 0
    for r in range(1, R):
        x = rng.integers(1, np.maximum(j - w.local + 1, 2), size=(B, H, S))
        keep = (j - w.local >= 1) & (rng.random((B, H, S)) < 0.7) & np.all(sel[..., :r] != x[..., None], axis=-1)
        sel[..., r] = np.where(keep, x, -1)
    return sel


@pytest.mark.parametrize("name", ["sweep", "long"])
def test_stage_attend_hot_block(gpu_lib, name):
    """A block that every eligible token selects: its pair list spans many work items of the remote
    kernel, while the other slots spread over random blocks with short lists."""
    mdr = gpu_lib
    w = small(name)
    inp = synth.make_core_inputs(w, 7)
    sel = hot_block_selection(w, 7)
    cfg = cfg_of(mdr, w)
    dt = io_dtype(w)
    q, k, v = (dev(inp[n], dt) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    mdr.mdr_stage_attend(cfg, q, k, v, dev(sel), out, mdr.workspace(cfg))
    torch.cuda.synchronize()
    out = host(out)
    err = 0.0
    for b in range(w.batch):
        for h in range(w.heads):
            ref = attention_rows(w, inp, sel[b, h], b, h, None, dense=w.seq <= 4096)
            err = max(err, float(np.abs(out[b, h] - ref).max()))
    print(f"{name}: block 0 pairs per head {int((sel[0, 0] == 0).sum())}, max abs err {err:.3g}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("over", [dict(seq=16384), dict(seq=12288, remote=3)])
def test_stage_attend_binned_hot_block(gpu_lib, over):
    """Past 8,192 tokens the forward bins its pairs, each taking the next slot of its block by an LDS
    atomic, so the order inside a list varies between calls.  A hot block's list then spans many work
    items; R = 3 takes the path that stages the entries in LDS.  Sampled tokens (every token of the
    first and last query blocks, and a seeded spread) against the oracle, and two calls bit for bit
    (each pair's partial depends on its own query alone)."""
    mdr = gpu_lib
    w = synth.workload("sweep", heads=2, **over)
    inp = synth.make_core_inputs(w, 9)
    sel = hot_block_selection(w, 9)
    cfg = cfg_of(mdr, w)
    dt = io_dtype(w)
    q, k, v = (dev(inp[n], dt) for n in ("q", "k", "v"))
    ws = mdr.workspace(cfg)
    outs = []
    for _ in range(2):
        out = torch.empty_like(q)
        mdr.mdr_stage_attend(cfg, q, k, v, dev(sel), out, ws)
        torch.cuda.synchronize()
        outs.append(host(out))
    assert np.array_equal(outs[0], outs[1])
    rng = np.random.default_rng(9)
    toks = np.unique(np.concatenate([np.arange(w.block), np.arange(w.seq - w.block, w.seq),
                                     rng.choice(w.seq, 384, replace=False)]))
    err = 0.0
    for b in range(w.batch):
        for h in range(w.heads):
            ref = attention_rows(w, inp, sel[b, h][toks], b, h, toks)
            err = max(err, float(np.abs(outs[0][b, h, toks] - ref).max()))
    print(f"{over}: block 0 pairs per head {int((sel[0, 0] == 0).sum())}, sampled max abs err {err:.3g}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("marked", [None, 2, 3])
def test_profiled_form_gives_the_same_results(gpu_lib, marked):
    """mdr_routed_attention_profiled with every event, or with events around one kernel only (null
    entries elsewhere), runs the same kernels: results bit for bit those of the plain call, and
    every recorded interval is non-negative."""
    mdr = gpu_lib
    w = small("recall", batch=2)
    inp = synth.make_core_inputs(w, 8)
    plain = run_core(mdr, w, inp)
    cfg = cfg_of(mdr, w)
    q, k, v = (dev(inp[n], io_dtype(w)) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    rt = mdr.routing_buffers(cfg)
    from bench import HipEvents

    hip = HipEvents()
    nk = mdr.MDR_CORE_KERNELS
    handles = hip.create(nk + 1)
    events = list(handles) if marked is None else [
        handles[i] if i in (marked, marked + 1) else None for i in range(nk + 1)]
    mdr.mdr_routed_attention_profiled(cfg, q, k, v, dev(inp["codebook"], torch.float32), None, None, out, events,
                                      rt, mdr.workspace(cfg))
    torch.cuda.synchronize()
    pairs = [(i, i + 1) for i in range(nk)] if marked is None else [(marked, marked + 1)]
    assert all(hip.elapsed_ms(handles[a], handles[b]) >= 0 for a, b in pairs)
    hip.destroy(handles)
    assert np.array_equal(host(out), plain["out"])
    for n, t in rt.items():
        assert np.array_equal(host(t), plain[n]), n


@pytest.mark.parametrize("case", ["routing_limits", "block_limit"])
def test_size_limits(gpu_lib, case):
    """The largest sizes the library accepts.  routing_limits: 4 subspaces of 8 codes (4096
    addresses, the address limit), 16 probes and 16 remote blocks (both limits), through the
    generic probe kernel, checked on every token.  block_limit: 8192 blocks of 32 tokens (262144
    tokens, the block limit), checked on sampled tokens."""
    mdr = gpu_lib
    if case == "routing_limits":
        w = synth.workload("tiny", seq=16384, subspaces=4, codes=8, capacity=2, probes=16, remote=16, local=1)
        toks = None
    else:
        w = synth.workload("tiny", seq=8192 * 32, capacity=4, probes=2, remote=2)
        rng = np.random.default_rng(11)
        toks = np.unique(np.concatenate([rng.choice(w.seq, 64, replace=False), [0, w.seq - 1]]))
    assert mdr.mdr_check_config(cfg_of(mdr, w)) == 0
    inp = synth.make_core_inputs(w, 4)
    res = run_core(mdr, w, inp)
    _, near = check_head_routing(w, inp, res, 0, 0, tokens=toks)
    rows = np.arange(w.seq) if toks is None else toks
    ref = attention_rows(w, inp, res["sel"][0, 0][rows], 0, 0, toks)
    err = float(np.abs(res["out"][0, 0][rows] - ref).max())
    print(f"{case}: {w.nblocks} blocks, {w.addresses} addresses, P{w.probes} R{w.remote}, "
          f"selection near-ties {near}, max abs err {err:.3g}")
    assert err <= TOL[w.dtype]
