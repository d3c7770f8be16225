"""Parity of the streaming decode path (ring-buffer posting lists, mdr_decode_*)
with the CPU oracle on the GPU.

A decoded token must get the routing and output the oracle gives that token
in the full sequence (the ring buffers hold exactly the prefill views), so the
oracle of the prefill path is the reference: routing bit-exact wherever the
oracle's margin exceeds 1e-4, attention within 1e-5 (fp32) / 2e-2 (bf16).
The K/V cache rows after the current position hold NaN until their token is
appended, so any read of the future would poison the outputs.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import (NEAR, TOL, cfg_of, compare_addresses, compare_selection, dev, host, integer_inputs, io_dtype,
                        run_core, small)

pytestmark = pytest.mark.gpu


def decode_run(mdr, w, inp, n0, chunk, force=None):
    """Prime on the first n0 tokens, then decode the rest `chunk` tokens at a time (never across a
    block boundary).  Returns host arrays out [B,H,S-n0,D], sel [B,H,S-n0,R] and the state views."""
    cfg = cfg_of(mdr, w)
    dt = io_dtype(w)
    B, H, S, D, R, blk = w.batch, w.heads, w.seq, w.head_dim, w.remote, w.block
    q, k, v = (dev(inp[n], dt) for n in ("q", "k", "v"))
    kc = torch.full_like(k, float("nan"))
    vc = torch.full_like(v, float("nan"))
    kc[:, :, :n0] = k[:, :, :n0]
    vc[:, :, :n0] = v[:, :, :n0]
    cb = dev(inp["codebook"], torch.float32)
    bias = None if inp["bias"] is None else dev(inp["bias"], torch.float32)
    fd = None if force is None else dev(force)
    state = mdr.decode_state(cfg)
    mdr.mdr_decode_prime(cfg, kc, cb, bias, n0, state)
    outs, sels = [], []
    pos = n0
    while pos < S:
        n = min(chunk, blk - pos % blk, S - pos)
        kc[:, :, pos:pos + n] = k[:, :, pos:pos + n]
        vc[:, :, pos:pos + n] = v[:, :, pos:pos + n]
        out = torch.empty(B, H, n, D, dtype=dt, device="cuda")
        sel = torch.empty(B, H, n, R, dtype=torch.int32, device="cuda")
        f = None if fd is None else fd[:, :, pos:pos + n].contiguous()
        mdr.mdr_decode_step(cfg, q[:, :, pos:pos + n].contiguous(), kc, vc, cb, bias, f, pos, out, sel, state)
        outs.append(out)
        sels.append(sel)
        pos += n
    torch.cuda.synchronize()
    view = {n: host(t) for n, t in mdr.mdr_decode_state_view(cfg, state).items()}
    return host(torch.cat(outs, dim=2)), host(torch.cat(sels, dim=2)), view


def compare_addresses_prefix(w, inp, addr_g, b, h):
    """compare_addresses on the first len(addr_g) blocks (those the decode state has filed)."""
    ks = oracle.block_summaries(inp["k"][b, h], w.block)
    bias = None if inp["bias"] is None else inp["bias"][h]
    _, own, _ = oracle.block_addresses(ks, inp["codebook"][h], bias)
    full = own.copy()
    full[:len(addr_g)] = addr_g
    return compare_addresses(w, inp, full, b, h)


def check_against_oracle(w, inp, n0, out, sel, view, force=None):
    toks = np.arange(n0, w.seq)
    near = 0
    err = 0.0
    A = w.codes ** w.subspaces
    last_j = (w.seq - 1) // w.block
    for b in range(w.batch):
        for h in range(w.heads):
            bias = None if inp["bias"] is None else inp["bias"][h]
            f = None if force is None else force[b, h]
            filed = max(0, last_j - w.local + 1)
            # the decode state's addresses (near-ties allowed), then the oracle routed on them
            addr_g = np.asarray(view["addr"][b, h][:filed])
            na = compare_addresses_prefix(w, inp, addr_g, b, h)
            ad = None
            if na:
                ad = np.zeros(w.nblocks, dtype=np.int64)
                ad[:filed] = addr_g
                ks = oracle.block_summaries(inp["k"][b, h], w.block)
                _, own, _ = oracle.block_addresses(ks, inp["codebook"][h], bias)
                ad[filed:] = own[filed:]  # blocks never filed: their addresses do not matter
            r = oracle.route_head(inp["q"][b, h], inp["k"][b, h], inp["codebook"][h], bias, w, f, tokens=toks,
                                  addr=ad)
            # the rings hold the prefill views of the last query block
            assert view["filed"][b, h] == filed
            assert view["overflow"][b, h] == oracle.posting_overflow(r["lists"], w.capacity)
            for a in range(A):
                n = int(view["ring_n"][b, h, a])
                assert n == len(r["lists"][a]), (b, h, a)
                ring = [int(view["ring"][b, h, a, (n - 1 - e) % w.capacity]) for e in range(min(n, w.capacity))]
                assert ring == oracle.posting_view(r["lists"], a, last_j, w.local, w.capacity), (b, h, a)
            near += compare_selection(r, sel[b, h], w=w, inp=inp, b=b, h=h, force=f)
            ref = oracle.attention_packed(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], sel[b, h], w.block,
                                          w.local, tokens=toks)
            err = max(err, float(np.abs(out[b, h] - ref).max()))
    assert np.isfinite(out).all()
    assert err <= TOL[w.dtype], err
    return near, err


@pytest.mark.parametrize("name,n0,chunk", [
    ("tiny", 100, 1),       # fp32, D32 block 32, 16 addresses
    ("tiny_cap1", 100, 5),  # the same with capacity 1: every repeated address evicts
    ("recall", 1000, 7),    # fp32, P16, M5
    ("sweep", 3000, 1),     # bf16, balanced addresses
    ("skew", 15900, 16),    # bf16, D128, zipf-biased codes at 16K: hot rings overflow
    ("long", 5000, 64),     # bf16, D128 block 128, R4
    ("sweep_full", 32704, 1),  # the benchmark's decode: 32K context, 8 heads, one token per call
])
def test_decode_matches_oracle(gpu_lib, name, n0, chunk):
    mdr = gpu_lib
    over = {"tiny_cap1": dict(capacity=1), "recall": dict(batch=2), "sweep": dict(seq=4096),
            "skew": dict(batch=1, heads=2, seq=16384), "long": dict(heads=1, seq=8192),
            "sweep_full": dict(seq=32768)}.get(name, {})
    w = small(name.split("_")[0], **over)
    inp = synth.make_core_inputs(w, 0)
    out, sel, view = decode_run(mdr, w, inp, n0, chunk)
    near, err = check_against_oracle(w, inp, n0, out, sel, view)
    if name in ("tiny_cap1", "skew"):
        assert view["overflow"].sum() > 0
    print(f"{name}: decoded {w.seq - n0} tokens, selection near-ties {near}, max abs err {err:.3g}, "
          f"overflow {view['overflow'].sum()}")


@pytest.mark.parametrize("name,n0,chunk,cap", [("tiny", 100, 1, 1), ("recall", 1000, 7, None), ("sweep", 3000, 1, None)])
def test_decode_integer_scores_exactly(gpu_lib, name, n0, chunk, cap):
    """Integer-valued inputs make every score exact on both sides: each decoded token's selection
    must equal the oracle's, ties included, with no near-tie allowance."""
    mdr = gpu_lib
    over = {"recall": dict(batch=2), "sweep": dict(seq=4096)}.get(name, {})
    if cap is not None:
        over["capacity"] = cap
    w = small(name, **over)
    inp = integer_inputs(w, 4)
    out, sel, view = decode_run(mdr, w, inp, n0, chunk)
    toks = np.arange(n0, w.seq)
    ties = 0
    for b in range(w.batch):
        for h in range(w.heads):
            r = oracle.route_head(inp["q"][b, h], inp["k"][b, h], inp["codebook"][h],
                                  None if inp["bias"] is None else inp["bias"][h], w, tokens=toks)
            assert np.array_equal(sel[b, h], r["sel"]), (b, h)
            assert view["overflow"][b, h] == oracle.posting_overflow(r["lists"], w.capacity)
            ties += int(((r["probe_margin"] <= NEAR) | (r["sel_margin"] <= NEAR)).sum())
    assert np.isfinite(out).all()
    print(f"{name}: decoded {w.seq - n0} tokens, tied rankings {ties}, overflow {view['overflow'].sum()}, all matched")


def test_decode_matches_prefill_kernels(gpu_lib):
    """The decode path and the prefill path agree on the same tokens (GPU against GPU)."""
    mdr = gpu_lib
    w = small("sweep", seq=2048)
    inp = synth.make_core_inputs(w, 1)
    n0 = 1500
    out, sel, _ = decode_run(mdr, w, inp, n0, 5)
    res = run_core(mdr, w, inp)
    diff_rows = 0
    for b in range(w.batch):
        for h in range(w.heads):
            r = oracle.route_head(inp["q"][b, h], inp["k"][b, h], inp["codebook"][h], None, w,
                                  tokens=np.arange(n0, w.seq))
            sure = (r["probe_margin"] > NEAR) & (r["sel_margin"] > NEAR)
            same = np.all(sel[b, h] == res["sel"][b, h, n0:], axis=1)
            assert np.all(same | ~sure)
            diff_rows += int((~same).sum())
            ok = same
            np.testing.assert_allclose(out[b, h][ok], res["out"][b, h, n0:][ok], atol=TOL[w.dtype], rtol=0)
    print(f"decode vs prefill: {diff_rows} rows routed differently (near-ties)")


def test_decode_forced_target(gpu_lib):
    mdr = gpu_lib
    w = small("recall", batch=2)
    inp = synth.make_core_inputs(w, 0)
    force = inp["force"]
    n0 = w.seq - w.block  # decode the last query block, where the planted block is forced
    out, sel, view = decode_run(mdr, w, inp, n0, 1, force=force)
    check_against_oracle(w, inp, n0, out, sel, view, force=force)
    for b in range(w.batch):
        for h in range(w.heads):
            f = force[b, h, n0:]
            hit = np.any(sel[b, h] == f[:, None], axis=1) | (f < 0)
            assert hit.all()


def test_decode_from_an_empty_cache(gpu_lib):
    """Priming on zero tokens: the first L blocks have no eligible remote block at all."""
    mdr = gpu_lib
    w = small("tiny")
    inp = synth.make_core_inputs(w, 3)
    out, sel, view = decode_run(mdr, w, inp, 0, 3)
    check_against_oracle(w, inp, 0, out, sel, view)
    assert np.all(sel[:, :, : w.local * w.block] == -1)


def test_decode_rejects_a_step_across_blocks(gpu_lib):
    mdr = gpu_lib
    w = small("tiny")
    cfg = cfg_of(mdr, w)
    dt = io_dtype(w)
    q = torch.zeros(1, 1, 2, w.head_dim, dtype=dt, device="cuda")
    kc = torch.zeros(1, 1, w.seq, w.head_dim, dtype=dt, device="cuda")
    cb = torch.zeros(1, w.subspaces, w.codes, w.head_dim, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    state = mdr.decode_state(cfg)
    mdr.mdr_decode_prime(cfg, kc, cb, None, w.block - 1, state)
    with pytest.raises(mdr.MdrError) as e:
        mdr.mdr_decode_step(cfg, q, kc, kc, cb, None, None, w.block - 1, out, None, state)
    assert e.value.status == mdr.MDR_ERR_INVALID_ARG
