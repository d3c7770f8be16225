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


def run_core(mdr, w, inp, force=None, policy="drop"):
    """mdr_routed_attention with every routing output requested; returns host arrays."""
    cfg = cfg_of(mdr, w, policy)
    dt = io_dtype(w)
    q, k, v = (dev(inp[n], dt) for n in ("q", "k", "v"))
    cb = dev(inp["codebook"], torch.float32)
    bias = None if inp["bias"] is None else dev(inp["bias"], torch.float32)
    f = None if force is None else dev(force)
    out = torch.empty_like(q)
    rt = mdr.routing_buffers(cfg)
    ws = mdr.workspace(cfg)
    mdr.mdr_routed_attention(cfg, q, k, v, cb, bias, f, out, rt, ws)
    torch.cuda.synchronize()
    res = {n: host(t) for n, t in rt.items()}
    res["out"] = host(out)
    return res


def compare_addresses(w, inp, addr_gpu, b, h):
    """GPU addresses vs the oracle's; returns (oracle route pieces, number of near-ties)."""
    ks = oracle.block_summaries(inp["k"][b, h], w.block)
    bias = None if inp["bias"] is None else inp["bias"][h]
    _, addr, margin = oracle.block_addresses(ks, inp["codebook"][h], bias)
    sure = margin.min(axis=1) > NEAR
    assert np.array_equal(addr_gpu[sure], addr[sure]), (b, h)
    return int((~sure).sum())


def compare_selection(route, sel_gpu, rows=None):
    """sel rows vs the oracle route (same token order); returns the number of near-tie tokens."""
    sel_o = route["sel"]
    sure = (route["probe_margin"] > NEAR) & (route["sel_margin"] > NEAR)
    g = sel_gpu if rows is None else sel_gpu[rows]
    bad = np.nonzero(sure & np.any(g != sel_o, axis=1))[0]
    assert len(bad) == 0, f"selection mismatch at rows {bad[:8]}: gpu {g[bad[:4]]} oracle {sel_o[bad[:4]]}"
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
