"""The stateless mixer on the GPU against the oracle, through mdr_mixer_forward: the fused Q/K/V
projection (RoPE, block summaries and addresses in its epilogue; blocks of up to 64 tokens and a
width divisible by 8) and the unfused path (k_gemm, k_rope, the address kernel) for the rest.

Q, K, V are held in the io dtype between the projection and the core, so the oracle rounds them the
same way (oracle.mixer_forward, io_dtype).  Checks: block summaries (fp32 1e-5 relative; bf16 2e-3
relative: the fused epilogue averages the stored bf16 rows, the oracle the same rounded rows in fp32
from an fp64 product, so only bf16 rounding flips of single elements differ), addresses and
alternates under the near-tie rule, selections under the near-tie rule, and the delta with the GPU's
selection (1e-5 fp32 / 2e-2 bf16).
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import NEAR, TOL, cfg_of, check_head_routing, compare_selection, dev, host, io_dtype

pytestmark = pytest.mark.gpu

BASE = synth.workload("tiny")
CASES = {
    # fused: fp32, D32, block 32, width 64 (the tiny mixer)
    "tiny": dict(),
    # fused: bf16, D64, block 64, 2x16 codes
    "bf16_d64": dict(batch=1, heads=4, seq=2048, head_dim=64, block=64, width=256, subspaces=2, codes=16,
                     capacity=4, probes=4, dtype="bf16"),
    # fused: block 32 with seq % 64 == 32, so one 64-row tile holds the last block of one sequence and
    # the first block of the next
    "straddle": dict(batch=2, heads=2, seq=1056, head_dim=32, block=32, width=96),
    # fused + redirect policy: bf16, D128, 3x8 codes, capacity 1 and a skewing code bias (lists
    # overflow), alternates in the epilogue
    "redirect": dict(batch=1, heads=2, seq=2048, head_dim=128, block=64, width=128, subspaces=3, codes=8,
                     capacity=1, probes=6, remote=4, dtype="bf16", zipf_kappa=1.0),
    # fused bf16 with width 96: the projection's contraction (96) is not a whole number of 64-wide
    # steps, so it takes the register-staged loop; the output projection (64) takes the direct loop
    "bf16_w96": dict(batch=1, heads=2, seq=1024, head_dim=32, block=32, width=96, dtype="bf16"),
    # fused, one sequence of 1056 tokens: the last 64-row tile holds 32 rows (rows past the end read
    # the last row and are never stored)
    "row_tail": dict(batch=1, heads=2, seq=1056, head_dim=32, block=32, width=96),
    # unfused: block 128
    "block128": dict(batch=1, heads=2, seq=1024, head_dim=128, block=128, width=128, codes=8, capacity=4,
                     probes=4),
    # unfused: width not a multiple of 8
    "width60": dict(batch=1, heads=2, seq=512, head_dim=32, block=32, width=60),
}


@pytest.mark.parametrize("name", list(CASES))
def test_mixer_matches_oracle(gpu_lib, name):
    mdr = gpu_lib
    w = dataclasses.replace(BASE, **CASES[name])
    policy = "redirect" if name == "redirect" else "drop"
    inp = synth.make_mixer_inputs(w, 0)
    cfg = cfg_of(mdr, w, policy)
    dt = io_dtype(w)
    t = {n: dev(inp[n], dt) for n in ("x", "wq", "wk", "wv", "wo")}
    cb = dev(inp["codebook"], torch.float32)
    bias = synth.zipf_code_bias(w.heads, w.subspaces, w.codes, w.zipf_kappa) if w.zipf_kappa else None
    delta = torch.empty_like(t["x"])
    rt = mdr.routing_buffers(cfg)
    mdr.mdr_mixer_forward(cfg, t["x"], t["wq"], t["wk"], t["wv"], t["wo"], cb,
                          None if bias is None else dev(bias), delta, rt, mdr.workspace(cfg))
    torch.cuda.synchronize()
    res = {n: host(v) for n, v in rt.items()}
    ref, routes = oracle.mixer_forward(inp["x"], inp["wq"], inp["wk"], inp["wv"], inp["wo"], inp["codebook"], bias,
                                       w, sel_override=res["sel"], io_dtype=w.dtype, policy=policy)
    near_a = near_s = 0
    ktol = 1e-5 if w.dtype == "f32" else 2e-3
    q, k, _ = oracle.mixer_qkv(inp["x"], inp["wq"], inp["wk"], inp["wv"], w)
    if w.dtype == "bf16":
        q, k = oracle.round_to_bf16(q), oracle.round_to_bf16(k)
    heads_inp = {"q": q.astype(np.float32), "k": k.astype(np.float32), "codebook": inp["codebook"], "bias": bias}
    for b in range(w.batch):
        for h in range(w.heads):
            r = routes[b][h]
            scale = max(1.0, float(np.abs(r["ksum"]).max()))
            np.testing.assert_allclose(res["ksum"][b, h], r["ksum"], rtol=0, atol=ktol * scale)
            na, ns = check_head_routing(w, heads_inp, res, b, h, policy=policy)
            near_a += na
            near_s += ns
    err = float(np.abs(host(delta) - ref).max())
    print(f"{name}: address near-ties {near_a}, selection near-ties {near_s}, max abs err {err:.3g}, "
          f"overflow {int(res['overflow'].sum())}")
    assert err <= TOL[w.dtype]
    if name == "redirect":
        assert int(res["overflow"].sum()) >= 0 and int(res["redir_off"][..., -1].sum()) > 0


def test_mixer_large_tiles(gpu_lib):
    """16384 rows: the output projection takes its 128-row tiles.  Summaries and addresses of every
    block against the oracle's projections, and the delta on sampled tokens (gathered attention with
    the GPU's selection, then the output projection)."""
    mdr = gpu_lib
    w = dataclasses.replace(BASE, batch=1, heads=2, seq=16384, head_dim=64, block=64, width=256, subspaces=2,
                            codes=16, capacity=4, probes=4, dtype="bf16")
    inp = synth.make_mixer_inputs(w, 1)
    cfg = cfg_of(mdr, w)
    t = {n: dev(inp[n], torch.bfloat16) for n in ("x", "wq", "wk", "wv", "wo")}
    cb = dev(inp["codebook"], torch.float32)
    delta = torch.empty_like(t["x"])
    rt = mdr.routing_buffers(cfg)
    mdr.mdr_mixer_forward(cfg, t["x"], t["wq"], t["wk"], t["wv"], t["wo"], cb, None, delta, rt, mdr.workspace(cfg))
    torch.cuda.synchronize()
    res = {n: host(v) for n, v in rt.items()}
    q, k, v = (oracle.round_to_bf16(a) for a in oracle.mixer_qkv(inp["x"], inp["wq"], inp["wk"], inp["wv"], w))
    rng = np.random.default_rng(3)
    toks = np.sort(rng.choice(w.seq, size=64, replace=False))
    o = np.zeros((len(toks), w.heads * w.head_dim))
    near = 0
    for h in range(w.heads):
        ks = oracle.block_summaries(k[0, h].astype(np.float32), w.block)
        scale = max(1.0, float(np.abs(ks).max()))
        np.testing.assert_allclose(res["ksum"][0, h], ks, rtol=0, atol=2e-3 * scale)
        _, addr, margin = oracle.block_addresses(ks, inp["codebook"][h], None)
        sure = margin.min(axis=1) > NEAR
        near += int((~sure).sum())
        assert np.array_equal(res["addr"][0, h][sure], addr[sure]), h
        o[:, h * w.head_dim:(h + 1) * w.head_dim] = oracle.attention_packed(
            q[0, h], k[0, h], v[0, h], res["sel"][0, h][toks], w.block, w.local, tokens=toks)
    ref = o @ inp["wo"].astype(np.float64)
    err = float(np.abs(host(delta)[0, toks] - ref).max())
    print(f"large tiles: address near-ties {near}, sampled delta max abs err {err:.3g}")
    assert err <= TOL["bf16"]


def test_mixer_full_size_sampled(gpu_lib):
    """The benchmark's mixer at full size in its launch configuration (B1 S32768 W512, 8 heads of 64,
    bf16): summaries and addresses of every block against the oracle's projections, routing of sampled
    tokens of every head under the near-tie rule (on the GPU's addresses where a head has an address
    near-tie), and the delta on those tokens (gathered attention with the GPU's selection, then the
    output projection)."""
    mdr = gpu_lib
    w = dataclasses.replace(synth.workload("sweep", seq=32768), width=512)
    inp = synth.make_mixer_inputs(w, 0)
    cfg = cfg_of(mdr, w)
    t = {n: dev(inp[n], torch.bfloat16) for n in ("x", "wq", "wk", "wv", "wo")}
    cb = dev(inp["codebook"], torch.float32)
    delta = torch.empty_like(t["x"])
    rt = mdr.routing_buffers(cfg)
    mdr.mdr_mixer_forward(cfg, t["x"], t["wq"], t["wk"], t["wv"], t["wo"], cb, None, delta, rt, mdr.workspace(cfg))
    torch.cuda.synchronize()
    res = {n: host(v) for n, v in rt.items()}
    q, k, v = (oracle.round_to_bf16(a) for a in oracle.mixer_qkv(inp["x"], inp["wq"], inp["wk"], inp["wv"], w))
    heads_inp = {"q": q.astype(np.float32), "k": k.astype(np.float32), "codebook": inp["codebook"], "bias": None}
    rng = np.random.default_rng(11)
    toks = np.unique(np.concatenate([rng.choice(w.seq, size=96, replace=False), [0, w.block - 1, w.seq - 1]]))
    o = np.zeros((len(toks), w.heads * w.head_dim))
    near_a = near_s = 0
    for h in range(w.heads):
        ks = oracle.block_summaries(k[0, h].astype(np.float32), w.block)
        scale = max(1.0, float(np.abs(ks).max()))
        np.testing.assert_allclose(res["ksum"][0, h], ks, rtol=0, atol=2e-3 * scale)
        na, ns = check_head_routing(w, heads_inp, res, 0, h, tokens=toks)
        near_a += na
        near_s += ns
        o[:, h * w.head_dim:(h + 1) * w.head_dim] = oracle.attention_packed(
            q[0, h], k[0, h], v[0, h], res["sel"][0, h][toks], w.block, w.local, tokens=toks)
    ref = o @ inp["wo"].astype(np.float64)
    err = float(np.abs(host(delta)[0, toks] - ref).max())
    print(f"mixer full size: address near-ties {near_a}, sampled selection near-ties {near_s}, "
          f"sampled delta max abs err {err:.3g}")
    assert err <= TOL["bf16"]
