"""Parity of the attention backward (mdr_stage_attend_lse + mdr_stage_attend_backward) with the
CPU oracle on the GPU, the selection held fixed.

The selection comes either from the library's own routing (the realistic distribution of pairs
over remote blocks) or from a seeded random draw with empty, repeated and ineligible entries (the
kernel must ignore the same entries the forward ignores).  Tolerances, as a fraction of the largest
magnitude of each gradient in the (b, h) compared:
  fp32  2e-5: fp32 products and sums throughout, the exponent from the hardware exp2 and the
        stored fp32 normaliser (a few fp32 ulps per term over at most a few thousand terms); the
        largest error seen is about 4e-6.
  bf16  2e-2: the MFMA operands P and dS are rounded to bf16 (2^-9 relative), as are the stored
        output (used in D = dO . O), each remote block's dQ share and the final gradients.
The normaliser lse (fp32 arithmetic for either io dtype) must match the oracle's within 1e-5
absolute in log2 units (about 1e-6 seen).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import cfg_of, dev, host, io_dtype, run_core, small

pytestmark = pytest.mark.gpu

GTOL = {"f32": 2e-5, "bf16": 2e-2}
LTOL = {"f32": 1e-5, "bf16": 1e-5}


def clean_selection(sel, block, local):
    """The entries the forward uses (0 <= i <= j - L, first of a repeat); others become -1."""
    S, R = sel.shape
    out = np.full_like(sel, -1)
    for t in range(S):
        hi = t // block - local
        seen = []
        for r in range(R):
            i = int(sel[t, r])
            if 0 <= i <= hi and i not in seen:
                seen.append(i)
                out[t, r] = i
    return out


def random_selection(rng, w):
    """[B,H,S,R] entries in [-2, nb): empty, repeated and ineligible (i > j - L) ones included."""
    B, H, S, R = w.batch, w.heads, w.seq, w.remote
    sel = rng.integers(-2, w.nblocks, size=(B, H, S, R))
    rep = rng.random((B, H, S, R)) < 0.15
    sel[..., 1:] = np.where(rep[..., 1:], sel[..., :1], sel[..., 1:])
    return sel.astype(np.int32)


def run_backward(mdr, w, inp, sel, d_out, repeat=1):
    cfg = cfg_of(mdr, w)
    dt = io_dtype(w)
    q, k, v = (dev(inp[n], dt) for n in ("q", "k", "v"))
    sd = dev(sel)
    g = dev(d_out, dt)
    out = torch.empty_like(q)
    lse = torch.empty(w.batch, w.heads, w.seq, dtype=torch.float32, device="cuda")
    ws = mdr.workspace(cfg)
    mdr.mdr_stage_attend_lse(cfg, q, k, v, sd, out, lse, ws)
    res = []
    for _ in range(repeat):
        dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
        mdr.mdr_stage_attend_backward(cfg, q, k, v, sd, out, lse, g, dq, dk, dv, ws)
        torch.cuda.synchronize()
        res.append({"dq": host(dq), "dk": host(dk), "dv": host(dv)})
    return host(out), host(lse), res


def check(w, inp, sel, d_out, out, lse, grads, heads=None, packed=False):
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0, "lse": 0.0}
    pairs = [(b, h) for b in range(w.batch) for h in range(w.heads)] if heads is None else heads
    for b, h in pairs:
        q, k, v = (inp[n][b, h] for n in ("q", "k", "v"))
        rows = clean_selection(sel[b, h], w.block, w.local)
        lref = oracle.attention_lse2(q, k, rows, w.block, w.local) if not packed else None
        fn = oracle.attention_backward_packed if packed else oracle.attention_backward_dense
        ref = dict(zip(("dq", "dk", "dv"), fn(q, k, v, rows, w.block, w.local, d_out[b, h])))
        if lref is not None:
            e = float(np.abs(lse[b, h] - lref).max())
            worst["lse"] = max(worst["lse"], e)
            assert e <= LTOL[w.dtype], (b, h, e)
        for n in ("dq", "dk", "dv"):
            g = grads[n][b, h]
            assert np.isfinite(g).all(), (n, b, h)
            e = float(np.abs(g - ref[n]).max()) / max(1.0, float(np.abs(ref[n]).max()))
            worst[n] = max(worst[n], e)
            assert e <= GTOL[w.dtype], (n, b, h, e)
    return worst


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),                                  # fp32, D32, block 32
    ("recall", dict(batch=2)),                     # fp32, D64, block 64
    ("sweep", dict(heads=2)),                      # bf16, D64, block 64, 4096 tokens
    ("long", dict(heads=1, seq=4096)),             # bf16, D128, block 128, R4
    ("skew", dict(batch=1, heads=2, seq=4096)),    # bf16, D128, block 64, R8, hot blocks
])
def test_backward_matches_oracle_on_routed_selections(gpu_lib, name, over):
    mdr = gpu_lib
    w = small(name, **over)
    inp = synth.make_core_inputs(w, 0)
    sel = run_core(mdr, w, inp)["sel"]
    d_out = synth.make_grad_inputs(w, 0)
    out, lse, (grads,) = run_backward(mdr, w, inp, sel, d_out)
    worst = check(w, inp, sel, d_out, out, lse, grads)
    print(f"{name}: worst relative errors {worst}")


@pytest.mark.parametrize("name,over", [
    ("tiny", dict(local=1)),
    ("tiny", dict(local=3, remote=5)),
    ("sweep", dict(seq=2048, heads=1, local=1, remote=3)),
    ("long", dict(heads=1, seq=2048, local=3)),
])
def test_backward_random_selection(gpu_lib, name, over):
    """Empty, repeated and ineligible entries count exactly as in the forward."""
    mdr = gpu_lib
    w = small(name, **over)
    inp = synth.make_core_inputs(w, 1)
    sel = random_selection(np.random.default_rng(5), w)
    d_out = synth.make_grad_inputs(w, 1)
    out, lse, (grads,) = run_backward(mdr, w, inp, sel, d_out)
    print(f"{name} {over}: worst relative errors {check(w, inp, sel, d_out, out, lse, grads)}")


def test_backward_every_token_selects_one_block(gpu_lib):
    """Every token selects block 0 (and block 1): those blocks' pair lists hold a pair of nearly every
    token and span many work items."""
    mdr = gpu_lib
    w = small("tiny", seq=8192)  # 256 blocks of 32: about 8,100 pairs for block 0, 64 work items
    inp = synth.make_core_inputs(w, 2)
    sel = np.zeros((1, 1, w.seq, w.remote), dtype=np.int32)
    sel[..., 1] = 1
    d_out = synth.make_grad_inputs(w, 2)
    out, lse, (grads,) = run_backward(mdr, w, inp, sel, d_out)
    print(f"one hot block: worst relative errors {check(w, inp, sel, d_out, out, lse, grads, packed=True)}")


@pytest.mark.parametrize("over", [dict(remote=0), dict(seq=64)])
def test_backward_local_only(gpu_lib, over):
    """No remote block: R = 0, or a sequence of L blocks."""
    mdr = gpu_lib
    w = small("tiny", **over)
    inp = synth.make_core_inputs(w, 3)
    sel = np.full((1, 1, w.seq, w.remote), -1, dtype=np.int32)
    d_out = synth.make_grad_inputs(w, 3)
    out, lse, (grads,) = run_backward(mdr, w, inp, sel, d_out)
    check(w, inp, sel, d_out, out, lse, grads)


def test_backward_is_deterministic(gpu_lib):
    mdr = gpu_lib
    w = small("skew", batch=1, heads=2, seq=4096)
    inp = synth.make_core_inputs(w, 4)
    sel = run_core(mdr, w, inp)["sel"]
    _, _, runs = run_backward(mdr, w, inp, sel, synth.make_grad_inputs(w, 4), repeat=2)
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(runs[0][n], runs[1][n]), n


def test_backward_full_size_heads(gpu_lib):
    """The 32768-token, 8-head bf16 workload in full; two heads checked token by token."""
    mdr = gpu_lib
    w = synth.workload("sweep")
    inp = synth.make_core_inputs(w, 0)
    sel = run_core(mdr, w, inp)["sel"]
    d_out = synth.make_grad_inputs(w, 0)
    out, lse, (grads,) = run_backward(mdr, w, inp, sel, d_out)
    worst = check(w, inp, sel, d_out, out, lse, grads, heads=[(0, 0), (0, 5)], packed=True)
    print(f"full size: worst relative errors {worst}")


def test_backward_profiled_form_gives_the_same_gradients(gpu_lib):
    """The event-recording entry point runs the same kernels: bit-identical results."""
    mdr = gpu_lib
    w = small("tiny")
    inp = synth.make_core_inputs(w, 6)
    sel = run_core(mdr, w, inp)["sel"]
    _, _, (plain,) = run_backward(mdr, w, inp, sel, synth.make_grad_inputs(w, 6))
    cfg = cfg_of(mdr, w)
    q, k, v = (dev(inp[n], io_dtype(w)) for n in ("q", "k", "v"))
    sd, g = dev(sel), dev(synth.make_grad_inputs(w, 6), io_dtype(w))
    out = torch.empty_like(q)
    lse = torch.empty(w.batch, w.heads, w.seq, dtype=torch.float32, device="cuda")
    ws = mdr.workspace(cfg)
    mdr.mdr_stage_attend_lse(cfg, q, k, v, sd, out, lse, ws)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    from bench import HipEvents

    hip = HipEvents()
    handles = hip.create(mdr.MDR_BACKWARD_KERNELS + 1)
    mdr.mdr_stage_attend_backward_profiled(cfg, q, k, v, sd, out, lse, g, dq, dk, dv, handles, ws)
    torch.cuda.synchronize()
    times = [hip.elapsed_ms(handles[i], handles[i + 1]) for i in range(mdr.MDR_BACKWARD_KERNELS)]
    hip.destroy(handles)
    assert all(t >= 0 for t in times)
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.array_equal(host(t), plain[n]), n
