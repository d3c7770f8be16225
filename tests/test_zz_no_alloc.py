"""The entry point that allocates nothing (mdr_routed_attention_noalloc, for callers that cannot allocate:
graph capture, serving loops, harnesses that forbid it) against mdr_routed_attention with a caller
workspace: the same kernels, so every output must be bit-identical.  Two calls in a row on the shared
static scratch, the second on a smaller input (its leftovers from the first call must not leak), then a
configuration beyond the scratch, which is rejected before anything runs."""

import numpy as np
import pytest
import torch

import synth
from tests._gpu import cfg_of, dev, host, io_dtype

pytestmark = pytest.mark.gpu


def _both(mdr, w, seed, force=False):
    inp = synth.make_core_inputs(w, seed)
    cfg = cfg_of(mdr, w)
    dt = io_dtype(w)
    q, k, v = (dev(inp[n], dt) for n in ("q", "k", "v"))
    cb = dev(inp["codebook"], torch.float32)
    bias = None if inp["bias"] is None else dev(inp["bias"], torch.float32)
    f = dev(inp["force"]) if force and inp.get("force") is not None else None
    outs = []
    for noalloc in (False, True):
        out = torch.empty_like(q)
        rt = mdr.routing_buffers(cfg)
        if noalloc:
            mdr.mdr_routed_attention_noalloc(cfg, q, k, v, cb, bias, f, out, rt)
        else:
            mdr.mdr_routed_attention(cfg, q, k, v, cb, bias, f, out, rt, mdr.workspace(cfg))
        torch.cuda.synchronize()
        res = {n: host(t) for n, t in rt.items()}
        res["out"] = host(out)
        outs.append(res)
    return outs


def test_noalloc_equals_the_workspace_entry_point(gpu_lib):
    mdr = gpu_lib
    cases = [(synth.workload("skew", batch=1, heads=4, seq=4096), 1, False),   # the larger call first
             (synth.workload("sweep", seq=4096, heads=2), 2, False),           # then a smaller one
             (synth.workload("recall", batch=2), 3, True)]                     # fp32, forced targets
    for w, seed, force in cases:
        assert mdr.mdr_workspace_size(cfg_of(mdr, w)) <= mdr.MDR_NOALLOC_SCRATCH_BYTES
        a, b = _both(mdr, w, seed, force)
        for n in a:
            assert np.array_equal(a[n], b[n]), (w.name, n)
        print(f"{w.name} S{w.seq} H{w.heads}: noalloc bit-identical, R_eff {float((b['sel'] >= 0).sum(-1).mean()):.3f}")


def test_noalloc_rejects_a_workspace_beyond_its_scratch(gpu_lib):
    mdr = gpu_lib
    w = synth.workload("sweep")  # 32K tokens, 8 heads: more workspace than the scratch holds
    cfg = cfg_of(mdr, w)
    assert mdr.mdr_workspace_size(cfg) > mdr.MDR_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    cb = torch.zeros(8, 2, 16, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(mdr.MdrError) as e:
        mdr.mdr_routed_attention_noalloc(cfg, x, x, x, cb, None, None, x)
    assert e.value.status == 3  # MDR_ERR_WORKSPACE
