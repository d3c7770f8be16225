"""The kernels' index arithmetic checked on the CPU (mdr_selfcheck_indices): the functions the kernels
use to map work-groups to work and to address their buffers, run over every launch index of each
configuration, must stay inside the workspace regions -- for the five workload families at full size,
the size limits, and seeded random configurations."""

import numpy as np
import pytest

import synth
from tests.test_abi import _ensure_built


@pytest.fixture(scope="module")
def mdr():
    _ensure_built()
    import learned_product_hash_amd as m

    return m


def _cfg(mdr, w, **over):
    f = dict(batch=w.batch, seq=w.seq, heads=w.heads, head_dim=w.head_dim, width=w.width, block=w.block,
             subspaces=w.subspaces, codes=w.codes, capacity=w.capacity, probes=w.probes, max_cand=w.max_cand,
             remote=w.remote, local=w.local, dtype=w.dtype, rope_base=w.rope_base)
    f.update(over)
    return mdr.config(**f)


@pytest.mark.parametrize("name", ["tiny", "recall", "sweep", "long", "skew"])
def test_full_size_workloads(mdr, name):
    w = synth.workload(name)
    for policy in ("drop", "redirect"):
        assert mdr.mdr_selfcheck_indices(_cfg(mdr, w, overflow_policy=policy)) == ""


@pytest.mark.parametrize("over", [
    dict(seq=8192 * 32, block=32, capacity=4, probes=2, remote=2),          # the block limit
    dict(seq=16384, subspaces=4, codes=8, probes=16, remote=16, local=1),   # address, probe, remote limits
    dict(seq=64, local=2),                                                   # nothing eligible
    dict(seq=128 * 3, block=128, head_dim=128, local=1, remote=16, batch=3, heads=5),
])
def test_limits_and_edges(mdr, over):
    w = synth.workload("tiny")
    assert mdr.mdr_selfcheck_indices(_cfg(mdr, w, **over)) == ""


def test_random_configurations(mdr):
    rng = np.random.default_rng(0)
    n = 0
    while n < 60:
        blk = int(rng.choice([32, 64, 128]))
        f = dict(batch=int(rng.integers(1, 5)), heads=int(rng.integers(1, 17)), seq=blk * int(rng.integers(1, 300)),
                 head_dim=int(rng.choice([32, 64, 128])), block=blk, subspaces=int(rng.integers(1, 4)),
                 codes=int(rng.integers(2, 9)), capacity=int(rng.integers(1, 9)), probes=1,
                 remote=int(rng.integers(0, 17)), local=int(rng.integers(1, 4)), dtype=str(rng.choice(["f32", "bf16"])))
        f["probes"] = int(rng.integers(1, min(16, f["codes"] ** f["subspaces"]) + 1))
        cfg = mdr.config(**f)
        if mdr.mdr_check_config(cfg) != 0:
            continue
        assert mdr.mdr_selfcheck_indices(cfg) == "", f
        n += 1
