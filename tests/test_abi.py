"""The C-ABI library on the host (no GPU needed): it loads, exports every function
include/mdr.h declares, and rejects bad arguments before anything is launched."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mdr.h")
LIB = os.path.join(ROOT, "learned_product_hash_amd", "libmdr.so")


def _ensure_built():
    if not os.path.exists(LIB):
        import __graft_entry__

        __graft_entry__.build()


@pytest.fixture(scope="module")
def mdr():
    _ensure_built()
    import learned_product_hash_amd as m

    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mdr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mdr_routed_attention", "mdr_mixer_forward", "mdr_stage_address", "mdr_stage_post",
              "mdr_stage_probe_rerank", "mdr_stage_attend", "mdr_stage_attend_lse", "mdr_stage_attend_backward",
              "mdr_workspace_size", "mdr_check_config"):
        assert n in names


def test_library_exports_every_declared_symbol(mdr):
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert mdr.mdr_abi_version() == 4


def test_binding_has_every_declared_entry_point(mdr):
    """The Python binding is the thin layer over the C ABI: one function of the same name per
    declared entry point."""
    for name in declared_functions():
        assert callable(getattr(mdr, name, None)), name
        assert name in mdr.__all__, name


def _good(**over):
    f = dict(batch=1, seq=4096, heads=8, head_dim=64, block=64, subspaces=2, codes=16, capacity=2, probes=4,
             remote=2, local=2, dtype="bf16")
    f.update(over)
    return f


def test_valid_configs_pass(mdr):
    assert mdr.mdr_check_config(mdr.config(**_good())) == 0
    for w in ("tiny", "recall", "sweep", "long", "skew"):
        import synth

        wl = synth.workload(w)
        c = mdr.config(batch=wl.batch, seq=wl.seq, heads=wl.heads, head_dim=wl.head_dim, width=wl.width,
                       block=wl.block, subspaces=wl.subspaces, codes=wl.codes, capacity=wl.capacity,
                       probes=wl.probes, max_cand=wl.max_cand, remote=wl.remote, local=wl.local,
                       dtype=wl.dtype, rope_base=wl.rope_base)
        assert mdr.mdr_check_config(c) == 0, w
        assert mdr.mdr_workspace_size(c) > 0


@pytest.mark.parametrize("over,status", [
    (dict(seq=4000), 1),            # seq % block != 0
    (dict(batch=0), 1),
    (dict(local=0), 1),
    (dict(capacity=0), 1),
    (dict(probes=0), 1),
    (dict(remote=-1), 1),
    (dict(dtype=7), 1),
    (dict(overflow_policy=2), 1),
    (dict(probes=300, codes=16), 1),  # more probes than addresses (A = 256)
    (dict(head_dim=48), 2),
    (dict(block=16), 2),
    (dict(remote=17), 2),
    (dict(probes=17), 2),
    (dict(subspaces=5, codes=2), 2),
    (dict(codes=128), 2),           # 2 x 128 codes exceed the 64 logits per query
    (dict(subspaces=4, codes=16), 2),  # 65536 addresses
    (dict(seq=64 * 9000), 2),       # more than 8192 blocks
])
def test_invalid_configs_are_rejected_on_the_host(mdr, over, status):
    cfg = mdr.config(**_good(**over))
    assert mdr.mdr_check_config(cfg) == status
    with pytest.raises(mdr.MdrError) as e:
        mdr.mdr_workspace_size(cfg)
    assert e.value.status == status


def test_entry_points_validate_before_launching(mdr):
    """Null pointers, misalignment and short workspaces return a status; no device is touched."""
    lib = mdr.lib
    cfg = mdr.config(**_good())
    need = mdr.mdr_workspace_size(cfg)
    p = 1 << 20  # a fake, 256-byte aligned address: never dereferenced on these paths
    c = ctypes.byref(cfg)
    assert lib.mdr_routed_attention(c, None, p, p, p, None, None, p, None, p, need, None) == 1
    assert lib.mdr_routed_attention(c, p + 2, p, p, p, None, None, p, None, p, need, None) == 1
    assert lib.mdr_routed_attention(c, p, p, p, p, None, None, p, None, p, need - 1, None) == 3
    assert lib.mdr_routed_attention(c, p, p, p, p, None, None, p, None, p + 16, need, None) == 1
    assert lib.mdr_stage_attend(c, p, p, p, p, p, p, need - 1, None) == 3
    assert lib.mdr_stage_attend(c, p, p, p, None, p, p, need, None) == 1
    assert lib.mdr_stage_attend_lse(c, p, p, p, p, p, p, p, need - 1, None) == 3
    assert lib.mdr_stage_attend_lse(c, p, p, p, p, p + 4, p, p, need, None) == 1
    bwd = lib.mdr_stage_attend_backward
    assert bwd(c, p, p, p, p, p, None, p, p, p, p, p, need, None) == 1        # no lse
    assert bwd(c, p, p, p, p, p, p, None, p, p, p, p, need, None) == 1        # no d_out
    assert bwd(c, p, p, p, p, p, p, p, p + 8, p, p, p, need, None) == 1       # misaligned dq
    assert bwd(c, p, p, p, None, p, p, p, p, p, p, p, need, None) == 1        # no selection with R > 0
    assert bwd(c, p, p, p, p, p, p, p, p, p, p, p, need - 1, None) == 3
    assert lib.mdr_stage_post(c, None, None, p, p, None, None, None, p, None) == 1
    assert lib.mdr_stage_address(c, p, p, None, p + 4, p, None, None) == 1
    assert lib.mdr_stage_probe_rerank(c, p, p, None, p, p, p, None, None, None, None, None, None, None, None) == 1
    red = mdr.config(**_good(overflow_policy="redirect"))
    cr = ctypes.byref(red)
    assert mdr.mdr_check_config(red) == 0
    assert lib.mdr_stage_post(cr, p, None, p, p, p, p, p, p, None) == 1        # redirect needs alt
    assert lib.mdr_stage_post(cr, p, p, p, p, None, p, p, p, None) == 1        # and the redirect lists
    assert lib.mdr_stage_probe_rerank(cr, p, p, None, p, p, p, None, p, p, None, p, None, None, None) == 1
    mix = mdr.config(**_good(width=0))
    assert lib.mdr_mixer_forward(ctypes.byref(mix), p, p, p, p, p, p, None, p, None, p, 1 << 40, None) == 1
    assert mdr.mdr_status_string(3) == "MDR_ERR_WORKSPACE"


def test_workspace_grows_with_the_mixer_buffers(mdr):
    core = mdr.mdr_workspace_size(mdr.config(**_good()))
    mixer = mdr.mdr_workspace_size(mdr.config(**_good(width=512, rope_base=10000.0)))
    assert mixer > core


def test_workspace_breakdown_sums_to_the_workspace_size(mdr):
    for over in ({}, dict(width=512, rope_base=10000.0), dict(overflow_policy="redirect"), dict(remote=0)):
        cfg = mdr.config(**_good(**over))
        parts = mdr.workspace_breakdown(cfg)
        assert parts["total"] == mdr.mdr_workspace_size(cfg)
        assert sum(v for k, v in parts.items() if k != "total") == parts["total"]
        assert (parts["mixer"] > 0) == ("width" in over)
        assert all(v % 256 == 0 for v in parts.values())
    with pytest.raises(mdr.MdrError):
        mdr.workspace_breakdown(mdr.config(**_good(seq=4000)))


def test_noalloc_validates_before_touching_the_device(mdr):
    """The entry point without a workspace checks the configuration and its scratch limit on the host:
    a workspace beyond MDR_NOALLOC_SCRATCH_BYTES is MDR_ERR_WORKSPACE, nothing launched."""
    text = open(HEADER).read()
    assert "#define MDR_NOALLOC_SCRATCH_BYTES (64u << 20)" in text
    assert mdr.MDR_NOALLOC_SCRATCH_BYTES == 64 << 20
    big = mdr.config(**_good(seq=32768))
    assert mdr.mdr_workspace_size(big) > mdr.MDR_NOALLOC_SCRATCH_BYTES
    fake = 1 << 20  # aligned non-null pointers: never dereferenced, the call returns first
    for cfg, status in ((big, 3), (mdr.config(**_good(seq=4000)), 1)):
        with pytest.raises(mdr.MdrError) as e:
            mdr.mdr_routed_attention_noalloc(cfg, fake, fake, fake, fake, None, None, fake, stream=0)
        assert e.value.status == status
    with pytest.raises(mdr.MdrError) as e:  # a null input
        mdr.mdr_routed_attention_noalloc(mdr.config(**_good()), None, fake, fake, fake, None, None, fake, stream=0)
    assert e.value.status == 1


def test_decode_state_size_and_view(mdr):
    cfg = mdr.config(**_good())
    n = mdr.mdr_decode_state_size(cfg)
    A = 16 * 16
    nb = 4096 // 64
    assert n >= 8 * (A * 3 + nb) * 4 + 8 * nb * 64 * 4
    # (remote + local) * block above 4096 keys, or an invalid config: no state
    assert mdr.lib.mdr_decode_state_size(ctypes.byref(mdr.config(**_good(remote=16, local=60)))) == 0
    assert mdr.lib.mdr_decode_state_size(ctypes.byref(mdr.config(**_good(seq=4000)))) == 0
    v = mdr.MdrDecodeView()
    base = 1 << 20
    assert mdr.lib.mdr_decode_state_view(ctypes.byref(cfg), base, ctypes.byref(v)) == 0
    ptrs = [v.ring, v.overflow, v.summarized, v.filed, v.addr, v.ksum]
    assert ptrs == sorted(ptrs) and ptrs[0] == base and ptrs[-1] + nb * 64 * 4 * 8 <= base + n
    assert all(p % 256 == 0 for p in ptrs)
    assert mdr.lib.mdr_decode_state_view(ctypes.byref(cfg), base + 4, ctypes.byref(v)) == 1


def test_decode_entry_points_validate_before_launching(mdr):
    lib = mdr.lib
    cfg = mdr.config(**_good())
    c = ctypes.byref(cfg)
    n = mdr.mdr_decode_state_size(cfg)
    p = 1 << 20
    assert lib.mdr_decode_prime(c, p, p, None, 100, p, n - 1, None) == 3      # short state
    assert lib.mdr_decode_prime(c, p, p, None, -1, p, n, None) == 1           # n_tokens < 0
    assert lib.mdr_decode_prime(c, p, p, None, 4096, p, n, None) == 1         # nothing left to decode
    assert lib.mdr_decode_prime(c, None, p, None, 100, p, n, None) == 1
    # tokens 63 and 64 lie in two blocks
    assert lib.mdr_decode_step(c, p, p, p, p, None, None, 63, 2, p, None, p, n, None) == 1
    assert lib.mdr_decode_step(c, p, p, p, p, None, None, 4095, 2, p, None, p, n, None) == 1  # past seq
    assert lib.mdr_decode_step(c, p, p, p, p, None, None, 10, 0, p, None, p, n, None) == 1
    assert lib.mdr_decode_step(c, p, p, p, p, None, None, 10, 1, p + 2, None, p, n, None) == 1  # misaligned out
    assert lib.mdr_decode_step(c, p, p, p, p, None, None, 10, 1, p, None, p + 16, n, None) == 1  # state alignment


def test_redirect_policy_is_prefill_only(mdr):
    """The decode state has no redirect lists: a redirect config is rejected before any launch."""
    red = mdr.config(**_good(overflow_policy="redirect"))
    assert mdr.mdr_check_config(red) == 0
    with pytest.raises(mdr.MdrError) as e:
        mdr.mdr_decode_state_size(red)
    assert e.value.status == 2
    drop = mdr.mdr_workspace_size(mdr.config(**_good()))
    assert mdr.mdr_workspace_size(red) > drop  # alternates and redirect lists
