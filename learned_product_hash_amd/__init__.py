"""Python binding of libmdr.so, the gfx950 HIP library of Monodratic routed sparse
causal attention: the routed forward path, the stateless mixer around it, the
streaming decode step, and the attention backward under a fixed selection.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch supplies device memory and streams; it is imported before the
library so the library binds to the HIP runtime torch has already loaded.

The functions carry the names of the C entry points declared in
``include/mdr.h`` and raise :class:`MdrError` on any status other than MDR_OK.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library must share)

__all__ = [
    "LIB_PATH", "MdrError", "MdrConfig", "MdrRouting", "MdrDecodeView", "MDR_F32", "MDR_BF16",
    "MDR_OVERFLOW_DROP", "MDR_OVERFLOW_REDIRECT", "config", "lib",
    "mdr_abi_version", "mdr_status_string", "mdr_check_config", "mdr_workspace_size", "MdrWorkspaceParts",
    "mdr_workspace_breakdown", "workspace_breakdown", "mdr_selfcheck_indices",
    "mdr_routed_attention", "mdr_routed_attention_profiled", "MDR_CORE_KERNELS", "CORE_KERNELS",
    "mdr_routed_attention_noalloc", "MDR_NOALLOC_SCRATCH_BYTES",
    "mdr_mixer_forward", "mdr_stage_address", "mdr_stage_post",
    "mdr_stage_probe_rerank", "mdr_stage_attend", "mdr_stage_attend_lse", "mdr_stage_attend_backward",
    "mdr_stage_attend_backward_profiled", "MDR_BACKWARD_KERNELS", "BACKWARD_KERNELS",
    "mdr_decode_state_size", "decode_state", "mdr_decode_state_view", "mdr_decode_prime", "mdr_decode_step",
    "workspace", "routing_buffers",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmdr.so")

MDR_OK, MDR_ERR_INVALID_ARG, MDR_ERR_UNSUPPORTED, MDR_ERR_WORKSPACE, MDR_ERR_HIP = range(5)
MDR_F32, MDR_BF16 = 0, 1
MDR_OVERFLOW_DROP, MDR_OVERFLOW_REDIRECT = 0, 1


class MdrError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {mdr_status_string(status)} ({status})")


class MdrConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seq", "heads", "head_dim", "width", "block", "subspaces", "codes", "capacity",
        "probes", "max_cand", "remote", "local", "dtype")] + [
        ("rope_base", ctypes.c_float), ("softmax_scale", ctypes.c_float), ("overflow_policy", ctypes.c_int32)]


class MdrRouting(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "ksum", "addr", "post_off", "post_idx", "overflow", "sel", "n_cand", "n_drop", "alt", "redir_off",
        "redir_idx", "redir_time", "probes", "sel_score", "probe_margin", "sel_margin", "addr_margin")]


class MdrWorkspaceParts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "summaries", "posting_lists", "selection", "pair_lists", "partials", "backward", "mixer", "total")]


class MdrDecodeView(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "ring", "overflow", "summarized", "filed", "addr", "ksum")]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python learned_product_hash_amd/build.py`")
    return ctypes.CDLL(LIB_PATH)


lib = _load()

_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_cfgp = ctypes.POINTER(MdrConfig)
_rtp = ctypes.POINTER(MdrRouting)
_SIGS = {
    "mdr_abi_version": ([], _i32),
    "mdr_status_string": ([_i32], ctypes.c_char_p),
    "mdr_check_config": ([_cfgp], _i32),
    "mdr_workspace_size": ([_cfgp, ctypes.POINTER(_sz)], _i32),
    "mdr_workspace_breakdown": ([_cfgp, ctypes.POINTER(MdrWorkspaceParts)], _i32),
    "mdr_selfcheck_indices": ([_cfgp, ctypes.c_char_p, _sz], _i32),
    "mdr_routed_attention": ([_cfgp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _rtp, _vp, _sz, _vp], _i32),
    "mdr_routed_attention_profiled": ([_cfgp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _rtp, _vp, _sz,
                                       ctypes.POINTER(_vp), _vp], _i32),
    "mdr_routed_attention_noalloc": ([_cfgp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _rtp, _vp], _i32),
    "mdr_mixer_forward": ([_cfgp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _rtp, _vp, _sz, _vp], _i32),
    "mdr_stage_address": ([_cfgp] + [_vp] * 7, _i32),
    "mdr_stage_post": ([_cfgp] + [_vp] * 9, _i32),
    "mdr_stage_probe_rerank": ([_cfgp] + [_vp] * 14, _i32),
    "mdr_stage_attend": ([_cfgp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "mdr_stage_attend_lse": ([_cfgp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "mdr_stage_attend_backward": ([_cfgp] + [_vp] * 11 + [_sz, _vp], _i32),
    "mdr_stage_attend_backward_profiled": ([_cfgp] + [_vp] * 11 + [_sz, ctypes.POINTER(_vp), _vp], _i32),
    "mdr_decode_state_size": ([_cfgp], _sz),
    "mdr_decode_state_view": ([_cfgp, _vp, ctypes.POINTER(MdrDecodeView)], _i32),
    "mdr_decode_prime": ([_cfgp, _vp, _vp, _vp, ctypes.c_int32, _vp, _sz, _vp], _i32),
    "mdr_decode_step": ([_cfgp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp, _sz,
                         _vp], _i32),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


def config(**fields) -> MdrConfig:
    """An MdrConfig with unspecified fields zero (dtype accepts "f32"/"bf16", overflow_policy
    "drop"/"redirect")."""
    f = dict(fields)
    if isinstance(f.get("dtype"), str):
        f["dtype"] = {"f32": MDR_F32, "bf16": MDR_BF16}[f["dtype"]]
    if isinstance(f.get("overflow_policy"), str):
        f["overflow_policy"] = {"drop": MDR_OVERFLOW_DROP, "redirect": MDR_OVERFLOW_REDIRECT}[f["overflow_policy"]]
    return MdrConfig(**f)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmdr must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(status: int, where: str):
    if status != MDR_OK:
        raise MdrError(status, where)


def _routing(r):
    if r is None:
        return None
    if isinstance(r, MdrRouting):
        return ctypes.byref(r)
    rt = MdrRouting(**{k: _ptr(v) for k, v in r.items() if v is not None})
    return ctypes.byref(rt)


def mdr_abi_version() -> int:
    return lib.mdr_abi_version()


def mdr_status_string(status: int) -> str:
    return lib.mdr_status_string(status).decode()


def mdr_check_config(cfg: MdrConfig) -> int:
    """Returns the status code (does not raise)."""
    return lib.mdr_check_config(ctypes.byref(cfg))


def mdr_workspace_size(cfg: MdrConfig) -> int:
    n = _sz(0)
    _check(lib.mdr_workspace_size(ctypes.byref(cfg), ctypes.byref(n)), "mdr_workspace_size")
    return n.value


def mdr_workspace_breakdown(cfg: MdrConfig) -> MdrWorkspaceParts:
    p = MdrWorkspaceParts()
    _check(lib.mdr_workspace_breakdown(ctypes.byref(cfg), ctypes.byref(p)), "mdr_workspace_breakdown")
    return p


def workspace_breakdown(cfg: MdrConfig) -> dict:
    """mdr_workspace_breakdown as a dict of byte counts."""
    p = mdr_workspace_breakdown(cfg)
    return {n: getattr(p, n) for n, _ in MdrWorkspaceParts._fields_}


def mdr_selfcheck_indices(cfg: MdrConfig) -> str:
    """Host-only check of the kernels' index arithmetic for ``cfg``; returns "" when every index is in
    bounds, else the first violation."""
    buf = ctypes.create_string_buffer(256)
    st = lib.mdr_selfcheck_indices(ctypes.byref(cfg), buf, 256)
    if st not in (MDR_OK, MDR_ERR_INVALID_ARG):
        raise MdrError(st, "mdr_selfcheck_indices")
    return buf.value.decode() if st != MDR_OK else ""


def workspace(cfg: MdrConfig, device="cuda") -> torch.Tensor:
    """A device buffer of mdr_workspace_size(cfg) bytes."""
    return torch.empty(max(1, mdr_workspace_size(cfg)), dtype=torch.uint8, device=device)


def routing_buffers(cfg: MdrConfig, device="cuda", diag=False) -> dict:
    """Device tensors for every routing output of ``cfg`` (with ``diag`` also the routing diagnostics:
    probes, selection scores and the decision margins)."""
    B, H, S, D = cfg.batch, cfg.heads, cfg.seq, cfg.head_dim
    nb = S // cfg.block
    A = cfg.codes ** cfg.subspaces
    i32 = dict(dtype=torch.int32, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    extra = {}
    if diag:
        extra = dict(probes=torch.empty(B, H, S, cfg.probes, **i32), sel_score=torch.empty(B, H, S, cfg.remote, **f32),
                     probe_margin=torch.empty(B, H, S, **f32), sel_margin=torch.empty(B, H, S, **f32),
                     addr_margin=torch.empty(B, H, nb, **f32))
    return dict(**extra, ksum=torch.empty(B, H, nb, D, dtype=torch.float32, device=device),
                addr=torch.empty(B, H, nb, **i32), post_off=torch.empty(B, H, A + 1, **i32),
                post_idx=torch.empty(B, H, nb, **i32), overflow=torch.empty(B, H, **i32),
                sel=torch.empty(B, H, S, cfg.remote, **i32), n_cand=torch.empty(B, H, S, **i32),
                n_drop=torch.empty(B, H, S, **i32),
                **(dict(alt=torch.empty(B, H, nb, **i32), redir_off=torch.empty(B, H, A + 1, **i32),
                        redir_idx=torch.empty(B, H, nb, **i32), redir_time=torch.empty(B, H, nb, **i32))
                   if cfg.overflow_policy == MDR_OVERFLOW_REDIRECT else {}))


def _ws(ws):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())


def mdr_routed_attention(cfg, q, k, v, codebook, code_bias, force, out, routing=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib.mdr_routed_attention(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(codebook),
                                    _ptr(code_bias), _ptr(force), _ptr(out), _routing(routing), wp, wn,
                                    _stream(stream)), "mdr_routed_attention")


MDR_NOALLOC_SCRATCH_BYTES = 64 << 20


def mdr_routed_attention_noalloc(cfg, q, k, v, codebook, code_bias, force, out, routing=None, stream=None):
    """mdr_routed_attention on the library's static per-GPU scratch (no workspace argument)."""
    _check(lib.mdr_routed_attention_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(codebook),
                                            _ptr(code_bias), _ptr(force), _ptr(out), _routing(routing),
                                            _stream(stream)), "mdr_routed_attention_noalloc")


MDR_CORE_KERNELS = 6
CORE_KERNELS = ("address", "post", "probe_rerank", "attn_bin", "attn_remote", "attn_local")


def mdr_routed_attention_profiled(cfg, q, k, v, codebook, code_bias, force, out, events, routing=None, ws=None,
                                  stream=None):
    """``events``: MDR_CORE_KERNELS + 1 raw hipEvent_t handles (ints) created by the caller."""
    wp, wn = _ws(ws)
    arr = (_vp * (MDR_CORE_KERNELS + 1))(*events)
    _check(lib.mdr_routed_attention_profiled(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(codebook),
                                             _ptr(code_bias), _ptr(force), _ptr(out), _routing(routing), wp, wn,
                                             arr, _stream(stream)), "mdr_routed_attention_profiled")


def mdr_mixer_forward(cfg, x, wq, wk, wv, wo, codebook, code_bias, delta, routing=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib.mdr_mixer_forward(ctypes.byref(cfg), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo),
                                 _ptr(codebook), _ptr(code_bias), _ptr(delta), _routing(routing), wp, wn,
                                 _stream(stream)), "mdr_mixer_forward")


def mdr_stage_address(cfg, k, codebook, code_bias, ksum, addr, alt=None, stream=None):
    _check(lib.mdr_stage_address(ctypes.byref(cfg), _ptr(k), _ptr(codebook), _ptr(code_bias), _ptr(ksum),
                                 _ptr(addr), _ptr(alt), _stream(stream)), "mdr_stage_address")


def mdr_stage_post(cfg, addr, post_off, post_idx, overflow, alt=None, redir_off=None, redir_idx=None,
                   redir_time=None, stream=None):
    _check(lib.mdr_stage_post(ctypes.byref(cfg), _ptr(addr), _ptr(alt), _ptr(post_off), _ptr(post_idx),
                              _ptr(redir_off), _ptr(redir_idx), _ptr(redir_time), _ptr(overflow),
                              _stream(stream)), "mdr_stage_post")


def mdr_stage_probe_rerank(cfg, q, codebook, code_bias, ksum, post_off, post_idx, force, sel, n_cand=None,
                           redir_off=None, redir_idx=None, redir_time=None, n_drop=None, stream=None):
    _check(lib.mdr_stage_probe_rerank(ctypes.byref(cfg), _ptr(q), _ptr(codebook), _ptr(code_bias), _ptr(ksum),
                                      _ptr(post_off), _ptr(post_idx), _ptr(redir_off), _ptr(redir_idx),
                                      _ptr(redir_time), _ptr(force), _ptr(sel), _ptr(n_cand), _ptr(n_drop),
                                      _stream(stream)), "mdr_stage_probe_rerank")


def mdr_stage_attend(cfg, q, k, v, sel, out, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib.mdr_stage_attend(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(out), wp, wn,
                                _stream(stream)), "mdr_stage_attend")


def mdr_stage_attend_lse(cfg, q, k, v, sel, out, lse, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib.mdr_stage_attend_lse(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(out), _ptr(lse),
                                    wp, wn, _stream(stream)), "mdr_stage_attend_lse")


def mdr_stage_attend_backward(cfg, q, k, v, sel, out, lse, d_out, dq, dk, dv, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib.mdr_stage_attend_backward(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(sel), _ptr(out),
                                         _ptr(lse), _ptr(d_out), _ptr(dq), _ptr(dk), _ptr(dv), wp, wn,
                                         _stream(stream)), "mdr_stage_attend_backward")


MDR_BACKWARD_KERNELS = 4
BACKWARD_KERNELS = ("pair_bin", "bwd_dot", "bwd_kv", "bwd_q")


def mdr_stage_attend_backward_profiled(cfg, q, k, v, sel, out, lse, d_out, dq, dk, dv, events, ws, stream=None):
    """``events``: MDR_BACKWARD_KERNELS + 1 raw hipEvent_t handles (ints) created by the caller."""
    wp, wn = _ws(ws)
    arr = (_vp * (MDR_BACKWARD_KERNELS + 1))(*events)
    _check(lib.mdr_stage_attend_backward_profiled(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(sel),
                                                  _ptr(out), _ptr(lse), _ptr(d_out), _ptr(dq), _ptr(dk), _ptr(dv),
                                                  wp, wn, arr, _stream(stream)),
           "mdr_stage_attend_backward_profiled")


# ---- streaming decode

def mdr_decode_state_size(cfg) -> int:
    n = lib.mdr_decode_state_size(ctypes.byref(cfg))
    if n == 0:
        raise MdrError(MDR_ERR_UNSUPPORTED if mdr_check_config(cfg) == MDR_OK else mdr_check_config(cfg),
                       "mdr_decode_state_size")
    return n


def decode_state(cfg, device="cuda") -> torch.Tensor:
    """A device buffer of mdr_decode_state_size(cfg) bytes."""
    return torch.empty(mdr_decode_state_size(cfg), dtype=torch.uint8, device=device)


def mdr_decode_state_view(cfg, state) -> dict:
    """Tensors viewing the regions of a decode state (no copy)."""
    v = MdrDecodeView()
    _check(lib.mdr_decode_state_view(ctypes.byref(cfg), _ptr(state), ctypes.byref(v)), "mdr_decode_state_view")
    B, H, D, cap = cfg.batch, cfg.heads, cfg.head_dim, cfg.capacity
    nb = cfg.seq // cfg.block
    A = cfg.codes ** cfg.subspaces
    base = state.data_ptr()

    def region(ptr, shape, dtype):
        n = 1
        for x in shape:
            n *= x
        off = ptr - base
        return state[off:off + n * 4].view(dtype).view(*shape)

    ring = region(v.ring, (B, H, A, cap + 1), torch.int32)
    return dict(ring=ring[..., 1:], ring_n=ring[..., 0],
                overflow=region(v.overflow, (B, H), torch.int32), summarized=region(v.summarized, (B, H), torch.int32),
                filed=region(v.filed, (B, H), torch.int32), addr=region(v.addr, (B, H, nb), torch.int32),
                ksum=region(v.ksum, (B, H, nb, D), torch.float32))


def mdr_decode_prime(cfg, k_cache, codebook, code_bias, n_tokens, state, stream=None):
    _check(lib.mdr_decode_prime(ctypes.byref(cfg), _ptr(k_cache), _ptr(codebook), _ptr(code_bias), int(n_tokens),
                                _ptr(state), state.numel(), _stream(stream)), "mdr_decode_prime")


def mdr_decode_step(cfg, q_new, k_cache, v_cache, codebook, code_bias, force, pos, out, sel, state, stream=None):
    n_new = q_new.shape[2]
    _check(lib.mdr_decode_step(ctypes.byref(cfg), _ptr(q_new), _ptr(k_cache), _ptr(v_cache), _ptr(codebook),
                               _ptr(code_bias), _ptr(force), int(pos), int(n_new), _ptr(out), _ptr(sel), _ptr(state),
                               state.numel(), _stream(stream)), "mdr_decode_step")
