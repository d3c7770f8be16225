"""Seeded generators for the five workloads of routed sparse causal attention.

Every array is drawn from ``numpy.random.default_rng(seed)`` in a fixed order
(codebook, then Q, K, V -- or x and the projections -- then the planted
structure), so a seed regenerates the same bytes.  bf16 workloads are rounded
once to bf16 (round to nearest even) here, and that rounded array is what both
the oracle and the GPU receive.

The workload shapes follow the method's descriptions: a tiny mixer case, an
associative-recall-shaped case with one planted key block per sequence, a
balanced scaling sweep (the pages describe their timing runs as a "fixed,
balanced setup" with zero posting overflow), a long-context case and a
skewed/batched case whose address use is pushed towards a Zipf law so that
posting lists overflow.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seq: int
    head_dim: int
    block: int
    subspaces: int
    codes: int
    capacity: int
    probes: int
    max_cand: int  # 0 means probes * capacity
    remote: int
    local: int
    dtype: str  # "f32" or "bf16"
    width: int = 0  # mixer only
    plant: str = "none"  # none | recall | balanced | zipf
    rope_base: float = 10000.0
    plant_gain: float = 1.5  # balanced planting: logit added to each planted code
    zipf_kappa: float = 0.0  # code bias slope for the zipf plant

    @property
    def nblocks(self) -> int:
        return self.seq // self.block

    @property
    def addresses(self) -> int:
        return self.codes ** self.subspaces

    @property
    def cand_limit(self) -> int:
        return self.max_cand if self.max_cand > 0 else self.probes * self.capacity

    def as_dict(self) -> dict:
        return dataclasses.asdict(self)


def _sweep_capacity(seq: int, block: int, addresses: int) -> int:
    return 2 * math.ceil((seq // block) / addresses)


WORKLOADS = {
    # [batch, seq, width] mixer case; fp32.
    "tiny": Workload("tiny", batch=1, heads=1, seq=512, head_dim=32, block=32, subspaces=2, codes=4,
                     capacity=8, probes=2, max_cand=0, remote=2, local=2, dtype="f32", width=64),
    # Associative-recall shaped: one planted key block per sequence, five eligible candidates, R=2.
    "recall": Workload("recall", batch=16, heads=4, seq=2048, head_dim=64, block=64, subspaces=2, codes=8,
                       capacity=8, probes=16, max_cand=5, remote=2, local=2, dtype="f32", plant="recall"),
    # Scaling sweep at its largest length; balanced addresses so no list overflows.
    "sweep": Workload("sweep", batch=1, heads=8, seq=32768, head_dim=64, block=64, subspaces=2, codes=16,
                      capacity=_sweep_capacity(32768, 64, 256), probes=4, max_cand=0, remote=2, local=2,
                      dtype="bf16", plant="balanced"),
    "long": Workload("long", batch=1, heads=16, seq=131072, head_dim=128, block=128, subspaces=2, codes=32,
                     capacity=16, probes=4, max_cand=0, remote=4, local=2, dtype="bf16"),
    # Skewed/batched: code biases -kappa*ln(c+1) concentrate address use (kappa chosen so the ranked
    # address-use histogram of Gaussian keys has a log-log slope near -1.1).
    "skew": Workload("skew", batch=8, heads=32, seq=16384, head_dim=128, block=64, subspaces=3, codes=8,
                     capacity=8, probes=6, max_cand=0, remote=8, local=2, dtype="bf16", plant="zipf",
                     zipf_kappa=0.11),
}

SWEEP_SEQS = (4096, 8192, 16384, 32768)


def workload(name: str, **over) -> Workload:
    """A named workload, optionally with fields replaced (e.g. a shorter ``seq`` for tests).

    For the sweep the posting capacity follows the sequence length
    (2 * ceil(blocks / addresses)) unless ``capacity`` is given explicitly.
    """
    w = WORKLOADS[name]
    if name == "sweep" and "capacity" not in over:
        seq = over.get("seq", w.seq)
        block = over.get("block", w.block)
        codes = over.get("codes", w.codes)
        sub = over.get("subspaces", w.subspaces)
        over = dict(over, capacity=_sweep_capacity(seq, block, codes ** sub))
    return dataclasses.replace(w, **over)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); returns float32."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    u = x.view(np.uint32)
    flat = u.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):  # chunked to bound temporaries; finite inputs cannot overflow
        c = flat[s:s + step]
        lsb = (c >> 16) & 1
        c += np.uint32(0x7FFF)
        c += lsb
        c &= np.uint32(0xFFFF0000)
    return x


def zipf_code_bias(H: int, G: int, C: int, kappa: float) -> np.ndarray:
    """Code bias -kappa * ln(c + 1) for every head and subspace [H, G, C] float32: the larger kappa,
    the more the low codes (and so a few addresses) attract blocks and queries."""
    c = np.arange(C, dtype=np.float64)
    row = (-kappa * np.log(c + 1.0)).astype(np.float32)
    return np.broadcast_to(row, (H, G, C)).copy()


def _normal(rng, shape, std=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def make_core_inputs(w: Workload, seed: int) -> dict:
    """Post-RoPE Q, K, V [B,H,S,D], codebook [H,G,C,D] and code bias [H,G,C] (or None).

    Q, K, V are float32 arrays; for bf16 workloads they hold bf16-rounded values.
    Extra keys describe the planted structure:
      recall:   ``planted`` [B] (the planted block) and ``force`` [B,H,S] (planted block on the last
                query block's tokens, -1 elsewhere).
      balanced: ``target_addr`` [H, nb] (the address each block's keys were pushed towards).
    """
    B, H, S, D = w.batch, w.heads, w.seq, w.head_dim
    G, C, blk = w.subspaces, w.codes, w.block
    if S % blk:
        raise ValueError("seq must be a multiple of block")
    nb = S // blk
    rng = np.random.default_rng(seed)
    codebook = _normal(rng, (H, G, C, D), 1.0 / math.sqrt(D))
    q = _normal(rng, (B, H, S, D))
    k = _normal(rng, (B, H, S, D))
    v = _normal(rng, (B, H, S, D))
    bias = None
    out = {}
    if w.plant == "recall":
        n_elig = nb - w.local  # blocks eligible for the last query block: 0 .. nb-1-L
        if n_elig < 1:
            raise ValueError("recall plant needs at least one eligible block")
        planted = rng.integers(0, n_elig, size=B)
        last = slice((nb - 1) * blk, S)
        force = np.full((B, H, S), -1, dtype=np.int32)
        for b in range(B):
            p = int(planted[b])
            for h in range(H):
                u = q[b, h, last].astype(np.float64).mean(axis=0)
                u /= np.linalg.norm(u)
                noise = _normal(rng, (blk, D), 0.1)
                k[b, h, p * blk:(p + 1) * blk] = (math.sqrt(D) * u).astype(np.float32)[None, :] + noise
            force[b, :, last] = p
        out["planted"] = planted.astype(np.int32)
        out["force"] = force
    elif w.plant == "balanced":
        A = C ** G
        target = np.empty((H, nb), dtype=np.int32)
        for h in range(H):
            target[h] = (rng.permutation(nb) % A).astype(np.int32)
            # One-hot pattern of the target codes (digits of the address, most significant subspace
            # first); the push is its least-squares preimage under the stacked codebook rows, so it
            # raises each planted code's logit by plant_gain and leaves the other codes' logits alone.
            onehot = np.zeros((nb, G, C))
            for g in range(G):
                onehot[np.arange(nb), g, (target[h] // C ** (G - 1 - g)) % C] = 1.0
            rows = codebook[h].reshape(G * C, D).astype(np.float64)
            push = w.plant_gain * onehot.reshape(nb, G * C) @ np.linalg.pinv(rows).T
            k[:, h] += np.repeat(push.astype(np.float32), blk, axis=0)[None]
        out["target_addr"] = target
    elif w.plant == "zipf":
        bias = zipf_code_bias(H, G, C, w.zipf_kappa)
    elif w.plant != "none":
        raise ValueError(f"unknown plant {w.plant!r}")
    if w.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    elif w.dtype != "f32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    out.update(q=q, k=k, v=v, codebook=codebook, bias=bias)
    return out


def make_grad_inputs(w: Workload, seed: int) -> np.ndarray:
    """Upstream gradient of the attention output, d_out [B,H,S,D] ~ N(0, 1) (bf16-rounded for bf16
    workloads), drawn from its own stream so the forward inputs of the same seed are unchanged."""
    rng = np.random.default_rng([seed, 0x6772])
    g = _normal(rng, (w.batch, w.heads, w.seq, w.head_dim))
    return bf16_round(g) if w.dtype == "bf16" else g


def make_mixer_inputs(w: Workload, seed: int) -> dict:
    """x [B,S,W], wq/wk/wv [W, H*D], wo [H*D, W] (std 1/sqrt(fan_in)), codebook, bias=None."""
    B, H, S, D, W = w.batch, w.heads, w.seq, w.head_dim, w.width
    G, C = w.subspaces, w.codes
    if W <= 0:
        raise ValueError("mixer workloads need a width")
    rng = np.random.default_rng(seed)
    codebook = _normal(rng, (H, G, C, D), 1.0 / math.sqrt(D))
    x = _normal(rng, (B, S, W))
    wq = _normal(rng, (W, H * D), 1.0 / math.sqrt(W))
    wk = _normal(rng, (W, H * D), 1.0 / math.sqrt(W))
    wv = _normal(rng, (W, H * D), 1.0 / math.sqrt(W))
    wo = _normal(rng, (H * D, W), 1.0 / math.sqrt(H * D))
    if w.dtype == "bf16":
        x, wq, wk, wv, wo = (bf16_round(a) for a in (x, wq, wk, wv, wo))
    return dict(x=x, wq=wq, wk=wk, wv=wv, wo=wo, codebook=codebook, bias=None)
