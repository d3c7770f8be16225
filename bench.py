"""Benchmark of routed sparse causal attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the whole hot path -- block addresses, posting lists,
probe + rerank, selected-set attention -- over the scaling-sweep workload at
32K tokens (B=1, H=8, D=64, block 64, 2x16 codes, capacity 4, 4 probes, R=2
remote + 2 local blocks, bf16 Q/K/V with fp32 routing and softmax, balanced
addresses), with inputs already resident in HBM.  An untimed pass of K calls
of the library's profiling entry point, with an event before every kernel,
gives each kernel's average duration; the timed region is then K consecutive
calls of the same entry point, bracketed by torch.cuda.synchronize(), with
events on the call's stream around the selected-set attention stage only (the
remote and local attention kernels, which run last), whose average over that
region is the roofline's duration.

Prints one JSON line: tokens/s (B*S*K / wall time), the roofline of the
attention stage (its compulsory bytes -- Q, K, V and O once plus the selection
-- per call / its average duration, against 8 TB/s), every kernel's time, the
memory split, the fitted timing exponent over 4K-32K, and the CPU oracle timed
on the host's cores over a bounded sample of the same workload.

    python bench.py --ingest-pmc FETCH.csv WRITE.csv
turns two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of
``python bench.py --steps 3 --warmup 1 --calib-copy --no-cpu --no-sweep --no-decode --no-backward --no-stress
--no-mixer --no-cold`` into
profiles/traffic_<workload>.json (per-launch HBM bytes of every kernel,
scaled by what the counters read for a plain elementwise copy of known size).
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X dense, published (fp32: no fp32 MFMA figure; vector)
def _has(sym, name):
    """sym (a substring, or a tuple of alternatives: rocprofv3 prints some names demangled and leaves
    others, such as those with bf16 template arguments, mangled) occurs in the kernel name."""
    return any(x in name for x in (sym if isinstance(sym, tuple) else (sym,)))


def _label(sym):
    return sym[0] if isinstance(sym, tuple) else sym


KERNEL_SYMBOL = {  # substrings of the kernels' symbol names in rocprofv3 output
    "address": "k_address",
    "post": "k_post",
    "probe_rerank": "k_probe",
    "attn_bin": ("k_pair_scatter<false>", "k_pair_scatterILb0E"),  # the forward's (unordered) filing
    "attn_remote": "k_attn_remote",
    "attn_local": "k_attn_local",
}
# The selected-set attention stage (mdr_sel_attn) of the roofline: the remote partials and the local window
# with the merge.  The pair binning that feeds it (attn_bin, the selection turned into per-block pair lists)
# is timed with it and reported beside it (attention_stage.with_binning).
STAGE_KERNELS = ("attn_remote", "attn_local")
KERNEL_SOURCE = {
    "address": "mdr_route.hip", "post": "mdr_route.hip", "probe_rerank": "mdr_route.hip",
    "attn_bin": "mdr_pairs.hip", "attn_remote": "mdr_attn.hip", "attn_local": "mdr_attn.hip",
}
MIXER_SYMBOL = {  # every listed substring must occur in the (mangled) kernel name
    "qkv (fused projections + RoPE + summaries + addresses)": ("k_mm", "Lb0ELb1E"),
    "output projection": ("k_mm", "Lb1ELb0E"),
    "weight transposes": ("k_transpose",),
}
BACKWARD_SYMBOL = {
    "pair_bin (count)": "k_pair_count",
    "pair_bin (ordered scatter)": ("k_pair_scatter<true>", "k_pair_scatterILb1E"),
    "bwd_dot": "k_bwd_dot",
    "bwd_kv": "k_bwd_kv",
    "bwd_q": "k_bwd_q",
}
CALIB_BYTES = 512 << 20
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)
PMC_COMMANDS = [  # run from the repository root on one MI355X, TMPDIR=/tmp
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmcf -o f -- "
    "python3 bench.py --steps 3 --warmup 1 --calib-copy --no-cpu --no-sweep --no-decode --no-backward --no-stress --no-mixer --no-cold",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmcw -o w -- "
    "python3 bench.py --steps 3 --warmup 1 --calib-copy --no-cpu --no-sweep --no-decode --no-backward --no-stress --no-mixer --no-cold",
]


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sweep", choices=["sweep", "long", "skew", "recall", "tiny"])
    ap.add_argument("--seq", type=int, default=0, help="override the sequence length")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 4K-32K exponent sweep")
    ap.add_argument("--no-decode", action="store_true", help="skip the streaming-decode timing")
    ap.add_argument("--no-backward", action="store_true", help="skip the attention-backward timing")
    ap.add_argument("--no-stress", action="store_true", help="skip the overflow stress test")
    ap.add_argument("--no-mixer", action="store_true", help="skip the mixer timing")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache steps")
    ap.add_argument("--mixer-only", action="store_true", help="time the mixer alone and print its JSON")
    ap.add_argument("--profile-name", default="routed_attention_kernels",
                    help="with --summarize-rocprof: file name stem of the summary under profiles/")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one elementwise copy of 512 MiB first (counter calibration)")
    ap.add_argument("--cpu-heads", type=int, default=8)
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--bench-log", default=None, help="with --summarize-rocprof: bench.py's stdout of the same run")
    ap.add_argument("--summarize-rocprof", nargs=2, metavar=("KERNEL_STATS_CSV", "COMMAND"),
                    help="write profiles/routed_attention_kernels_<workload>.md from a rocprofv3 --stats CSV")
    return ap.parse_args(argv)


# ----------------------------------------------------------------------------- HIP events

class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded (the one the library uses)."""

    def __init__(self):
        import ctypes

        path = None
        for line in open("/proc/self/maps"):
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
        if path is None:
            raise RuntimeError("libamdhip64 is not mapped; initialise torch.cuda first")
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = self.ct.c_void_p()
            # without the system-scope fence an event adds ~1 us instead of ~5 us between kernels, so the
            # per-kernel intervals agree with rocprofv3's kernel durations
            if self.hip.hipEventCreateWithFlags(self.ct.byref(h), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            out.append(h.value)
        return out

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


# ----------------------------------------------------------------------------- workload

def make_workload(name, seq):
    import synth

    over = {"seq": seq} if seq else {}
    return synth.workload(name, **over)


def describe(w):
    return (f"{w.name} B{w.batch} H{w.heads} S{w.seq} D{w.head_dim} block{w.block} "
            f"{w.subspaces}x{w.codes} codes cap{w.capacity} P{w.probes} M{w.cand_limit} R{w.remote} "
            f"L{w.local} {w.dtype} plant={w.plant}")


class Run:
    """Device inputs, workspace and routing buffers of one workload."""

    def __init__(self, mdr, w, seed, policy="drop", bias=None, inputs=None):
        import torch

        import synth

        self.w = w
        self.mdr = mdr
        inp = synth.make_core_inputs(w, seed) if inputs is None else inputs
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.q, self.k, self.v = (torch.from_numpy(inp[n]).to("cuda").to(dt) for n in ("q", "k", "v"))
        self.cb = torch.from_numpy(inp["codebook"]).cuda()
        b = inp["bias"] if bias is None else bias
        self.bias = None if b is None else torch.from_numpy(b).cuda()
        self.out = torch.empty_like(self.q)
        self.cfg = mdr.config(batch=w.batch, seq=w.seq, heads=w.heads, head_dim=w.head_dim, block=w.block,
                              subspaces=w.subspaces, codes=w.codes, capacity=w.capacity, probes=w.probes,
                              max_cand=w.max_cand, remote=w.remote, local=w.local, dtype=w.dtype,
                              overflow_policy=policy)
        self.ws = mdr.workspace(self.cfg)
        self.rt = mdr.routing_buffers(self.cfg)
        self.inputs = inp

    def step(self, events=None):
        if events is None:
            self.mdr.mdr_routed_attention(self.cfg, self.q, self.k, self.v, self.cb, self.bias, None, self.out,
                                          self.rt, self.ws)
        else:
            self.mdr.mdr_routed_attention_profiled(self.cfg, self.q, self.k, self.v, self.cb, self.bias, None,
                                                   self.out, events, self.rt, self.ws)

    def routing_stats(self):
        import torch

        sel = self.rt["sel"]
        valid = (sel >= 0)
        pairs = int(valid.sum().item())
        nb, blk = self.w.nblocks, self.w.block
        BH = self.w.batch * self.w.heads
        used = torch.zeros(BH * nb, dtype=torch.bool, device=sel.device)
        flat = (sel.reshape(BH, -1) + (torch.arange(BH, device=sel.device) * nb)[:, None]).reshape(-1)
        used[flat[valid.reshape(-1)].long()] = True
        return dict(pairs=pairs, blocks_used=int(used.sum().item()),
                    R_eff=pairs / float(self.w.batch * self.w.heads * self.w.seq),
                    overflow=int(self.rt["overflow"].sum().item()),
                    n_cand_mean=float(self.rt["n_cand"].float().mean().item()))


def design_bytes(w, st):
    """Bytes each kernel moves per launch by this design's own data flow (each byte once), including what the
    design adds beyond the method's compulsory bytes (per-pair query gathers, the remote partials' round
    trip, pair lists).  Reported per kernel; the roofline uses the stage's compulsory bytes instead."""
    e = 2 if w.dtype == "bf16" else 4
    B, H, S, D, nb, blk = w.batch, w.heads, w.seq, w.head_dim, w.nblocks, w.block
    A, R, G, C = w.addresses, w.remote, w.subspaces, w.codes
    ne = max(0, nb - w.local)
    BH = B * H
    qkv = BH * S * D * e
    cb = H * G * C * D * 4
    pairs, used = st["pairs"], st["blocks_used"]
    part = D * e + 4  # a remote partial: normalised output row and its log2 normaliser
    tbin = ((S + 15) // 16 + 255) // 256 * 256  # tokens per range of the pair binning
    ng = (S + tbin - 1) // tbin
    return {
        "address": qkv + BH * nb * D * 4 + 2 * BH * nb * 4 + cb,
        "post": BH * nb * 4 + BH * (A + 1) * 4 + BH * nb * 4 + BH * 4,
        "probe_rerank": qkv + cb + BH * (A + 1 + nb) * 4 + BH * nb * D * 4 + BH * S * (R + 1) * 4,
        "attn_bin": BH * S * R * 4 + BH * ng * ne * 4 + pairs * 4 + BH * (ne + 1) * 4,
        "attn_remote": pairs * (4 + D * e + part) + used * 2 * blk * D * e,
        "attn_local": 4 * qkv + BH * S * R * 4 + pairs * part,
    }


def stage_bytes(w):
    """The attention stage's compulsory bytes: Q, K, V and O once plus the selection."""
    e = 2 if w.dtype == "bf16" else 4
    BH = w.batch * w.heads
    return 4 * BH * w.seq * w.head_dim * e + BH * w.seq * w.remote * 4


def strip_comments(text):
    """C++ source without its comments and blank lines (a comment edit does not change a kernel)."""
    text = re.sub(rb"/\*.*?\*/", b"", text, flags=re.S)
    text = re.sub(rb"//[^\n]*", b"", text)
    return b"\n".join(line.rstrip() for line in text.split(b"\n") if line.strip())


def source_digest(kernel):
    """Digest of the code (comments stripped) of the kernel's source file and every project header
    it includes (transitively)."""
    csrc = os.path.join(ROOT, "learned_product_hash_amd", "csrc")
    seen, todo = [], [KERNEL_SOURCE[kernel]]
    while todo:
        f = todo.pop(0)
        if f in seen:
            continue
        seen.append(f)
        path = os.path.join(csrc, f) if f != "mdr.h" else os.path.join(ROOT, "include", f)
        text = open(path, "rb").read()
        todo += [m.decode() for m in re.findall(rb'#include "([^"]+)"', text)]
    h = hashlib.sha256()
    for f in sorted(seen):
        path = os.path.join(csrc, f) if f != "mdr.h" else os.path.join(ROOT, "include", f)
        h.update(strip_comments(open(path, "rb").read()))
    return h.hexdigest()[:16]


def traffic_path(w):
    return os.path.join(ROOT, "profiles", f"traffic_{w.name}_{w.seq // 1024}k.json")


def load_traffic(w, kernel):
    p = traffic_path(w)
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    k = t.get("kernels", {}).get(kernel)
    if not k or k.get("source_sha") != source_digest(kernel):
        return None  # counters were taken on another version of the kernel
    return k["bytes_per_launch"]


def selected_set_bytes(w, pairs):
    """What a per-query gather with no reuse across queries would read and write: per (token, head)
    q, o and the local window's K/V (L blocks amortised per query block: L * D * 2e per token), plus
    blk K/V rows per selected remote (token, slot) pair."""
    e = 2 if w.dtype == "bf16" else 4
    return w.batch * w.heads * w.seq * (2 * w.head_dim * e + w.local * w.head_dim * 2 * e) + \
        pairs * w.block * w.head_dim * 2 * e


def attention_stage(w, t_att, pairs, stage_names, t_bin=None):
    """The selected-set attention stage against the HBM peak, three ways: (i) compulsory bytes (Q, K, V,
    O once + sel) / time -- the roofline's fraction; (ii) L2-to-fabric bytes (FETCH_SIZE + WRITE_SIZE of
    the stage's kernels, when counters for these sources exist) / time, an upper bound on what HBM served
    (the 256 MB last-level cache serves part of it); (iii) the selected-set bytes of a gather without reuse
    / time, which counts cache-served and regrouped re-reads and so is not an HBM bandwidth.  With t_bin
    (the pair binning's average), (i) and (ii) again for the stage together with the binning that feeds it."""
    alg = stage_bytes(w)
    sel_b = selected_set_bytes(w, pairs)
    out = {"ms": round(t_att, 5), "alg_bytes": alg,
           "frac_of_hbm_peak": round(alg / (t_att * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "selected_set_bytes": sel_b,
           "selected_set_gbps_not_hbm": round(sel_b / (t_att * 1e-3) / 1e9, 1)}
    tr = [load_traffic(w, k) for k in stage_names]
    if all(t is not None for t in tr):
        gbps = sum(tr) / (t_att * 1e-3) / 1e9
        out.update(l2_fabric_bytes=round(sum(tr)), l2_fabric_gbps=round(gbps, 1),
                   l2_fabric_over_compulsory=round(sum(tr) / alg, 3))
    if t_bin is not None:
        t = t_att + t_bin
        wb = {"kernels": ["attn_bin", *stage_names], "ms": round(t, 5),
              "frac_of_hbm_peak": round(alg / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        trb = [load_traffic(w, k) for k in ("attn_bin", *stage_names)]
        if all(x is not None for x in trb):
            wb.update(l2_fabric_bytes=round(sum(trb)), l2_fabric_over_compulsory=round(sum(trb) / alg, 3))
        out["with_binning"] = wb
    return out


# ----------------------------------------------------------------------------- timing

def event_overhead(hip, steps):
    """Cost of one event on the stream: an interval between two events also holds the second
    event's own cost, so it is measured with back-to-back pairs and taken off kernel intervals."""
    import torch

    pairs = hip.create(2 * steps)
    stream = torch.cuda.current_stream().cuda_stream
    for s in range(steps):
        hip.record(pairs[2 * s], stream)
        hip.record(pairs[2 * s + 1], stream)
    torch.cuda.synchronize()
    overhead = sum(hip.elapsed_ms(pairs[2 * s], pairs[2 * s + 1]) for s in range(steps)) / steps
    hip.destroy(pairs)
    return overhead


def stage_span(names):
    """Event indices bracketing the selected-set attention stage (mdr_sel_attn): the STAGE_KERNELS, which
    run last in the core path."""
    idx = [i for i, n in enumerate(names) if n in STAGE_KERNELS]
    return idx[0], idx[-1] + 1


def timed_region(run, hip, steps, warmup):
    """W warm-up steps; then K steps with an event before every kernel (untimed: every kernel's
    average); then the timed region, K steps with events around the attention stage only (its
    first kernel to the end of its last) on every other step, so that the step rate carries one event
    per step on average instead of one per kernel.  Returns the timed wall time, the per-kernel averages, the event cost and the stage's
    average over the timed region."""
    import numpy as np
    import torch

    mdr = run.mdr
    nk = mdr.MDR_CORE_KERNELS
    for _ in range(warmup):
        run.step()
    events = hip.create(steps * (nk + 1))
    torch.cuda.synchronize()
    for s in range(steps):
        run.step(events[s * (nk + 1):(s + 1) * (nk + 1)])
    torch.cuda.synchronize()
    per = [0.0] * nk
    totals = []
    for s in range(steps):
        ev = events[s * (nk + 1):(s + 1) * (nk + 1)]
        for i in range(nk):
            per[i] += hip.elapsed_ms(ev[i], ev[i + 1])
        totals.append(hip.elapsed_ms(ev[0], ev[nk]))
    hip.destroy(events)
    run.step_quantiles = [round(float(x), 4) for x in np.percentile(totals, [10, 50, 90])]
    overhead = event_overhead(hip, steps)
    per = [max(0.0, p / steps - overhead) for p in per]
    a, b = stage_span(list(mdr.CORE_KERNELS))
    # the stage's two events on every other step of the timed region (each event costs the GPU a few
    # microseconds, which the other half of the steps then does not pay)
    sampled = list(range(0, steps, 2))
    marks = hip.create(2 * len(sampled))
    arrays = [[None] * (nk + 1) for _ in range(steps)]
    for x, s in enumerate(sampled):
        arrays[s][a], arrays[s][b] = marks[2 * x], marks[2 * x + 1]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        run.step(arrays[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = max(0.0, sum(hip.elapsed_ms(marks[2 * x], marks[2 * x + 1]) for x in range(len(sampled))) /
                   len(sampled) - overhead)
    hip.destroy(marks)
    return wall, per, overhead, stage_ms


def cold_region(run, hip, steps, overhead):
    """Steps with the caches cold: before each step a 512 MiB buffer is written (twice the 256 MB
    last-level cache of the chip, so neither it nor the L2s hold the inputs), outside the events
    that bracket the step.  Returns the p10 / p50 / p90 step time and each kernel's average (ms)."""
    import numpy as np
    import torch

    nk = run.mdr.MDR_CORE_KERNELS
    flush = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device="cuda")
    events = hip.create(steps * (nk + 1))
    for s in range(steps):
        flush.fill_(float(s))
        run.step(events[s * (nk + 1):(s + 1) * (nk + 1)])
    torch.cuda.synchronize()
    per = [0.0] * nk
    totals = []
    for s in range(steps):
        ev = events[s * (nk + 1):(s + 1) * (nk + 1)]
        for i in range(nk):
            per[i] += hip.elapsed_ms(ev[i], ev[i + 1])
        totals.append(hip.elapsed_ms(ev[0], ev[nk]))
    hip.destroy(events)
    del flush
    q = [round(float(x), 4) for x in np.percentile(totals, [10, 50, 90])]
    return q, [max(0.0, p / steps - overhead) for p in per]


def plain_region(run, steps):
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run.step()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def attended_pairs(w, pairs):
    """(query, key) pairs the attention visits: remote pairs * block + each token's local window."""
    import numpy as np

    t = np.arange(w.seq)
    lo = np.maximum(0, (t // w.block - w.local + 1) * w.block)
    return pairs * w.block + w.batch * w.heads * int((t - lo + 1).sum())


def exponent_sweep(mdr, seqs, seed):
    """OLS slope of ln(time) against ln(S), and against ln(attended pairs), over the sweep lengths."""
    import numpy as np

    rows = []
    for s in seqs:
        run = Run(mdr, make_workload("sweep", s), seed)
        for _ in range(3):
            run.step()
        ms = plain_region(run, 20) / 20 * 1e3  # wall time per call of the plain entry point
        st = run.routing_stats()
        rows.append(dict(seq=s, ms=ms, R_eff=st["R_eff"], overflow=st["overflow"],
                         attended=attended_pairs(run.w, st["pairs"])))
        del run
    lt = np.log([r["ms"] for r in rows])
    slope = float(np.polyfit(np.log([r["seq"] for r in rows]), lt, 1)[0])
    slope_work = float(np.polyfit(np.log([r["attended"] for r in rows]), lt, 1)[0])
    return dict(seqs=[r["seq"] for r in rows], ms=[round(r["ms"], 4) for r in rows],
                R_eff=[round(r["R_eff"], 3) for r in rows], overflow=[r["overflow"] for r in rows],
                attended_pairs=[r["attended"] for r in rows],
                ps_per_attended_pair=[round(r["ms"] * 1e9 / r["attended"], 2) for r in rows],
                slope_vs_seq=round(slope, 3), slope_vs_attended_pairs=round(slope_work, 3),
                note="context only: the pages report 0.993 for their packed CPU routing over 4K-32K "
                     "(fixed, balanced setup; CPU hardware not stated)")


def decode_bench(run, batch, steps=48, warmup=4):
    """Streaming decode on the same workload: the cache holds the workload's K/V (replicated over
    `batch` sequences), the state is primed on all but the last block, and single-token steps
    continue from there.  Returns time per step and its compulsory bytes (per decoded token and
    head: q, o, the K/V rows of the selected remote blocks and of the local window, the summaries
    of its candidates)."""
    import torch

    mdr, w = run.mdr, run.w
    B, H, S, D, blk = batch, w.heads, w.seq, w.head_dim, w.block
    e = 2 if w.dtype == "bf16" else 4
    rep = lambda t: t.expand(B, *t.shape[1:]).contiguous() if B != t.shape[0] else t
    q, k, v = rep(run.q), rep(run.k), rep(run.v)
    cfg = mdr.config(batch=B, seq=S, heads=H, head_dim=D, block=blk, subspaces=w.subspaces, codes=w.codes,
                     capacity=w.capacity, probes=w.probes, max_cand=w.max_cand, remote=w.remote, local=w.local,
                     dtype=w.dtype)
    state = mdr.decode_state(cfg)
    n0 = S - blk
    mdr.mdr_decode_prime(cfg, k, run.cb, run.bias, n0, state)
    out = torch.empty(B, H, 1, D, dtype=q.dtype, device="cuda")
    sel = torch.empty(B, H, 1, w.remote, dtype=torch.int32, device="cuda")
    qs = [q[:, :, t:t + 1].contiguous() for t in range(n0, n0 + warmup + steps)]
    sels = []
    for i in range(warmup):
        mdr.mdr_decode_step(cfg, qs[i], k, v, run.cb, run.bias, None, n0 + i, out, sel, state)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(warmup, warmup + steps):
        mdr.mdr_decode_step(cfg, qs[i], k, v, run.cb, run.bias, None, n0 + i, out, sel, state)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # compulsory bytes of the timed steps, from their selections (re-run untimed to read them)
    mdr.mdr_decode_prime(cfg, k, run.cb, run.bias, n0, state)
    nbytes = 0
    for i in range(warmup + steps):
        t = n0 + i
        mdr.mdr_decode_step(cfg, qs[i], k, v, run.cb, run.bias, None, t, out, sel, state)
        if i >= warmup:
            nsel = int((sel >= 0).sum().item())
            local = t - max(0, (t // blk - w.local + 1) * blk) + 1
            nbytes += 2 * D * e * B * H + nsel * blk * 2 * D * e + B * H * local * 2 * D * e
    nbytes /= steps
    return {"workload": f"sweep context {n0}-{n0 + warmup + steps} tokens, B{B} H{H}, one new token per call",
            "batch": B, "ms_per_step": round(ms, 5), "tokens_per_s": round(B / (ms * 1e-3), 1),
            "alg_bytes_per_step": int(nbytes), "alg_gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def backward_bench(run, hip, overhead, steps=20, warmup=3):
    """The attention backward (dQ, dK, dV under the forward's selection) on the same workload, timed
    per kernel with HIP events like the forward.  Compulsory bytes: Q, K, V, O, dO read and dQ, dK,
    dV written once, plus the selection and the fp32 normaliser; algorithmic flops 10 D per visited
    (query, key) pair (S, dP, dV, dK, dQ; the forward's S and PV count 4 D)."""
    import torch

    import synth

    mdr, w = run.mdr, run.w
    B, H, S, D, R = w.batch, w.heads, w.seq, w.head_dim, w.remote
    e = 2 if w.dtype == "bf16" else 4
    sel = run.rt["sel"]
    g = torch.from_numpy(synth.make_grad_inputs(w, 1)).to("cuda").to(run.q.dtype)
    out = torch.empty_like(run.q)
    lse = torch.empty(B, H, S, dtype=torch.float32, device="cuda")
    mdr.mdr_stage_attend_lse(run.cfg, run.q, run.k, run.v, sel, out, lse, run.ws)
    dq, dk, dv = (torch.empty_like(run.q) for _ in range(3))
    args = (run.cfg, run.q, run.k, run.v, sel, out, lse, g, dq, dk, dv)
    for _ in range(warmup):
        mdr.mdr_stage_attend_backward(*args, run.ws)
    nk = mdr.MDR_BACKWARD_KERNELS
    events = hip.create(steps * (nk + 1))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        mdr.mdr_stage_attend_backward_profiled(*args, events[i * (nk + 1):(i + 1) * (nk + 1)], run.ws)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    per = [max(0.0, sum(hip.elapsed_ms(events[i * (nk + 1) + k], events[i * (nk + 1) + k + 1])
                        for i in range(steps)) / steps - overhead) for k in range(nk)]
    hip.destroy(events)
    pairs = int((sel >= 0).sum().item())
    qkv = B * H * S * D * e
    alg_bytes = 8 * qkv + B * H * S * (R * 4 + 4)
    flops = 10 * D * attended_pairs(w, pairs)
    total = sum(per)
    return {"workload": describe(w) + ", upstream gradient ~ N(0, 1), the forward's own selection",
            "ms_per_call": round(wall * 1e3, 4), "kernels_ms": {n: round(x, 5) for n, x in zip(mdr.BACKWARD_KERNELS, per)},
            "alg_bytes": alg_bytes, "alg_flops": flops, "tokens_per_s": round(B * S / wall, 1),
            "hbm_frac": round(alg_bytes / (total * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "mfma_frac": round(flops / (total * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype], 4)}


def overflow_stress(mdr, seed, steps=20, warmup=3):
    """The overflow stress test the pages ask for (remio.ai, "What sparse attention researchers
    should watch next"): skewed code biases -kappa ln(c + 1) send many blocks and queries to few
    addresses; for the drop and redirect policies report overflow, dropped candidates per token,
    candidates per token, the step time's spread, and route recall of a planted block.
      skew shape:   B2 H8 S16384 D128 block 64, 3x8 codes, capacity 8, P6, R8, bf16, kappa 0 .. 1
      recall shape: B16 H4 S2048 D64 block 64, 2x8 codes, capacity 2, P16, M5, R2, fp32; route recall =
                    share of the last query block's tokens whose selection holds the planted block."""
    import numpy as np
    import torch

    import synth

    def timed(run):
        for _ in range(warmup):
            run.step()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(steps):
            run.step()
            ev[i + 1].record()
        torch.cuda.synchronize()
        ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
        return [round(float(x), 4) for x in np.percentile(ms, [10, 50, 90])] + [round(float(ms.max()), 4)]

    out = {"skew": [], "recall": []}
    ws = make_workload("skew", 0)
    ws = __import__("dataclasses").replace(ws, batch=2, heads=8)
    inp = synth.make_core_inputs(ws, seed)
    for kappa in (0.0, 0.11, 0.5, 1.0):
        bias = synth.zipf_code_bias(ws.heads, ws.subspaces, ws.codes, kappa)
        row = {"kappa": kappa}
        for policy in ("drop", "redirect"):
            run = Run(mdr, ws, seed, policy, bias=bias, inputs=inp)
            q = timed(run)
            rt = run.rt
            row[policy] = {"overflow": int(rt["overflow"].sum().item()),
                           "dropped_per_token": round(float(rt["n_drop"].float().mean().item()), 3),
                           "cand_per_token": round(float(rt["n_cand"].float().mean().item()), 3),
                           "step_ms_p10_p50_p90_max": q}
            del run
        out["skew"].append(row)
    wr = __import__("dataclasses").replace(make_workload("recall", 0), capacity=2)
    inp = synth.make_core_inputs(wr, seed)
    planted = torch.from_numpy(inp["planted"]).cuda().long()
    last = slice((wr.nblocks - 1) * wr.block, wr.seq)
    for kappa in (0.0, 0.5, 1.0, 2.0):
        bias = synth.zipf_code_bias(wr.heads, wr.subspaces, wr.codes, kappa)
        row = {"kappa": kappa}
        for policy in ("drop", "redirect"):
            run = Run(mdr, wr, seed, policy, bias=bias, inputs=inp)
            run.step()
            torch.cuda.synchronize()
            sel = run.rt["sel"][:, :, last].long()
            hit = (sel == planted[:, None, None, None]).any(dim=-1)
            row[policy] = {"route_recall": round(float(hit.float().mean().item()), 4),
                           "overflow": int(run.rt["overflow"].sum().item()),
                           "dropped_per_token": round(float(run.rt["n_drop"].float().mean().item()), 3)}
            del run
        out["recall"].append(row)
    out["note"] = ("synthetic keys and untrained random codebooks: the recall figures describe the overflow "
                   "mechanism, not the pages' trained-router result")
    return out


def mixer_bench(mdr, hip, seed, steps=20, warmup=3):
    """The stateless mixer [B, S, W] -> delta on the 32K sweep shape with width H*D = 512: the fused
    Q/K/V projection (RoPE, block summaries and addresses in its epilogue), the core, the output
    projection.  Timed per call with HIP events; projection flops 2 * B*S * W * 3HD (+ 2 * B*S * HD * W)."""
    import dataclasses

    import torch

    import synth

    w = dataclasses.replace(make_workload("sweep", 0), width=512)
    inp = synth.make_mixer_inputs(w, seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {n: torch.from_numpy(inp[n]).to("cuda").to(dt) for n in ("x", "wq", "wk", "wv", "wo")}
    cb = torch.from_numpy(inp["codebook"]).cuda()
    cfg = mdr.config(batch=w.batch, seq=w.seq, heads=w.heads, head_dim=w.head_dim, width=w.width, block=w.block,
                     subspaces=w.subspaces, codes=w.codes, capacity=w.capacity, probes=w.probes,
                     max_cand=w.max_cand, remote=w.remote, local=w.local, dtype=w.dtype, rope_base=w.rope_base)
    ws = mdr.workspace(cfg)
    delta = torch.empty_like(t["x"])
    call = lambda: mdr.mdr_mixer_forward(cfg, t["x"], t["wq"], t["wk"], t["wv"], t["wo"], cb, None, delta, None, ws)
    for _ in range(warmup):
        call()
    ev = hip.create(2)
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    hip.record(ev[0], stream)
    for _ in range(steps):
        call()
    hip.record(ev[1], stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(ev[0], ev[1]) / steps
    hip.destroy(ev)
    M, HD = w.batch * w.seq, w.heads * w.head_dim
    return {"workload": f"mixer B{w.batch} S{w.seq} W{w.width} H{w.heads} D{w.head_dim} block{w.block} "
                        f"{w.subspaces}x{w.codes} codes cap{w.capacity} P{w.probes} R{w.remote} L{w.local} {w.dtype}",
            "ms_per_call": round(ms, 4), "tokens_per_s": round(M / (ms * 1e-3), 1),
            "projection_flops": 2 * M * w.width * 3 * HD + 2 * M * HD * w.width}


_CPU_JOB = {}  # the workload and its inputs, set before the worker processes are forked


def _cpu_task(task):
    """One share of the CPU baseline: the packed C oracle (oracle/mdr_packed.c: routing with its head's
    index build, then gathered fp64 attention) over a contiguous token range of one head, on one thread.
    With kind "numpy" the NumPy oracle does the same share instead."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    kind, h, t0, t1 = task
    w, inp = _CPU_JOB["w"], _CPU_JOB["inputs"]
    q, k, v = (inp[n][0, h] for n in ("q", "k", "v"))
    bias = None if inp["bias"] is None else inp["bias"][h]
    if kind == "packed":
        from oracle import packed

        packed.packed_forward(q, k, v, inp["codebook"][h], bias, w, t0, t1)
        return t1 - t0
    import oracle

    toks = np.arange(t0, t1)
    with threadpool_limits(1):
        r = oracle.route_head(q, k, inp["codebook"][h], bias, w, tokens=toks)
        oracle.attention_packed(q, k, v, r["sel"], w.block, w.local, tokens=toks)
    return t1 - t0


def host_cpu():
    """(usable cores for the pool, cores this process may run on, CPU model name)."""
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return max(1, min(avail, 16)), avail, model


def cpu_baseline(w, inputs, heads, seed=0, sweep=True):
    """The oracle on the host's cores: the packed C oracle (the timed value) and the NumPy oracle beside
    it, each over (head, token range) shares of the sample on a pool of forked worker processes (one
    thread each) so every core has work, then on one thread over one head for the per-core rate; with
    sweep, the packed oracle's one-thread time on one head at 4K-32K tokens and its fitted exponent.
    Runs before the process initialises the GPU, so forking is safe."""
    import multiprocessing as mp

    import synth
    from oracle import packed

    packed._load()  # built (if needed) before the workers fork
    heads = min(heads, w.heads)
    cores, avail, model = host_cpu()
    parts = max(1, -(-cores // heads))
    bounds = [(w.seq * p) // parts for p in range(parts + 1)]
    _CPU_JOB.update(w=w, inputs=inputs)

    def pooled(kind, reps=1):
        tasks = [(kind, h, bounds[p], bounds[p + 1]) for h in range(heads) for p in range(parts)] * reps
        t0 = time.perf_counter()
        with mp.get_context("fork").Pool(cores) as pool:
            done = sum(pool.map(_cpu_task, tasks, chunksize=1))
        dt = time.perf_counter() - t0
        t1 = time.perf_counter()
        _cpu_task((kind, 0, 0, w.seq))
        dt1 = time.perf_counter() - t1
        return done / w.heads / dt, w.seq / w.heads / dt1, dt, dt1, len(tasks) // reps

    rate, rate1, dt, dt1, ntasks = pooled("packed", reps=3)  # the sample three times: about 10 s of CPU work
    nrate, nrate1, ndt, ndt1, _ = pooled("numpy")
    res = {"value": round(rate, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "cpu_model": model, "host_cpus_visible": avail,
           "one_thread_tokens_per_s": round(rate1, 2),
           "sample": f"the packed C oracle (oracle/mdr_packed.c, gcc -O2, one thread per process): batch 0, heads "
                     f"0-{heads - 1} of {w.heads}, all {w.seq} tokens each, split into {ntasks} (head, token range) "
                     f"shares over {cores} forked worker processes; each share routes its tokens (with its head's "
                     f"index build) and runs gathered fp64 attention; the shares three times over; tokens/s "
                     f"counts a token as all {w.heads} heads; {dt:.2f} s wall. One thread, head 0 alone: {dt1:.2f} s",
           "numpy_oracle": {"tokens_per_s": round(nrate, 2), "one_thread_tokens_per_s": round(nrate1, 2),
                            "note": f"the NumPy oracle (oracle/mdr_oracle.py) on the same shares: {ndt:.1f} s wall; "
                                    f"one thread, head 0: {ndt1:.1f} s"}}
    if sweep and w.name == "sweep":
        import numpy as np

        seqs, secs, pairs = [4096, 8192, 16384, 32768], [], []
        for S in seqs:
            ws = synth.workload("sweep", seq=S)
            inp = inputs if S == w.seq else synth.make_core_inputs(ws, seed)
            bias = None if inp["bias"] is None else inp["bias"][0]
            args = [inp[n][0, 0] for n in ("q", "k", "v")] + [inp["codebook"][0], bias, ws]
            best = float("inf")
            for _ in range(2):  # the faster of two runs
                t1 = time.perf_counter()
                sel, _ = packed.packed_forward(*args)
                best = min(best, time.perf_counter() - t1)
            secs.append(best)
            t = np.arange(S)
            local = t - np.maximum(0, (t // ws.block - ws.local + 1) * ws.block) + 1
            pairs.append(int((sel >= 0).sum()) * ws.block + int(local.sum()))
        slope = float(np.polyfit(np.log(seqs), np.log(secs), 1)[0])
        pslope = float(np.polyfit(np.log(pairs), np.log(secs), 1)[0])
        res["exponent"] = {"seqs": seqs, "s_one_head_one_thread": [round(x, 4) for x in secs],
                           "attended_pairs_one_head": pairs, "slope_vs_seq": round(slope, 3),
                           "slope_vs_attended_pairs": round(pslope, 3),
                           "note": "the packed C oracle on head 0 of the sweep workload at each length, one thread, "
                                   "the faster of two runs (routing with the index build, and gathered attention); "
                                   "the pages report 0.993 "
                                   "for their packed CPU routing over 4K-32K (CPU not stated)"}
    return res


# ----------------------------------------------------------------------------- PMC ingest

def _read_pmc(path):
    rows = list(csv.DictReader(open(path)))
    out = []
    for r in rows:
        name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
        cname = r.get("Counter_Name") or r.get("Counter") or ""
        val = float(r.get("Counter_Value") or r.get("Value") or 0.0)
        disp = r.get("Dispatch_Id") or r.get("Dispatch_ID") or r.get("Correlation_Id") or ""
        out.append((disp, name, cname, val))
    return out


def ingest_pmc(fetch_csv, write_csv, w):
    """Per-launch HBM bytes of each kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), calibrated on a
    plain elementwise copy of CALIB_BYTES (read CALIB_BYTES, write CALIB_BYTES)."""
    def per_kernel(path, counter):
        acc = {}
        for disp, name, cname, val in _read_pmc(path):
            if cname != counter:
                continue
            acc.setdefault(name, {}).setdefault(disp, 0.0)
            acc[name][disp] += val
        return {n: sum(d.values()) / len(d) for n, d in acc.items()}, {n: len(d) for n, d in acc.items()}

    fetch, nf = per_kernel(fetch_csv, "FETCH_SIZE")
    write, nw = per_kernel(write_csv, "WRITE_SIZE")
    calib_f = [v for n, v in fetch.items() if "neg" in n.lower()]
    calib_w = [v for n, v in write.items() if "neg" in n.lower()]
    if not calib_f or not calib_w:
        raise SystemExit("no calibration copy dispatch found (run bench.py with --calib-copy)")
    kib = CALIB_BYTES / 1024.0
    sf, sw = kib / calib_f[0], kib / calib_w[0]
    res = {"workload": describe(w), "commands": PMC_COMMANDS, "calibration": {"copy_bytes": CALIB_BYTES, "fetch_kib": calib_f[0],
                                                   "write_kib": calib_w[0], "fetch_scale": sf, "write_scale": sw},
           "kernels": {}}
    for k, sym in KERNEL_SYMBOL.items():
        fn = [n for n in fetch if _has(sym, n)]
        wn = [n for n in write if _has(sym, n)]
        if not fn or not wn:
            continue
        fb = fetch[fn[0]] * sf * 1024
        wb = write[wn[0]] * sw * 1024
        res["kernels"][k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb,
                             "dispatches": nf[fn[0]], "source_sha": source_digest(k)}
    os.makedirs(os.path.dirname(traffic_path(w)), exist_ok=True)
    json.dump(res, open(traffic_path(w), "w"), indent=1)
    print(json.dumps(res, indent=1))


# ----------------------------------------------------------------------------- main

def summarize_rocprof(stats_csv, command, w, bench_log=None, stem="routed_attention_kernels"):
    """Short markdown table of the library's kernels from a rocprofv3 kernel_stats.csv, with the
    HIP-event averages bench.py printed in the same run (bench_log: its stdout) beside them."""
    rows = list(csv.DictReader(open(stats_csv)))
    events, timed = {}, None
    if bench_log:
        for line in open(bench_log):
            if line.startswith("{"):
                rec = json.loads(line)
                ks = rec.get("kernels", {})
                events = {k: v["ms"] * 1e3 for k, v in ks.items()}
                if "roofline" in rec:
                    timed = (rec["roofline"]["kernel"], rec["roofline"]["ms_timed_region"] * 1e3)
    lines = [f"# rocprofv3 kernel statistics: routed attention, {describe(w)}", "",
             "Command (run from the repository root on one MI355X):", "", f"    {command}", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time | bench.py HIP-event avg us |",
             "|---|---|---|---|---|---|---|"]
    for k, sym in KERNEL_SYMBOL.items():
        for r in rows:
            if _has(sym, r["Name"]):
                ev = f"{events[k]:.2f}" if k in events else "-"
                lines.append(f"| {k} (`{_label(sym)}`) | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                             f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                             f"{float(r['Percentage']):.1f}% | {ev} |")
    if timed:
        stage = list(STAGE_KERNELS)
        avgs = [next((float(r["AverageNs"]) / 1e3 for r in rows if _has(KERNEL_SYMBOL[k], r["Name"])), None)
                for k in stage]
        tot = sum(avgs) if all(x is not None for x in avgs) else None
        lines += ["", f"The HIP-event column is bench.py's pass with an event before every kernel.  In its timed "
                      f"region (events around the attention stage only) {timed[0]} averaged {timed[1]:.2f} us"
                      + (f"; rocprofv3, every launch in the run, sums the stage's kernels to {tot:.2f} us." if tot
                         else ".")]
    bwd = {}
    if bench_log:
        for line in open(bench_log):
            if line.startswith("{") and "backward" in json.loads(line):
                bwd = {k: v * 1e3 for k, v in json.loads(line)["backward"]["kernels_ms"].items()}
    bl = []
    for k, sym in BACKWARD_SYMBOL.items():
        for r in rows:
            if _has(sym, r["Name"]):
                ev = f"{bwd[k]:.2f}" if k in bwd else "-"
                bl.append(f"| {k} (`{_label(sym)}`) | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                          f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                          f"{float(r['Percentage']):.1f}% | {ev} |")
    if bl:
        lines += ["", "Backward (mdr_stage_attend_backward on the forward's selection):", "",
                  "| kernel | calls | avg us | min us | max us | share of GPU time | bench.py HIP-event avg us |",
                  "|---|---|---|---|---|---|---|"] + bl
    ml = []
    for k, subs in MIXER_SYMBOL.items():
        for r in rows:
            if all(x in r["Name"] for x in subs):
                ml.append(f"| {k} (`{subs[0]}`) | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                          f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                          f"{float(r['Percentage']):.1f}% |")
    if ml:
        lines += ["", "Mixer (mdr_mixer_forward at width 512; its core kernels are counted in the table above):", "",
                  "| kernel | calls | avg us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"] + ml
    known = list(KERNEL_SYMBOL.values()) + list(BACKWARD_SYMBOL.values()) + [v[0] for v in MIXER_SYMBOL.values()]
    other = sum(float(r["Percentage"]) for r in rows if not any(_has(sym, r["Name"]) for sym in known))
    lines += ["", f"Other kernels (input generation, torch copies, routing statistics): {other:.1f}% of GPU time.", ""]
    out = os.path.join(ROOT, "profiles", f"{stem}_{w.name}_{w.seq // 1024}k.md")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    open(out, "w").write("\n".join(lines))
    print(open(out).read())


def memory_split(mdr, w, cfg):
    """Device memory of one call, split the way the pages ask (remio.ai, "What sparse attention
    researchers should watch next": weights, routing buffers, posting lists and K/V reported apart)."""
    e = 2 if w.dtype == "bf16" else 4
    BH = w.batch * w.heads
    parts = mdr.workspace_breakdown(cfg)
    row = BH * w.seq * w.head_dim * e
    return {"weights_and_codebook": w.heads * w.subspaces * w.codes * (w.head_dim + 1) * 4,
            "k_v": 2 * row, "q_and_out": 2 * row,
            "posting_lists": parts["posting_lists"],
            "routing_buffers": {k: parts[k] for k in ("summaries", "selection", "pair_lists", "partials")},
            "backward_scratch": parts["backward"], "workspace_total": parts["total"],
            "note": "bytes; the workspace is caller-owned and sized by mdr_workspace_size; weights are the "
                    "fp32 codebook and bias (the core takes post-RoPE Q/K/V, so it has no projection weights)"}


def main(argv=None):
    a = parse(argv)
    w = make_workload(a.workload, a.seq)
    if a.ingest_pmc:
        ingest_pmc(*a.ingest_pmc, w)
        return 0
    if a.summarize_rocprof:
        summarize_rocprof(*a.summarize_rocprof, w, a.bench_log, a.profile_name)
        return 0
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only: the path shards over (batch, head) with no "
                                   "communication, so N GPUs would each run this benchmark on their own share; "
                                   "run with --gpus 1"}))
        return 2
    import synth

    inputs = None
    cpu = None
    if not a.no_cpu and not a.mixer_only:
        # the CPU baseline forks worker processes, so it runs before anything touches the GPU
        inputs = synth.make_core_inputs(w, a.seed)
        cpu = cpu_baseline(w, inputs, a.cpu_heads, a.seed, sweep=not a.no_sweep)
    import torch

    import learned_product_hash_amd as mdr

    torch.cuda.init()
    hip = HipEvents()
    if a.mixer_only:
        print(json.dumps({"mixer": mixer_bench(mdr, hip, a.seed)}))
        return 0
    if a.calib_copy:
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    run = Run(mdr, w, a.seed, inputs=inputs)
    wall, per, ev_overhead, stage_ms = timed_region(run, hip, a.steps, a.warmup)
    plain = plain_region(run, a.steps)
    cold_q, cold_per = (None, None) if a.no_cold else cold_region(run, hip, min(a.steps, 20), ev_overhead)
    st = run.routing_stats()
    names = list(mdr.CORE_KERNELS)
    dbytes = design_bytes(w, st)
    kernels = {}
    for n, ms in zip(names, per):
        kernels[n] = {"ms": round(ms, 5), "design_bytes": dbytes.get(n),
                      "design_gbps": round(dbytes[n] / (ms * 1e-3) / 1e9, 1) if ms > 0 and n in dbytes else None}
    stage_names = [n for n in names if n in STAGE_KERNELS]
    alg = stage_bytes(w)
    achieved = alg / (stage_ms * 1e-3) / 1e9
    tr = [load_traffic(w, n) for n in stage_names]
    traffic = None if any(t is None for t in tr) else round(sum(tr))
    tokens = w.batch * w.seq
    res = {
        "metric": "routed-attention tokens/sec at 32K seq; achieved HBM GB/s vs peak",
        "value": round(tokens * a.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(wall / a.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian Q/K/V with balanced planted block addresses)",
        "config": {"workload": describe(w), "global_batch": w.batch, "seq_len": w.seq, "heads": w.heads,
                   "head_dim": w.head_dim, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "mdr_sel_attn (" + " + ".join(stage_names) + ")",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "alg_bytes": alg, "ms_timed_region": round(stage_ms, 5),
                     "note": "achieved = compulsory bytes of the stage (Q, K, V and O once, plus the selection) / "
                             "the stage's average duration over the timed region (HIP events on the call's stream "
                             "before its first kernel and after its last); traffic = FETCH_SIZE + WRITE_SIZE of the "
                             "stage's kernels per call, calibrated on a plain copy: bytes between the L2s and the "
                             "fabric, served by HBM or the 256 MB last-level cache, so an upper bound on DRAM bytes. "
                             "The pair binning that feeds the stage (attn_bin) is in attention_stage.with_binning"},
        "kernels": kernels,
        "attention_stage": attention_stage(w, stage_ms, st["pairs"], stage_names,
                                           kernels["attn_bin"]["ms"] if "attn_bin" in kernels else None),
        "plain_entry_point_ms_per_step": round(plain / a.steps * 1e3, 4),
        "event_overhead_ms": round(ev_overhead, 5),
        "profiled_step_ms_p10_p50_p90": run.step_quantiles,
        "cold_caches": None if cold_q is None else {
            "note": "a 512 MiB write before each step evicts the last-level cache and the L2s; the step is "
                    "bracketed by events, the write is not",
            "step_ms_p10_p50_p90": cold_q, "kernels_ms": {n: round(ms, 5) for n, ms in zip(names, cold_per)}},
        "routing": st,
        "memory": memory_split(mdr, w, run.cfg),
    }
    if not a.no_decode and a.workload == "sweep":
        res["decode"] = [decode_bench(run, b) for b in (1, 16)]
    if not a.no_backward:
        res["backward"] = backward_bench(run, hip, ev_overhead)
    if not a.no_mixer and a.workload == "sweep":
        res["mixer"] = mixer_bench(mdr, hip, a.seed)
    if not a.no_stress and a.workload == "sweep":
        res["overflow_stress"] = overflow_stress(mdr, a.seed)
    if not a.no_sweep and a.workload == "sweep":
        res["exponent"] = exponent_sweep(mdr, (4096, 8192, 16384, 32768), a.seed)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
