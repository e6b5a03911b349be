#!/usr/bin/env python3
"""Benchmark of the GDN speculative-verify hot path on one MI355X.

A step is one speculative pass over a 48-GDN-layer model (32 heads per layer,
dk = dv = 128, bf16 q/k/v, fp32 state): one gdn_commit_verify launch over all
48 layers commits the block pending from the previous pass at that pass's
accepted length n ~ Uniform{0..8} (the same n for all layers, read on the
device) and verifies the next T = 8 block.  The headline value is committed
tokens per second; the accepted lengths come in pairs (n, 8 - n), so every
timed window commits exactly 4 tokens a pass on average.

The same passes as separate gdn_verify_block + gdn_commit calls, each kernel
alone, the chunked prefill (one layer, 32 heads, 4,096-token prompt, chunk 64;
and 48 layers x 32,768 tokens followed by 256 rounds on the prefilled state),
plain decode, acceptance, the full-attention layers and the GDN mixer are
timed in the same run and reported beside it.

Inputs are synthetic (speculative_verify_amd.inputs) and already resident in
HBM.  Four independent buffer sets rotate across passes, so no kernel finds
its state still in the 256 MB Infinity Cache from the previous kernel.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
KERNEL_SOURCES = ["speculative_verify_amd/csrc/verify.hip", "speculative_verify_amd/csrc/commit.hip",
                  "speculative_verify_amd/csrc/prefill.hip", "speculative_verify_amd/csrc/gdn_internal.h"]

# Workload sizes.
LAYERS, HEADS, DK, DV, T = 48, 32, 128, 128, 8
PF_B, PF_H, PF_L, PF_C = 1, 32, 4096, 64
PFL_B, PFL_L = 48, 32768   # the long-context prompt: all 48 GDN layers, 32K tokens
RING, LAG = 4, 2


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--prefill-reps", type=int, default=20)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-accept", action="store_true")
    p.add_argument("--no-attn", action="store_true")
    p.add_argument("--no-mixer", action="store_true")
    p.add_argument("--no-prefill-long", action="store_true",
                   help="skip the 48-layer, 32,768-token prefill (about 65 GB of device memory)")
    p.add_argument("--decode-steps", type=int, default=10000)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=15.0)
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="after the bench, run 3 plain device copies of this many MiB (a "
                        "reference kernel of known traffic for hardware counters)")
    p.add_argument("--summarize", metavar="DIR", default=None,
                   help="no GPU work: turn the rocprofv3 outputs under DIR (stats/, fetch/, "
                        "write/ and commands.txt) into the summaries under profiles/")
    return p.parse_args()


def verify_bytes(B, H, dk, dv, T, es):
    """Algorithmic HBM bytes of one verify launch: state read once, the block's
    inputs read once, outputs and the block record written once."""
    state = B * H * dv * dk * 4
    inputs = B * T * H * (2 * dk + dv) * es + B * T * H * 8
    outputs = B * T * H * dv * 4
    record = B * T * H * (dv * 4 + dk * es + 4) + B * 16
    return state + inputs + outputs + record


def commit_bytes(B, H, dk, dv, n, es):
    """Algorithmic HBM bytes of one commit launch at accepted length n (same n
    for every instance): the state read and written once when n >= 1, plus the
    record rows it replays; n = 0 touches only the control words."""
    ctrl = B * (16 + 4 + 4)
    if n == 0:
        return ctrl
    return 2 * B * H * dv * dk * 4 + B * n * H * (dv * 4 + dk * es + 4) + ctrl


def fused_bytes(B, H, dk, dv, T, n, es):
    """Algorithmic HBM bytes of one gdn_commit_verify launch at accepted length n:
    the verify's bytes plus the commit's, less the commit's state read (the state
    is read once for both)."""
    extra = commit_bytes(B, H, dk, dv, n, es)
    if n > 0:
        extra -= B * H * dv * dk * 4
    return verify_bytes(B, H, dk, dv, T, es) + extra


def mixer_fused_bytes(B, H, Hk, d, T, n):
    """Algorithmic HBM bytes of one gdn_mixer_commit_verify launch at accepted
    length n: those of gdn_commit_verify with bf16 inputs, with the block's q, k,
    v replaced by the raw rows (q/k channels once per q/k head), the filter
    history, the output gate z, and the filter taps and norm weight; the gate
    pre-activations a, b take the place of g, beta byte for byte."""
    cdim = 2 * Hk * d + H * d
    qkv = B * T * H * 3 * d * 2
    raw = B * T * cdim * 2 + B * 3 * cdim * 2 + B * T * H * d * 2 + cdim * 16 + d * 4 + H * 8
    return fused_bytes(B, H, d, d, T, n, 2) - qkv + raw


def prefill_bytes(B, H, dk, dv, L):
    return B * L * H * (2 * dk + dv) * 2 + B * L * H * 8 + B * L * H * dv * 4 + 2 * B * H * dv * dk * 4


def prefill_flops(B, H, dk, dv, L, C):
    """Causal flop count of the chunk form per token and head:
    state-coupled 6 dk dv (K S^T, Q S^T, the state update), intra-chunk
    C (3 dk + 2 dv) (causal halves of K K^T, Q K^T, Tm V, Tm K and P D) and the
    triangular solve C^2 / 3."""
    per = 6 * dk * dv + C * (3 * dk + 2 * dv) + C * C / 3
    return B * L * H * per


def sources_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "hbm_traffic_verify_commit_48x32_T8_prefill_32x4096.json")
STATS_MD = os.path.join(ROOT, "profiles", "kernel_stats_verify_commit_48x32_T8_prefill_32x4096.md")
MFMA_JSON = os.path.join(ROOT, "profiles", "mfma_prefill_32x4096_and_48x32x32768.json")


def load_mfma(leg):
    """The MFMA counter summary of a prefill leg, only if it was taken on the
    current kernel sources."""
    try:
        with open(MFMA_JSON) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256_16") != sources_hash():
        return None
    k = t.get("legs", {}).get(leg)
    return None if k is None else {c: k[c] for c in ("executed_over_algorithmic", "executed_frac_of_peak",
                                                     "mfma_busy_frac")}


def load_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, only if
    it was taken on the current kernel sources."""
    path = TRAFFIC_JSON
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256_16") != sources_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def accept_plan(args):
    """The accepted lengths of every region, in launch order: warmup and headline
    passes of the fused kernel, the separate calls' commits, the commit-alone
    region's commits.  Each region draws its own paired sequence (n, 8 - n)."""
    from speculative_verify_amd.inputs import make_accepts_paired

    return {"warm": [int(v) for v in make_accepts_paired(args.warmup, T, seed=args.seed)],
            "head": [int(v) for v in make_accepts_paired(args.steps, T, seed=args.seed + 1)],
            "sep": [int(v) for v in make_accepts_paired(args.steps, T, seed=args.seed + 2)],
            "com": [int(v) for v in make_accepts_paired(args.steps, T, seed=args.seed + 3)]}


class KernelEvents:
    """Timing events on the launch stream.  HIP events created with
    hipEventDisableSystemFence: an event without the flag releases to system
    scope when it completes, which adds a few microseconds to the interval
    around a 30 us kernel.  Falls back to torch's events if the HIP runtime
    cannot be reached."""

    def __init__(self, torch, stream):
        import ctypes

        self.ctypes, self.torch = ctypes, torch
        self.stream = ctypes.c_void_p(stream.cuda_stream)
        try:
            self.hip = ctypes.CDLL("libamdhip64.so.7")
            e = self._create()
            self.hip.hipEventDestroy(e)
            self.kind = "hipEvent, hipEventDisableSystemFence"
        except (OSError, RuntimeError):
            self.hip = None
            self.kind = "torch.cuda.Event"

    def _create(self):
        e = self.ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ctypes.byref(e), self.ctypes.c_uint(0x20000000)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e

    def new(self):
        return self._create() if self.hip else self.torch.cuda.Event(enable_timing=True)

    def record(self, e):
        if self.hip:
            if self.hip.hipEventRecord(e, self.stream) != 0:
                raise RuntimeError("hipEventRecord failed")
        else:
            e.record()

    def ms(self, a, b):
        if not self.hip:
            return a.elapsed_time(b)
        f = self.ctypes.c_float()
        if self.hip.hipEventElapsedTime(self.ctypes.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def free(self, evs):
        if self.hip:
            for e in evs:
                self.hip.hipEventDestroy(e)


def cpu_baseline(args):
    """The fp64 oracle on a bounded sample of the same pass: verify + commit of
    the 48-layer block, repeated until about cpu_budget_s seconds of work."""
    import numpy as np
    import torch

    import oracle
    from speculative_verify_amd.inputs import make_accepts_paired, make_inputs

    x = make_inputs(LAYERS, HEADS, DK, DV, T, seed=args.seed + 1000)
    f64 = [t.double().numpy() for t in (x.S0, x.q, x.k, x.v, x.g, x.beta)]
    ns = make_accepts_paired(64, T, seed=args.seed + 1000).numpy()
    passes, tokens = 0, 0
    t0 = time.perf_counter()
    while True:
        n = int(ns[passes % len(ns)])
        oracle.verify(*f64)
        oracle.commit(*f64, np.full(LAYERS, n, np.int32))
        passes += 1
        tokens += n
        if time.perf_counter() - t0 >= args.cpu_budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{passes} passes (48 layers x 32 heads, d=128, T=8, verify + commit at "
                      f"n~U{{0..8}}, {tokens} tokens) in {dt:.1f} s, fp64"}


def main():
    args = parse()
    if args.summarize:
        summarize_profiles(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the GDN path is "
              f"single-GPU by design and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch

    import speculative_verify_amd.gdn as G
    from speculative_verify_amd.inputs import make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16
    es = 2

    # Buffer sets: state, block inputs, outputs, two records (alternating).  Four
    # sets rotate, so no kernel finds its 96 MiB state still in the 256 MB
    # Infinity Cache from the previous kernel.
    sets = []
    for r in range(RING):
        x = make_inputs(LAYERS, HEADS, DK, DV, T, dtype=dt, seed=args.seed + r, device=dev,
                        device_gen=True)
        o = torch.empty(LAYERS, T, HEADS, DV, dtype=torch.float32, device=dev)
        recs = [G.new_record(x.S0, T, dt) for _ in range(3)]
        sets.append((x, o, recs))
    # Accepted lengths: every region draws its own paired sequence (n, 8 - n), so
    # each timed window commits exactly 4 tokens per pass on average.
    plan = accept_plan(args)
    n_head, n_sep, n_com = plan["head"], plan["sep"], plan["com"]
    per_layer = lambda n: torch.tensor(n, dtype=torch.int32).view(-1, 1).expand(-1, LAYERS).contiguous().to(dev)
    n_head_d, n_sep_d, n_com_d = per_layer(n_head), per_layer(n_sep), per_layer(n_com)
    pos = torch.zeros(LAYERS, dtype=torch.int32, device=dev)

    # Fused path (the headline): step s runs on set s % RING one
    # gdn_commit_verify -- commit the block pending there at n[s], then verify
    # the set's next block -- alternating the set's first two records.
    def fused(s, n):
        x, o, recs = sets[s % RING]
        visit = s // RING
        G.gdn_commit_verify(x.S0, recs[visit % 2], n, x.q, x.k, x.v, x.g, x.beta, o, recs[(visit + 1) % 2],
                            pos=pos)

    for r in range(RING):  # a pending block on every set
        x, o, recs = sets[r]
        G.gdn_verify_block(x.S0, x.q, x.k, x.v, x.g, x.beta, o, recs[0])
    warm_n = per_layer(plan["warm"]) if args.warmup else None
    for s in range(args.warmup):
        fused(s, warm_n[s])
    torch.cuda.synchronize()

    # Headline region: exactly `steps` passes back to back, nothing between the
    # launches.  The wall clock runs between device synchronisations; two events
    # on the launch stream bracket the same launches, so their interval over
    # `steps` is the kernel's average duration per launch (back-to-back launches,
    # no per-launch events), never above the wall time per step.
    kev = KernelEvents(torch, torch.cuda.current_stream())
    ev_a, ev_b = kev.new(), kev.new()
    t0 = time.perf_counter()
    kev.record(ev_a)
    for i in range(args.steps):
        fused(args.warmup + i, n_head_d[i])
    kev.record(ev_b)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_fus_ms = kev.ms(ev_a, ev_b) / args.steps
    n_timed = [int(v) for v in n_head]
    tokens = sum(n_timed)
    s1 = args.warmup + args.steps

    # Separate calls: the same passes as gdn_verify_block + gdn_commit.  Pass p is
    # verified on set p % RING and committed LAG steps later (so that a commit
    # never finds the state its verify just read in the cache); the set's third
    # record carries the block.
    def verify(p):
        x, o, recs = sets[p % RING]
        G.gdn_verify_block(x.S0, x.q, x.k, x.v, x.g, x.beta, o, recs[2])

    def commit(p, n):
        x, _, recs = sets[p % RING]
        G.gdn_commit(x.S0, recs[2], n, pos)

    s2 = s1
    for p in range(s2, s2 + LAG):
        verify(p)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        verify(s2 + i + LAG)
        commit(s2 + i, n_sep_d[i])
    torch.cuda.synchronize()
    wall_sep = time.perf_counter() - t0
    tokens_sep = sum(int(v) for v in n_sep)
    for p in range(s2 + args.steps, s2 + args.steps + LAG):  # the pending blocks left: committed, untimed
        commit(p, n_sep_d[0])
    torch.cuda.synchronize()

    # Verify alone: `steps` launches back to back over the rotating sets (verify
    # never writes the state), bracketed by two events.
    kev.record(ev_a)
    for i in range(args.steps):
        verify(i)
    kev.record(ev_b)
    torch.cuda.synchronize()
    avg_ver_ms = kev.ms(ev_a, ev_b) / args.steps

    # Commit alone: a pool of states, each with a pending block verified (untimed)
    # and the caches flushed, then the pool's commits back to back between two
    # events; repeated until `steps` commits are timed.  The flush reads a 512 MiB
    # buffer: it evicts the states (writing back whatever the verifies left dirty,
    # untimed) and leaves only clean lines, so the timed commits write back
    # nothing of the flush's.
    POOL = min(args.steps, 8)
    pool = []
    for _ in range(POOL):
        S_p = torch.empty_like(sets[0][0].S0)
        pool.append((S_p, G.new_record(S_p, T, dt)))
    flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
    com_ms, done = 0.0, 0
    while done < args.steps:
        cnt = min(POOL, args.steps - done)
        for j in range(cnt):
            x, o, _ = sets[j % RING]
            pool[j][0].copy_(x.S0)
            G.gdn_verify_block(pool[j][0], x.q, x.k, x.v, x.g, x.beta, o, pool[j][1])
        flush.sum(dtype=torch.int64)
        torch.cuda.synchronize()
        kev.record(ev_a)
        for j in range(cnt):
            G.gdn_commit(pool[j][0], pool[j][1], n_com_d[done + j], pos)
        kev.record(ev_b)
        torch.cuda.synchronize()
        com_ms += kev.ms(ev_a, ev_b)
        done += cnt
    avg_com_ms = com_ms / args.steps
    kev.free([ev_a, ev_b])
    del pool, flush
    torch.cuda.empty_cache()

    vb = verify_bytes(LAYERS, HEADS, DK, DV, T, es)
    fb_avg = sum(fused_bytes(LAYERS, HEADS, DK, DV, T, n, es) for n in n_timed) / len(n_timed)
    cb_avg = sum(commit_bytes(LAYERS, HEADS, DK, DV, int(n), es) for n in n_com) / len(n_com)
    fus_gbs = fb_avg / (avg_fus_ms * 1e-3) / 1e9
    ver_gbs = vb / (avg_ver_ms * 1e-3) / 1e9
    com_gbs = cb_avg / (avg_com_ms * 1e-3) / 1e9

    def entry(gbs, ms, nbytes, traffic):
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "avg_launch_us": round(ms * 1e3, 2),
                "algorithmic_bytes_per_launch": round(nbytes), "traffic": traffic}

    kernels = {
        "gdn_commit_verify": entry(fus_gbs, avg_fus_ms, fb_avg, load_traffic("commit_verify_kernel")),
        "gdn_verify": entry(ver_gbs, avg_ver_ms, vb, load_traffic("verify_kernel")),
        "gdn_commit": entry(com_gbs, avg_com_ms, cb_avg, load_traffic("commit_kernel")),
    }
    roof = dict(kernels["gdn_commit_verify"])
    roof["kernel"] = "gdn_commit_verify"

    result = {
        "metric": "GDN verify tokens/s (48 layers, T=8) + % HBM peak; prefill tok/s + % MFMA peak",
        "value": round(tokens / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "speculative verify pass: 48 GDN layers x 32 heads, dk=dv=128, T=8 "
                               "(7 draft + 1 anchor), bf16 q/k/v, fp32 state, verify + commit at "
                               "n~U{0..8}",
                   "path": "gdn_commit_verify (commit of the pending block and verify of the next "
                           "in one pass over the state)",
                   "layers": LAYERS, "heads": HEADS, "dk": DK, "dv": DV, "T": T,
                   "input_dtype": "bf16", "tokens_committed": tokens,
                   "accepted_lengths": "pairs (n, 8 - n), n ~ U{0..8}: every even window averages 4"},
        "rows_per_s": round(T * args.steps / wall, 1),
        "pass_hbm_frac": round(fus_gbs / HBM_PEAK_GBS, 4),
        "separate_calls": {"tokens_per_s": round(tokens_sep / wall_sep, 1),
                           "ms_per_step": round(wall_sep / args.steps * 1e3, 4),
                           "path": "gdn_verify_block + gdn_commit"},
        "kernel_timing": {"events": kev.kind,
                          "region": f"two events bracketing {args.steps} back-to-back launches on the launch "
                                    f"stream: gdn_commit_verify over the headline region itself, gdn_verify_block "
                                    f"over its own region, gdn_commit over batches of {POOL} pending states "
                                    f"(each batch after a cache flush); average = interval / launches"},
        "sources_sha256_16": sources_hash(),
        "roofline": roof,
        "kernels": kernels,
    }

    result["copy_ceiling"] = copy_ceiling(dev)
    result["copy_same_size"] = copy_same_size(dev, roof["algorithmic_bytes_per_launch"], roof["achieved"])
    if not args.no_prefill:
        result["prefill"] = bench_prefill(args, G, dev)
    if not args.no_prefill_long:
        result["prefill_long"] = bench_prefill(args, G, dev, B=PFL_B, L=PFL_L, reps=3, flush_mib=0, traffic_key=None,
                                               rounds=256)
    if not args.no_decode:
        result["decode"] = bench_decode(args, G, dev)
    if not args.no_accept:
        result["accept"] = bench_accept(args, G, dev)
    if not args.no_attn:
        result["attn"] = bench_attn(args, G, dev)
    if not args.no_mixer:
        result["mixer"] = bench_mixer(args, G, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 18  # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration"] = {"bytes_read": n * 4, "bytes_written": n * 4, "launches": 3}
    print(json.dumps(result), flush=True)


def copy_same_size(dev, nbytes, pass_gbs, pairs=6, reps=30):
    """Achieved GB/s of a device-to-device copy that moves as many bytes as one
    launch of the headline pass (half read, half written), rotated over `pairs`
    buffer pairs so that no copy finds its source in the 256 MB last-level cache.
    A launch's ramp-up and drain weigh more at this size than at 1 GiB, so this
    is the ceiling the pass itself runs against; `pass_vs_copy` is the pass's
    rate over the copy's."""
    import torch

    n = max(1, nbytes // 8)  # fp32 elements per side
    bufs = [(torch.ones(n, dtype=torch.float32, device=dev), torch.empty(n, dtype=torch.float32, device=dev))
            for _ in range(pairs)]
    for s_, d_ in bufs:
        d_.copy_(s_)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        s_, d_ = bufs[i % pairs]
        d_.copy_(s_)
    b.record()
    torch.cuda.synchronize()
    gbs = 2 * n * 4 * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del bufs
    torch.cuda.empty_cache()
    return {"kernel": "torch copy_", "bytes_per_copy": 2 * n * 4, "pairs": pairs, "achieved": round(gbs, 1),
            "unit": "GB/s", "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "pass_vs_copy": round(pass_gbs / gbs, 4)}


def copy_ceiling(dev, mib=1024, reps=10):
    """Achieved GB/s of a plain device-to-device copy (bytes read + written): the
    practical HBM ceiling on this device, reported beside the peak for context."""
    import torch

    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 2 * src.numel() * 4 * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"kernel": "torch copy_", "mib": mib, "achieved": round(gbs, 1), "unit": "GB/s",
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def _read_csv(pattern):
    import csv
    import glob

    paths = sorted(glob.glob(pattern, recursive=True))
    if not paths:
        raise SystemExit(f"no file matches {pattern}")
    with open(paths[0]) as f:
        return list(csv.DictReader(f))


def _cmd_arg(cmd, flag, default):
    """The integer value of `flag` in a command line, else `default`."""
    parts = cmd.split()
    return int(parts[parts.index(flag) + 1]) if flag in parts else default


def summarize_profiles(args):
    """Write the profile summaries from one directory of rocprofv3 output:
      stats/**/*kernel_stats.csv            --kernel-trace --stats run of bench.py
      fetch/**/*counter_collection.csv      --pmc FETCH_SIZE run
      write/**/*counter_collection.csv      --pmc WRITE_SIZE run (same command)
      commands.txt                          the three commands, one a line
    The counter runs must use --copy-calibration-mib; the copy's bytes scale the
    raw counters (per dispatch, KiB) to bytes.  --steps/--warmup/--seed must be
    those of the counter runs: the commit's accepted lengths, and so its
    algorithmic bytes, follow from them."""
    d = args.summarize
    with open(os.path.join(d, "commands.txt")) as f:
        commands = [ln.rstrip("\n") for ln in f if ln.strip()]

    # Kernel-trace statistics.
    stats = _read_csv(os.path.join(d, "stats", "**", "*kernel_stats.csv"))
    lines = ["# Kernel time: verify + commit (48 layers x 32 heads, d=128, T=8), the same pass with the GDN "
             "mixer, chunked prefill (32 heads, L=4096; 48 layers x 32 heads, L=32768), plain decode (32 heads, "
             "T=1), acceptance (T=8, V=151,936) and full attention (16 layers, 32,760 cached positions)", "",
             "rocprofv3 `--kernel-trace --stats` of the benchmark, GPU kernels of libgdn only "
             "(torch's input generation and copies omitted).", "", "Command:", "", "```",
             commands[0], "```", "", "| kernel | calls | average us | min us | max us | share of listed time |",
             "|---|---|---|---|---|---|"]
    rows = [r for r in stats if "gdn::" in r["Name"]]
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("void gdn::(anonymous namespace)::", "").split("(")[0]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / total:.3f} |")
    # The headline region alone: the fused 48-layer kernel's launches after the
    # warmup, by launch order in the kernel trace (the long prompt's rounds run the
    # same kernel later in the run).
    trace = _read_csv(os.path.join(d, "stats", "**", "*kernel_trace.csv"))
    fus = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in trace
                 if "verify_kernel" in r["Kernel_Name"] and ", true, 4, false>" in r["Kernel_Name"])
    steps, warm = _cmd_arg(commands[0], "--steps", 500), _cmd_arg(commands[0], "--warmup", 20)
    head = fus[warm:warm + steps]
    if head:
        avg = sum(e - b for b, e in head) / len(head) / 1e3
        span = (head[-1][1] - head[0][0]) / len(head) / 1e3
        lines += ["", f"Headline region (`gdn_commit_verify`, 48 layers x 32 heads, T=8, launches {warm} .. "
                      f"{warm + steps - 1} of that kernel): average kernel duration {avg:.2f} us over {len(head)} "
                      f"launches; first start to last end {span:.2f} us per launch."]
    with open(STATS_MD, "w") as f:
        f.write("\n".join(lines) + "\n")

    # Hardware counters: FETCH_SIZE and WRITE_SIZE per dispatch (KiB), scaled by
    # what they read for a plain copy of known size.
    def per_dispatch(sub):
        out = {}
        for r in _read_csv(os.path.join(d, sub, "**", "*counter_collection.csv")):
            key = int(r["Dispatch_Id"])
            e = out.setdefault(key, {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]), "kib": 0.0})
            e["kib"] += float(r["Counter_Value"])
        return out

    fetch, write = per_dispatch("fetch"), per_dispatch("write")
    calib_kib = None
    for c in commands:
        if "--copy-calibration-mib" in c:
            calib_kib = int(c.split("--copy-calibration-mib")[1].split()[0]) * 1024
    if calib_kib is None:
        raise SystemExit("the counter runs need --copy-calibration-mib")
    # The calibration copies are the dispatches whose WRITE_SIZE is the copy's size.
    cal = [k for k, e in write.items() if "copyBuffer" in e["name"] and abs(e["kib"] - calib_kib) < 0.02 * calib_kib]
    cal = [k for k in cal if k in fetch and fetch[k]["grid"] == write[k]["grid"]]
    if not cal:
        raise SystemExit("calibration copy dispatches not found")
    fetch_factor = calib_kib / (sum(fetch[k]["kib"] for k in cal) / len(cal))
    write_factor = calib_kib / (sum(write[k]["kib"] for k in cal) / len(cal))

    def kernel_rows(tag, also=""):
        ids = sorted(k for k, e in fetch.items() if tag in e["name"] and also in e["name"] and k in write)
        return [(k, fetch[k]["kib"] * 1024 * fetch_factor, write[k]["kib"] * 1024 * write_factor) for k in ids]

    es = 2
    # The kernel sources the counter runs measured: their own bench output names
    # them; fall back to the tree's sources if that output is missing.
    src_hash = sources_hash()
    try:
        with open(os.path.join(d, "fetch.json")) as f:
            src_hash = json.loads(f.read().strip().splitlines()[-1]).get("sources_sha256_16", src_hash)
    except (OSError, ValueError, IndexError):
        pass
    summary = {"sources_sha256_16": src_hash, "commands": commands,
               "calibration": {"copy_kib": calib_kib, "dispatches": len(cal),
                               "fetch_factor": round(fetch_factor, 4), "write_factor": round(write_factor, 4)},
               "kernels": {}}
    plan = accept_plan(args)

    def summarize(rows, alg):
        fr = sum(r[1] for r in rows) / len(rows)
        wr = sum(r[2] for r in rows) / len(rows)
        ab = sum(alg) / len(alg)
        return {"dispatches": len(rows), "read_bytes": round(fr), "write_bytes": round(wr),
                "hbm_bytes_per_launch": round(fr + wr), "algorithmic_bytes_per_launch": round(ab),
                "traffic_over_algorithmic": round((fr + wr) / ab, 3)}

    # The fused kernel's dispatches run the warmup passes, then the headline
    # passes; the separate calls' commits come first among the commit kernel's
    # dispatches, then the commit-alone region's.  (Four tiles a wave: the
    # 48-layer launches; the plain-decode leg's few-heads launches and the
    # long-prompt rounds are not in the counter runs.)
    fus_n = plan["warm"] + plan["head"]
    fus = kernel_rows("verify_kernel", ", true, 4, false>")
    if fus:
        fus = fus[:len(fus_n)]
        summary["kernels"]["commit_verify_kernel"] = summarize(
            fus, [fused_bytes(LAYERS, HEADS, DK, DV, T, fus_n[i], es) for i in range(len(fus))])
    ver = kernel_rows("verify_kernel", ", false, 4, false>")
    if ver:
        vb = verify_bytes(LAYERS, HEADS, DK, DV, T, es)
        fr = sum(r[1] for r in ver) / len(ver)
        wr = sum(r[2] for r in ver) / len(ver)
        summary["kernels"]["verify_kernel"] = {
            "dispatches": len(ver), "read_bytes": round(fr), "write_bytes": round(wr),
            "hbm_bytes_per_launch": round(fr + wr), "algorithmic_bytes_per_launch": vb,
            "traffic_over_algorithmic": round((fr + wr) / vb, 3)}
    com_n = plan["sep"] + [plan["sep"][0]] * LAG + plan["com"]
    com = kernel_rows("commit_kernel")
    if com:
        com = com[:len(com_n)]
        summary["kernels"]["commit_kernel"] = summarize(
            com, [commit_bytes(LAYERS, HEADS, DK, DV, com_n[i], es) for i in range(len(com))])
    # Prefill: every call launches either prefill_kernel, or one prep launch and
    # one stage launch per chunk segment; per call.
    pk = kernel_rows("prefill_kernel<") + kernel_rows("prefill_pass_kernel<")
    pp = kernel_rows("prefill_prep_kernel")
    ps = kernel_rows("prefill_stage_kernel")
    calls = len(pp) if pp else len(pk)
    if calls:
        fr = (sum(r[1] for r in pk + pp + ps)) / calls
        wr = (sum(r[2] for r in pk + pp + ps)) / calls
        pb = prefill_bytes(PF_B, PF_H, DK, DV, PF_L)
        summary["kernels"]["prefill"] = {
            "calls": calls, "kernels": sorted({e["name"].replace("void gdn::(anonymous namespace)::", "").split("(")[0]
                                               for k, e in fetch.items() if "prefill" in e["name"]}),
            "read_bytes": round(fr), "write_bytes": round(wr), "hbm_bytes_per_launch": round(fr + wr),
            "algorithmic_bytes_per_launch": pb, "traffic_over_algorithmic": round((fr + wr) / pb, 3)}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(summary, f, indent=1)
        f.write("\n")
    print(f"wrote {STATS_MD} and {TRAFFIC_JSON}")
    if os.path.isdir(os.path.join(d, "mfma")):
        summarize_mfma(d, commands, src_hash)


def summarize_mfma(d, commands, src_hash):
    """MFMA counters of the prefill calls (the bf16 MFMA operations executed, and
    the matrix pipes' busy cycles against the kernel's active cycles), from a
    --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE run
    The calls' durations come from the plain benchmark run of the same tree
    (bench.json: counter collection slows the calls down), else from the counter
    run's own output (mfma.json).  GRBM_GUI_ACTIVE reads the sum over the 8 XCDs
    of the active cycles; the busy cycles are summed over the 1,024 SIMDs."""
    rows = _read_csv(os.path.join(d, "mfma", "**", "*counter_collection.csv"))
    disp = {}
    for r in rows:
        e = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    bench_out, timed_by = None, None
    for name in ("bench.json", "mfma.json"):
        try:
            with open(os.path.join(d, name)) as f:
                bench_out, timed_by = json.loads(f.read().strip().splitlines()[-1]), name
            break
        except (OSError, ValueError, IndexError):
            continue
    if bench_out is None:
        raise SystemExit("no benchmark output next to the MFMA counters")
    out = {"sources_sha256_16": src_hash, "command": next((c for c in commands if "--pmc SQ_INSTS_VALU_MFMA" in c), None),
           "durations_from": "plain benchmark run" if timed_by == "bench.json" else "the counter run", "legs": {}}
    for leg, tags in (("prefill", ("prefill_prep_kernel", "prefill_stage_kernel")),
                      ("prefill_long", ("prefill_pass_kernel<", "prefill_kernel<"))):
        ds = [e for e in disp.values() if any(t in e["name"] for t in tags)]
        b = bench_out.get(leg, {})
        if not ds or "avg_launch_us" not in b:
            continue
        calls = sum(1 for e in ds if tags[0] in e["name"])
        flops = sum(e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for e in ds) * 512 / calls
        busy = sum(e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for e in ds)
        active = sum(e.get("GRBM_GUI_ACTIVE", 0.0) for e in ds) / 8 * 1024
        us = b["avg_launch_us"]
        out["legs"][leg] = {
            "workload": b.get("workload"), "calls": calls, "avg_launch_us": us,
            "mfma_bf16_flops_executed_per_call": round(flops),
            "algorithmic_flops_per_call": round(b["mfma"]["flops_per_launch"]),
            "executed_over_algorithmic": round(flops / b["mfma"]["flops_per_launch"], 3),
            "executed_tflops": round(flops / (us * 1e-6) / 1e12, 2),
            "executed_frac_of_peak": round(flops / (us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "mfma_busy_frac": round(busy / active, 4) if active else None}
    with open(MFMA_JSON, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(f"wrote {MFMA_JSON}")


def bench_decode(args, G, dev):
    """Plain decode, T = 1: one GDN layer, 32 heads, d = 128, bf16, a chain of
    decode steps carrying the 2 MiB state, each step one gdn_commit_verify
    (commit the previous token, n = 1, and verify the next).  Timed eagerly over
    the whole chain and as a HIP graph of 100 chained steps replayed back to back.
    The 2 MiB state stays in the caches between steps, so the effective rate is
    not an HBM figure; the step is launch- and latency-bound."""
    import torch

    from speculative_verify_amd.inputs import make_inputs

    B, H, L = 1, HEADS, args.decode_steps
    x = make_inputs(B, H, DK, DV, L, seed=args.seed + 91, device=dev, device_gen=True)
    S = x.S0.clone()
    o = torch.empty(B, L, H, DV, dtype=torch.float32, device=dev)
    recs = [G.new_record(S, 1, torch.bfloat16) for _ in range(2)]
    one = torch.ones(B, dtype=torch.int32, device=dev)
    sl = lambda a, t: a[:, t:t + 1]

    def step(t):  # commits token t - 1, verifies token t
        G.gdn_commit_verify(S, recs[(t + 1) % 2], one, sl(x.q, t), sl(x.k, t), sl(x.v, t), sl(x.g, t),
                            sl(x.beta, t), sl(o, t), recs[t % 2])

    G.gdn_verify_block(S, sl(x.q, 0), sl(x.k, 0), sl(x.v, 0), sl(x.g, 0), sl(x.beta, 0), sl(o, 0), recs[0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(1, L):
        step(t)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) / (L - 1) * 1e6

    # A graph of 100 chained steps (an even count, so the records alternate
    # consistently from one replay to the next).
    GS = 100
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for t in range(2, 2 + GS):
                step(t)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, (L - 1) // GS)
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) / (reps * GS) * 1e6
    nbytes = fused_bytes(B, H, DK, DV, 1, 1, 2)
    return {"workload": f"plain decode: 1 layer x {H} heads, dk=dv={DK}, T=1, bf16, fp32 state (2 MiB), "
                        f"{L} chained steps, one gdn_commit_verify per step",
            "us_per_step_eager": round(eager_us, 2), "us_per_step_graph": round(graph_us, 2),
            "tokens_per_s_graph": round(1e6 / graph_us, 1),
            "algorithmic_bytes_per_step": nbytes,
            "effective_GBs_graph": round(nbytes / (graph_us * 1e-6) / 1e9, 1),
            "note": "state cache-resident between steps"}


ACC_V = 151936   # the Qwen3 tokenizer's vocabulary (the pages' targets are Qwen3-family models)
HIST_C = 8192    # filter channels of one GDN layer: q, k (16 heads x 128) and v (32 heads x 128)
HIST_W = 3       # history rows of a width-4 causal filter


def accept_bytes(B, T, V, es, sampled):
    """Algorithmic HBM bytes of one acceptance call: every target row (and, when
    sampled, every drafter row) read once, the draft tokens and uniforms read and
    n and the emitted token written."""
    rows = 2 * T - 1 if sampled else T
    return B * rows * V * es + B * (T - 1) * (8 if sampled else 4) + B * (12 if sampled else 8)


def bench_accept(args, G, dev):
    """On-device acceptance of one verify block (one sequence, T = 8 rows, the
    Qwen3 vocabulary, bf16 logits), greedy and sampled, and the filter-history
    rewind of all 48 GDN layers (history [48][3][8192] bf16).  Each timed over
    200 calls back to back, eagerly and as a HIP graph of 20 calls."""
    import torch

    from speculative_verify_amd.inputs import make_accept_inputs, make_history_inputs

    B, Tb, V = 1, T, ACC_V
    x = make_accept_inputs(B, Tb, V, dtype=torch.bfloat16, seed=args.seed + 55, device=dev, peak=16.0)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    wg = torch.empty(G.gdn_accept_workspace_bytes(x.target, False), dtype=torch.uint8, device=dev)
    wsamp = torch.empty(G.gdn_accept_workspace_bytes(x.target, True), dtype=torch.uint8, device=dev)
    hist, rows = make_history_inputs(LAYERS, HIST_W, Tb, HIST_C, seed=args.seed + 56, device=dev)
    nh = torch.full((LAYERS,), 5, dtype=torch.int32, device=dev)
    calls = {
        "greedy": lambda: G.gdn_accept_greedy(x.target, x.tokens, n, nxt, ws=wg),
        "sampled": lambda: G.gdn_accept_sampled(x.target, x.draft, x.tokens, x.u_accept, x.u_sample, 1.0, n, nxt,
                                                ws=wsamp),
        "history_rewind": lambda: G.gdn_history_rewind(hist, rows, nh),
    }
    nbytes = {"greedy": accept_bytes(B, Tb, V, 2, False), "sampled": accept_bytes(B, Tb, V, 2, True),
              "history_rewind": LAYERS * HIST_C * 2 * 2 * HIST_W + LAYERS * 4}   # W rows read, W written
    out = {"workload": f"acceptance of one verify block: 1 sequence, T={Tb} rows (anchor + {Tb - 1} drafts), "
                       f"V={V}, bf16 logits; filter-history rewind of {LAYERS} layers x {HIST_W} rows x "
                       f"{HIST_C} channels, bf16, n=5"}
    N, GS = 200, 20
    for name, fn in calls.items():
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(N):
            fn()
        b.record()
        torch.cuda.synchronize()
        eager = a.elapsed_time(b) / N * 1e3
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for _ in range(GS):
                    fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        a.record()
        for _ in range(N // GS):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        gus = a.elapsed_time(b) / N * 1e3
        out[name] = {"us_per_call_eager": round(eager, 2), "us_per_call_graph": round(gus, 2),
                     "algorithmic_bytes": nbytes[name],
                     "effective_GBs_graph": round(nbytes[name] / (gus * 1e-6) / 1e9, 1)}
    return out


ATT_LAYERS, ATT_HQ, ATT_HKV, ATT_D = 16, 16, 2, 256   # the 16 full-attention layers (Qwen3-Next-style heads)
MIX_HK = 16   # q/k heads of the GDN mixer (value heads: HEADS)


def bench_mixer(args, G, dev):
    """The 48-layer pass with the GDN mixer fused around the recurrence: one
    gdn_mixer_commit_verify per pass (filter, norms and gates from the raw
    in-projection rows; gated RMS norm on the outputs) against one
    gdn_commit_verify on ready q, k, v, at the same accepted lengths.  Four state
    buffers rotate, as in the headline, so that no launch finds its state still in
    the last-level cache."""
    import torch

    from speculative_verify_amd.inputs import make_accepts_paired, make_inputs, make_mixer_inputs

    L, H, NSET = LAYERS, HEADS, 4
    x = make_inputs(L, H, DK, DV, T, seed=args.seed + 61, device=dev, device_gen=True)
    m = make_mixer_inputs(L, T, H, MIX_HK, DK, seed=args.seed + 61, device=dev)
    ns = make_accepts_paired(64, T, seed=args.seed + 61)
    nt = [torch.full((L,), int(v), dtype=torch.int32, device=dev) for v in ns]
    y = torch.empty(L, T, H, DV, dtype=torch.float32, device=dev)
    Ss = [x.S0.clone() for _ in range(NSET)]
    recs = [[G.new_record(Ss[j], T, torch.bfloat16) for _ in range(2)] for j in range(NSET)]
    out = {"workload": f"{L} GDN layers x {H} value heads ({MIX_HK} q/k heads), d={DK}, T={T}: commit + verify "
                       f"per pass, n~U{{0..8}}, {NSET} rotating state buffers"}
    for name in ("mixer_commit_verify", "commit_verify"):
        def step(i):
            j, c = i % NSET, i // NSET
            rp, rn = recs[j][c % 2], recs[j][(c + 1) % 2]
            if name == "mixer_commit_verify":
                G.gdn_mixer_commit_verify(Ss[j], rp, nt[i % len(nt)], m, y, rn)
            else:
                G.gdn_commit_verify(Ss[j], rp, nt[i % len(nt)], x.q, x.k, x.v, x.g, x.beta, y, rn)
        for j in range(NSET):   # a pending block on every set
            if name == "mixer_commit_verify":
                G.gdn_mixer_verify(Ss[j], m, y, recs[j][0])
            else:
                G.gdn_verify_block(Ss[j], x.q, x.k, x.v, x.g, x.beta, y, recs[j][0])
        for i in range(12):
            step(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 100
        a.record()
        for i in range(12, 12 + n):
            step(i)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / n * 1e3
        out[name + "_us"] = round(us, 2)
        nv = [int(ns[i % len(ns)]) for i in range(12, 12 + n)]
        nb = [mixer_fused_bytes(L, H, MIX_HK, DK, T, v) if name == "mixer_commit_verify" else
              fused_bytes(L, H, DK, DV, T, v, 2) for v in nv]
        out[name + "_bytes"] = int(sum(nb) / n)
        out[name + "_tbs"] = round(sum(nb) / n / us * 1e-6, 3)
    return out


def attn_bytes(B, T, Hq, Hkv, d, ctx):
    """Algorithmic HBM bytes of one attention call: the cached keys and values
    read once, the block's queries, keys and values read, the outputs written
    and the block's rows appended to the cache."""
    return (B * ctx * Hkv * d * 2 * 2 + B * T * (Hq + 2 * Hkv) * d * 2 + B * T * Hq * d * 4
            + B * T * Hkv * d * 2 * 2)


def bench_attn(args, G, dev):
    """The verify pass's 16 full-attention layers (16 query / 2 key-value heads,
    d = 256, bf16 cache), T = 8, at 32,760 and at 120 cached positions; timed
    over 20 calls with events, caches flushed by the 1 GiB working set itself."""
    import torch

    from speculative_verify_amd.inputs import make_attn_inputs

    B, Tb, Lmax = ATT_LAYERS, T, 32768
    out = {"workload": f"full-attention verify: {B} layers x {ATT_HQ} query / {ATT_HKV} key-value heads, "
                       f"d={ATT_D}, T={Tb}, bf16 K/V cache of {Lmax} positions"}
    x = make_attn_inputs(B, Tb, ATT_HQ, ATT_HKV, ATT_D, Lmax, [Lmax - Tb] * B, seed=args.seed + 33, device=dev,
                         device_gen=True)
    o = torch.empty(B, Tb, ATT_HQ, ATT_D, dtype=torch.float32, device=dev)
    ws = torch.empty(G.gdn_attn_workspace_bytes(x.q, x.k_cache), dtype=torch.uint8, device=dev)
    for name, ctx in (("ctx_32760", Lmax - Tb), ("ctx_120", 120)):
        c = torch.full((B,), ctx, dtype=torch.int32, device=dev)
        G.gdn_attn_verify(x.q, x.k_new, x.v_new, x.k_cache, x.v_cache, c, o, ws=ws)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 20
        a.record()
        for _ in range(n):
            G.gdn_attn_verify(x.q, x.k_new, x.v_new, x.k_cache, x.v_cache, c, o, ws=ws)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / n * 1e3
        nb = attn_bytes(B, Tb, ATT_HQ, ATT_HKV, ATT_D, ctx)
        gbs = nb / (us * 1e-6) / 1e9
        out[name] = {"us_per_call": round(us, 2), "algorithmic_bytes": nb, "achieved_GBs": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "workspace_bytes": ws.numel()}
    return out


def bench_rounds(G, dev, S, rounds, seed):
    """Speculative rounds on a prefilled state: `rounds` gdn_commit_verify launches
    back to back on the one state S [B][H][dv][dk] (the model's own: no rotation,
    so the 256 MB last-level cache may hold part of it), each committing the
    previous round's block at its accepted length and verifying the next T = 8
    block; paired accepted lengths, so the rounds commit exactly 4 tokens each on
    average.  Timed with two events around the launches."""
    import torch

    from speculative_verify_amd.inputs import make_accepts_paired, make_inputs

    B, H = S.shape[0], S.shape[1]
    blocks = [make_inputs(B, H, DK, DV, T, seed=seed + i, device=dev, device_gen=True) for i in range(8)]
    recs = [G.new_record(S, T, torch.bfloat16) for _ in range(2)]
    ns = make_accepts_paired(rounds, T, seed=seed)
    nd = ns.view(-1, 1).expand(-1, B).contiguous().to(dev)
    o = torch.empty(B, T, H, DV, dtype=torch.float32, device=dev)
    pos = torch.zeros(B, dtype=torch.int32, device=dev)
    x0 = blocks[0]
    G.gdn_verify_block(S, x0.q, x0.k, x0.v, x0.g, x0.beta, o, recs[0])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for r in range(rounds):
        x = blocks[(r + 1) % len(blocks)]
        G.gdn_commit_verify(S, recs[r % 2], nd[r], x.q, x.k, x.v, x.g, x.beta, o, recs[(r + 1) % 2], pos=pos)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / rounds * 1e3
    tokens = int(ns.sum())
    nbytes = sum(fused_bytes(B, H, DK, DV, T, int(v), 2) for v in ns) / rounds
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"{rounds} speculative rounds (gdn_commit_verify, T={T}, n~U{{0..8}} in pairs) on the "
                        f"state of the {B}-layer prefill, one state, back to back",
            "rounds": rounds, "tokens_committed": tokens, "us_per_round": round(us, 2),
            "tokens_per_s": round(tokens / (us * 1e-6 * rounds), 1),
            "hbm": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": round(nbytes)}}


def bench_prefill(args, G, dev, B=PF_B, L=PF_L, reps=None, flush_mib=512, traffic_key="prefill", rounds=0):
    """Chunked prefill of B layers x PF_H heads over an L-token prompt, timed with
    events over `reps` calls; a token counts once it has passed all B layers.
    With `rounds`, that many speculative rounds then run on the prefilled state."""
    import torch

    from speculative_verify_amd.inputs import make_inputs

    reps = args.prefill_reps if reps is None else reps
    x = make_inputs(B, PF_H, DK, DV, L, seed=args.seed + 77, device=dev, device_gen=True)
    o = torch.empty(B, L, PF_H, DV, dtype=torch.float32, device=dev)
    S = x.S0.clone()
    need = G.gdn_prefill_workspace_bytes(S, L, PF_C)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None
    try:
        G.gdn_prefill_chunked(S, x.q, x.k, x.v, x.g, x.beta, o, chunk=PF_C, ws=ws)
    except G.GdnError as e:
        return {"status": f"unavailable: {e}"}
    # A buffer rewritten between reps pushes the prompt out of the caches (not
    # needed when the prompt itself is many times the cache).
    flush = torch.empty(flush_mib << 20, dtype=torch.uint8, device=dev) if flush_mib else None
    t_ms = []
    for _ in range(reps):
        if flush is not None:
            flush.fill_(1)
        S.copy_(x.S0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        G.gdn_prefill_chunked(S, x.q, x.k, x.v, x.g, x.beta, o, chunk=PF_C, ws=ws)
        b.record()
        torch.cuda.synchronize()
        t_ms.append(a.elapsed_time(b))
    del x, o, ws, flush
    torch.cuda.empty_cache()
    rounds_out = bench_rounds(G, dev, S, rounds, args.seed + 333) if rounds else None
    del S
    torch.cuda.empty_cache()
    avg = sum(t_ms) / len(t_ms)
    fl = prefill_flops(B, PF_H, DK, DV, L, PF_C)
    by = prefill_bytes(B, PF_H, DK, DV, L)
    tf = fl / (avg * 1e-3) / 1e12
    gbs = by / (avg * 1e-3) / 1e9
    return {"workload": f"chunked prefill: {B} layer{'s' if B > 1 else ''} x {PF_H} heads, dk=dv={DK}, L={L}, "
                        f"chunk {PF_C}, bf16 in, fp32 state, cold caches",
            "schedule": "two-phase (chunk prep, scan; prep of each segment beside the scan of the previous)" if need else "one-pass",
            "workspace_bytes": need, "reps": reps,
            "tokens_per_s": round(L / (avg * 1e-3), 1), "avg_launch_us": round(avg * 1e3, 2),
            "mfma": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                     "flops_per_launch": fl, "flop_convention": "causal"},
            "hbm": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": by,
                    "traffic": load_traffic(traffic_key) if traffic_key else None},
            "mfma_counters": load_mfma("prefill" if B == PF_B and L == PF_L else "prefill_long"),
            **({"rounds_after": rounds_out} if rounds_out else {})}


if __name__ == "__main__":
    main()
