"""Benchmark of the Gated DeltaNet layer on one MI355X.

Default workload: the decode step at B = 64 sequences, 16 K/Q heads expanded to
32 V heads, d_k = d_v = 128, conv K = 4, bf16 inputs, fp32 state [64,32,128,128]
(~N(0, 0.1)) and conv state, 256 consecutive steps with fresh inputs per step.
A "step" is one gdn_decode_step call (conv + SiLU, split, GQA, L2 norm, scale,
one recurrence step for every (sequence, V head)).

Timing: W untimed warm-up steps, then exactly K steps bracketed by
torch.cuda.synchronize(); inputs are resident in HBM before the clock starts.
HIP events on the launch stream split the K steps into R = 5 consecutive
repetitions (no synchronisation between them, so the launches stay pipelined, as
the mlxcel benchmark notes advise): the per-launch kernel time is reported as the
median over the repetitions with its spread (max - min) / median, and a row
whose spread exceeds 4% of the median is marked untrustworthy (the spread guard
of those notes). The roofline uses the median.
Cold-cache mode: 4 independent state replicas rotate, so the 128 MiB state a
step reads was last touched 4 steps (512 MiB of state) earlier and cannot sit
in the 256 MB Infinity Cache; this is the reported value. With --warm the
warm-cache rate (one replica) is timed too.

The default run also measures the device's achievable ceilings (HBM read, write
and copy over 1 GiB; an MFMA throughput loop; libgdn_ceiling.so), records run
metadata (build commit and source digest, ROCm, GPU, CUs, clocks, host CPU),
times the fp64 oracle on a bounded sample on the host (all threads, and one
thread), and times the other workloads of the layer (prefill L = 4096, the
ragged 8-sequence prefill, the verify block and its commit) into `workloads`,
each with its own median, spread and roofline. --no-extras skips them.

Other workloads as the main line (--workload verify | prefill | ragged | commit
| decode_fused | prefill_fused | ragged_fused | spec_round_copy |
spec_round_slots | packed_short, 512 prompts of 64 tokens packed in one prefill call;
--verify-t sets the verify block width, --prefill-rows and --prefill-len the prompts
of prefill and prefill_fused) print the same kind of JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gated DeltaNet tokens/s + % roofline (decode HBM GB/s; prefill MFMA util)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 (and fp16) MFMA, published
PROFILES = os.path.join(ROOT, "profiles")
PKG = os.path.join(ROOT, "linear_attention_sequence_amd")
CSRC = os.path.join(PKG, "csrc")
REPS = 5                       # repetitions per timed region
SPREAD_GUARD = 0.04            # spread / median above this marks a row untrustworthy


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counters(name, digest):
    """Committed rocprofv3 --pmc figures for a workload (profiles/<name>_counters.json),
    or None when absent or taken from other kernel sources."""
    path = os.path.join(PROFILES, f"{name}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    return c if c.get("source_digest") == digest else None


def traffic_from_counters(c):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by
    what the same counter reads for a plain device copy of known size in the same run."""
    if c is None:
        return None
    fetch = c["fetch_kib_per_dispatch"] * 1024.0 * c["copy_read_bytes"] / (c["copy_fetch_kib"] * 1024.0)
    write = c["write_kib_per_dispatch"] * 1024.0 * c["copy_write_bytes"] / (c["copy_write_kib"] * 1024.0)
    return fetch + write


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------
def run_timed(torch, step_fn, steps, warmup, reps=REPS):
    """W untimed steps, then K timed steps launched back to back. HIP events on the launch
    stream (torch's current stream, which the binding launches on) split the K steps into
    R consecutive repetitions without synchronising; the host clock with a synchronize on
    both sides gives the wall time of all K. Returns (wall seconds, per-step ms per rep)."""
    for i in range(warmup):
        step_fn(i)
    torch.cuda.synchronize()
    R = max(1, min(reps, steps))
    bounds = [round(steps * r / R) for r in range(R + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for r in range(R):
        for i in range(bounds[r], bounds[r + 1]):
            step_fn(warmup + i)
        ev[r + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[r].elapsed_time(ev[r + 1]) / (bounds[r + 1] - bounds[r]) for r in range(R)]
    return wall, per


def summary(per_ms):
    med = statistics.median(per_ms)
    spread = (max(per_ms) - min(per_ms)) / med if med > 0 else 0.0
    return {"reps": len(per_ms), "median_us": med * 1e3, "min_us": min(per_ms) * 1e3,
            "max_us": max(per_ms) * 1e3, "spread": spread, "trustworthy": spread <= SPREAD_GUARD,
            "per_rep_us": [round(x * 1e3, 2) for x in per_ms]}


# ---------------------------------------------------------------------------
# measured ceilings and run metadata
# ---------------------------------------------------------------------------
def _ceiling_lib():
    path = os.path.join(PKG, "libgdn_ceiling.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    V, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.gdn_ceiling_read.argtypes = [V, SZ, V, I, V]
    lib.gdn_ceiling_write.argtypes = [V, SZ, I, I, V]
    lib.gdn_ceiling_copy.argtypes = [V, V, SZ, I, I, V]
    lib.gdn_ceiling_mfma.argtypes = [V, I, I, I, V]
    lib.gdn_ceiling_device_info.argtypes = [I] + [ctypes.POINTER(I)] * 4
    lib.gdn_ceiling_read_blocked.argtypes = [V, SZ, V, I, V]
    lib.gdn_ceiling_write_blocked.argtypes = [V, SZ, I, I, V]
    lib.gdn_ceiling_copy_blocked.argtypes = [V, V, SZ, I, I, V]
    return lib


def measure_ceilings(torch, lib, cus):
    """Best median rate over a few grid sizes for HBM read / write / copy of 1 GiB, and the
    MFMA loop at fp16 and bf16 (5 repetitions each)."""
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(1 << 16, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def rate(fn, units, per_rep=10):
        """units per second: median over REPS of per_rep launches back to back (pipelined,
        as the layer's kernels are timed)"""
        fn()
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(REPS):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(per_rep):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1) / per_rep)
        return units / (statistics.median(ms) * 1e-3)

    def check(st):
        if st != 0:
            raise RuntimeError(f"ceiling kernel failed ({st})")

    grids = [cus * k for k in (4, 8, 16, 32)]
    per_thread = (4, 8, 16)
    out, best = {}, {}

    def best_of(key, forms):
        """forms: (label, fn, units); keeps the fastest and which form it was"""
        rates = [(rate(fn, units), label) for label, fn, units in forms]
        r, label = max(rates)
        out[key] = r / 1e9
        best[key] = label

    best_of("hbm_read_GBs",
            [(f"grid-stride, {g // cus} workgroups/CU",
              lambda g=g: check(lib.gdn_ceiling_read(P(src), nbytes, P(sink), g, s)), nbytes) for g in grids] +
            [(f"blocked, {u} per thread", lambda u=u: check(lib.gdn_ceiling_read_blocked(P(src), nbytes, P(sink), u, s)),
              nbytes) for u in per_thread])
    for nt, key in ((1, "hbm_write_nt_GBs"), (0, "hbm_write_GBs")):
        best_of(key,
                [(f"grid-stride, {g // cus} workgroups/CU",
                  lambda g=g: check(lib.gdn_ceiling_write(P(dst), nbytes, nt, g, s)), nbytes) for g in grids] +
                [(f"blocked, {u} per thread", lambda u=u: check(lib.gdn_ceiling_write_blocked(P(dst), nbytes, nt, u, s)),
                  nbytes) for u in per_thread])
    for nt, key in ((1, "hbm_copy_nt_GBs"), (0, "hbm_copy_GBs")):
        best_of(key,
                [(f"grid-stride, {g // cus} workgroups/CU",
                  lambda g=g: check(lib.gdn_ceiling_copy(P(src), P(dst), nbytes, nt, g, s)), 2 * nbytes) for g in grids] +
                [(f"blocked, {u} per thread",
                  lambda u=u: check(lib.gdn_ceiling_copy_blocked(P(src), P(dst), nbytes, nt, u, s)), 2 * nbytes)
                 for u in per_thread])
    iters = 2000
    for dt, key, fl in ((0, "mfma_f16_16x16x32_TFLOPs", 16384), (1, "mfma_bf16_16x16x32_TFLOPs", 16384),
                        (2, "mfma_f16_32x32x16_TFLOPs", 32768), (3, "mfma_bf16_32x32x16_TFLOPs", 32768)):
        out[key] = max(rate(lambda g=g, dt=dt: check(lib.gdn_ceiling_mfma(P(sink), g, iters, dt, s)),
                            g * 4 * iters * 8 * fl, per_rep=3) for g in (cus * 2, cus * 4)) / 1e12
    out["mfma_f16_TFLOPs"] = max(out["mfma_f16_16x16x32_TFLOPs"], out["mfma_f16_32x32x16_TFLOPs"])
    out["copy_best_GBs"] = max(out["hbm_copy_GBs"], out["hbm_copy_nt_GBs"])
    out["best_form"] = best
    out["note"] = ("1 GiB per memory kernel (4x the Infinity Cache): grid-stride loops at 4-32 workgroups per CU and "
                   "blocked forms (4, 8 or 16 granules per thread, all loads before the stores); median of 5 "
                   "repetitions of 10 launches back to back, best form; copy counts read + write bytes; MFMA: 8 "
                   "independent chains per wave, 2 or 4 workgroups of 4 waves per CU")
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


def run_metadata(torch, lib):
    meta = {"source_digest_now": None, "build": None}
    try:
        import linear_attention_sequence_amd.build as b
        meta["source_digest_now"] = b.source_digest()
        with open(b.BUILD_INFO) as f:
            meta["build"] = json.load(f)
    except (OSError, ValueError, ImportError):
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            meta["rocm"] = f.read().strip()
    except OSError:
        meta["rocm"] = None
    pr = torch.cuda.get_device_properties(0)
    meta.update({"gpu": pr.name or f"AMD Instinct, {pr.gcnArchName.split(':')[0]}",   # the box reports no name
                 "arch": pr.gcnArchName, "cus": pr.multi_processor_count,
                 "hbm_bytes": pr.total_memory, "torch": torch.__version__, "python": platform.python_version()})
    if lib is not None:
        v = [ctypes.c_int() for _ in range(4)]
        if lib.gdn_ceiling_device_info(0, *[ctypes.byref(x) for x in v]) == 0:
            meta.update({"sclk_mhz": v[1].value / 1000.0, "mclk_mhz": v[2].value / 1000.0, "mem_bus_bits": v[3].value})
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count()
    meta.update({"host_cpu": cpu, "host_threads": threads})
    return meta


# ---------------------------------------------------------------------------
# decode (default)
# ---------------------------------------------------------------------------
def decode_bytes(sh, B, fused):
    n = (B * sh.Hv * sh.dk * sh.dv * 4 * 2          # S read + write
         + B * sh.D * 2                              # qkv
         + B * sh.D * (sh.K - 1) * 2 * 2             # conv state read + write
         + sh.D * sh.K * 2                           # conv weight
         + B * sh.Hv * 2 * 2                         # gate, beta
         + B * sh.Hv * sh.dv * 4)                    # o
    if fused:
        n += B * sh.Hv * sh.dv * 2 + (2 * sh.Hv + sh.dv) * 2   # z; A_log, dt_bias, norm weight
    return n


def bench_decode(args, torch, gdn, gi, fused=False):
    sh, w_ = gi.QWEN, gi.WORKLOADS[1]
    seed, B, NSTEP = w_.seed, gi.DECODE_B, gi.DECODE_STEPS
    p = gdn.GdnParams(sh.Hk, sh.Hv, sh.dk, sh.dv, sh.K, True, 1e-6, gdn.GDN_BF16)
    dev = lambda a, bf=True: (torch.from_numpy(a).cuda().to(torch.bfloat16) if bf else torch.from_numpy(a).cuda())
    log("generating decode inputs ...")
    xs = [dev(gi.qkv(sh, B, 1, seed, "bf16", step=s)) for s in range(NSTEP)]
    if fused:   # raw a/b through the prologue, gated RMSNorm epilogue with z
        gs = [dev(gi.a_raw(sh, B, 1, seed, "bf16", step=s)) for s in range(NSTEP)]
        bs = [dev(gi.b_raw(sh, B, 1, seed, "bf16", step=s)) for s in range(NSTEP)]
        zs = [dev(gi.z_gate(sh, B, 1, seed, "bf16", step=s)) for s in range(NSTEP)]
        fus = [gdn.GdnFusion(dev(gi.a_log(sh, seed, "bf16")), dev(gi.dt_bias(sh, seed, "bf16")), z,
                             dev(gi.norm_weight(sh, seed, "bf16")), 1e-6) for z in zs]
    else:
        gs = [dev(gi.gate(sh, B, 1, seed, "bf16", step=s)) for s in range(NSTEP)]
        bs = [dev(gi.beta(sh, B, 1, seed, "bf16", step=s)) for s in range(NSTEP)]
    w = dev(gi.conv_weight(sh, seed, "bf16"))
    S0 = dev(gi.state0(sh, B, seed, 0.1), bf=False)
    c0 = dev(gi.conv_state0(sh, B, seed, 1.0, "bf16"))
    o = torch.empty((B, 1, sh.Hv, sh.dv), device="cuda")

    def make(replicas):
        S = [S0.clone() for _ in range(replicas)]
        conv = [[c0.clone(), torch.empty_like(c0)] for _ in range(replicas)]
        par = [0] * replicas

        def step(i):
            r = i % replicas
            ci, co = conv[r][par[r]], conv[r][1 - par[r]]
            j = i % NSTEP
            if fused:
                gdn.gdn_decode_step_ex(p, fus[j], xs[j], gs[j], bs[j], w, ci, co, S[r], o)
            else:
                gdn.gdn_decode_step(p, xs[j], gs[j], bs[j], w, ci, co, S[r], o)
            par[r] ^= 1
        return step

    wall, per = run_timed(torch, make(4), args.steps, args.warmup)
    t = summary(per)
    nbytes = decode_bytes(sh, B, fused)
    achieved = nbytes / (t["median_us"] * 1e-6) / 1e9
    digest = source_digest(["gdn_recurrent.hip", "gdn_common.hpp"])
    traffic = traffic_from_counters(counters("decode_fused_B64_d128" if fused else "decode_B64_d128", digest))
    res = {
        "metric": METRIC, "value": B * args.steps / wall, "unit": "tokens/s",
        "ms_per_step": 1e3 * wall / args.steps,
        "config": {"workload": w_.name + ("+gate_beta_prologue+gated_rmsnorm_epilogue" if fused else ""),
                   "B": B, "Hk": sh.Hk, "Hv": sh.Hv, "dk": sh.dk, "dv": sh.dv,
                   "conv_K": sh.K, "inputs": "bf16", "state": "fp32",
                   "cache": "cold: 4 rotating state replicas"},
        "dtype": "f32",
        "timing": t,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "recurrent_kernel (decode)", "algorithmic_bytes_per_launch": nbytes,
                     "avg_kernel_us": t["median_us"]},
    }
    if args.warm:
        wall_w, per_w = run_timed(torch, make(1), args.steps, args.warmup)
        tw = summary(per_w)
        res["warm"] = {"value": B * args.steps / wall_w, "ms_per_step": 1e3 * wall_w / args.steps,
                       "timing": tw, "achieved_GBs": nbytes / (tw["median_us"] * 1e-6) / 1e9}
    return res


def cpu_baseline_decode(gi, sh, seed, B, nthreads, budget_s):
    """The fp64 oracle, unmodified, on decode steps of the same workload (all 64
    sequences, all heads), one step per call with both states carried, until about
    budget_s seconds of CPU work have run."""
    import oracle
    op = oracle.OracleParams.of(sh)
    S = gi.state0(sh, B, seed, 0.1).astype(np.float64)
    c = gi.conv_state0(sh, B, seed, 1.0, "bf16").astype(np.float64)
    w = gi.conv_weight(sh, seed, "bf16")
    done, el = 0, 0.0
    while el < budget_s and done < gi.DECODE_STEPS:
        x = gi.qkv(sh, B, 1, seed, "bf16", step=done)
        g = gi.gate(sh, B, 1, seed, "bf16", step=done)
        b = gi.beta(sh, B, 1, seed, "bf16", step=done)
        t0 = time.perf_counter()
        r = oracle.gdn_forward(op, x, g, b, w, c, S, nthreads=nthreads)
        el += time.perf_counter() - t0
        S, c = r["S"], r["conv_out"]
        done += 1
    return {"value": B * done / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{done} consecutive decode steps of the same workload (B={B}, all 32 V heads), "
                      f"{el:.1f} s of oracle time"}


def cpu_baseline(gi):
    import oracle
    sh, seed, B = gi.QWEN, gi.WORKLOADS[1].seed, gi.DECODE_B
    nthreads = min(oracle.default_threads(), 16)
    res = cpu_baseline_decode(gi, sh, seed, B, nthreads, 12.0)
    res["single_thread"] = cpu_baseline_decode(gi, sh, seed, B, 1, 6.0)
    return res


# ---------------------------------------------------------------------------
# verify (B = 128, T = 4) and commit
# ---------------------------------------------------------------------------
def bench_verify(args, torch, gdn, gi, commit=False, rnd=None):
    """verify (one gdn_verify_block), commit (one gdn_verify_commit), or a whole
    speculative round: rnd == "copy" is verify + commit of the accepted state,
    rnd == "slots" is gdn_verify_block_slots from the previous block's snapshots
    (updated in place) + a window-only commit."""
    sh, w_ = gi.QWEN, gi.WORKLOADS[4]
    seed, B, T = w_.seed, gi.VERIFY_B, args.verify_t
    p = gdn.GdnParams(sh.Hk, sh.Hv, sh.dk, sh.dv, sh.K, True, 1e-6, gdn.GDN_BF16)
    dev = lambda a, bf=True: (torch.from_numpy(a).cuda().to(torch.bfloat16) if bf else torch.from_numpy(a).cuda())
    x = dev(gi.qkv(sh, B, T, seed, "bf16"))
    g = dev(gi.gate(sh, B, T, seed, "bf16"))
    b = dev(gi.beta(sh, B, T, seed, "bf16"))
    w = dev(gi.conv_weight(sh, seed, "bf16"))
    S_in = dev(gi.state0(sh, B, seed, 0.1), bf=False)
    c0 = dev(gi.conv_state0(sh, B, seed, 1.0, "bf16"))
    acc = torch.from_numpy(gi.accept_len(B, T, seed)).cuda()
    snap = torch.empty((B, T, sh.Hv, sh.dk, sh.dv), device="cuda")
    o = torch.empty((B, T, sh.Hv, sh.dv), device="cuda")
    S_out = torch.empty_like(S_in)
    c_out = torch.empty_like(c0)
    gdn.gdn_verify_block(p, x, g, b, w, c0, S_in, snap, o)
    # commit alone: the calls rotate the accepted lengths over the T slots and alternate
    # between two outputs, so that each reads and writes 268 MB the last one did not
    # (repeating one set would leave part of it in the 256 MB Infinity Cache)
    accs = [torch.from_numpy(((gi.accept_len(B, T, seed) + r) % T).astype(np.int32)).cuda() for r in range(T)]
    S_outs = [S_out, torch.empty_like(S_in)] if commit else [S_out]

    def step(i):
        if rnd == "copy":       # the committed state ping-pongs between S_in and S_out
            src, dst = (S_in, S_out) if i % 2 == 0 else (S_out, S_in)
            gdn.gdn_verify_block(p, x, g, b, w, c0, src, snap, o)
            gdn.gdn_verify_commit(p, acc, x, c0, snap, c_out, dst)
        elif rnd == "slots":
            gdn.gdn_verify_block_slots(p, None, x, g, b, w, c0, snap, acc, snap, o)
            gdn.gdn_verify_commit(p, acc, x, c0, None, c_out, None)
        elif commit:
            gdn.gdn_verify_commit(p, accs[i % T], x, c0, snap, c_out, S_outs[i % 2])
        else:
            gdn.gdn_verify_block(p, x, g, b, w, c0, S_in, snap, o)

    wall, per = run_timed(torch, step, args.steps, args.warmup)
    t = summary(per)
    tile = sh.dk * sh.dv * 4
    conv_b = B * sh.D * (sh.K - 1) * 2 * 2 + B * sh.D * T * 2 + B * 4   # window roll of a commit
    vbytes = (B * sh.Hv * tile * (1 + T) + B * sh.D * T * 2 + B * sh.D * (sh.K - 1) * 2
              + sh.D * sh.K * 2 + B * T * sh.Hv * 2 * 2 + B * T * sh.Hv * sh.dv * 4)
    if rnd is not None:
        nbytes = vbytes + conv_b + (B * sh.Hv * tile * 2 if rnd == "copy" else B * 4)
        name = f"spec_round_{rnd}_B{B}_T{T}_Hk16_Hv32_d128"
        kern = "speculative round: verify + commit (two launches, timed together)"
        cname = None
    elif commit:
        nbytes = B * sh.Hv * tile * 2 + conv_b
        name, kern = f"verify_commit_B{B}_T{T}_d128", "commit_kernel"
        cname = f"verify_commit_B{B}_T{T}_d128"
    else:
        nbytes = vbytes
        name, kern = (w_.name if T == gi.VERIFY_T else f"verify_B{B}_T{T}_Hk16_Hv32_d128"), f"recurrent_kernel (verify, T={T})"
        cname = f"verify_B{B}_T{T}_d128"
    digest = source_digest(["gdn_recurrent.hip", "gdn_common.hpp"])
    traffic = traffic_from_counters(counters(cname, digest)) if cname else None
    achieved = nbytes / (t["median_us"] * 1e-6) / 1e9
    return {
        "metric": METRIC, "value": (B if commit else B * T) * args.steps / wall, "unit": "tokens/s",
        "ms_per_step": 1e3 * wall / args.steps,
        "config": {"workload": name, "B": B, "T": T, "Hk": sh.Hk, "Hv": sh.Hv, "dk": sh.dk, "dv": sh.dv,
                   "cache": ("accepted slot rotated over the T snapshots, two alternating outputs" if commit
                             else "single working set of >1.3 GB (no rotation needed)")},
        "dtype": "f32",
        "timing": t,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": kern,
                     "algorithmic_bytes_per_launch": nbytes, "avg_kernel_us": t["median_us"]},
    }


# ---------------------------------------------------------------------------
# prefill (L = 4096) and ragged prefill (8 sequences)
# ---------------------------------------------------------------------------
PREFILL_FLOP_PER_TOKEN_HEAD = 163840   # bf16-MFMA-shaped work of the chunked form, C = 64, d = 128
PREFILL_SOURCES = ["gdn_prefill_mfma.hip", "gdn_prefill_plan.hpp", "gdn_packed.hpp", "gdn_prefill.hip", "gdn_common.hpp",
                   "gdn_mfma.hpp", "gdn_api.cpp"]


def prefill_bytes(sh, L, N, fused):
    """Algorithmic HBM bytes of one call: qkv, gate, beta, conv weight and states in, o out,
    the final state written (and read: it is carried in place)."""
    n = (sh.D * L * 2 + 2 * L * sh.Hv * 2 + sh.D * sh.K * 2 + 2 * N * sh.D * (sh.K - 1) * 2
         + L * sh.Hv * sh.dv * 4 + 2 * N * sh.Hv * sh.dk * sh.dv * 4)
    if fused:
        n += L * sh.Hv * sh.dv * 2 + (2 * sh.Hv + sh.dv) * 2
    return n


SHORT_N, SHORT_LEN = 512, 64   # many short prompts packed in one call


def bench_prefill(args, torch, gdn, gi, ragged=False, fused=False, short=False):
    sh = gi.QWEN
    w_ = gi.WORKLOADS[3 if ragged or short else 2]
    seed = w_.seed
    if short:   # the ragged workload's inputs, cut into SHORT_N sequences of SHORT_LEN tokens
        cu_np = gi.cu_seqlens(np.full(SHORT_N, SHORT_LEN))
        L, N = SHORT_N * SHORT_LEN, SHORT_N
        ragged = True
    elif ragged:
        lens = gi.seq_lens(gi.RAGGED_N, gi.RAGGED_LO, gi.RAGGED_HI, seed)
        cu_np = gi.cu_seqlens(lens)
        L, N = int(cu_np[-1]), gi.RAGGED_N
    else:
        L, N = args.prefill_len, args.prefill_rows
    B = 1 if ragged else N   # rows of the input: one packed row, or N unpacked rows of L tokens
    standard = ragged or (B == 1 and L == gi.PREFILL_L)
    p = gdn.GdnParams(sh.Hk, sh.Hv, sh.dk, sh.dv, sh.K, True, 1e-6, gdn.GDN_BF16)
    dev = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    # input replicas so that the calls read qkv cold: the 64 MiB of the 4096-token prompt
    # takes 4 to exceed the 256 MB cache; larger inputs fewer
    reps = 1 if ragged else max(1, min(4, (512 << 20) // (B * L * sh.D * 2)))
    xs = [dev(gi.qkv(sh, B, L, seed + 100 * r, "bf16")) for r in range(reps)]
    if fused:   # raw a/b through the prologue, gated RMSNorm epilogue with z
        g = dev(gi.a_raw(sh, B, L, seed, "bf16"))
        b = dev(gi.b_raw(sh, B, L, seed, "bf16"))
        fus = gdn.GdnFusion(dev(gi.a_log(sh, seed, "bf16")), dev(gi.dt_bias(sh, seed, "bf16")),
                            dev(gi.z_gate(sh, B, L, seed, "bf16")), dev(gi.norm_weight(sh, seed, "bf16")), 1e-6)
    else:
        g = dev(gi.gate(sh, B, L, seed, "bf16"))
        b = dev(gi.beta(sh, B, L, seed, "bf16"))
    w = dev(gi.conv_weight(sh, seed, "bf16"))
    c0 = torch.zeros((N, sh.D, sh.K - 1), device="cuda", dtype=torch.bfloat16)
    c_out = torch.empty_like(c0)
    S = torch.zeros((N, sh.Hv, sh.dk, sh.dv), device="cuda")
    o = torch.empty((B, L, sh.Hv, sh.dv), device="cuda")
    cu = torch.from_numpy(cu_np).cuda() if ragged else None
    ws = gdn.prefill_workspace(p, B, L, N)

    def step(i):
        # the state is carried in place, so each call continues from the last one's
        # final state: the work per call is the same whatever S holds
        if fused:
            gdn.gdn_prefill_ex(p, fus, xs[i % reps], g, b, w, c0, c_out, S, o, ws, cu_seqlens=cu)
        else:
            gdn.gdn_prefill(p, xs[i % reps], g, b, w, c0, c_out, S, o, ws, cu_seqlens=cu)

    wall, per = run_timed(torch, step, args.steps, args.warmup)
    t = summary(per)
    flops = PREFILL_FLOP_PER_TOKEN_HEAD * B * L * sh.Hv
    achieved = flops / (t["median_us"] * 1e-6) / 1e12
    nbytes = prefill_bytes(sh, B * L, N, fused)
    cname = ("ragged_prefill_8seqs_d128" if ragged else "prefill_L4096_d128") + ("_fused" if fused else "")
    c = counters(cname, source_digest(PREFILL_SOURCES)) if standard and not short else None
    roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / BF16_PEAK_TFLOPS, "traffic": traffic_from_counters(c),
            "kernel": "gdn_prefill (all kernels of one call)",
            "algorithmic_flops_per_call": flops, "algorithmic_bytes_per_call": nbytes,
            "achieved_GBs": nbytes / (t["median_us"] * 1e-6) / 1e9, "avg_call_us": t["median_us"]}
    if c is not None and "mfma_busy" in c:
        roof["mfma_busy"] = c["mfma_busy"]
    return {
        "metric": METRIC, "value": B * L * args.steps / wall, "unit": "tokens/s",
        "ms_per_step": 1e3 * wall / args.steps,
        "config": {"workload": (f"packed prefill, {SHORT_N} sequences of {SHORT_LEN} tokens" if short else
                                w_.name if standard else f"prefill_B{B}_L{L}_Hk16_Hv32_d128_chunk64")
                   + ("+gate_beta_prologue+gated_rmsnorm_epilogue" if fused else ""),
                   "L_total": B * L, "N": N, "Hk": sh.Hk, "Hv": sh.Hv, "dk": sh.dk,
                   "dv": sh.dv, "chunk": 64, "cache": f"{reps} input replicas"},
        "dtype": "f32",
        "timing": t,
        "roofline": roof,
    }


# (timed steps, untimed warm-up steps). Every workload keeps the GPU busy for 10-40 ms
# before timing: the prefill calls' time still fell by about 10% over the first ~10 ms of
# back-to-back calls (the clocks settling), which a 3 ms warm-up left in the timed
# region, and decode's first repetition after a 1.6 ms warm-up ran about 3% slow.
DEFAULT_STEPS = {"decode": (256, 256), "decode_fused": (256, 256), "verify": (50, 40), "commit": (50, 100),
                 "prefill": (60, 200), "ragged": (20, 40), "prefill_fused": (60, 200), "ragged_fused": (20, 40),
                 "spec_round_copy": (50, 30), "spec_round_slots": (50, 40), "packed_short": (20, 30)}
EXTRAS = ("prefill", "ragged", "verify", "commit")


def bench_fn(name):
    return {"decode": bench_decode, "verify": bench_verify,
            "decode_fused": lambda a, t, g, i: bench_decode(a, t, g, i, fused=True),
            "commit": lambda a, t, g, i: bench_verify(a, t, g, i, commit=True),
            "prefill": bench_prefill,
            "ragged": lambda a, t, g, i: bench_prefill(a, t, g, i, ragged=True),
            "prefill_fused": lambda a, t, g, i: bench_prefill(a, t, g, i, fused=True),
            "spec_round_copy": lambda a, t, g, i: bench_verify(a, t, g, i, rnd="copy"),
            "spec_round_slots": lambda a, t, g, i: bench_verify(a, t, g, i, rnd="slots"),
            "ragged_fused": lambda a, t, g, i: bench_prefill(a, t, g, i, ragged=True, fused=True),
            "packed_short": lambda a, t, g, i: bench_prefill(a, t, g, i, short=True)}[name]


def with_measured(res, ceil):
    """frac_of_measured: the achieved rate over the measured ceiling of the same unit (HBM:
    the best copy, which like these kernels reads and writes; MFMA: the fp16 loop, the
    operand type of the prefill products)."""
    if ceil is None:
        return res
    r = res["roofline"]
    if r["bound"] == "hbm":
        r["measured_peak"] = ceil["copy_best_GBs"]
    else:
        r["measured_peak"] = ceil["mfma_f16_TFLOPs"]
    r["frac_of_measured"] = r["achieved"] / r["measured_peak"]
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode", choices=sorted(DEFAULT_STEPS))
    ap.add_argument("--verify-t", type=int, default=4,
                    help="verify/commit/spec_round_*: block width T (tokens per sequence per block)")
    ap.add_argument("--prefill-rows", type=int, default=1,
                    help="prefill/prefill_fused: unpacked rows (prompts) per call")
    ap.add_argument("--prefill-len", type=int, default=4096,
                    help="prefill/prefill_fused: tokens per row")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--no-extras", dest="extras", action="store_false",
                    help="skip the ceilings and the other workloads (profiling runs)")
    ap.add_argument("--warm", action="store_true",
                    help="decode: also time the warm-cache rate (one state replica)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run one plain 256 MiB device copy (reads and writes 268435456 B), "
                         "so that HBM counters can be scaled by a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the layer's path is built and measured on a single "
              f"MI355X (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    defaults = DEFAULT_STEPS[args.workload]
    args.steps = defaults[0] if args.steps is None else args.steps
    args.warmup = defaults[1] if args.warmup is None else args.warmup
    main_is_decode = args.workload == "decode"
    if not main_is_decode:
        args.cpu_baseline = False
        args.extras = False

    import torch
    import gdn_inputs as gi
    import linear_attention_sequence_amd as gdn
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    gdn.load()
    if args.calibration_copy:
        src = torch.ones(64 << 20, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    clib = _ceiling_lib()
    meta = run_metadata(torch, clib)
    ceil = None
    if args.extras and clib is not None:
        log("measuring ceilings ...")
        ceil = measure_ceilings(torch, clib, meta["cus"])
    res = with_measured(bench_fn(args.workload)(args, torch, gdn, gi), ceil)
    out = {"metric": res.pop("metric"), "value": res.pop("value"), "unit": res.pop("unit"),
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": res.pop("dtype"), "data": "synthetic (seeded)",
           "config": res.pop("config")}
    out.update(res)
    if args.extras:
        wl = {}
        for name in EXTRAS:
            log(f"workload {name} ...")
            a = argparse.Namespace(**vars(args))
            a.steps, a.warmup = DEFAULT_STEPS[name]
            r = with_measured(bench_fn(name)(a, torch, gdn, gi), ceil)
            wl[r["config"]["workload"]] = {"value": r["value"], "unit": r["unit"], "steps": a.steps,
                                           "warmup": a.warmup, "ms_per_step": r["ms_per_step"],
                                           "config": r["config"], "timing": r["timing"],
                                           "roofline": r["roofline"]}
            torch.cuda.empty_cache()
        out["workloads"] = wl
    if ceil is not None:
        out["ceilings"] = ceil
    out["run"] = meta
    if args.cpu_baseline:
        log("timing the oracle on the host ...")
        out["cpu_baseline"] = cpu_baseline(gi)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
