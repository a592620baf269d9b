#!/usr/bin/env python3
"""Benchmark of the speculative-sampling verify step on one MI355X.

Default workload: B=256 sequences, K=7 draft positions, V=262144 vocabulary,
bf16 logits (target N(0,3^2) plus a Zipf(1.1) log-prior, draft = target +
N(0,0.7^2) noise, draft tokens sampled from the draft softmax), temperature 1,
SAMPLE mode.  One step = one spec_verify call over the whole batch with its
inputs already resident in HBM.

Prints ONE JSON line on stdout:
  value      verified draft positions per second, B*(K+1) / step time, the
             step time taken over `--steps` uninstrumented calls
  roofline   the row-statistics kernel (the dominant one): algorithmic bytes
             per launch (every logit of target and draft rows 0..K-1 read
             once) / its average duration from HIP events recorded on the
             launch stream around every launch in a second pass over the same
             steps, against MI355X's 8 TB/s HBM peak; `traffic` is HBM bytes
             per launch from the rocprofv3 PMC summary in profiles/ when that
             summary matches the current kernel source, else null.
             Beside the peak: the measured rate of a read-only stream of the
             same loads (spec_read_stream_probe) and of a device copy.
  acceptance alpha observed (accepted drafts / accept tests taken), mean
             tokens per verify and the closed form at that alpha.
  cpu_baseline  the fp64 oracle timed on this host's cores on a sample of the
             same batch (it is a baseline, not a target); untimed on the same
             sample: mean beta = sum_v min(P_t, P_d) with the exact expected
             tokens per verify, and a decision-level comparison of the GPU
             outputs with the oracle (disagreements, excused ties, failures).
  early_exit the position-by-position schedule on the same batch (identical
             outputs; rows after each sequence's first rejection not read).
  kv_commit  the KV-cache commit of that batch's accepted drafts on a
             Llama-3-8B-like cache layout (bytes moved, HBM rate).
  greedy, small_batches, shortlist_head
             (default workload, unless --no-extras) GREEDY mode on the same
             batch; the smaller batch configurations (B=1, 8, 64), warm and
             cold; the shortlisted drafter head with full-vocabulary verify,
             its sparse-draft form and the static shared shortlist head.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
LLC_BYTES = 256 << 20   # MI355X last-level (Infinity) cache
MFMA_BF16_PEAK_TFLOPS = 2500.0
HEAD_WORKLOAD = "shortlist_head_b32_k4_d4096_v128256"
PROFILE_PMC = os.path.join(ROOT, "profiles", "stats_kernel_b256_k7_v262144_bf16_pmc.md")
HEAD_PROFILE_PMC = os.path.join(ROOT, "profiles", "head_mfma_kernel_shortlist_b32_k4_d4096_v128256_pmc.md")
CSRC = os.path.join(ROOT, "speculative_sampling_verification_vocab_amd", "csrc")
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("sv_verify.hip", "sv_common.h")]
HEAD_SOURCES = [os.path.join(CSRC, f) for f in ("sv_head.hip", "sv_common.h")]
STATIC_PROFILE_PMC = os.path.join(ROOT, "profiles", "head_static_kernel_frspec_m128_n32768_d4096_pmc.md")
STATIC_SOURCES = [os.path.join(CSRC, f) for f in ("sv_static.hip", "sv_common.h")]
MFMA_PROFILE_PMC = os.path.join(ROOT, "profiles", "head_kernels_mfma_busy_pmc.md")
MFMA_SOURCES = [os.path.join(CSRC, f) for f in ("sv_head.hip", "sv_static.hip", "sv_common.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_value(path, key, sources):
    """A figure recorded as `key: value` in a committed rocprofv3 summary, if
    the summary was taken on the current kernel source (its source_sha256)."""
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"source_sha256:\s*([0-9a-f]+)", txt)
    m_v = re.search(re.escape(key) + r":\s*([0-9.eE+-]+)", txt)
    if not m_hash or not m_v or m_hash.group(1) != source_hash(sources):
        return None
    return float(m_v.group(1))


def traffic_from_profile(path=PROFILE_PMC, sources=KERNEL_SOURCES):
    """HBM bytes per launch of the dominant kernel from a committed PMC
    summary, if it was taken on the current kernel source."""
    return profile_value(path, "hbm_bytes_per_launch", sources)


def cpu_baseline(case, res, args, K):
    """The fp64 C oracle on the host cores, timed on a bounded sample of the
    same batch: the first --cpu-sample sequences, repeated until about
    --cpu-seconds of thread time has been spent (at most 20 repetitions)."""
    import numpy as np

    import oracle
    B = case.B
    nb = min(args.cpu_sample, B)
    sl = slice(0, nb)
    greedy = args.mode == "greedy"
    tgt_h = case.target[sl].cpu()
    dr_h = None if greedy else case.draft[sl].cpu()
    tok_h = case.draft_tokens[sl].cpu()
    uni_h = None if greedy else case.uniforms[sl].cpu()
    threads = oracle.default_threads()
    mode = oracle.GREEDY if greedy else oracle.SAMPLE
    reps, wall = 0, 0.0
    while reps < 20 and (reps == 0 or wall * threads < args.cpu_seconds):
        t1 = time.perf_counter()
        orc = oracle.verify(tgt_h, dr_h, tok_h, uni_h, case.temperature, mode=mode, threads=threads)
        wall += time.perf_counter() - t1
        reps += 1
    agree = int(np.sum(orc["accepted_len"] == res[0][sl].cpu().numpy()))
    # The same sample, untimed: decision-level agreement with the GPU outputs
    # (the tie accounting of the parity tests) and, in sample mode, the
    # per-position acceptance probabilities beta = sum_v min(P_t, P_d).
    from tests.parity_util import compare, probe_tokens
    g_len, g_out = res[0][sl].cpu().numpy(), res[1][sl].cpu().numpy()
    orc_p = oracle.verify(tgt_h, dr_h, tok_h, uni_h, case.temperature, mode=mode, threads=threads,
                          probe_token=None if greedy else probe_tokens(g_len, g_out))
    rep = compare(g_len, g_out, orc_p, K, greedy=greedy)
    parity = {"sequences": nb, "decisions": rep.decisions, "disagreements": rep.excused + len(rep.failures),
              "excused_ties": rep.excused, "failures": len(rep.failures),
              "rule": "a disagreement is excused only within 1e-6 of the oracle's decision boundary"}
    beta = None
    if not greedy and K > 0:
        b = oracle.overlap(tgt_h[:, :K].contiguous(), dr_h, case.temperature, threads=threads)
        prod = np.ones(nb)
        expect = np.zeros(nb)
        for i in range(K + 1):
            expect += prod
            if i < K:
                prod = prod * b[:, i]
        a = float(np.mean(b))
        beta = {"alpha_mean_beta": a, "expected_tokens_per_verify_exact": float(np.mean(expect)),
                "closed_form_tokens_at_mean_beta": (1 - a ** (K + 1)) / (1 - a) if a < 1 else float(K + 1),
                "observed_mean_tokens_per_verify": float(np.mean(g_len[g_len >= 0] + 1)),
                "sample": f"first {nb} sequences, fp64 oracle"}
    # one thread on a smaller slice of the same sample, for the per-core rate
    n1 = max(1, min(nb, 16))
    t1 = time.perf_counter()
    oracle.verify(tgt_h[:n1], None if dr_h is None else dr_h[:n1], tok_h[:n1], None if uni_h is None else uni_h[:n1],
                  case.temperature, mode=mode, threads=1)
    w1 = time.perf_counter() - t1
    return {"value": reps * nb * (K + 1) / wall, "unit": "positions/s", "cores": threads, "kind": "oracle",
            "single_thread_value": n1 * (K + 1) / w1,
            "sample": f"first {nb} of {B} sequences of the same batch x {reps} repetitions, fp64 C oracle, "
                      f"{threads} threads, {wall:.2f} s wall; accepted_len agrees on {agree}/{nb}; "
                      f"single thread: first {n1} sequences once, {w1:.2f} s",
            "parity_sample": parity, "acceptance_sample": beta}


def acceptance_report(n, K):
    """Acceptance from the GPU outputs of one step: alpha = accepted drafts /
    accept tests taken (a sequence that accepted n drafts took min(n + 1, K)
    tests), the mean tokens emitted per verify, and the closed form
    (1 - alpha^(K+1)) / (1 - alpha) for i.i.d. acceptance at that alpha."""
    import numpy as np
    n = np.asarray(n)
    n = n[n >= 0].astype(np.int64)
    tests = int(np.minimum(n + 1, K).sum()) if K > 0 else 0
    alpha = float(n.sum()) / tests if tests else float("nan")
    closed = None
    if tests:
        closed = (1 - alpha ** (K + 1)) / (1 - alpha) if alpha < 1 else float(K + 1)
    return {"alpha_observed": alpha, "accept_tests": tests, "accepted_drafts": int(n.sum()),
            "mean_tokens_per_verify": float(np.mean(n + 1)) if n.size else float("nan"),
            "closed_form_tokens_at_alpha_observed": closed}


def copy_reference(dev, gib=1.0, reps=5):
    """Measured bandwidth of a plain device copy (torch's copy kernel), bytes
    read + written per second: the practical ceiling beside the 8 TB/s peak."""
    import numpy as np
    import torch
    n = int(gib * (1 << 30)) // 4
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        b.copy_(a)
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.median([x.elapsed_time(y) for x, y in ev]))
    del a, b
    return 2.0 * n * 4 / (ms * 1e-3) / 1e9


def read_stream_reference(dev, gib=2.0, reps=9):
    """Measured read-only streaming rate (spec_read_stream_probe: the
    statistics pass's loads with no arithmetic) over `gib` GiB, larger than
    the last-level cache, alternating two halves so no call re-reads what the
    previous one left cached: the like-for-like ceiling for the read-only
    passes beside the 8 TB/s peak."""
    import ctypes

    import numpy as np
    import torch

    import speculative_sampling_verification_vocab_amd as sv
    lib = sv._native.load()
    half = (int(gib * (1 << 30)) // 2) // 32768 * 32768
    buf = torch.ones(2 * half // 2, dtype=torch.bfloat16, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def run(i):
        sv._native.check(lib.spec_read_stream_probe(ctypes.c_void_p(buf.data_ptr() + (i % 2) * half), half,
                                                    ctypes.c_void_p(sink.data_ptr()), st), "read probe")

    run(0)
    run(1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        run(i)
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.median([x.elapsed_time(y) for x, y in ev]))
    del buf
    return half / (ms * 1e-3) / 1e9


def cold_warm(call, input_bytes, dev, reps=20):
    """Median HIP-event time of one call with its inputs cache-resident (warm)
    and after reading 512 MiB of other data, which evicts them from the
    256 MB last-level cache (cold).  The eviction reads rather than writes so
    that the cold call does not also pay for writing back dirty lines.  Only
    meaningful for inputs well under 256 MB."""
    import numpy as np
    import torch
    flush = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    out = {}
    for kind in ("warm", "cold"):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        call()
        for e0, e1 in ev:
            if kind == "cold":
                torch.sum(flush, dim=0, out=sink)
            e0.record()
            call()
            e1.record()
        torch.cuda.synchronize()
        out[kind + "_us"] = float(np.median([x.elapsed_time(y) for x, y in ev])) * 1e3
    del flush
    out["input_bytes"] = input_bytes
    out["cold_gbs"] = input_bytes / (out["cold_us"] * 1e-6) / 1e9
    out["note"] = "median of %d calls, events around the call only; cold = after a 512 MiB read" % reps
    return out


def bench_kv_commit(accepted_len, K, steps, dev):
    """KV-cache commit of one verify step's accepted drafts (spec_kv_commit)
    on a Llama-3-8B-like layout: 32 layers x {K, V} planes, 8 KV heads x 128
    dims, bf16, 128 cache positions, B sequences.  Bytes moved = 2 (read and
    write) x sum over committed sequences of n x planes x row bytes.  Each
    timed call restores the lengths first (outside the events), so every call
    moves the same rows.  Sampled rows are checked against the staging buffer."""
    import numpy as np
    import torch

    import speculative_sampling_verification_vocab_amd as sv
    from workloads import KV_WORKLOAD, kv_case

    w = KV_WORKLOAD
    B = int(accepted_len.numel())
    kc = kv_case(w["P"], B, K, w["Lmax"], w["E"], device=dev)
    ln0 = kc.cache_len.clone()
    stream = torch.cuda.current_stream(dev)
    acc = accepted_len.to(torch.int32)
    st = sv.spec_kv_commit(kc.cache, kc.staging, acc, kc.cache_len)
    torch.cuda.synchronize()
    n = acc.cpu().numpy()
    l0 = ln0.cpu().numpy()
    ok = st.cpu().numpy() == 0
    rng = np.random.default_rng(11)
    checked = 0
    for _ in range(16):
        b = int(rng.integers(B))
        p = int(rng.integers(w["P"]))
        if not ok[b] or n[b] == 0:
            continue
        got = kc.cache[p, b, l0[b]:l0[b] + n[b]]
        assert torch.equal(got, kc.staging[p, b, :n[b]]), "kv commit: committed rows differ from staging"
        checked += 1
    row_bytes = w["E"] * 2
    moved = int(2 * n[ok].clip(min=0).sum()) * w["P"] * row_bytes
    times = []
    for _ in range(steps):
        kc.cache_len.copy_(ln0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sv.spec_kv_commit(kc.cache, kc.staging, acc, kc.cache_len, status=st)
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in times]))
    del kc
    return {"workload": w["name"].replace("b256", f"b{B}"), "P": w["P"], "E": w["E"], "L_max": w["Lmax"],
            "ms_per_call": ms, "bytes_moved": moved, "achieved_gbs": moved / (ms * 1e-3) / 1e9,
            "hbm_frac": moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "committed_sequences": int(ok.sum()),
            "mean_committed_entries": float(n[ok].mean()) if ok.any() else 0.0, "sampled_rows_checked": checked}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="b256_k7_v262144_bf16")
    ap.add_argument("--mode", default="sample", choices=["sample", "greedy", "sample_early_exit"])
    ap.add_argument("--no-kv-commit", action="store_true",
                    help="skip the KV-cache commit of the verify step's accepted drafts in sample mode")
    ap.add_argument("--no-early-exit", action="store_true",
                    help="skip the extra timing of the early-exit schedule in sample mode")
    ap.add_argument("--cpu-sample", type=int, default=256, help="sequences timed on the CPU oracle")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="thread-seconds of oracle work to time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the small-batch, greedy and drafter-head measurements of the default run")
    ap.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                    help="also run one plain device copy of this many GiB (PMC scaling reference)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(verify shards over sequences with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import speculative_sampling_verification_vocab_amd as sv
    from workloads import workload_case

    dev = torch.device("cuda", 0)
    if args.calibrate_copy_gib > 0:
        n = int(args.calibrate_copy_gib * (1 << 30)) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"calibration copy: {n * 4} bytes read, {n * 4} bytes written")
        del a, b
    if args.workload == HEAD_WORKLOAD:
        print(json.dumps(bench_shortlist(args, dev)), flush=True)
        return
    t0 = time.time()
    case = workload_case(args.workload, device=dev, greedy=args.mode == "greedy")
    torch.cuda.synchronize()
    B, K, V = case.B, case.K, case.V
    esz = 2 if case.dtype == "bf16" else 4
    log(f"inputs generated in {time.time() - t0:.1f}s: B={B} K={K} V={V} {case.dtype} T={case.temperature}")

    ws = sv.Workspace(dev)
    stream = torch.cuda.current_stream(dev)
    # Inputs larger than the 256 MB last-level cache: consecutive steps
    # alternate between two copies of the batch (same values, other
    # addresses).  With one copy, the rows that step i's sampling pass reads
    # (~240 MB at B=256, K=7, V=262144) are still cached when step i+1's
    # statistics pass reads them again, which no serving loop sees: new
    # logits arrive every step.
    in_bytes = case.target.numel() * esz + (case.draft.numel() * esz if case.draft is not None else 0)
    sets = [case]
    if in_bytes > LLC_BYTES:
        sets.append(type(case)(case.target.clone(), case.draft.clone() if case.draft is not None else None,
                               case.draft_tokens.clone(), case.uniforms.clone(), case.temperature, case.dtype))
        torch.cuda.synchronize()

    def timed(mode, steps, warmup):
        """Two passes of `steps` verify calls after `warmup` untimed ones.
        Pass 1 (no instrumentation): mean wall ms per step between two device
        synchronisations.  Pass 2: the same calls with a HIP event recorded on
        the launch stream before every kernel launch and after the last, for
        per-kernel durations, mean and median over the steps (an event record
        between dependent launches adds ~3 us, so pass 2 is not used for the
        step time)."""
        L = sv.spec_verify_launch_count(B, K, V, case.target.dtype, mode)
        NE = L + 1
        # A serving loop's call: outputs and workspace allocated once (VerifyPlan)
        plan = sv.VerifyPlan(B, K, V, case.target.dtype, mode, device=dev, stream=stream)

        def step(i, evs=None):
            c = sets[i % len(sets)]
            return plan(c.target, c.draft, c.draft_tokens, c.uniforms, c.temperature, events=evs)

        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        start = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - start) * 1e3 / steps
        res = [t.clone() for t in step(0)]  # outputs of the first copy (the batch itself)
        torch.cuda.synchronize()

        evs = [torch.cuda.Event(enable_timing=True) for _ in range(NE * steps)]
        for e in evs:
            e.record(stream)  # creates the underlying hipEvent
        torch.cuda.synchronize()
        for s in range(steps):
            step(s, evs[NE * s:NE * s + NE])
        torch.cuda.synchronize()

        def span(i, j, f=np.mean):
            return float(f([evs[NE * s + i].elapsed_time(evs[NE * s + j]) for s in range(steps)]))

        launch_ms = [span(k, k + 1) for k in range(L)]
        timed.medians = {"launches": [span(k, k + 1, np.median) for k in range(L)],
                         "events_step": span(0, L, np.median)}
        return ms, launch_ms, span(0, L), res

    ms_step, launch_ms, ev_step, res = timed(args.mode, args.steps, args.warmup)
    k_ms = {"launches": launch_ms, "events_step": ev_step, "median": timed.medians}
    acc = res[0].float()
    mean_tokens = float((acc[acc >= 0] + 1).mean()) if (acc >= 0).any() else float("nan")

    early = None
    if args.mode == "sample" and not args.no_early_exit:
        # The early-exit schedule on the same batch: identical outputs, rows after
        # each sequence's first rejection are not read.
        ee_ms, ee_launch, ee_ev, ee_res = timed("sample_early_exit", args.steps, args.warmup)
        same = bool(torch.equal(ee_res[0], res[0]) and torch.equal(ee_res[1], res[1]))
        n = res[0].cpu().numpy()
        rows = np.where(n >= 0, np.minimum(n, K - 1) + 1, 0) if K > 0 else np.zeros(B)
        need = int(2 * rows.sum()) * V * esz            # target and draft rows 0..min(n, K-1)
        # launches 0..K-1: position i's statistics (and the decision of i - 1),
        # then the sampling pass (decides K - 1) and the pick
        phase_ms = float(sum(ee_launch[0:K]))
        early = {
            "mode": "sample_early_exit",
            "value": B * (K + 1) / (ee_ms * 1e-3),
            "unit": "positions/s",
            "ms_per_step": ee_ms,
            "outputs_identical_to_full_schedule": same,
            "rows_read_fraction": float(rows.sum()) / max(1, B * K),
            "statistics_bytes_needed": need,
            "phase_launches_ms": phase_ms,
            "sampling_ms": float(ee_launch[K]) if len(ee_launch) > K else None,
            "pick_ms": float(ee_launch[K + 1]) if len(ee_launch) > K + 1 else None,
            "statistics_gbs": need / (phase_ms * 1e-3) / 1e9 if phase_ms > 0 else None,
            "kernels_ms": {"launches": ee_launch, "events_step": ee_ev},
        }

    positions = B * (K + 1)
    value = positions / (ms_step * 1e-3)
    if args.mode == "sample":
        step_bytes = B * (2 * K + 1) * V * esz          # every logit read once
        dom_bytes = B * 2 * K * V * esz                 # launch 0: rows 0..K-1 of target and draft
        dom_name, dom_ms = "stats_kernel (per-tile max and exp sums of the proposal rows)", launch_ms[0]
    elif args.mode == "sample_early_exit":
        # bytes the rule needs: target and draft rows up to the first rejection,
        # plus the bonus row where every draft was accepted
        n = res[0].cpu().numpy()
        rows = np.where(n >= 0, np.minimum(n, K - 1) + 1, 0) if K > 0 else np.zeros(B, dtype=np.int64)
        dom_bytes = int(2 * rows.sum()) * V * esz
        step_bytes = dom_bytes + int((n == K).sum()) * V * esz
        dom_name = "ee_phase_kernel, all positions (statistics of the rows up to each first rejection)"
        dom_ms = float(sum(launch_ms[0:K])) if K > 0 else launch_ms[0]
    else:
        step_bytes = B * (K + 1) * V * esz
        dom_bytes = step_bytes
        dom_name, dom_ms = "greedy_kernel (per-tile argmax)", launch_ms[0]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = traffic_from_profile() if (args.workload == "b256_k7_v262144_bf16" and args.mode == "sample") else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, res, args, K)
    copy_gbs = copy_reference(dev)
    read_gbs = read_stream_reference(dev)
    cache = None
    in_bytes = step_bytes + B * K * 4 + B * (K + 1) * 8
    if in_bytes < 256_000_000:
        # inputs that fit the 256 MB last-level cache: report cold and warm calls
        plan = sv.VerifyPlan(B, K, V, case.target.dtype, args.mode, device=dev)
        cache = cold_warm(lambda: plan(case.target, case.draft, case.draft_tokens, case.uniforms, case.temperature),
                          in_bytes, dev)
    kv = None
    if args.mode == "sample" and not args.no_kv_commit:
        kv = bench_kv_commit(res[0], K, args.steps, dev)
    extras = {}
    if args.mode == "sample" and not args.no_extras and args.workload == "b256_k7_v262144_bf16":
        # the other rows of the path, measured in the same run: GREEDY on this
        # batch, the smaller batch configurations, and the drafter heads
        log("greedy on the benchmark batch")
        extras["greedy"] = bench_greedy(case, sets, args.steps, args.warmup, dev)
        log("small batch configurations")
        extras["small_batches"] = bench_small_batches(dev)
        log("drafter heads (shortlist gather-GEMM + verify, sparse draft, static shortlist)")
        head = bench_shortlist(args, dev)
        extras["shortlist_head"] = {k: head[k] for k in ("ms_per_step", "value", "unit", "config", "kernels_ms",
                                                         "roofline", "mfma", "acceptance", "sparse_draft",
                                                         "static_head", "cache_residency_verify")}

    out = {
        "metric": "verified draft positions/sec (B*(K+1)) and achieved HBM GB/s vs peak",
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic (seeded generators; no dataset or model weights)",
        "config": {"workload": args.workload, "B": B, "K": K, "V": V, "logits": case.dtype,
                   "temperature": case.temperature, "mode": args.mode},
        "achieved_gbs_step": step_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_frac_step": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernels_ms": k_ms,
        "mean_tokens_per_verify": mean_tokens,
        "acceptance": acceptance_report(res[0].cpu().numpy(), K),
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": dom_bytes,
                     "measured_read_stream_gbs": read_gbs, "frac_of_read_stream": achieved / read_gbs,
                     "measured_copy_gbs": copy_gbs,
                     "references": "measured_read_stream_gbs: read-only stream with the statistics pass's "
                                   "loads and no arithmetic (the like-for-like ceiling); measured_copy_gbs: "
                                   "torch device copy, bytes read + written"},
        "cpu_baseline": cpu,
    }
    if cache is not None:
        out["cache_residency"] = cache
    if early is not None:
        out["early_exit"] = early
    if kv is not None:
        out["kv_commit"] = kv
    out.update(extras)
    print(json.dumps(out), flush=True)


def bench_shortlist(args, dev):
    """Shortlisted drafter head (bf16 MFMA) followed by full-vocabulary verify:
    B=32 contexts, K=4, d=4096, V=128256 in 256 clusters of 501, top-16 clusters
    per context; target N(0,3^2)+Zipf(1.1); T=1.  One step = head + verify."""
    import numpy as np
    import torch

    import speculative_sampling_verification_vocab_amd as sv
    from workloads import gumbel_max_tokens, head_case, normal_logits, verify_uniforms

    hc = head_case(device=dev)
    B, K, d = hc.h.shape
    V = hc.W.shape[0]
    cs, n_sel = hc.cluster_size, hc.cluster_ids.shape[1]
    target = normal_logits((B, K + 1, V), 3.0, 1.1, (0, 5, 0, 0, 0), dev).to(torch.bfloat16)
    _, dense = sv.spec_draft_head_shortlist(hc.h, hc.W, hc.cluster_ids, cs, compact=False,
                                            dense_dtype=torch.bfloat16)
    tok = gumbel_max_tokens(dense, 1.0, (0, 5, 0, 2, 0))
    uni = verify_uniforms(B, K, (0, 5, 0, 3, 0), dev)
    ws = sv.Workspace(dev)
    stream = torch.cuda.current_stream(dev)
    L = sv.spec_verify_launch_count(B, K + 1 - 1, V, torch.bfloat16, "sample")
    NE = L + 1

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        _, dn = sv.spec_draft_head_shortlist(hc.h, hc.W, hc.cluster_ids, cs, compact=False,
                                             dense_dtype=torch.bfloat16)
        if evs is not None:
            evs[1].record(stream)
        return sv.spec_verify(target, dn, tok, uni, 1.0, "sample", workspace=ws,
                              events=evs[2:] if evs is not None else None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        res = step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # second pass with an event around every launch, for per-kernel durations
    evs = [torch.cuda.Event(enable_timing=True) for _ in range((NE + 2) * args.steps)]
    for e in evs:
        e.record(stream)
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(evs[(NE + 2) * s:(NE + 2) * (s + 1)])
    torch.cuda.synchronize()

    def span(i, j):
        return float(np.mean([evs[(NE + 2) * s + i].elapsed_time(evs[(NE + 2) * s + j]) for s in range(args.steps)]))

    head_ms = span(0, 1)
    k_ms = {"head": head_ms, "verify_launches": [span(2 + k, 3 + k) for k in range(L)],
            "events_step": span(0, 2 + L)}
    sel = torch.unique(hc.cluster_ids).numel()
    w_bytes = sel * cs * d * 2
    head_bytes = w_bytes + B * K * d * 2 + B * K * V * 2          # W of the selected clusters, h, dense bf16 out
    flops = 2.0 * B * K * n_sel * cs * d
    achieved = head_bytes / (head_ms * 1e-3) / 1e9
    tflops = flops / (head_ms * 1e-3) / 1e12
    acc = res[0].float()
    out = {
        "metric": "verified draft positions/sec (B*(K+1)) and achieved HBM GB/s vs peak",
        "value": B * (K + 1) / (ms_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded generators; no dataset or model weights)",
        "config": {"workload": HEAD_WORKLOAD, "B": B, "K": K, "d": d, "V": V, "clusters": V // cs,
                   "cluster_size": cs, "n_sel": n_sel, "selected_clusters_union": sel, "temperature": 1.0},
        "kernels_ms": k_ms,
        "mean_tokens_per_verify": float((acc[acc >= 0] + 1).mean()),
        "acceptance": acceptance_report(res[0].cpu().numpy(), K),
        "roofline": {"bound": "hbm", "kernel": "head_mfma_kernel (shortlist gather-GEMM)", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_from_profile(HEAD_PROFILE_PMC, HEAD_SOURCES),
                     "algorithmic_bytes_per_launch": head_bytes},
        "mfma": {"achieved_tflops": tflops, "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                 "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "flops_per_launch": flops,
                 "busy_frac_pmc": profile_value(MFMA_PROFILE_PMC, "mfma_busy_frac head_mfma_kernel", MFMA_SOURCES),
                 "ridge_note": f"{flops / head_bytes:.1f} flop/byte against a ridge of "
                               f"{MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):.0f}: HBM-bound"},
        "cpu_baseline": None,
    }
    vb = B * (2 * K + 1) * V * 2 + B * K * 4 + B * (K + 1) * 8
    out["cache_residency_verify"] = cold_warm(
        lambda: sv.spec_verify(target, dense, tok, uni, 1.0, "sample", workspace=ws), vb, dev)
    out["roofline"]["measured_read_stream_gbs"] = read_stream_reference(dev)
    out["roofline"]["frac_of_read_stream"] = achieved / out["roofline"]["measured_read_stream_gbs"]
    out["roofline"]["measured_copy_gbs"] = copy_reference(dev)
    out["sparse_draft"] = bench_sparse_draft(hc, target, uni, args.steps, args.warmup, dev)
    out["static_head"] = bench_static_head(hc, args.steps, args.warmup, dev)
    return out


SMALL_BATCHES = (("b1_k4_v32000_f32", (0.5,)), ("b8_k5_v128256_bf16", (0.2, 1.0)),
                 ("b64_k4_v151936_bf16", (0.1, 0.5, 1.0, 2.0)))


def bench_small_batches(dev):
    """The smaller verify configurations, one call at a time as a serving loop
    makes them (VerifyPlan: no allocation per call): B=1, K=4, V=32000 f32;
    B=8, K=5, V=128256 bf16 at draft noise sigma 0.2 and 1.0 (T=0.8), and its
    greedy run on argmax drafts; B=64, K=4, V=151936 bf16 at sigma 0.1, 0.5,
    1.0, 2.0 (T=1).  Median call time with HIP events around the call, with
    the inputs cache-resident (warm) and after a 512 MiB read (cold), and the
    acceptance the call produced beside the closed form at that alpha."""
    import torch

    import speculative_sampling_verification_vocab_amd as sv
    from workloads import workload_case

    out = []
    for name, sigmas in SMALL_BATCHES:
        runs = [(sw, sig, "sample") for sw, sig in enumerate(sigmas)]
        if name.startswith("b8_"):
            runs.append((0, sigmas[0], "greedy"))
        for sw, sig, mode in runs:
            case = workload_case(name, sweep=sw, device=dev, greedy=mode == "greedy")
            B, K, V = case.B, case.K, case.V
            esz = 2 if case.dtype == "bf16" else 4
            plan = sv.VerifyPlan(B, K, V, case.target.dtype, mode, device=dev)
            args = (case.target, case.draft, case.draft_tokens, case.uniforms, case.temperature)
            res = plan(*args)
            torch.cuda.synchronize()
            acc = acceptance_report(res[0].cpu().numpy(), K)
            rows = (K + 1) if mode == "greedy" else (2 * K + 1)
            t = cold_warm(lambda: plan(*args), B * rows * V * esz, dev)
            out.append({"workload": name, "mode": mode, "sigma": sig, "temperature": case.temperature,
                        "launches": sv.spec_verify_launch_count(B, K, V, case.target.dtype, mode),
                        "warm_us": t["warm_us"], "cold_us": t["cold_us"], "logit_bytes": t["input_bytes"],
                        "cold_gbs": t["cold_gbs"], "hbm_frac_cold": t["cold_gbs"] / HBM_PEAK_GBS,
                        "acceptance": acc})
            del case, plan, res
    return out


def bench_greedy(case, sets, steps, warmup, dev):
    """GREEDY mode on the benchmark batch: argmax of every target row and the
    longest matching prefix.  Mean step time (no instrumentation) and the
    argmax pass's rate on its B*(K+1)*V logits (HIP events on its launch)."""
    import numpy as np
    import torch

    import speculative_sampling_verification_vocab_amd as sv

    B, K, V = case.B, case.K, case.V
    esz = 2 if case.dtype == "bf16" else 4
    plan = sv.VerifyPlan(B, K, V, case.target.dtype, "greedy", device=dev)

    def step(i, evs=None):
        c = sets[i % len(sets)]
        return plan(c.target, None, c.draft_tokens, None, 0.0, events=evs)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e3 in evs:
        for e in e3:
            e.record()  # creates the underlying hipEvent the library records into
    torch.cuda.synchronize()
    for i, e3 in enumerate(evs):
        step(i, e3)
    torch.cuda.synchronize()
    argmax_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    fin_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    nbytes = B * (K + 1) * V * esz
    return {"mode": "greedy", "ms_per_step": ms, "value": B * (K + 1) / (ms * 1e-3), "unit": "positions/s",
            "argmax_kernel_ms": argmax_ms, "finalize_kernel_ms": fin_ms, "logit_bytes": nbytes,
            "argmax_gbs": nbytes / (argmax_ms * 1e-3) / 1e9,
            "argmax_hbm_frac": nbytes / (argmax_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def bench_static_head(hc, steps, warmup, dev):
    """Drafter head over one static shortlist shared by all 128 contexts
    (FR-Spec / VocabTrim): the same h and W, a fixed set of 32768 token ids at
    cluster size 1 (FR-Spec's shortlist size) and of 16 clusters of 501
    (N = 8016).  Times spec_draft_head_static (W rows gathered inside the
    kernel) with fp32 and bf16 logits.  Each timed call takes the next of 8
    different shortlists of that size, so W_S is read from HBM rather than
    left in the 256 MB last-level cache by the previous call (the figure
    with one shortlist repeated is reported as `us_fp32_out_warm`).  Narrow
    shortlists split d over blocks through a workspace; the single-launch
    form is reported beside it.  For context, torch's bf16 GEMM (F.linear,
    i.e. hipBLASLt) on a pre-gathered contiguous W_S, warm."""
    import numpy as np
    import torch
    import torch.nn.functional as F

    import speculative_sampling_verification_vocab_amd as sv

    B, K, d = hc.h.shape
    V = hc.W.shape[0]
    M = B * K
    h2 = hc.h.reshape(M, d)
    ws = sv.Workspace(dev)

    def med(fn, n):
        for i in range(warmup):
            fn(i)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i, (e0, e1) in enumerate(ev):
            e0.record()
            fn(i)
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    shapes = []
    for name, cs, n_sel, seed in (("frspec_32768_tokens", 1, 32768, 11), ("clusters_16x501", 501, 16, 12)):
        sets = []
        for r in range(8):
            g = torch.Generator().manual_seed(seed + 1000 * r)
            sets.append(torch.sort(torch.randperm(V // cs, generator=g)[:n_sel]).values.to(torch.int32).to(dev))
        N = n_sel * cs
        o32 = torch.empty((M, N), dtype=torch.float32, device=dev)
        o16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        n = max(steps, 24)
        ms32 = med(lambda i: sv.spec_draft_head_static(h2, hc.W, sets[i % 8], cs, out=o32, workspace=ws), n)
        ms16 = med(lambda i: sv.spec_draft_head_static(h2, hc.W, sets[i % 8], cs, dtype=torch.bfloat16, out=o16,
                                                       workspace=ws), n)
        ms32_one = med(lambda i: sv.spec_draft_head_static(h2, hc.W, sets[i % 8], cs, out=o32, split=False), n)
        ms32_warm = med(lambda i: sv.spec_draft_head_static(h2, hc.W, sets[0], cs, out=o32, workspace=ws), n)
        rows = (sets[0].long()[:, None] * cs + torch.arange(cs, device=dev)[None, :]).reshape(-1)
        Ws = hc.W[rows].contiguous()
        ms_blas = med(lambda i: F.linear(h2, Ws), n)
        del Ws
        flops = 2.0 * M * N * d
        b32 = N * d * 2 + M * d * 2 + M * N * 4
        b16 = N * d * 2 + M * d * 2 + M * N * 2
        ach = b32 / (ms32 * 1e-3) / 1e9
        split = sv._native.load().spec_draft_head_static_workspace_bytes(M, d, V, cs, n_sel) > 0
        shapes.append({
            "shortlist": name, "M": M, "N": N, "d": d, "cluster_size": cs, "k_split": split,
            "us_fp32_out": ms32 * 1e3, "us_bf16_out": ms16 * 1e3, "us_fp32_out_single_launch": ms32_one * 1e3,
            "us_fp32_out_warm": ms32_warm * 1e3,
            "roofline": {"bound": "hbm", "kernel": "head_static_dma_kernel", "achieved": ach, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                         "traffic": traffic_from_profile(STATIC_PROFILE_PMC, STATIC_SOURCES)
                         if name.startswith("frspec") else None,
                         "algorithmic_bytes_per_launch": b32},
            "bf16_out_gbs": b16 / (ms16 * 1e-3) / 1e9,
            "mfma": {"achieved_tflops": flops / (ms32 * 1e-3) / 1e12, "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                     "frac": flops / (ms32 * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "busy_frac_pmc": profile_value(MFMA_PROFILE_PMC, "mfma_busy_frac head_static_kernel "
                                                    + ("n32768_fp32" if name.startswith("frspec") else "n8016"),
                                                    MFMA_SOURCES)},
            "blas_reference": {"op": "torch F.linear bf16 on a pre-gathered contiguous W_S (hipBLASLt), warm",
                               "us": ms_blas * 1e3},
        })
    return shapes


def bench_sparse_draft(hc, target, uni, steps, warmup, dev):
    """The same contexts with DynaSpec's position-aware budget (k_max = 16:
    16, 16, 2, 2 clusters at positions 0..3): per-position head straight into
    the compact layout (bf16), then spec_verify_sparse_draft, which reads the
    compact draft instead of -inf-filled dense rows.  Draft tokens are sampled
    from the compact draft (Gumbel-max on its dense form, outside the timed
    region)."""
    import numpy as np
    import torch

    import speculative_sampling_verification_vocab_amd as sv
    from workloads import gumbel_max_tokens, normal_logits, top_clusters

    B, K, d = hc.h.shape
    V = hc.W.shape[0]
    cs = hc.cluster_size
    nc = V // cs
    n_sel = [sv.position_budget(t, 16) for t in range(K)]
    S = max(n_sel)
    cids = torch.full((B, K, S), -1, dtype=torch.int32, device=dev)
    for k in range(K):
        cids[:, k, :n_sel[k]] = top_clusters(normal_logits((B, nc), 1.0, 0.0, (0, 5, 1, 4, k), dev), n_sel[k])
    comp = sv.spec_draft_head_positions(hc.h, hc.W, cids, n_sel, cs)
    dense = torch.full((B, K, V), float("-inf"), dtype=torch.bfloat16, device=dev)
    for k in range(K):
        ids = (cids[:, k, :n_sel[k]].long()[:, :, None] * cs + torch.arange(cs, device=dev)).reshape(B, -1)
        dense[:, k].scatter_(1, ids, comp[:, k, :ids.shape[1]])
    tok = gumbel_max_tokens(dense, 1.0, (0, 5, 1, 2, 0))
    del dense
    ws = sv.Workspace(dev)
    stream = torch.cuda.current_stream(dev)

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        cp = sv.spec_draft_head_positions(hc.h, hc.W, cids, n_sel, cs, out=comp)
        if evs:
            evs[1].record(stream)
        r = sv.spec_verify_sparse_draft(target, cp, cids, n_sel, cs, tok, uni, 1.0, workspace=ws)
        if evs:
            evs[2].record(stream)
        return r

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        res = step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e3 in evs:
        step(e3)
    torch.cuda.synchronize()
    head_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    ver_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    short = int(sum(n_sel)) * cs
    verify_bytes = B * (K + 1) * V * 2 + B * short * 2       # target rows + compact draft
    dense_verify_bytes = B * (2 * K + 1) * V * 2
    acc = res[0].float()
    return {"n_sel_per_position": n_sel, "ms_per_step": ms, "value": B * (K + 1) / (ms * 1e-3),
            "unit": "positions/s", "head_ms": head_ms, "verify_ms": ver_ms,
            "verify_bytes": verify_bytes, "dense_verify_bytes_same_shape": dense_verify_bytes,
            "verify_gbs": verify_bytes / (ver_ms * 1e-3) / 1e9,
            "mean_shortlist_tokens": short / K,
            "mean_tokens_per_verify": float((acc[acc >= 0] + 1).mean())}


if __name__ == "__main__":
    main()
