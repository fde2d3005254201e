#!/usr/bin/env python3
"""Benchmark of the packing + document-causal attention path on one MI355X.

One step = the whole path over one synthetic batch already resident in HBM:
  1. GPU packing of the workload's document stream (psc_pack_build),
  2. attention forward over the packed rows' segments (psc_varlen_attn_fwd),
  3. attention backward (psc_varlen_attn_bwd), unless the workload is
     forward-only.
Throughput counts only in-document causal FLOPs: forward
4 * D * Hq * sum over real segments of L(L+1)/2, backward 2.5x that (padding
segments are computed but not counted).  The default workload is the
2 x 32768-token log-normal pack with GQA 32/8 heads, head_dim 128, bf16.

Prints one JSON line.  Besides the standard fields it carries
  roofline:     the dominant kernel's algorithmic FLOP rate (HIP events
                recorded by the library around that kernel alone on its
                stream, summed over the timed steps; an untimed pass with every
                kernel's events picks it and gives kernels_ms_per_step)
                against the bf16 MFMA peak;
  cpu_baseline: the fp64 CPU oracle timed on a bounded sample of the same
                workload (whole documents in order until ~--cpu-seconds of
                work), in the same unit;
  clock:        graphics clock and socket power read with amd-smi while the
                step loops after the timed region, and the rate against the
                peak at that clock;
  workloads:    the same step on every other bf16 workload;
  seed1:        the default workload drawn from seed 1;
  rope, rope_step, data_steps: the rotary embedding pass, the step with the
                rotation separate and fused, and the packer's follow-up data
                steps.
Defaults: 10 untimed warm-up steps, then 50 timed steps.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402  (seeded synthetic inputs; no torch at import)

METRIC = "varlen causal attn fwd+bwd TFLOP/s (in-doc FLOPs) & % MFMA peak, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 dense bf16 FLOP/clk x 2.4 GHz (published 2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0
BF16_WORKLOADS = ["lognormal_32k", "uniform_8k", "seqpar_share_128k", "skewed_32k"]


# HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (each
# scaled by the factor a plain 1 GiB copy gives: 2.0 for FETCH_SIZE, 1.0 for
# WRITE_SIZE), for (kernel, workload), valid only while the kernel's sources
# hash to the recorded value (profiles/hbm_counters_<workload>.md).
KERNEL_SOURCES = {
    "attn_fwd": ["packed_sequence_causal_amd/csrc/attn_fwd.hip", "packed_sequence_causal_amd/csrc/attn_common.h",
                 "packed_sequence_causal_amd/csrc/rope_common.h"],
    "attn_bwd_dkdv": ["packed_sequence_causal_amd/csrc/attn_bwd.hip", "packed_sequence_causal_amd/csrc/attn_common.h",
                      "packed_sequence_causal_amd/csrc/rope_common.h"],
    "attn_bwd_dq": ["packed_sequence_causal_amd/csrc/attn_bwd.hip", "packed_sequence_causal_amd/csrc/attn_common.h",
                    "packed_sequence_causal_amd/csrc/rope_common.h"],
}
MEASURED_TRAFFIC = {
    # (kernel, workload): (sources sha256 prefix, read bytes, write bytes)
    ("attn_fwd", "lognormal_32k"): ("2290f70f7c66f31f", 2.0 * 418581.0 * 1024, 1.0 * 533345.1 * 1024),
    ("attn_bwd_dkdv", "lognormal_32k"): ("8ef2a2d29357273e", 2.0 * 4180083.1 * 1024, 1.0 * 532863.3 * 1024),
    ("attn_bwd_dq", "lognormal_32k"): ("8ef2a2d29357273e", 2.0 * 964721.2 * 1024, 1.0 * 1066056.9 * 1024),
}


def sources_sha(kernel):
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    rec = MEASURED_TRAFFIC.get((kernel, workload))
    if not rec or rec[0] != sources_sha(kernel):
        return None
    return {"read_bytes": rec[1], "write_bytes": rec[2], "bytes": rec[1] + rec[2]}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="lognormal_32k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only --workload (by default the line also carries every other bf16 workload)")
    ap.add_argument("--no-clock", action="store_true", help="skip the amd-smi clock and power reading")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the separate RoPE, fused-RoPE step and data-step measurements (profiles of the "
                         "step's own kernels use this)")
    ap.add_argument("--doc-sweep", action="store_true",
                    help="time each 32K document layout with its document mask and as one whole-row causal "
                         "segment (same kernels); one JSON line per layout")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (3 launches) and exit; "
                         "its HBM counters scale the counters read for the path's kernels")
    return ap.parse_args()


def calibrate_copy(mib):
    import torch

    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "launches": 3}), flush=True)


def real_segments(w, cu):
    """Boolean per segment: True for documents, False for padding tails."""
    import numpy as np

    if w.attn_is_pad is not None:
        return ~np.asarray(w.attn_is_pad, dtype=bool)
    return np.ones(len(cu) - 1, dtype=bool)


def cpu_model():
    """The host CPU's model name, as lscpu reports it (else /proc/cpuinfo)."""
    import subprocess

    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, q, k, v, do, cu, real, budget_s):
    """The oracle as it stands, on whole documents in order until the budget."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attn_ref

    a = w.attn
    lens = np.diff(cu)
    flops, docs, heads_done = 0.0, 0, 0
    t0 = time.perf_counter()
    for i in range(len(lens)):
        if not real[i]:
            continue
        s, e = int(cu[i]), int(cu[i + 1])
        one = np.array([0, e - s])
        # one key/value group (its hq/hkv query heads) per document keeps the sample bounded
        g = docs % a.hkv
        G = a.hq // a.hkv
        qs = q[s:e, g * G:(g + 1) * G]
        ks, vs, dos = k[s:e, g:g + 1], v[s:e, g:g + 1], do[s:e, g * G:(g + 1) * G]
        attn_ref.attn_fwd(qs, ks, vs, one)
        mult = 1.0
        if a.backward:
            attn_ref.attn_bwd(qs, ks, vs, dos, one)
            mult += 2.5
        L = e - s
        flops += mult * 4.0 * a.head_dim * G * L * (L + 1) / 2
        docs += 1
        heads_done += G
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "cpu_model": cpu_model(),
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"fp64 NumPy oracle, fwd{'+bwd' if a.backward else ''} of the first {docs} documents "
                  f"(one key/value group of {a.hq // a.hkv} query heads each), {flops:.3e} in-doc FLOP "
                  f"in {dt:.1f} s",
        "seconds": dt,
    }


def rope_rate(psc, torch, np, qd, kd, pk, w, args):
    """Rotary embedding of the workload's q and k in place (positions = the
    packer's indexes), timed apart from the step: HBM-bound, algorithmic bytes
    = q and k read and written once + positions."""
    T, hq, D = qd.shape
    hkv = kd.shape[1]
    pos = pk["indexes"][: w.pack.keep_rows].reshape(-1)[:T].contiguous()
    if pos.numel() != T:
        return None
    q2, k2 = qd.clone(), kd.clone()
    for _ in range(3):
        psc.rope(q2, k2, pos)
    torch.cuda.synchronize()
    psc.timing_reset()
    psc.timing_enable(True)
    n = 20
    for _ in range(n):
        psc.rope(q2, k2, pos)
    torch.cuda.synchronize()
    psc.timing_enable(False)
    ms_total, launches = psc.timing_read()["rope"]
    ms = ms_total / max(launches, 1)
    nbytes = 2 * (q2.numel() + k2.numel()) * q2.element_size() + 4 * T
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "rope", "bound": "hbm", "ms": round(ms, 4), "bytes": nbytes, "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "launches": launches}


def rope_step_rate(psc, torch, np, ctx, w, steps):
    """The step with the rotary embedding of q and k at the packer's indexes,
    two ways, same inputs, timed by events around each whole step:
      separate: psc_rope on q, k; attention fwd and bwd on the rotated q, k;
                psc_rope's inverse on the fp32 dq, dk (gradients of the
                unrotated q, k);
      fused:    psc_varlen_attn_fwd_rope (k turned by the rotation kernel, q
                inside the forward) and psc_varlen_attn_bwd_rope (dq, dk turned
                back in the dQ and dK kernels' epilogues).
    Results are bit-identical (tests/test_gpu_rope_fused.py)."""
    a = w.attn
    qd, kd = ctx["qd"], ctx["kd"]
    T, hq, D = qd.shape
    if not a.backward or a.dtype != "bf16" or D not in (64, 128):
        return None
    pos = ctx["pk"]["indexes"][: w.pack.keep_rows].reshape(-1)[:T].contiguous()
    if pos.numel() != T:
        return None
    cu, ml, nseg = ctx["cu"], ctx["max_seqlen"], ctx["n_seg"]
    vd, dod = ctx["vd"], ctx["dod"]
    q2, k2 = qd.clone(), kd.clone()
    o = torch.empty_like(qd)
    lse = torch.empty(hq, T, dtype=torch.float32, device=qd.device)
    f32 = dict(dtype=torch.float32, device=qd.device)
    g = (torch.empty(T, hq, D, **f32), torch.empty(T, kd.shape[1], D, **f32), torch.empty(T, kd.shape[1], D, **f32))
    dt = psc.BF16

    def sizes(pass_):
        return torch.empty(psc.varlen_attn_workspace(pass_, dt, T, nseg, ml, hq, kd.shape[1], D), dtype=torch.uint8,
                           device=qd.device)

    wf, wb, wfr, wbr = sizes(0), sizes(1), sizes(2), sizes(3)

    def sep():
        psc.rope(q2, k2, pos)
        psc.varlen_attn_fwd(q2, k2, vd, cu, ml, n_segments=nseg, out=o, lse=lse, workspace=wf)
        psc.varlen_attn_bwd(q2, k2, vd, o, dod, lse, cu, ml, n_segments=nseg, dq=g[0], dk=g[1], dv=g[2],
                            workspace=wb)
        psc.rope(g[0], g[1], pos, inverse=True)

    def fus():
        psc.varlen_attn_fwd_rope(q2, k2, vd, cu, ml, pos, n_segments=nseg, out=o, lse=lse, workspace=wfr)
        psc.varlen_attn_bwd_rope(q2, k2, vd, o, dod, lse, cu, ml, pos, n_segments=nseg, dq=g[0], dk=g[1], dv=g[2],
                                 workspace=wbr)

    res = {}
    for rnd in range(2):  # alternate the two, twice, and keep the second round
        for name, fn in (("separate", sep), ("fused", fus)):
            q2.copy_(qd)
            k2.copy_(kd)
            for _ in range(2):
                fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            torch.cuda.synchronize()
            ev[0].record()
            for i in range(steps):
                fn()
                ev[i + 1].record()
            torch.cuda.synchronize()
            res[name] = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))
    return {"separate_ms": round(res["separate"], 4), "fused_ms": round(res["fused"], 4),
            "saving_ms": round(res["separate"] - res["fused"], 4), "steps": steps,
            "what": "rope(q,k)+fwd+bwd+rope^-1(dq,dk) vs fwd_rope+bwd_rope, fp32 gradients"}


def data_steps_rate(psc, torch, np, pk, w):
    """The data steps after the packer on this workload's packer output, timed
    apart from the step: per-row max_seqlen, unpack_data with the workload's
    micro_bsz / SEQ_LEN, and the tp = 8 split of input_ids, labels and indexes.
    Algorithmic bytes: every int32 read and written once."""
    mb, sl = w.pack.micro_bsz, w.pack.seq_len
    rows, PL = pk["input_ids"].shape
    tp = 8 if PL % 8 == 0 else 1

    def once():
        psc.row_max_seqlen(pk)
        psc.unpack_data(pk, mb, sl)
        for key in ("input_ids", "labels", "indexes"):
            psc.split_sequence(pk[key], tp, tp - 1)

    for _ in range(3):
        once()
    torch.cuda.synchronize()
    psc.timing_reset()
    psc.timing_enable(True)
    n = 20
    for _ in range(n):
        once()
    torch.cuda.synchronize()
    psc.timing_enable(False)
    ms_total, launches = psc.timing_read()["data_steps"]
    ms = ms_total / n
    nseg = pk["cu_seqlens"].numel()
    nbytes = 4 * ((rows + 1) + nseg + rows)                       # row max_seqlen
    nbytes += 4 * (2 * rows * PL + 2 * rows * mb * sl + nseg + 2 * rows)  # unpack_data (upper bound on reads)
    nbytes += 3 * 4 * 2 * rows * (PL // tp)                       # three splits
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernels": "row_max_seqlen+unpack_data+split_sequence x3", "bound": "hbm", "ms": round(ms, 4),
            "launches_per_call": launches // n, "bytes": nbytes, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "tp": tp}


def doc_sweep(args):
    """The Sample Packing page's document-length measurement (section 5.3) on
    this kernel: each layout of one 32768-token row with its document mask,
    and the same row as one causal segment (cu_seqlens = [0, 32768]), at the
    lognormal_32k head configuration (GQA 32/8, D 128, bf16)."""
    import numpy as np
    import torch

    import packed_sequence_causal_amd as psc
    import workloads

    dev = torch.device("cuda:0")
    hq, hkv, D = 32, 8, 128
    S = workloads.DOC_SWEEP_ROW
    q, k, v, do = (x.to(dev) for x in workloads.qkv_do(S, hq, hkv, D, seed=args.seed, dtype="bf16"))

    def timed(cu_np):
        cu = torch.from_numpy(cu_np).to(dev)
        n_seg = cu.numel() - 1
        ml = int(np.diff(cu_np).max())
        o, lse = psc.varlen_attn_fwd(q, k, v, cu, ml, n_segments=n_seg)
        g = psc.varlen_attn_bwd(q, k, v, o, do, lse, cu, ml, n_segments=n_seg)
        wf = torch.empty(psc.varlen_attn_workspace(0, psc.BF16, S, n_seg, ml, hq, hkv, D), dtype=torch.uint8,
                         device=dev)
        wb = torch.empty(psc.varlen_attn_workspace(1, psc.BF16, S, n_seg, ml, hq, hkv, D), dtype=torch.uint8,
                         device=dev)
        fw, bw = [], []
        for i in range(args.warmup + args.steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            psc.varlen_attn_fwd(q, k, v, cu, ml, n_segments=n_seg, out=o, lse=lse, workspace=wf)
            e[1].record()
            psc.varlen_attn_bwd(q, k, v, o, do, lse, cu, ml, n_segments=n_seg, dq=g[0], dk=g[1], dv=g[2],
                                workspace=wb)
            e[2].record()
            torch.cuda.synchronize()
            if i >= args.warmup:
                fw.append(e[0].elapsed_time(e[1]))
                bw.append(e[1].elapsed_time(e[2]))
        return float(np.median(fw)), float(np.median(bw))

    for name, lens in workloads.DOC_SWEEP.items():
        L = np.asarray(lens, dtype=np.int64)
        pairs = float((L * (L + 1) // 2).sum())
        whole = float(S * (S + 1) // 2)
        f_doc, b_doc = timed(workloads.doc_sweep_cu(name))
        f_row, b_row = timed(workloads.doc_sweep_cu(name, whole_row=True))
        ff = 4.0 * D * hq
        line = {
            "layout": name, "row_tokens": S, "max_doc": int(L.max()), "hq": hq, "hkv": hkv, "head_dim": D,
            "mask_zero_fraction": round(1.0 - pairs / (S * S), 4),
            "whole_row_over_in_doc_work": round(whole / pairs, 3),
            "doc_mask": {"fwd_ms": round(f_doc, 4), "bwd_ms": round(b_doc, 4),
                         "fwd_tflops": round(ff * pairs / (f_doc * 1e-3) / 1e12, 1),
                         "bwd_tflops": round(2.5 * ff * pairs / (b_doc * 1e-3) / 1e12, 1)},
            "whole_row": {"fwd_ms": round(f_row, 4), "bwd_ms": round(b_row, 4),
                          "fwd_tflops": round(ff * whole / (f_row * 1e-3) / 1e12, 1),
                          "bwd_tflops": round(2.5 * ff * whole / (b_row * 1e-3) / 1e12, 1)},
            "speedup_fwd": round(f_row / f_doc, 3), "speedup_bwd": round(b_row / b_doc, 3),
            "steps": args.steps, "warmup": args.warmup, "seed": args.seed,
        }
        print(json.dumps(line), flush=True)


def measure(w, args, steps, warmup, torch, np, psc):
    """Times `steps` steps (pack + fwd [+ bwd]) of workload w after `warmup`
    untimed ones, with the library's per-kernel HIP-event timing on.
    Returns (summary dict, context for the extra rows)."""
    dev = torch.device("cuda:0")
    a = w.attn
    mode = psc.PACK if w.pack.mode == "pack" else psc.UNPACK

    toks = torch.from_numpy(w.pack.tokens).to(dev)
    offs = torch.from_numpy(w.pack.doc_offsets).to(dev)
    pk = psc.pack_build(toks, offs, w.pack.micro_bsz, w.pack.seq_len, mode)
    torch.cuda.synchronize()
    if w.attn_cu_seqlens is None:
        # attention runs on the first keep_rows rows of the packer's own output
        n_seg = int(pk["row_seg_ptr"][w.pack.keep_rows].item())
        cu = pk["cu_seqlens"][: n_seg + 1]
    else:
        cu = torch.from_numpy(np.asarray(w.attn_cu_seqlens, dtype=np.int32)).to(dev)
        n_seg = cu.numel() - 1
    cu_h = cu.cpu().numpy().astype(np.int64)
    T = int(cu_h[-1])
    lens = np.diff(cu_h)
    max_seqlen = int(lens.max())
    real = real_segments(w, cu_h)
    pairs = float((lens[real] * (lens[real] + 1) // 2).sum())
    real_tokens = int(lens[real].sum())
    fwd_flops = 4.0 * a.head_dim * a.hq * pairs
    bwd_flops = 2.5 * fwd_flops if a.backward else 0.0

    q, k, v, do = workloads.qkv_do(T, a.hq, a.hkv, a.head_dim, seed=args.seed, dtype=a.dtype)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    dt = psc.BF16 if a.dtype == "bf16" else psc.F32
    o, lse = psc.varlen_attn_fwd(qd, kd, vd, cu, max_seqlen, n_segments=n_seg)
    ws_f = torch.empty(psc.varlen_attn_workspace(0, dt, T, n_seg, max_seqlen, a.hq, a.hkv, a.head_dim),
                       dtype=torch.uint8, device=dev)
    grads = ws_b = None
    if a.backward:
        grads = psc.varlen_attn_bwd(qd, kd, vd, o, dod, lse, cu, max_seqlen, n_segments=n_seg)
        ws_b = torch.empty(psc.varlen_attn_workspace(1, dt, T, n_seg, max_seqlen, a.hq, a.hkv, a.head_dim),
                           dtype=torch.uint8, device=dev)
    pk_ws = pk["_workspace"]

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(e=None):
        if e:
            e[0].record()
        psc.pack_build(toks, offs, w.pack.micro_bsz, w.pack.seq_len, mode, out=pk, workspace=pk_ws)
        if e:
            e[1].record()
        psc.varlen_attn_fwd(qd, kd, vd, cu, max_seqlen, n_segments=n_seg, out=o, lse=lse, workspace=ws_f)
        if e:
            e[2].record()
        if a.backward:
            psc.varlen_attn_bwd(qd, kd, vd, o, dod, lse, cu, max_seqlen, n_segments=n_seg, dq=grads[0],
                                dk=grads[1], dv=grads[2], workspace=ws_b)
        if e:
            e[3].record()

    for _ in range(warmup):
        step()
    # untimed pass with the library's HIP events around every kernel: the
    # kernel breakdown, and which attention kernel dominates the step
    torch.cuda.synchronize()
    psc.timing_select(None)
    psc.timing_reset()
    psc.timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    psc.timing_enable(False)
    kt = psc.timing_read()
    algo = {"attn_fwd": fwd_flops}
    if a.backward:
        # forward = the two in-document products; dK/dV = S, dP, dV, dK (2.0x
        # forward); dQ = the dQ product only (0.5x forward; the S and dP it
        # recomputes are counted once, in dK/dV): the 2.5x convention
        algo.update({"attn_bwd_dkdv": 2.0 * fwd_flops, "attn_bwd_dq": 0.5 * fwd_flops})
    dom = max(algo, key=lambda n: kt[n][0])
    # the timed region: events around each phase, and the library's HIP events
    # around the dominant kernel alone (its launch durations for the roofline)
    psc.timing_select([dom])
    psc.timing_reset()
    psc.timing_enable(True)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(ev[i])
    t1.record()
    torch.cuda.synchronize()
    psc.timing_enable(False)
    psc.timing_select(None)
    kt_dom = psc.timing_read()[dom]
    ms = t0.elapsed_time(t1) / steps
    # the same number of steps once more with nothing recorded between them:
    # what the instrumentation costs (reported beside, not as the value)
    u0, u1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    u0.record()
    for _ in range(steps):
        step()
    u1.record()
    torch.cuda.synchronize()
    ms_plain = u0.elapsed_time(u1) / steps
    fwd_all = [e[1].elapsed_time(e[2]) for e in ev]
    bwd_all = [e[2].elapsed_time(e[3]) for e in ev]
    fwd_ms = float(np.median(fwd_all))
    bwd_ms = float(np.median(bwd_all)) if a.backward else 0.0
    value = (fwd_flops + bwd_flops) / (ms * 1e-3) / 1e12
    summary = {
        "workload": w.name, "tokens": T, "real_tokens": real_tokens, "segments": n_seg, "max_seqlen": max_seqlen,
        "hq": a.hq, "hkv": a.hkv, "head_dim": a.head_dim, "dtype": a.dtype,
        "passes": "pack+fwd+bwd" if a.backward else "pack+fwd", "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4), "tflops": round(value, 2),
        "ms_per_step_uninstrumented": round(ms_plain, 4),
        "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(real_tokens / (ms * 1e-3), 1),
        "pack_ms": round(float(np.median([e[0].elapsed_time(e[1]) for e in ev])), 4),
        "fwd": {"ms": round(fwd_ms, 4), "min_ms": round(float(min(fwd_all)), 4),
                "tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
                "pct_peak": round(100 * fwd_flops / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)},
        "kernels_ms_per_step": {n: round(t / steps, 4) for n, (t, c) in kt.items() if c},
    }
    if a.backward:
        summary["bwd"] = {"ms": round(bwd_ms, 4), "min_ms": round(float(min(bwd_all)), 4),
                          "tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
                          "pct_peak": round(100 * bwd_flops / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
    ctx = dict(q=q, k=k, v=v, do=do, qd=qd, kd=kd, vd=vd, dod=dod, pk=pk, cu=cu, cu_h=cu_h, n_seg=n_seg,
               max_seqlen=max_seqlen, real=real, kt=kt, ms=ms, value=value, fwd_flops=fwd_flops,
               bwd_flops=bwd_flops, step=step, algo=algo, dom=dom, kt_dom=kt_dom)
    return summary, ctx


def sustained_clock(step, torch, value):
    """Graphics clock and socket power while the step runs back to back,
    outside the timed region: `amd-smi metric -p -c` is read twice (per-XCD
    GFX clocks, socket power) while the loop keeps the GPU busy, and `value`
    is restated against the bf16 peak scaled to the mean clock read.  None
    where amd-smi is not installed or prints neither figure."""
    import re
    import shutil
    import subprocess
    import threading

    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    outs = []

    def poll():
        for _ in range(2):
            try:
                outs.append(subprocess.run([exe, "metric", "-p", "-c"], capture_output=True, text=True,
                                           timeout=30).stdout)
            except (OSError, subprocess.SubprocessError):
                pass

    t_end = time.perf_counter() + 0.5  # clocks settle under load before the first read
    n = 0
    while time.perf_counter() < t_end:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    th = threading.Thread(target=poll)
    th.start()
    while th.is_alive():
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    clk = [int(m) for o in outs for m in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", o)]
    pw = [int(m) for o in outs for m in re.findall(r"SOCKET_POWER:\s*(\d+)\s*W", o)]
    if not clk and not pw:
        return None
    res = {"source": "amd-smi metric -p -c, twice, while the step loops (untimed)", "steps_run": n,
           "socket_power_w": pw}
    if clk:
        mhz = sum(clk) / len(clk)
        res.update({"gfx_mhz_mean": round(mhz, 1), "gfx_mhz_min": min(clk), "gfx_mhz_max": max(clk),
                    "peak_at_clock_tflops": round(PEAK_BF16_TFLOPS * mhz / 2400.0, 1),
                    "pct_peak_at_clock": round(100 * value / (PEAK_BF16_TFLOPS * mhz / 2400.0), 2)})
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return
    if args.doc_sweep:
        doc_sweep(args)
        return

    import numpy as np
    import torch

    import packed_sequence_causal_amd as psc

    w = workloads.make(args.workload, args.seed)
    a = w.attn
    summ, ctx = measure(w, args, args.steps, args.warmup, torch, np, psc)
    # dominant kernel (from the untimed pass) and its algorithmic work per
    # launch; its launch durations are the ones recorded in the timed region
    algo, dom = ctx["algo"], ctx["dom"]
    dom_ms, dom_n = ctx["kt_dom"]
    dom_avg = dom_ms / max(dom_n, 1)
    achieved = algo[dom] / (dom_avg * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom, w.name),
                "avg_launch_ms": round(dom_avg, 4), "launches": dom_n}

    result = {
        "metric": METRIC,
        "value": summ["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": summ["ms_per_step"],
        "ms_per_step_uninstrumented": summ["ms_per_step_uninstrumented"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": a.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": summ["tokens"], "real_tokens": summ["real_tokens"],
                   "segments": summ["segments"], "max_seqlen": summ["max_seqlen"], "hq": a.hq, "hkv": a.hkv,
                   "head_dim": a.head_dim,
                   "packer": f"{w.pack.mode}(micro_bsz={w.pack.micro_bsz}, seq_len={w.pack.seq_len}), "
                             f"{len(w.pack.docs)} docs",
                   "passes": summ["passes"], "seed": args.seed},
        "pct_peak": summ["pct_peak"],
        "tokens_per_s": summ["tokens_per_s"],
        "pack_ms": summ["pack_ms"],
        "fwd": summ["fwd"],
        "kernels_ms_per_step": summ["kernels_ms_per_step"],
        "roofline": roofline,
    }
    if a.backward:
        result["bwd"] = summ["bwd"]
    if not args.no_clock:
        result["clock"] = sustained_clock(ctx["step"], torch, summ["tflops"])
    if not args.no_extras:
        result["rope"] = rope_rate(psc, torch, np, ctx["qd"], ctx["kd"], ctx["pk"], w, args)
        result["rope_step"] = rope_step_rate(psc, torch, np, ctx, w, min(args.steps, 10))
        result["data_steps"] = data_steps_rate(psc, torch, np, ctx["pk"], w)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, ctx["q"], ctx["k"], ctx["v"], ctx["do"], ctx["cu_h"], ctx["real"],
                                              args.cpu_seconds)
    # the other bf16 workloads, same step, fewer timed steps: their own lines
    # in one object so that every workload's rate is in the driver's record
    if not args.no_other_workloads:
        del ctx
        others = {}
        for name in BF16_WORKLOADS:
            if name == w.name:
                continue
            torch.cuda.empty_cache()
            wo = workloads.make(name, args.seed)
            s_o, _ = measure(wo, args, args.steps, args.warmup, torch, np, psc)
            others[name] = s_o
            print(f"# {name}: {s_o['ms_per_step']} ms/step, fwd {s_o['fwd']['pct_peak']} %"
                  + (f", bwd {s_o['bwd']['pct_peak']} %" if "bwd" in s_o else ""), file=sys.stderr, flush=True)
        result["workloads"] = others
    # the same workload drawn from seed 1 (document lengths and values)
    if not args.no_other_workloads and args.seed == 0:
        torch.cuda.empty_cache()
        s_1, _ = measure(workloads.make(w.name, 1), args, args.steps, args.warmup, torch, np, psc)
        s_1["seed"] = 1
        result["seed1"] = s_1
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
