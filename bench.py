"""Benchmark one step of the sequence-parallel attention path on one MI355X.

A step is the whole path over one batch of synthetic input, all W virtual
ranks per launch: pad + send_recv_heads (Q, K, V in one launch, one move) ->
partition -> masked attention on every rank's local heads -> gather_heads +
gather_output_tokens (one move).  Inputs are resident in HBM before the timed
region.  The default workload is long_hires (B = 2, 32768 tokens, the largest
that the pages' long-sequence case describes); the others are available
through --config.

Prints one JSON line.  ``value`` is masked-attention TFLOP/s of the whole step
(algorithmic attention flops per step / step time); ``roofline`` is the
all-ranks attention launch, ``roofline_share`` the launch of one rank's share
alone (R = 1, what each GPU runs when the ranks are devices); the per-kernel
figures and the head-relayout bandwidth are added beside them.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config long_hires]
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILE_DIR = os.path.join(ROOT, "profiles")   # rocprofv3 summaries (read and written here)
sys.path.insert(0, ROOT)

METRIC = "masked-attention TFLOP/s (MFMA util %) + head relayout GB/s (HBM %), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_MFMA_TFLOPS = 157.3   # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """C++ source without comments and with whitespace runs collapsed: what
    the compiler sees, so that a comment edit does not change the hash."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_hash(*names) -> str:
    """Hash of the named kernel sources (their code, not their comments) and
    of the compiler flags they are built with (build.py), so that a profile
    taken on other code or flags is never reported as current."""
    from sequence_attention_video_amd import build as b
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sequence_attention_video_amd", "csrc", n), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
        flags = [f for f in b.compile_flags() + b.EXTRA_FLAGS.get(n, []) if not os.path.isabs(f)]
        h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str, src_hash: str, key: str = "bytes_per_launch"):
    """HBM bytes per attention launch (``key``: the all-ranks launch, or
    "share_bytes_per_launch" for one rank's share) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source;
    else None."""
    path = os.path.join(PROFILE_DIR, f"attention_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    m = re.search(r"^traffic_json:\s*(\{.*\})\s*$", text, flags=re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get(key)


COPY_PROBE_BYTES = 1 << 29   # plain device copy of known size for counter calibration


def traffic_probe(workload: str, launches: int = 3):
    """Run only what the HBM counter passes measure: one plain copy of
    COPY_PROBE_BYTES (calibration), then the step once, the all-ranks
    attention launch `launches` more times and rank 0's share alone (R = 1)
    `launches` + 1 times."""
    import numpy as np
    import torch

    from sequence_attention_video_amd import binding
    from sequence_attention_video_amd.pipeline import UlyssesStep
    from sequence_attention_video_amd.workloads import WORKLOADS, make_inputs
    wl = WORKLOADS[workload]
    x = make_inputs(wl)
    td = lambda a: (torch.from_numpy(a).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)).cuda()
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda").random_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    step = UlyssesStep(wl, td(x["q"]), td(x["k"]), td(x["v"]), td(x["mask"]) if x["mask"] is not None else None)
    step.run()
    for _ in range(launches):
        step.attention()
    tq = wl.q_tokens_pad
    need = binding.sp_masked_attention_workspace_size(1, wl.B, tq, wl.T_pad, wl.Hl, wl.D,
                                                      binding._dtype_code(step.kh), step.mask is not None, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    share_out = torch.empty_like(step.oh[0])
    for _ in range(launches + 1):
        step.attention_rank(0, share_out, ws)
    torch.cuda.synchronize()
    print("traffic probe done", workload, flush=True)


def mfma_probe(workload: str, launches: int = 3):
    """Run only what the MFMA counter pass measures: the step once, then the
    all-ranks attention launch `launches` times and rank 0's share alone
    (R = 1, split when the library splits it) `launches` + 1 times."""
    import numpy as np
    import torch

    from sequence_attention_video_amd import binding
    from sequence_attention_video_amd.pipeline import UlyssesStep
    from sequence_attention_video_amd.workloads import WORKLOADS, make_inputs
    wl = WORKLOADS[workload]
    x = make_inputs(wl)
    td = lambda a: (torch.from_numpy(a).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)).cuda()
    step = UlyssesStep(wl, td(x["q"]), td(x["k"]), td(x["v"]), td(x["mask"]) if x["mask"] is not None else None)
    step.run()
    for _ in range(launches):
        step.attention()
    tq = wl.q_tokens_pad if wl.cross else wl.T_pad
    need = binding.sp_masked_attention_workspace_size(1, wl.B, tq, wl.T_pad, wl.Hl, wl.D,
                                                      binding._dtype_code(step.kh), step.mask is not None, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    share_out = torch.empty_like(step.oh[0])
    for _ in range(launches + 1):
        step.attention_rank(0, share_out, ws)
    torch.cuda.synchronize()
    print("mfma probe done", workload, flush=True)


def attention_flops(wl) -> tuple:
    """Algorithmic attention flops (4*D per visible (query, key) pair and
    head, over every query row the path computes): (all W shares, one share)."""
    if wl.cross:
        pairs = wl.q_tokens_pad * wl.T
    elif wl.mask == "block_causal":
        from sequence_attention_video_amd.workloads import make_inputs
        m = make_inputs(wl)["mask"]
        pairs = int(m.astype("int64").sum()) // m.shape[0] + (wl.T_pad - wl.T) * wl.T   # pad rows see real keys
    else:
        pairs = wl.T_pad * wl.T
    total = 4 * wl.D * wl.H * wl.B * pairs
    return total, total // wl.W


MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"]
N_XCD, N_SIMD, PEAK_CLOCK_GHZ = 8, 1024, 2.4     # MI355X: 256 CUs x 4 SIMDs, published peak clock


def write_mfma_summary(workload: str, pmc_dir: str, cmds: list):
    """Turn one rocprofv3 --pmc pass over `bench.py --mfma-probe` into
    profiles/attention_mfma_<workload>.md.  Per attention launch kind: the
    MFMA flops the hardware executed (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)
    against the algorithmic flops; MFMA busy cycles per SIMD
    (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs) over the launch's duration at the
    published 2.4 GHz (utilisation in the terms of the published peak) and
    over the cycles the GPU was active (GRBM_GUI_ACTIVE, counted once per
    XCD: the clock the launch actually ran at)."""
    import collections

    from sequence_attention_video_amd.workloads import WORKLOADS
    wl = WORKLOADS[workload]
    flops_all, flops_share = attention_flops(wl)
    per = collections.defaultdict(dict)
    kname, dur = {}, {}
    for r in _counter_rows(pmc_dir):
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] = per[d].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        m = re.search(r"(attn_\w+<[^>]*>|\w+_kernel)\(", r["Kernel_Name"])
        kname[d] = m.group(1) if m else r["Kernel_Name"][:60]
        dur[d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    order = sorted(per)
    main = [d for d in order if kname[d].startswith("attn_") and "combine" not in kname[d]]
    # dispatch order of the probe: the step's attention launch, `n` all-ranks
    # launches, then n + 1 share launches (a split share runs a merge kernel
    # after each); the first launch of each kind is left out (cold)
    n = (len(main) - 2) // 2
    share = main[2 + n:]
    groups = [("all W rank shares (one launch)", main[1:1 + n], flops_all),
              ("rank 0's share alone (R = 1)", share, flops_share)]
    # a split launch's merge kernel follows its attention kernel: each merge
    # dispatch belongs to the attention dispatch before it
    merge_of = {}
    for d in order:
        if "combine" in kname[d]:
            prev = [m for m in main if m < d]
            if prev:
                merge_of[prev[-1]] = d
    rows, recs = [], []
    for label, ds, flops in groups:
        merge = [merge_of[d] for d in ds if d in merge_of]
        avg = lambda f: sum(f(d) for d in ds) / len(ds)
        busy = avg(lambda d: per[d]["SQ_VALU_MFMA_BUSY_CYCLES"]) / N_SIMD
        hw = avg(lambda d: per[d]["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) * 512
        t = avg(lambda d: dur[d])
        gui = avg(lambda d: per[d]["GRBM_GUI_ACTIVE"]) / N_XCD
        util_peak = busy / (t * PEAK_CLOCK_GHZ * 1e9)
        util_active = busy / gui
        rec = {"launch": label, "kernel": kname[ds[0]], "launches": len(ds), "us_per_launch": round(t * 1e6, 1),
               "algorithmic_flops": int(flops), "hw_mfma_flops": int(hw), "hw_over_algorithmic": round(hw / flops, 4),
               "mfma_busy_cycles_per_simd": int(busy), "mfma_util_at_peak_clock": round(util_peak, 4),
               "mfma_busy_of_active_cycles": round(util_active, 4), "active_cycles_per_xcd": int(gui),
               "implied_clock_ghz": round(gui / t / 1e9, 3)}
        if merge:
            rec["merge_kernel_us"] = round(sum(dur[d] for d in merge) / len(merge) * 1e6, 1)
        recs.append(rec)
        rows.append(f"| {label} | `{rec['kernel']}` | {rec['us_per_launch']} | {flops:.4g} | {hw:.4g} | "
                    f"{hw / flops:.3f} | {100 * util_peak:.1f}% | {100 * util_active:.1f}% | {rec['implied_clock_ghz']} |")
    out = {"workload": workload, "kernel_source_hash": kernel_hash("sp_attention.hip", "sp_internal.h"), "launches": recs}
    lines = [f"# MFMA utilisation of the attention kernel on {workload}", "",
             "Commands (run from the repository root on one MI355X):", "", "```"] + cmds + ["```", "",
             "* hw MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, against the algorithmic flops (4 D per visible "
             "(query, key) pair and head). The busy-cycle counter gives the same figure: summed over the SIMDs, "
             "SQ_VALU_MFMA_BUSY_CYCLES x 1024 flops equals the MOPS count.",
             "* MFMA util at 2.4 GHz = busy cycles per SIMD (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs) / (launch duration "
             "x 2.4 GHz): the matrix unit's utilisation in the terms of the published peak (the roofline fraction "
             "of the launch while counters are collected).",
             "* MFMA busy of active cycles = busy cycles per SIMD / (GRBM_GUI_ACTIVE / 8 XCDs): the same against the "
             "cycles the GPU actually ran, whatever its clock. GRBM_GUI_ACTIVE also counts some cycles around each "
             "dispatch, so the implied clock (active cycles / duration) reads high, and the fraction low, on "
             "launches of tens of microseconds; on launches of hundreds of microseconds and more it shows the "
             "engine clock under sustained MFMA load.",
             "* Averages over the probe's launches of each kind, the first (cold) launch of each left out; the "
             "durations are dispatch timestamps with counters on (a few percent above the bench's event times).",
             "",
             "| launch | kernel | us per launch | algorithmic flops | hw MFMA flops | hw / alg | MFMA util at 2.4 GHz | "
             "MFMA busy of active cycles | implied clock (GHz) |",
             "|---|---|---|---|---|---|---|---|---|"] + rows
    for r in recs:
        if "merge_kernel_us" in r:
            lines += ["", f"The split launch of {r['launch']} is followed by a merge kernel (`attn_combine_kernel`) "
                          f"of {r['merge_kernel_us']} us per launch (no MFMA work)."]
    lines += ["", "mfma_json: " + json.dumps(out)]
    path = os.path.join(PROFILE_DIR, f"attention_mfma_{workload}.md")
    with open(path, "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")
    print(open(path).read())


PIPE_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
                 "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_VALU",
                 "GRBM_GUI_ACTIVE"]


def write_pipe_summary(workload: str, pmc_dir: str, cmds: list):
    """Turn one rocprofv3 --pmc pass (PIPE_COUNTERS) over `bench.py
    --mfma-probe` into profiles/attention_pipes_<workload>.md: for the
    all-ranks attention launch, the instructions issued per MFMA (VALU,
    transcendental, LDS) and how much of the MFMA-busy time a VALU
    instruction issued beside it (co-execution)."""
    import collections
    per = collections.defaultdict(dict)
    kname = {}
    for r in _counter_rows(pmc_dir):
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] = per[d].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        m = re.search(r"(attn_\w+<[^>]*>|\w+_kernel)\(", r["Kernel_Name"])
        kname[d] = m.group(1) if m else r["Kernel_Name"][:60]
    main = [d for d in sorted(per) if kname[d].startswith("attn_") and "combine" not in kname[d]]
    n = (len(main) - 2) // 2
    ds = main[1:1 + n]                      # the all-ranks launches after the step's own
    avg = {c: sum(per[d].get(c, float("nan")) for d in ds) / len(ds) for c in PIPE_COUNTERS}
    mf = avg["SQ_INSTS_MFMA"]
    rows = [("VALU instructions per MFMA (SQ_INSTS_VALU / SQ_INSTS_MFMA)", avg["SQ_INSTS_VALU"] / mf),
            ("transcendentals per MFMA (SQ_INSTS_VALU_TRANS_F32 / SQ_INSTS_MFMA)", avg["SQ_INSTS_VALU_TRANS_F32"] / mf),
            ("LDS instructions per MFMA (SQ_INSTS_LDS / SQ_INSTS_MFMA)", avg["SQ_INSTS_LDS"] / mf),
            ("MFMA-busy cycles with a VALU instruction issued beside them "
             "(SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES)",
             avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / avg["SQ_VALU_MFMA_BUSY_CYCLES"]),
            ("MFMA busy of active cycles (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8))",
             avg["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (avg["GRBM_GUI_ACTIVE"] / 8))]
    rec = {"workload": workload, "kernel": kname[ds[0]], "launches": len(ds),
           "kernel_source_hash": kernel_hash("sp_attention.hip", "sp_internal.h"),
           "counters_per_launch": {c: avg[c] for c in PIPE_COUNTERS}}
    lines = [f"# Issue mix of the attention kernel on {workload}", "",
             "Commands (run from the repository root on one MI355X):", "", "```"] + cmds + ["```", "",
             f"All-ranks launch (`{rec['kernel']}`), averages over {len(ds)} launches (the probe's first, the step's, "
             "left out). SQ instruction counts are wave instructions summed over the GPU.", "",
             "| quantity | value |", "|---|---|"] + [f"| {q} | {v:.3f} |" for q, v in rows] +             ["", "pipe_json: " + json.dumps(rec)]
    path = os.path.join(PROFILE_DIR, f"attention_pipes_{workload}.md")
    with open(path, "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")
    print(open(path).read())


def _counter_rows(path):
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def write_traffic_summary(workload: str, fetch_dir: str, write_dir: str, cmds: list):
    """Turn the two counter passes over `bench.py --traffic-probe` into
    profiles/attention_traffic_<workload>.md: bytes per launch of the
    all-ranks attention launch, of one rank's share (the split launch and
    its merge together), of the mask classifier and of the step's copy
    kernels, each against the bytes the method must move."""
    import collections

    from sequence_attention_video_amd.workloads import WORKLOADS
    wl = WORKLOADS[workload]
    out = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = collections.defaultdict(float)
        kname, grid = {}, {}
        for r in _counter_rows(d):
            if r["Counter_Name"] != name:
                continue
            per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
            kname[int(r["Dispatch_Id"])] = r["Kernel_Name"]
            grid[int(r["Dispatch_Id"])] = int(r["Grid_Size"])
        ids = sorted(per)
        copy = [per[i] for i in ids if "copyBuffer" in kname[i]]
        copy_kib = max(copy) if copy else float("nan")
        scale = (COPY_PROBE_BYTES / 1024.0) / copy_kib        # true KiB per counted KiB
        is_attn = lambda i: "attn_bf16_kernel" in kname[i] or "attn_f32_kernel" in kname[i]
        # the probe's first attention dispatch is the step's (all W shares);
        # the share launches have another grid
        g_all = next((grid[i] for i in ids if is_attn(i)), None)
        # a split launch's merge kernel follows its attention kernel and
        # counts with it
        merged = dict((i, per[i]) for i in ids if is_attn(i))
        last = None
        for i in ids:
            if is_attn(i):
                last = i
            elif "attn_combine_kernel" in kname[i] and last is not None:
                merged[last] += per[i]
        all_ = [merged[i] for i in ids if is_attn(i) and grid[i] == g_all]
        share = [merged[i] for i in ids if is_attn(i) and grid[i] != g_all]
        cls = [per[i] for i in ids if "classify_mask_kernel" in kname[i]]
        avg = lambda v: sum(v) / len(v) if v else float("nan")
        first = lambda key: next((per[i] for i in ids if key in kname[i]), float("nan"))
        out[name] = {"copy_kib": copy_kib, "scale": scale,
                     "all_kib": avg(all_[1:]) if len(all_) > 1 else avg(all_),
                     "share_kib": avg(share[1:]),
                     "classify_kib": avg(cls), "send_kib": first("relayout_kernel"),
                     "pad_mask_kib": first("pad_mask_kernel"), "gather_kib": first("gather_heads_unpad_kernel")}
    b = lambda ctr, key: out[ctr][key] * out[ctr]["scale"] * 1024
    one = wl.B * wl.T_pad * wl.H * wl.D * wl.eb                 # one (B, T_pad, H, D) tensor
    tq = wl.q_tokens_pad
    q_o = 2 * wl.B * tq * wl.H * wl.D * wl.eb                    # Q read + O written
    alg_all = q_o + 2 * one                                      # + K and V read once
    rec = {"workload": workload, "kernel_source_hash": kernel_hash("sp_attention.hip", "sp_internal.h"),
           "bytes_per_launch": int(b("FETCH_SIZE", "all_kib") + b("WRITE_SIZE", "all_kib")),
           "fetch_bytes": int(b("FETCH_SIZE", "all_kib")), "write_bytes": int(b("WRITE_SIZE", "all_kib")),
           "algorithmic_bytes": alg_all,
           "share_bytes_per_launch": int(b("FETCH_SIZE", "share_kib") + b("WRITE_SIZE", "share_kib")),
           "share_algorithmic_bytes": alg_all // wl.W,
           "fetch_scale": out["FETCH_SIZE"]["scale"], "write_scale": out["WRITE_SIZE"]["scale"]}
    lines = [f"# HBM traffic of the attention launches and the step's moves on {workload}", "",
             "Commands (run from the repository root on one MI355X):", "", "```"] + cmds + ["```", "",
             f"Calibration: a plain {COPY_PROBE_BYTES >> 20} MiB device copy read "
             f"{out['FETCH_SIZE']['copy_kib']:.0f} KiB (FETCH_SIZE) and wrote {out['WRITE_SIZE']['copy_kib']:.0f} KiB "
             f"(WRITE_SIZE) against {COPY_PROBE_BYTES >> 10} KiB moved, so the counters are scaled by "
             f"{out['FETCH_SIZE']['scale']:.3f} and {out['WRITE_SIZE']['scale']:.3f}. Bytes below are scaled, per "
             "launch (averages over the probe's launches of each kind after the first).", "",
             "Algorithmic bytes of an attention launch: Q read, K and V read once, O written once (with a user "
             "mask the launch also reads the classifier's visibility words).", "",
             "| launch | fetched | written | total | algorithmic | total / algorithmic |", "|---|---|---|---|---|---|"]
    def row(label, key, alg):
        f_, w_ = b("FETCH_SIZE", key), b("WRITE_SIZE", key)
        ratio = (f_ + w_) / alg if alg else float("nan")
        lines.append(f"| {label} | {f_:.4g} | {w_:.4g} | {f_ + w_:.4g} | {alg:.4g} | {ratio:.3f} |")
    row("attention, all W rank shares (R = W; a split launch's merge included)", "all_kib", alg_all)
    row("attention, rank 0's share alone (R = 1; a split launch's merge included)", "share_kib", alg_all // wl.W)
    nrel = 2 if wl.cross else 3
    send_alg = nrel * (wl.B * wl.T * wl.H * wl.D * wl.eb + one)
    out_rows = wl.Tq if wl.cross else wl.T
    gather_alg = 2 * wl.B * out_rows * wl.H * wl.D * wl.eb
    row(f"pad + send_recv_heads, one move (`relayout_kernel`, {nrel} tensors)", "send_kib", send_alg)
    row("gather_heads + gather_output_tokens, one move (`gather_heads_unpad_kernel`)", "gather_kib", gather_alg)
    if wl.mask == "block_causal":
        T, Tp = wl.T, wl.T_pad
        row("user-mask extension (`pad_mask_kernel`)", "pad_mask_kib", T * T + Tp * Tp)
        nkt = -(-Tp // 64)
        row("mask classifier (`classify_mask_kernel`: mask read, classes and words written)", "classify_kib",
            Tp * Tp + Tp * nkt * 8)
    lines += ["", "traffic_json: " + json.dumps(rec)]
    path = os.path.join(PROFILE_DIR, f"attention_traffic_{workload}.md")
    with open(path, "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")
    print(open(path).read())


def write_kernel_trace_summary(trace_csv: str, bench_json: str, title: str, cmd: str, out_name: str):
    """Turn a rocprofv3 --kernel-trace kernel_trace.csv (and the bench line of
    the same run) into a short markdown summary under profiles/.  Dispatches
    are grouped by kernel and grid size, so that launches of one kernel with
    different shapes (the all-ranks attention launch and one rank's share)
    have averages of their own."""
    import collections
    import csv
    import statistics
    from sequence_attention_video_amd.workloads import WORKLOADS
    bench = json.loads([l for l in open(bench_json).read().splitlines() if l.startswith('{"metric"')][-1])
    wl = WORKLOADS[bench["config"]["workload"]]
    groups = collections.defaultdict(list)
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    for r in rows:
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups[(r["Kernel_Name"], grid)].append(dur)
    total = sum(sum(v) for v in groups.values())
    is_attn = lambda name: "attn_bf16_kernel" in name or "attn_f32_kernel" in name
    # the all-ranks launch is the attention grid launched most often; any
    # other attention grid is rank 0's share alone
    g_all = max(((g, len(v)) for (n, g), v in groups.items() if is_attn(n)), key=lambda t: t[1], default=(None, 0))[0]
    # a split launch's merge kernel follows its attention kernel: a merge
    # grid belongs to the attention launch dispatched before it
    merge_kind, last = {}, None
    for r in rows:
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        if is_attn(r["Kernel_Name"]):
            last = grid
        elif "attn_combine_kernel" in r["Kernel_Name"] and last is not None:
            merge_kind[(r["Kernel_Name"], grid)] = ("merge of the all-ranks launch" if last == g_all
                                                    else "merge of the split share")
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```", cmd, "```", "",
             "Dispatches grouped by kernel and grid size (threads).", "",
             "| kernel | grid | launch | calls | avg (us) | median (us) | min (us) | max (us) | share of time |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        if sum(v) < 0.001 * total and "attn_combine_kernel" not in name:
            continue
        short = name.replace("sp::(anonymous namespace)::", "")
        short = short if len(short) <= 80 else short[:77] + "..."
        kind = ("all ranks (R = %d)" % wl.W if grid == g_all else "one share (R = 1)") if is_attn(name) else (
            merge_kind.get((name, grid), "merge") if "attn_combine_kernel" in name else "")
        lines.append(f"| `{short}` | {grid} | {kind} | {len(v)} | {sum(v) / len(v):.1f} | "
                     f"{statistics.median(v):.1f} | {min(v):.1f} | {max(v):.1f} | {100 * sum(v) / total:.1f}% |")
    r, rs, k = bench["roofline"], bench.get("roofline_share") or {}, bench["kernels"]
    lines += ["", "The same run's bench line (HIP events on the launch stream):", "",
              f"* attention, all ranks{' (split + merge)' if r.get('split') else ''}: "
              f"{r['avg_launch_ms'] * 1e3:.1f} us per launch (median in the step), "
              f"{r['achieved']} TFLOP/s, {100 * r['frac']:.1f}% of the bf16 MFMA peak"]
    if rs:
        lines.append(f"* attention, one share (R = 1{', split + merge' if rs.get('split') else ''}): "
                     f"{rs['avg_launch_ms'] * 1e3:.1f} us per launch, {rs['achieved']} TFLOP/s, "
                     f"{100 * rs['frac']:.1f}% of the peak")
    for key, label in (("send_recv_heads_rotating", "send_recv_heads (Q, K, V, rotating buffers)"),
                       ("pad+send_recv_heads_fused_rotating", "pad + send_recv_heads, one move (rotating buffers)"),
                       ("gather_heads+gather_output_tokens_fused_rotating",
                        "gather_heads + gather_output_tokens, one move (rotating buffers)"),
                       ("gather_heads_rotating", "gather_heads alone (rotating buffers)"),
                       ("gather_output_tokens_rotating", "gather_output_tokens alone (rotating buffers)")):
        if key in k:
            lines.append(f"* {label}: {k[key]['ms'] * 1e3:.1f} us, {k[key]['GB/s']} GB/s "
                         f"({100 * k[key]['hbm_frac']:.1f}% of 8000 GB/s)")
    lines.append(f"* kernel source hash: `{bench['kernel_source_hash']}`")
    path = os.path.join(PROFILE_DIR, out_name)
    with open(path, "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")
    print(open(path).read())


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first; the clocks need ~0.1 s of sustained work to settle")
    ap.add_argument("--config", default="long_hires")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run only a calibration copy and attention launches (for rocprofv3 --pmc passes)")
    ap.add_argument("--write-traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/attention_traffic_<config>.md from two counter passes")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="run only the step and attention launches, all-ranks and one share (for the MFMA counter pass)")
    ap.add_argument("--write-mfma-summary", metavar="PMC_DIR",
                    help="write profiles/attention_mfma_<config>.md from one MFMA counter pass")
    ap.add_argument("--write-pipe-summary", metavar="PMC_DIR",
                    help="write profiles/attention_pipes_<config>.md from one issue-mix counter pass")
    ap.add_argument("--write-kernel-trace-summary", nargs=2, metavar=("TRACE_CSV", "BENCH_JSON"),
                    help="write profiles/kernel_trace_<config>.md from a rocprofv3 --kernel-trace run of bench.py")
    ap.add_argument("--profile-command", action="append", default=[],
                    help="the command line(s) that produced the profile, recorded in the summary")
    args = ap.parse_args()
    if args.write_traffic_summary:
        write_traffic_summary(args.config, *args.write_traffic_summary, args.profile_command)
        return
    if args.write_kernel_trace_summary:
        write_kernel_trace_summary(*args.write_kernel_trace_summary,
                                   f"rocprofv3 kernel trace: bench step on {args.config}",
                                   "\n".join(args.profile_command), f"kernel_trace_{args.config}.md")
        return
    if args.write_pipe_summary:
        write_pipe_summary(args.config, args.write_pipe_summary, args.profile_command)
        return
    if args.write_mfma_summary:
        write_mfma_summary(args.config, args.write_mfma_summary, args.profile_command)
        return
    if args.traffic_probe:
        traffic_probe(args.config)
        return
    if args.mfma_probe:
        mfma_probe(args.config)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py measures one GPU only: the W ranks of the sequence-parallel path are virtual "
               "ranks on a single device; runs on several GPUs are not supported")
        if int(os.environ.get("RANK", "0")) == 0:
            print(msg, file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from sequence_attention_video_amd import binding
    from sequence_attention_video_amd.pipeline import UlyssesStep
    from sequence_attention_video_amd.workloads import GRIDS, WORKLOADS, make_inputs

    binding.load()          # fails loudly if the HIP library is missing
    if args.config == "joint_av":
        bench_joint(args)
        return
    wl = WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    log("inputs", wl.name)
    x = make_inputs(wl)

    def to_dev(a):
        t = torch.from_numpy(a)
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    mask = to_dev(x["mask"]) if x["mask"] is not None else None
    step = UlyssesStep(wl, q, k, v, mask, device=dev)
    B, H, D, W, T, Tp, Hl = wl.B, wl.H, wl.D, wl.W, wl.T, wl.T_pad, wl.Hl
    eb = wl.eb

    # -- algorithmic work per step
    step.run()
    torch.cuda.synchronize()
    if wl.cross:
        pairs_per_bh = wl.Tq * T
        tq = wl.Tq
    elif mask is not None:
        pairs_per_bh = int(step.mask_ext.to(torch.int64).sum().item()) // step.mask_ext.shape[0]
        tq = Tp
    else:
        pairs_per_bh = Tp * T
        tq = Tp
    attn_flops = 4 * D * H * B * pairs_per_bh                       # all W rank shares
    n_relayed = 2 if wl.cross else 3
    relayout_bytes = 2 * n_relayed * B * Tp * H * D * eb            # read + write, Q/K/V (K/V for cross)
    relayout_o_bytes = 2 * B * tq * H * D * eb
    out_rows = wl.Tq if wl.cross else T
    gather_bytes = 2 * B * out_rows * H * D * eb
    pad_bytes = (n_relayed * B * (T + Tp) * H * D * eb) if step.need_pad else 0
    if step.need_pad and mask is not None:
        pad_bytes += mask.shape[0] * (T * T + Tp * Tp)

    # -- warmup, then K timed steps (events only around the K steps), then the
    #    same K steps again with per-stage events for the breakdown
    run_bytes_in = (n_relayed * B * T * H * D * eb) + (n_relayed * B * Tp * H * D * eb)   # fused pad + send
    if step.need_q_pad:
        run_bytes_in += B * (wl.Tq + wl.q_tokens_pad) * H * D * eb
    if step.need_pad and mask is not None:
        run_bytes_in += mask.shape[0] * (T * T + Tp * Tp)
    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    log("timed", args.steps)
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()            # no collector pause inside the timed regions (as timeit does)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        step.run()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        e = ev[i]
        e[0].record(stream)
        step.pad_send()
        _, lengths = step.partition()
        e[1].record(stream)
        step.attention()
        e[2].record(stream)
        step.gather_unpad(lengths)
        e[3].record(stream)
    torch.cuda.synchronize()
    # per-stage medians: a host stall inside one step's event pair (the GPU
    # idles until the next launch arrives) would otherwise weigh in a mean
    stage = lambda a, b: float(np.median([ev[i][a].elapsed_time(ev[i][b]) for i in range(args.steps)]))
    ms_pad_send = stage(0, 1)
    ms_attn_stage = stage(1, 2)
    ms_gather_fused = stage(2, 3)
    # the same step as the five separate calls (pad, send_recv_heads,
    # attention, gather_heads, gather_output_tokens), stage by stage
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        e = evs[i]
        e[0].record(stream)
        step.pad()
        _, lengths = step.partition()
        step.send_recv_heads()
        e[1].record(stream)
        step.attention()
        e[2].record(stream)
        step.gather_heads()
        e[3].record(stream)
        step.gather_output_tokens(lengths)
        e[4].record(stream)
    torch.cuda.synchronize()
    stage_s = lambda a, b: float(np.median([evs[i][a].elapsed_time(evs[i][b]) for i in range(args.steps)]))
    ms_pad_send_sep = stage_s(0, 1)
    ms_gh = stage_s(2, 3)
    ms_gather = stage_s(3, 4)
    ms_separate_step = float(np.median([evs[i][0].elapsed_time(evs[i][4]) for i in range(args.steps)]))
    # the dominant kernel's launch duration for the roofline: its in-step
    # median above; beside it, K launches back to back between one event pair
    # (the chip's clock runs lower under MFMA load with no copy in between)
    ms_attn = ms_attn_stage
    a0 = torch.cuda.Event(enable_timing=True)
    a1 = torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(args.steps):
        step.attention()
    a1.record(stream)
    torch.cuda.synchronize()
    ms_attn_b2b = a0.elapsed_time(a1) / args.steps
    gc.enable()
    per_step = [ev[i][0].elapsed_time(ev[i][3]) for i in range(args.steps)]
    per_attn = [ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)]
    spread = {"step_ms_median": round(float(np.median(per_step)), 4), "step_ms_min": round(float(np.min(per_step)), 4),
              "attention_ms_median": round(float(np.median(per_attn)), 4),
              "attention_ms_min": round(float(np.min(per_attn)), 4), "steps": args.steps,
              "note": "per-step event pairs (a second run of K steps with an event between stages)"}

    # -- the same step with both exchanges folded into attention's addressing
    #    (one device only: the head-side views are strided views of the
    #    token-side tensors); reported beside the step, not as the step
    ref_out = step.out.clone()
    for _ in range(max(3, args.warmup // 4)):
        step.run_zero_copy()
    z0 = torch.cuda.Event(enable_timing=True)
    z1 = torch.cuda.Event(enable_timing=True)
    z0.record(stream)
    for _ in range(args.steps):
        step.run_zero_copy()
    z1.record(stream)
    torch.cuda.synchronize()
    ms_zero = z0.elapsed_time(z1) / args.steps
    zero_equal = bool(torch.equal(step.outz.view(torch.uint8), ref_out.view(torch.uint8)))

    # -- the same step recorded once as a HIP graph and replayed (the kernels
    #    and their arguments are fixed; the per-launch host work and launch
    #    gaps go); reported beside the step
    graph = step.capture()
    for _ in range(max(3, args.warmup // 4)):
        graph.replay()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    ms_graph = g0.elapsed_time(g1) / args.steps
    graph_equal = bool(torch.equal(step.out.view(torch.uint8), ref_out.view(torch.uint8)))
    del graph, ref_out

    # -- the 2-D (height x width) split in place of the 1-D token split, for
    #    workloads that are one video grid; reported beside the step
    cp2d = None
    if args.config in GRIDS:
        from sequence_attention_video_amd.pipeline import Ulysses2DStep
        step2 = Ulysses2DStep(wl, GRIDS[args.config], q, k, v, device=dev)
        for _ in range(max(3, args.warmup // 4)):
            step2.run()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c2 = torch.cuda.Event(enable_timing=True)
        c3 = torch.cuda.Event(enable_timing=True)
        c4 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(args.steps):
            step2.run()
        c1.record(stream)
        for _ in range(args.steps):
            step2.split_cp_2d()
        c2.record(stream)
        for _ in range(args.steps):
            step2.split_send_heads()
        c3.record(stream)
        for _ in range(args.steps):
            step2.run_separate()
        c4.record(stream)
        torch.cuda.synchronize()
        ms_2d = c0.elapsed_time(c1) / args.steps
        ms_tile = c1.elapsed_time(c2) / args.steps
        ms_fused = c2.elapsed_time(c3) / args.steps
        ms_sep = c3.elapsed_time(c4) / args.steps
        tile_bytes = 2 * 3 * B * T * H * D * eb
        cp2d = {"ms": round(ms_2d, 4), "TFLOP/s": round(attn_flops / (ms_2d * 1e-3) / 1e12, 2),
                "split_hw": list(step2.split), "grid_fhw": list(GRIDS[args.config]),
                "split_send_heads_qkv": {"ms": round(ms_fused, 4), "bytes": tile_bytes,
                                         "GB/s": round(tile_bytes / (ms_fused * 1e-3) / 1e9, 1)},
                "split_cp_2d_qkv": {"ms": round(ms_tile, 4), "bytes": tile_bytes,
                                    "GB/s": round(tile_bytes / (ms_tile * 1e-3) / 1e9, 1)},
                "separate_moves_step_ms": round(ms_sep, 4),
                "max_abs_diff_vs_step": float((step2.out.float() - step.out.float()).abs().max().item())}
        del step2

    # -- the copy kernels back to back over rotating buffer sets (> 1 GB in
    #    flight defeats the 256 MB MALL).  Each is timed twice: as eager
    #    launches (the host's per-call work, Python and the binding included,
    #    is longer than a 100 MB copy, so the GPU waits between launches) and
    #    as one replay of the same launches recorded in a HIP graph (the
    #    kernels back to back on the device); GB/s is the graph figure.
    def rotating_ms(make_set, call, nbytes):
        n = min(16, max(2, int(math.ceil(1.2e9 / max(nbytes, 1)))))
        bufs = [make_set() for _ in range(n)]
        iters = max(args.steps, 2 * n)
        for i in range(n):
            call(*bufs[i])
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(iters):
            call(*bufs[i % n])
        t1.record(stream)
        torch.cuda.synchronize()
        eager = t0.elapsed_time(t1) / iters
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(iters):
                call(*bufs[i % n])
        g.replay()
        torch.cuda.synchronize()
        t0.record(stream)
        g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        graph = t0.elapsed_time(t1) / iters
        del g, bufs
        torch.cuda.empty_cache()
        return graph, eager, n

    def rand_like(t):
        u = torch.empty_like(t)
        u.view(torch.uint8).random_()
        return u

    dt = step.kh.dtype
    tok_view = (Tp // W * H * D, Tp * H * D)
    ms_relayout_rot, ms_relayout_eager, nsets = rotating_ms(
        lambda: ([rand_like(step.kh.new_empty((B, Tp, H, D))) for _ in range(n_relayed)],
                 [torch.empty((W, B, Tp, Hl, D), dtype=dt, device=dev) for _ in range(n_relayed)]),
        lambda srcs, dsts: binding.sp_relayout_heads(srcs, dsts, W, B, Tp, H, D, binding.SP_TOKENS_TO_HEADS,
                                                     tok_strides=tok_view),
        relayout_bytes)
    tq_pad = wl.q_tokens_pad if wl.cross else Tp
    t_out = wl.Tq if wl.cross else T
    ts_q = tq_pad // W
    # the two fused moves of the step, the same way
    unpadded = (B, T, H, D)
    fused_send_bytes = n_relayed * B * (T + Tp) * H * D * eb
    ms_ps_rot, ms_ps_eager, n_ps = rotating_ms(
        lambda: ([rand_like(step.k.new_empty(unpadded)) for _ in range(n_relayed)],
                 [torch.empty_like(step.kh) for _ in range(n_relayed)]),
        lambda srcs, dsts: binding.sp_pad_relayout_heads(srcs, dsts, W, B, T, Tp, H, D),
        fused_send_bytes)
    ms_ghu_rot, ms_ghu_eager, n_ghu = rotating_ms(
        lambda: (rand_like(step.oh), torch.empty_like(step.out)),
        lambda src, dst: binding.sp_gather_heads_unpad([src], [dst], W, B, tq_pad, H, D, t_out, counts=[ts_q] * W),
        gather_bytes)
    ms_gh_rot, ms_gh_eager, n_gh = rotating_ms(
        lambda: (rand_like(step.oh), torch.empty_like(step.ot)),
        lambda src, dst: binding.sp_relayout_heads([src], [dst], W, B, tq_pad, H, D, binding.SP_HEADS_TO_TOKENS),
        relayout_o_bytes)
    ms_gather_rot, ms_gather_eager, n_ga = rotating_ms(
        lambda: (rand_like(step.ot), torch.empty_like(step.out)),
        lambda src, dst: binding.sp_gather_unpad(src, dst, W, B, ts_q, H * D, t_out, counts=[ts_q] * W),
        gather_bytes)

    # -- one rank's share alone (R = 1): the attention launch each GPU runs when
    #    the W ranks are devices; few query tiles, so the library splits keys
    share_out = torch.empty_like(step.oh[0])
    mbs = 0
    if step.mask is not None and step.mask_ext.shape[0] > 1:
        mbs = step.mask_ext.stride(0)
    tq_share = wl.Tq if wl.cross else Tp
    need = binding.sp_masked_attention_workspace_size(1, B, tq_share, Tp, Hl, D, binding._dtype_code(step.kh),
                                                      step.mask is not None, mbs)
    # the mask part alone is what the (never split) fp32 kernel would need
    mask_part = binding.sp_masked_attention_workspace_size(1, B, tq_share, Tp, Hl, D, binding.SP_F32,
                                                           step.mask is not None, mbs)
    share_split = wl.dtype == "bf16" and need > mask_part
    # the all-ranks launch splits too where its query tiles leave a partly
    # filled last round (long_hires: 21 whole rounds of 256, then 128 tiles)
    all_split = wl.dtype == "bf16" and (
        binding.sp_masked_attention_workspace_size(W, B, tq_share, Tp, Hl, D, binding._dtype_code(step.kh),
                                                   step.mask is not None, mbs) >
        binding.sp_masked_attention_workspace_size(W, B, tq_share, Tp, Hl, D, binding.SP_F32,
                                                   step.mask is not None, mbs))
    share_ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    n_share = 10 if attn_flops > 4e12 else max(20, args.steps)
    for _ in range(n_share):
        step.attention_rank(0, share_out, share_ws)
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(n_share):
        step.attention_rank(0, share_out, share_ws)
    s1.record(stream)
    torch.cuda.synchronize()
    ms_share_b2b = s0.elapsed_time(s1) / n_share
    # per-launch event pairs (the split launch's two kernels between one
    # pair); the median is the share's launch time
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_share)]
    for a_, b_ in sev:
        a_.record(stream)
        step.attention_rank(0, share_out, share_ws)
        b_.record(stream)
    torch.cuda.synchronize()
    ms_share = float(np.median([a_.elapsed_time(b_) for a_, b_ in sev]))
    share_diff = float((share_out.float() - step.oh[0].float()).abs().max().item())
    share_flops = attn_flops // W
    share_tflops = share_flops / (ms_share * 1e-3) / 1e12
    del share_ws

    # -- oracle-free sanity on the timed buffers (parity proper lives in tests/)
    finite = bool(torch.isfinite(step.out.float()).all().item())
    back = torch.empty_like(step.kp)
    binding.sp_relayout_heads([step.kh], [back], W, B, Tp, H, D, binding.SP_HEADS_TO_TOKENS, tok_strides=tok_view)
    torch.cuda.synchronize()
    round_trip = bool(torch.equal(back.view(torch.uint8), step.kp.view(torch.uint8)))

    src_hash = kernel_hash("sp_attention.hip", "sp_internal.h")
    peak_mfma = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    attn_tflops = attn_flops / (ms_attn * 1e-3) / 1e12
    traffic = read_traffic(wl.name, src_hash)
    kname = ("attn_bf16_kernel<%d>" % D) if wl.dtype == "bf16" and D in (64, 128) else ("attn_f32_kernel<%d>" % D)
    roofline = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak_mfma, "unit": "TFLOP/s",
                "frac": round(attn_tflops / peak_mfma, 4), "traffic": traffic,
                "kernel": kname + (" + attn_combine_kernel" if all_split else ""), "flops_per_launch": attn_flops,
                "avg_launch_ms": round(ms_attn, 4), "R": W, "split": all_split}
    # one rank's share alone (R = 1): what each GPU runs when the ranks are
    # devices; a split launch is the attention kernel plus the merge kernel
    roofline_share = {"bound": "mfma", "achieved": round(share_tflops, 2), "peak": peak_mfma, "unit": "TFLOP/s",
                      "frac": round(share_tflops / peak_mfma, 4),
                      "traffic": read_traffic(wl.name, src_hash, "share_bytes_per_launch"),
                      "kernel": kname + (" + attn_combine_kernel" if share_split else ""),
                      "flops_per_launch": share_flops, "avg_launch_ms": round(ms_share, 4), "R": 1,
                      "split": share_split}
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    kernels = {
        "rotating_note": "copy kernels over rotating buffer sets: ms and GB/s from one replay of the launches "
                         "recorded in a HIP graph; eager_ms with the launches issued one by one from Python",
        "pad+send_recv_heads": {"ms": round(ms_pad_send, 4), "bytes": run_bytes_in,
                                "GB/s": round(gbs(run_bytes_in, ms_pad_send), 1),
                                "note": "in the step: one fused move (plus the mask extension and the query pad "
                                        "where the workload has them)"},
        "gather_heads+gather_output_tokens": {"ms": round(ms_gather_fused, 4), "bytes": gather_bytes,
                                              "GB/s": round(gbs(gather_bytes, ms_gather_fused), 1),
                                              "note": "in the step: one fused move"},
        "pad+send_recv_heads_fused_rotating": {"ms": round(ms_ps_rot, 4), "bytes": fused_send_bytes,
                                               "GB/s": round(gbs(fused_send_bytes, ms_ps_rot), 1),
                                               "hbm_frac": round(gbs(fused_send_bytes, ms_ps_rot) / PEAK_HBM_GBS, 4),
                                               "buffer_sets": n_ps, "eager_ms": round(ms_ps_eager, 4)},
        "gather_heads+gather_output_tokens_fused_rotating": {
            "ms": round(ms_ghu_rot, 4), "bytes": gather_bytes, "GB/s": round(gbs(gather_bytes, ms_ghu_rot), 1),
            "hbm_frac": round(gbs(gather_bytes, ms_ghu_rot) / PEAK_HBM_GBS, 4), "buffer_sets": n_ghu,
            "eager_ms": round(ms_ghu_eager, 4)},
        "separate_moves_step": {"ms": round(ms_separate_step, 4),
                                "pad+send_recv_heads_ms": round(ms_pad_send_sep, 4),
                                "bytes_pad+send": pad_bytes + relayout_bytes,
                                "note": "the step as five separate calls (median of per-step event pairs)"},
        "send_recv_heads_rotating": {"ms": round(ms_relayout_rot, 4), "bytes": relayout_bytes,
                                     "GB/s": round(gbs(relayout_bytes, ms_relayout_rot), 1),
                                     "hbm_frac": round(gbs(relayout_bytes, ms_relayout_rot) / PEAK_HBM_GBS, 4),
                                     "buffer_sets": nsets, "eager_ms": round(ms_relayout_eager, 4)},
        "masked_attention": {"ms": round(ms_attn, 4), "back_to_back_ms": round(ms_attn_b2b, 4),
                             "back_to_back_TFLOP/s": round(attn_flops / (ms_attn_b2b * 1e-3) / 1e12, 2),
                             "TFLOP/s": round(attn_tflops, 2),
                             "mfma_frac": round(attn_tflops / peak_mfma, 4)},
        "gather_heads": {"ms": round(ms_gh, 4), "bytes": relayout_o_bytes,
                         "GB/s": round(gbs(relayout_o_bytes, ms_gh), 1)},
        "gather_output_tokens": {"ms": round(ms_gather, 4), "bytes": gather_bytes,
                                 "GB/s": round(gbs(gather_bytes, ms_gather), 1)},
        "gather_heads_rotating": {"ms": round(ms_gh_rot, 4), "bytes": relayout_o_bytes,
                                  "GB/s": round(gbs(relayout_o_bytes, ms_gh_rot), 1),
                                  "hbm_frac": round(gbs(relayout_o_bytes, ms_gh_rot) / PEAK_HBM_GBS, 4),
                                  "buffer_sets": n_gh, "eager_ms": round(ms_gh_eager, 4)},
        "gather_output_tokens_rotating": {"ms": round(ms_gather_rot, 4), "bytes": gather_bytes,
                                          "GB/s": round(gbs(gather_bytes, ms_gather_rot), 1),
                                          "hbm_frac": round(gbs(gather_bytes, ms_gather_rot) / PEAK_HBM_GBS, 4),
                                          "buffer_sets": n_ga, "eager_ms": round(ms_gather_eager, 4)},
        "cp2d_step": cp2d,
        "zero_copy_step": {"ms": round(ms_zero, 4), "TFLOP/s": round(attn_flops / (ms_zero * 1e-3) / 1e12, 2),
                           "output_bytes_equal_to_step": zero_equal},
        "graph_step": {"ms": round(ms_graph, 4), "TFLOP/s": round(attn_flops / (ms_graph * 1e-3) / 1e12, 2),
                       "output_bytes_equal_to_step": graph_equal},
        "step_spread": spread,
        "masked_attention_rank_share": {"ms": round(ms_share, 4), "TFLOP/s": round(share_tflops, 2),
                                        "mfma_frac": round(share_tflops / peak_mfma, 4), "R": 1,
                                        "split": share_split, "back_to_back_ms": round(ms_share_b2b, 4),
                                        "max_abs_diff_vs_all_ranks": share_diff},
    }

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, x, args.cpu_seconds, step.out.float().cpu().numpy().astype(np.float64))

    value = attn_flops / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "T_pad": Tp, "W": W, "H": H, "Hl": Hl, "D": D,
                   "mask": wl.mask, "cross": wl.cross, "Tq": wl.Tq if wl.cross else T},
        "roofline": roofline,
        "roofline_share": roofline_share,
        "relayout": {"achieved": kernels["send_recv_heads_rotating"]["GB/s"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": kernels["send_recv_heads_rotating"]["hbm_frac"]},
        "cpu_baseline": cpu,
        "kernels": kernels,
        "attention_flops_per_step": attn_flops,
        "wall_s_timed": round(wall, 3),
        "checks": {"output_finite": finite, "relayout_round_trip_bytes_equal": round_trip},
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(out), flush=True)


def bench_joint(args):
    """The joint audio-video block: four attentions (video self, audio self,
    video->audio, audio->video), each through its whole path; a step runs all
    four.  value = attention flops of the four / step time."""
    import numpy as np
    import torch

    from sequence_attention_video_amd.pipeline import JointAVStep
    from sequence_attention_video_amd.workloads import JOINT_AV, make_joint_inputs

    jw = JOINT_AV
    log("inputs", jw.name)
    x = make_joint_inputs(jw)
    step = JointAVStep(jw, x)
    parts = jw.parts()
    flops = {n: 4 * wl.D * wl.H * wl.B * wl.q_tokens_pad * wl.T for n, wl in parts.items()}
    total = sum(flops.values())
    step.run()
    torch.cuda.synchronize()
    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    names = JointAVStep.PARTS
    n = len(names)
    # per step: n + 1 part boundaries, then the video self-attention launch's two
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 3)] for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    gc.collect()
    gc.disable()
    t0.record(stream)
    for i in range(args.steps):
        e = ev[i]
        for j, name in enumerate(names):
            e[j].record(stream)
            s_ = step.steps[name]
            s_.pad()
            _, lengths = s_.partition()
            s_.send_recv_heads()
            if name == "video_self":            # the dominant kernel, timed on its own
                e[n + 1].record(stream)
            s_.attention()
            if name == "video_self":
                e[n + 2].record(stream)
            s_.gather_heads()
            s_.gather_output_tokens(lengths)
        e[n].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    part_ms = {name: float(np.median([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
               for j, name in enumerate(names)}
    # the video self-attention launch: its in-step median (robust to a host
    # stall inside one event pair), and beside it K launches back to back
    ms_attn_v = float(np.median([ev[i][n + 1].elapsed_time(ev[i][n + 2]) for i in range(args.steps)]))
    v = step.steps["video_self"]
    a0 = torch.cuda.Event(enable_timing=True)
    a1 = torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(args.steps):
        v.attention()
    a1.record(stream)
    torch.cuda.synchronize()
    ms_attn_v_b2b = a0.elapsed_time(a1) / args.steps
    gc.enable()
    v_tflops = flops["video_self"] / (ms_attn_v * 1e-3) / 1e12
    finite = all(bool(torch.isfinite(o.float()).all().item()) for o in step.run().values())
    # the same block with the four parts on streams of their own (they share
    # no buffer); reported beside the sequential step
    ref = {name: o.clone() for name, o in step.run().items()}
    for _ in range(max(3, args.warmup // 4)):
        step.run_concurrent()
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(args.steps):
        outs_c = step.run_concurrent()
    c1.record(stream)
    torch.cuda.synchronize()
    ms_conc = c0.elapsed_time(c1) / args.steps
    conc_equal = all(torch.equal(outs_c[name].view(torch.uint8), ref[name].view(torch.uint8)) for name in names)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(parts["video_self"], x["video_self"], args.cpu_seconds)
    out = {
        "metric": METRIC,
        "value": round(total / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": jw.dtype,
        "data": "synthetic",
        "config": {"workload": jw.name, "B": jw.B, "W": jw.W, "H": jw.H, "Tv": jw.Tv, "Ta": jw.Ta,
                   "Dv": jw.Dv, "Da": jw.Da},
        "roofline": {"bound": "mfma", "achieved": round(v_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(v_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "attn_bf16_kernel<128> (video self-attention)",
                     "flops_per_launch": flops["video_self"], "avg_launch_ms": round(ms_attn_v, 4),
                     "back_to_back_ms": round(ms_attn_v_b2b, 4)},
        "cpu_baseline": cpu,
        "parts": {n: {"ms": round(part_ms[n], 4), "attention_flops": flops[n],
                      "TFLOP/s_over_path": round(flops[n] / (part_ms[n] * 1e-3) / 1e12, 2)} for n in names},
        "concurrent_step": {"ms": round(ms_conc, 4), "TFLOP/s": round(total / (ms_conc * 1e-3) / 1e12, 2),
                            "streams": len(names), "output_bytes_equal_to_step": conc_equal},
        "checks": {"output_finite": finite},
        "kernel_source_hash": kernel_hash("sp_attention.hip", "sp_internal.h"),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, x, budget_s: float, gpu_out=None):
    """The oracle as it stands, timed on the host on a bounded sample of the same
    workload: rank 0's local heads, query rows in blocks of 256, all keys.
    With gpu_out (the timed step's final output (B, T, H, D) as float64), the
    sampled oracle rows are also compared with it (outside the timed oracle
    calls): parity re-checked on the benchmarked buffers."""
    import numpy as np

    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    D, T, Tp, W, Hl = wl.D, wl.T, wl.T_pad, wl.W, wl.Hl
    scale = 1.0 / math.sqrt(D)
    widen = (lambda a: O.bf16_bits_to_f64(a)) if wl.dtype == "bf16" else (lambda a: a.astype(np.float64))
    mask = None if x["mask"] is None else O.extend_user_mask(x["mask"], Tp)[0]
    flops = 0
    rows_done = 0
    heads_done = []
    err = 0.0
    spent = 0.0
    t0 = time.perf_counter()
    for j in range(wl.H):                        # rank 0's heads first, then rank 1's, ...
        kj = widen(O.pad_tokens(x["k"][:, :, j], Tp)[0])
        vj = widen(O.pad_tokens(x["v"][:, :, j], Tp)[0])
        qsrc = x["q"][0, :, j] if wl.cross else O.pad_tokens(x["q"][:, :, j], Tp)[0]
        nq = qsrc.shape[0]
        kv_valid = T if mask is None else Tp
        for i0 in range(0, nq, 256):
            i1 = min(nq, i0 + 256)
            mrows = None if mask is None else mask[i0:i1]
            c0 = time.perf_counter()
            want = O.attention(widen(qsrc[i0:i1]), kj, vj, scale, kv_valid, mrows)
            spent += time.perf_counter() - c0
            vis = (i1 - i0) * min(kv_valid, kj.shape[0]) if mrows is None else int(mrows[:, :kv_valid].sum())
            flops += 4 * D * vis
            rows_done += i1 - i0
            if gpu_out is not None:
                keep = min(i1, gpu_out.shape[1]) - i0          # padded query rows are not in the output
                if keep > 0:
                    err = max(err, float(np.max(np.abs(gpu_out[0, i0:i0 + keep, j] - want[:keep]))))
            if spent > budget_s:
                break
        heads_done.append(j)
        if spent > budget_s:
            break
    dt = spent
    rec = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{rows_done} query rows (batch 0; heads {heads_done[0]}..{heads_done[-1]}, rank-major) "
                     f"against all {Tp} keys, float64 NumPy oracle, {dt:.1f} s; the whole step is "
                     f"{wl.H * wl.B} heads of {nq} query rows",
           "seconds": round(dt, 2)}
    if gpu_out is not None:
        tol = 2e-2 if wl.dtype == "bf16" else 1e-4
        rec["timed_output_vs_oracle"] = {"rows": rows_done, "max_abs_err": err, "tol": tol, "ok": err <= tol}
    # the copy oracle beside it: send_recv_heads of the relayed tensors (NumPy
    # moves, one core), in the same bytes-moved terms as the GPU relayout
    names = "kv" if wl.cross else "qkv"
    c0 = time.perf_counter()
    moved = 0
    for n in names:
        shards = O.token_shards(O.pad_tokens(x[n], Tp), W)
        O.send_recv_heads(shards)
        moved += 2 * shards.nbytes
    dc = time.perf_counter() - c0
    rec["relayout"] = {"value": round(moved / dc / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                       "sample": f"send_recv_heads of {', '.join(names.upper())} (pad, token shards, exchange; "
                                 f"{moved / 1e6:.1f} MB read + written), NumPy, {dc:.2f} s"}
    return rec


if __name__ == "__main__":
    main()
