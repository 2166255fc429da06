"""Benchmark of one draft-tree verify step on one MI355X.

A step is one pass of the whole path over one batch of the long-context
verify workload (B 4, P 131072, N 64 random trees of depth <= 8, Hq 32,
Hkv 8, D 128, bf16, page size 64): tree_build_masks -> tree_attention_prefix
-> tree_attention_window_merge -> verify_tree_greedy -> compact_window_rows
(K cache, V cache and a hidden-state table) -> tree_shift_positions(-1).
Inputs are resident in HBM before the timed region.

Prints one JSON line.  `value` is the KV bytes the step must read divided
by the step time; the roofline object is for the dominant kernel (the
split-K prefix), timed with HIP events on the stream it runs on, with the
HBM traffic of a committed counter summary when it was taken on the current
kernel source; `timing` holds the settle phase and the step and launch
statistics; `cpu_baseline` times the CPU fp64 oracle on a bounded sample of
rows of the same workload.
"""
import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import tree_attention_verify_amd as tav  # noqa: E402
from tree_attention_verify_amd import inputs as gen  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
# fp32 vector ALU without packed instructions: 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz = 39.3 T lane operations per second (157.3 TFLOP/s counts packed
# FMAs, two lanes' worth of two flops each)
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
METRIC = "tree-verify attention KV GB/s + rows/s, % of MI355X HBM peak at long ctx"
KERNEL_SRC = os.path.join(ROOT, "tree_attention_verify_amd", "csrc", "tree_attention.hip")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30          # plain copy used to calibrate the HBM byte counters
PREFIX_KERNEL = "k_prefix_mfma"
COPY_KERNEL = "copyBuffer"


def kernel_hash(src=None):
    return hashlib.sha256(open(src or KERNEL_SRC, "rb").read()).hexdigest()[:16]


def traffic_for(workload):
    """HBM bytes per prefix launch from the committed counter summary, or None
    when it is missing or the kernel source changed since it was taken."""
    f = os.path.join(PROFILES, "%s_prefix_traffic.json" % workload)
    if not os.path.exists(f):
        return None
    t = json.load(open(f))
    if t.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return t


def _csv_rows(pattern):
    rows = []
    for f in glob.glob(pattern, recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def summarize_traffic(workload, fetch_dir, write_dir, cmd):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the prefix kernel, each
    scaled by what the same counter reads for a plain 1 GiB copy."""
    def avg(rows, counter, name_has, largest=False):
        v = [float(r["Counter_Value"]) for r in rows
             if r["Counter_Name"] == counter and name_has in r["Kernel_Name"]]
        if largest and v:   # the 1 GiB calibration copies, not smaller copies of the run
            v = [x for x in v if x >= 0.9 * max(v)]
        return sum(v) / len(v) if v else float("nan"), len(v)
    fr = _csv_rows(os.path.join(fetch_dir, "**", "*counter_collection.csv"))
    wr = _csv_rows(os.path.join(write_dir, "**", "*counter_collection.csv"))
    pf, npf = avg(fr, "FETCH_SIZE", PREFIX_KERNEL)
    pw, npw = avg(wr, "WRITE_SIZE", PREFIX_KERNEL)
    cf, ncf = avg(fr, "FETCH_SIZE", COPY_KERNEL, largest=True)
    cw, ncw = avg(wr, "WRITE_SIZE", COPY_KERNEL, largest=True)
    f_scale = COPY_BYTES / (cf * 1024.0)
    w_scale = COPY_BYTES / (cw * 1024.0)
    wl = gen.WORKLOADS[workload]
    P_vis = min(wl.P, wl.prefix_window) if wl.prefix_window else wl.P
    e = ELEM_BYTES[wl.dtype]
    algo = kv_bytes(wl, P_vis, with_window=False) + wl.B * wl.R * wl.Hq * wl.D * e
    t = {"workload": workload, "kernel_source_sha256_16": kernel_hash(),
         "prefix_fetch_kib_per_dispatch": pf, "prefix_write_kib_per_dispatch": pw,
         "copy_fetch_kib_per_dispatch": cf, "copy_write_kib_per_dispatch": cw,
         "copy_bytes_each_way": COPY_BYTES, "fetch_scale": f_scale, "write_scale": w_scale,
         "prefix_read_bytes": pf * 1024 * f_scale, "prefix_write_bytes": pw * 1024 * w_scale,
         "prefix_traffic_bytes": pf * 1024 * f_scale + pw * 1024 * w_scale,
         "prefix_algorithmic_bytes": algo, "dispatches": [npf, npw, ncf, ncw], "command": cmd}
    os.makedirs(PROFILES, exist_ok=True)
    json.dump(t, open(os.path.join(PROFILES, "%s_prefix_traffic.json" % workload), "w"), indent=1)
    with open(os.path.join(PROFILES, "%s_prefix_traffic.md" % workload), "w") as f:
        f.write("# HBM traffic of the split-K prefix kernel, workload %s\n\n" % workload)
        f.write("Command (FETCH_SIZE pass, then the same with WRITE_SIZE):\n\n    %s\n\n" % cmd)
        f.write("| counter | prefix kernel (KiB/dispatch) | 1 GiB copy (KiB/dispatch) | scale |\n|---|---|---|---|\n")
        f.write("| FETCH_SIZE | %.0f | %.0f | %.4f |\n" % (pf, cf, f_scale))
        f.write("| WRITE_SIZE | %.0f | %.0f | %.4f |\n\n" % (pw, cw, w_scale))
        f.write("Scaled HBM bytes per launch: read %.4g, write %.4g, total %.4g; algorithmic "
                "bytes %.4g (ratio %.3f).  Kernel source sha256[:16] %s.\n"
                % (t["prefix_read_bytes"], t["prefix_write_bytes"], t["prefix_traffic_bytes"],
                   algo, t["prefix_traffic_bytes"] / algo, t["kernel_source_sha256_16"]))
    print(json.dumps(t))


MLA_SRC = os.path.join(ROOT, "tree_attention_verify_amd", "csrc", "tree_mla.hip")


def summarize_stats(workload, stats_dir, cmd, mla=False):
    """profiles/<workload>_kernel_stats.md from a rocprofv3 --kernel-trace
    --stats run (an MLA workload with mla=True)."""
    rows = _csv_rows(os.path.join(stats_dir, "**", "*kernel_stats.csv"))
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, "%s_kernel_stats.md" % workload)
    title = ("MLA cascade, workload %s" % gen.MLA_WORKLOADS[workload].describe()) if mla \
        else "workload %s" % workload
    with open(out, "w") as f:
        f.write("# rocprofv3 kernel statistics, %s\n\nCommand:\n\n    %s\n\n" % (title, cmd))
        f.write("| kernel | calls | average (us) | min (us) | max (us) | share |\n|---|---|---|---|---|---|\n")
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            name = r["Name"]
            name = name if len(name) < 90 else name[:87] + "..."
            f.write("| %s | %s | %.1f | %.1f | %.1f | %.1f%% |\n" % (
                name.replace("|", "/"), r["Calls"], float(r["AverageNs"]) / 1e3,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
        if mla:
            f.write("\nThe at::native and __amd_rocclr kernels are the seeded input generation and "
                    "host-to-device copies before the timed region; the MLA kernels count every "
                    "call: the untimed settle calls (back to back for 2 s), the warm-up and the "
                    "timed calls.  tree_mla.hip sha256[:16] %s.\n\n" % kernel_hash(MLA_SRC))
            f.write("k_mla_prefix is the split-K prefix over the latent rows (8 waves per 64 rows: "
                    "each scores one 16 x 16 tile on v_mfma_f32_16x16x32_bf16 and, in the same "
                    "pass, accumulates 64 value channels of the previous block); "
                    "k_mla_window_merge is the masked window and the merge. Under the FP8 latent "
                    "cache (KV8 = true) raw E4M3 rows land in a two-slot ring; at the end of a "
                    "trip each lane takes the chunks it loaded into registers and at the top of "
                    "the next widens them into the bf16 stage layout; the query is rounded to "
                    "E4M3 for every key.\n")
        else:
            f.write("\nThe at::native and __amd_rocclr kernels are the seeded input generation and "
                    "host-to-device copies before the timed region; the path's kernels count every "
                    "step run: the untimed settle steps (back to back for 2 s, so the board runs at "
                    "its steady clock), the warm-up and the timed steps.  Kernel source "
                    "sha256[:16] %s.\n" % kernel_hash())
    print(open(out).read())


N_XCD, N_SIMD = 8, 1024     # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def summarize_counters(workload, dirs, cmd, mla=False):
    """profiles/<workload>_counters.md from rocprofv3 --pmc runs (one
    directory per pass): per-dispatch averages of every counter for the
    prefix kernel (k_mla_prefix for an MLA workload), and what they imply
    (cycles, MFMA utilisation, vector and LDS instructions per unit of
    work)."""
    if mla:
        wl = gen.MLA_WORKLOADS[workload]
        kname, src = "k_mla_prefix", os.path.join(ROOT, "tree_attention_verify_amd", "csrc", "tree_mla.hip")
        Dk = wl.Dc + wl.Dr
        kvb = wl.B * wl.P * Dk * (1 if wl.kv == "fp8" else 2)
        scores = float(wl.B * wl.R * wl.Hq * wl.P)
        flops = scores * (2 * Dk + 2 * wl.Dc)
        # v_mfma_f32_16x16x32_bf16 per 1024 scores: 4 tiles of 16 x 16 over Dk / 32
        # steps, and Dc / 16 value tiles per 16 rows x 32 keys
        mfma_note = "%d = the exact work on 16x16x32 bf16" % (4 * Dk // 32 + 2 * wl.Dc // 16)
    else:
        wl = gen.WORKLOADS[workload]
        kname, src = prefix_kernel_name(wl), None
        mfma_note = "16 = the exact work on 32x32x16 bf16"
    vals, durs = {}, []
    for d in dirs:
        rows = [r for r in _csv_rows(os.path.join(d, "**", "*counter_collection.csv"))
                if kname + "<" in r["Kernel_Name"] or r["Kernel_Name"].endswith(kname)]
        per = {}
        for r in rows:
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            durs.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        for k, v in per.items():
            vals[k] = (sum(v) / len(v), len(v))
    if not mla:
        P_vis = min(wl.P, wl.prefix_window) if wl.prefix_window else wl.P
        kvb = kv_bytes(wl, P_vis, with_window=False)
        flops = 4.0 * wl.D * wl.Hq * wl.B * wl.R * P_vis
        scores = flops / (4.0 * wl.D)
    g = lambda k: vals.get(k, (float("nan"), 0))[0]
    dur_ns = float(np.median(durs)) if durs else float("nan")
    cyc = g("GRBM_GUI_ACTIVE") / N_XCD
    derived = [
        ("dispatch duration (median over passes), us", dur_ns / 1e3),
        ("kernel cycles (GRBM_GUI_ACTIVE / 8 XCDs)", cyc),
        ("engine clock during the dispatch, GHz", cyc / dur_ns if dur_ns else float("nan")),
        ("MFMA busy, share of SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles))",
         g("SQ_VALU_MFMA_BUSY_CYCLES") / (N_SIMD * cyc)),
        ("MFMA instructions per 1024 (row, key) scores (%s)" % mfma_note,
         g("SQ_INSTS_MFMA") / scores * 1024),
        ("vector ALU instructions other than MFMA, per 64 scores (one wave-wide op each)",
         (g("SQ_INSTS_VALU") - g("SQ_INSTS_MFMA")) / scores * 64),
        ("of which transcendental (v_exp), per 64 scores", g("SQ_INSTS_VALU_TRANS_F32") / scores * 64),
        ("LDS instructions per KiB of prefix K/V", g("SQ_INSTS_LDS") / (kvb / 1024)),

        ("MFMA/VALU co-execution, share of MFMA busy cycles",
         g("SQ_VALU_MFMA_COEXEC_CYCLES") / g("SQ_VALU_MFMA_BUSY_CYCLES")),
        ("LDS bank-conflict cycles per LDS instruction", g("SQ_LDS_BANK_CONFLICT") / g("SQ_INSTS_LDS")),
    ]
    if "SQ_LDS_IDX_ACTIVE" in vals:
        derived.append(("LDS busy, share of CU cycles (SQ_LDS_IDX_ACTIVE / (256 CUs x cycles))",
                        g("SQ_LDS_IDX_ACTIVE") / (N_SIMD / 4 * cyc)))
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, "%s_counters.md" % workload)
    with open(out, "w") as f:
        f.write("# rocprofv3 counters of %s, workload %s\n\n" % (kname, wl.describe()))
        f.write("Commands (one counter pass each; bench.py runs 10 steps after 2 warm-up ones):\n\n")
        for c in cmd.split(" ;; "):
            f.write("    %s\n" % c)
        f.write("\nWork per launch: %.4g bytes of prefix K/V, %.4g flops, %.4g (row, key) scores.\n\n"
                % (kvb, flops, scores))
        f.write("| counter | per dispatch (sum over the GPU) | dispatches |\n|---|---|---|\n")
        for k in sorted(vals):
            f.write("| %s | %.6g | %d |\n" % (k, vals[k][0], vals[k][1]))
        f.write("\n| derived | value |\n|---|---|\n")
        for k, v in derived:
            f.write("| %s | %.4g |\n" % (k, v))
        f.write("\nKernel source sha256[:16] %s.\n" % kernel_hash(src))
    print(open(out).read())


def prefix_kernel_name(wl):
    """The split-K prefix kernel the library launches for this shape."""
    if wl.dtype != "bf16":
        return "k_prefix_f32"
    wide = wl.R * (wl.Hq // wl.Hkv) > 128 and (wl.kv != "fp8" or wl.D == 128)
    return "k_prefix_mfma_pipe" if wide else "k_prefix_mfma"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}


def kv_bytes(wl, P_vis, with_window=True):
    e = ELEM_BYTES[wl.kv]
    keys = P_vis + (wl.W if with_window else 0)
    return wl.B * keys * wl.Hkv * wl.D * 2 * e


def attn_flops(wl, masks_np, P_vis):
    pop = sum(bin(int(x)).count("1") for x in masks_np.reshape(-1))
    return 4.0 * wl.D * wl.Hq * (wl.B * wl.R * P_vis + pop)


class Step:
    """Preallocated buffers and the ctypes calls of one verify step."""

    def __init__(self, wl, inp, hidden_dim=4096):
        self.wl, self.inp = wl, inp
        d = "cuda"
        self.L = tav.lib()
        t = lambda x, dt=torch.int32: torch.as_tensor(np.ascontiguousarray(x)).to(dt).to(d)
        self.parents = t(inp.parents)
        self.prefix_len = t(inp.prefix_len)
        self.page_table = t(inp.page_table)
        self.draft, self.target = t(inp.draft), t(inp.target)
        B, N, R = wl.B, wl.N, wl.R
        self.depth = torch.empty((B, N), dtype=torch.int32, device=d)
        self.masks = torch.empty((B, N), dtype=torch.int64, device=d)
        self.positions = torch.empty((B, N), dtype=torch.int32, device=d)
        self.tree_error = torch.empty((B,), dtype=torch.int32, device=d)
        self.out = torch.empty_like(inp.q)
        self.lse = torch.empty((B, R, wl.Hq), dtype=torch.float32, device=d)
        self.path = torch.empty((B, N), dtype=torch.int32, device=d)
        self.alen = torch.empty((B,), dtype=torch.int32, device=d)
        self.tokens = torch.empty((B, N), dtype=torch.int32, device=d)
        self.hidden = torch.randn((B, N, hidden_dim), device=d).to(torch.bfloat16)
        sp, sh, st, Hkv, ps = tav.kv_strides(inp.k_cache, inp.layout)
        self.kv = (sp, sh, st, inp.k_cache.shape[0], ps)
        self.code = tav._code(inp.q.dtype, inp.k_cache.dtype)
        nbytes = tav.tree_attention_workspace_size(inp.q.dtype, B, R, wl.Hq, wl.Hkv, wl.D, wl.P,
                                                   wl.prefix_window, ps, inp.k_cache.dtype)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=d)
        tables = [tav.RowTable.paged_kv(inp.k_cache, self.page_table, self.prefix_len),
                  tav.RowTable.paged_kv(inp.v_cache, self.page_table, self.prefix_len),
                  tav.RowTable.dense_rows(self.hidden)]
        self.tables = (tav.TavRows * 3)()
        for i, tb in enumerate(tables):
            self.tables[i] = tav.TavRows(
                tb.buf.data_ptr(), None if tb.page_table is None else tb.page_table.data_ptr(),
                None if tb.prefix_len is None else tb.prefix_len.data_ptr(),
                0 if tb.page_table is None else tb.page_table.shape[1], tb.page_size,
                tb.num_pages, tb.stride_page, tb.stride_token, tb.stride_head, tb.stride_batch,
                tb.n_heads, tb.row_bytes)
        self.stream = torch.cuda.current_stream().cuda_stream
        # draft lanes: the drafter's lane masks, and only the attention runs
        # (lanes are not verified, so there is no walk or compaction)
        self.lanes = wl.tree == "lanes"
        if self.lanes:
            self.masks = t(inp.lane_masks.view(np.int64), torch.int64)

    def _attn(self, fn):
        wl, inp = self.wl, self.inp
        sp, sh, st, npages, ps = self.kv
        rc = fn(inp.q.data_ptr(), inp.k_cache.data_ptr(), inp.v_cache.data_ptr(), self.code,
                sp, sh, st, npages, self.page_table.data_ptr(), self.page_table.shape[1], ps,
                self.prefix_len.data_ptr(), wl.P, wl.prefix_window, self.masks.data_ptr(),
                wl.W, wl.B, wl.R, wl.Hq, wl.Hkv, wl.D, 0.0, self.out.data_ptr(),
                self.lse.data_ptr(), self.ws.data_ptr(), self.ws.numel(), self.stream)
        assert rc == 0, self.L.tav_last_error()

    def run(self, ev=None):
        """One step.  ev: five events recorded at the step's start, before
        and after the prefix launch, after the window/merge launch and at the
        step's end (all on the step's stream)."""
        L, wl = self.L, self.wl
        B, N = wl.B, wl.N
        rec = (lambda i: ev[i].record() if ev[i] is not None else None) if ev is not None \
            else (lambda i: None)
        rec(0)
        if not self.lanes:
            assert L.tree_build_masks(self.parents.data_ptr(), B, N, self.prefix_len.data_ptr(),
                                      self.depth.data_ptr(), self.masks.data_ptr(),
                                      self.positions.data_ptr(), self.tree_error.data_ptr(),
                                      self.stream) == 0
        rec(1)
        self._attn(L.tree_attention_prefix)
        rec(2)
        self._attn(L.tree_attention_window_merge)
        rec(3)
        if self.lanes:
            rec(4)
            return
        assert L.verify_tree_greedy(self.draft.data_ptr(), self.target.data_ptr(),
                                    self.parents.data_ptr(), B, N, self.path.data_ptr(),
                                    self.alen.data_ptr(), self.tokens.data_ptr(),
                                    self.stream) == 0
        assert L.compact_window_rows(self.tables, 3, self.path.data_ptr(), self.alen.data_ptr(),
                                     B, N, self.stream) == 0
        assert L.tree_shift_positions(self.positions.data_ptr(), self.depth.data_ptr(), B, N, -1,
                                      self.stream) == 0
        rec(4)


def cpu_baseline(wl, inp, masks_np, budget_s):
    """The CPU fp64 oracle on a bounded sample of rows of the same workload."""
    import oracle
    kc, vc = gen.bf16_bits(inp.k_cache), gen.bf16_bits(inp.v_cache)
    q = gen.bf16_bits(inp.q)
    n_rows = wl.B * wl.R * wl.Hq
    rng = np.random.default_rng(0)
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = min(cores, int(omp)) if omp else cores
    n, total_t, done = 16, 0.0, 0
    while True:
        rows = rng.integers(0, n_rows, n)
        t0 = time.perf_counter()
        oracle.tree_attention(q, kc, vc, inp.strides, inp.page_table, wl.page_size,
                              inp.prefix_len, masks_np, wl.W, wl.Hkv,
                              prefix_window=wl.prefix_window, rows=rows)
        dt = time.perf_counter() - t0
        total_t += dt
        done += n
        if total_t >= budget_s or done >= n_rows:
            break
        n = int(min(n_rows - done, max(16, n * min(4.0, (budget_s - total_t) / max(dt, 1e-3)))))
    t_full = total_t * n_rows / done
    P_vis = min(wl.P, wl.prefix_window) if wl.prefix_window else wl.P
    return {"value": kv_bytes(wl, P_vis) / t_full / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle", "rows_per_s": n_rows / t_full,
            "sample": "%d of %d (request, row, head) rows of the same workload, %.1f s of fp64 "
                      "oracle time, scaled to the whole step" % (done, n_rows, total_t)}


SAMPLED_METRIC = "sampled tree verify: target logits GB/s (Gumbel-max draws + greedy walk)"
# vector ALU operations per logit of the Gumbel-max draw: a quarter of a
# Philox4x32-10 block (10 rounds of 2 32x32->64 multiplies and 2 three-way
# XORs), the uniform and its complement (2 conversions, 2 FMAs), the series
# (4 FMAs) and the two logarithms with their scalings (4), the select, the
# score FMA, the NaN clamp and the compare with its two selects (6), and
# the bf16 widening (1)
SAMPLE_OPS_PER_LOGIT = 10 + 4 + 4 + 4 + 1 + 6 + 1


def run_sampled(args):
    """Sampled verify on the EAGLE-style verify shape: 32 requests x 64 rows,
    a 128256-token vocabulary of bf16 logits (525 MB): one step is
    tree_sample_gumbel (the draws) then verify_tree_greedy over them."""
    L = tav.lib()
    wl = gen.WORKLOADS["eagle64"]
    B, N, V = wl.B, wl.N, gen.SAMPLE_VOCAB
    inp = gen.make_inputs(wl, args.seed, "cpu", with_tensors=False)
    # every request samples (temperature > 0): greedy rows would skip the noise
    s = gen.make_sample_inputs(B, N, V, args.seed, "bf16", "cuda", temperatures=(0.6, 1.0, 1.3))
    t = lambda x, dt=torch.int32: torch.as_tensor(np.ascontiguousarray(x)).to(dt).to("cuda")
    parents = t(inp.parents)
    m = tav.tree_build_masks(parents, vc=t(np.full(B, wl.P, np.int32)))
    positions = m["positions"]
    temp = t(s.temperature, torch.float32)
    seed = t(s.seed.view(np.int64), torch.int64)
    draft = t(inp.draft)
    ws = torch.empty(tav.tree_sample_workspace_size(B, N, V), dtype=torch.uint8, device="cuda")
    draws = torch.empty((B, N), dtype=torch.int32, device="cuda")
    path = torch.empty((B, N), dtype=torch.int32, device="cuda")
    alen = torch.empty((B,), dtype=torch.int32, device="cuda")
    toks = torch.empty((B, N), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    lg = s.logits

    def run(ev=None):
        if ev is not None:
            ev[0].record()
        assert L.tree_sample_gumbel(lg.data_ptr(), tav.TAV_BF16, lg.stride(1), V, B, N,
                                    temp.data_ptr(), seed.data_ptr(), positions.data_ptr(),
                                    draws.data_ptr(), ws.data_ptr(), ws.numel(), stream) == 0
        if ev is not None:
            ev[1].record()
        assert L.verify_tree_greedy(draft.data_ptr(), draws.data_ptr(), parents.data_ptr(), B, N,
                                    path.data_ptr(), alen.data_ptr(), toks.data_ptr(),
                                    stream) == 0

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    pairs = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
             for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        run(pairs[i])
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in pairs]))
    nbytes = B * N * V * 2
    ops = SAMPLE_OPS_PER_LOGIT * B * N * V
    res = {"metric": SAMPLED_METRIC, "value": round(nbytes / (ms_step * 1e-3) / 1e9, 2),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "sampled verify, %d requests x %d rows (EAGLE top-8 trees), "
                                  "vocabulary %d, bf16 logits N(0, 4)" % (B, N, V),
                      "temperatures": sorted(set(float(x) for x in s.temperature))},
           "rows_per_s": round(B * N / (ms_step * 1e-3), 1),
           "roofline": {"kernel": "k_gumbel_partial", "bound": "alu",
                        "achieved": round(ops / (k_ms * 1e-3) / 1e12, 2),
                        "peak": round(VALU_PEAK_TOPS, 2), "unit": "T ops/s",
                        "frac": round(ops / (k_ms * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4),
                        "ops_per_logit": SAMPLE_OPS_PER_LOGIT, "traffic": None,
                        "avg_launch_ms": round(k_ms, 4),
                        "hbm_gbs": round(nbytes / (k_ms * 1e-3) / 1e9, 1),
                        "hbm_frac": round(nbytes / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
    if args.cpu_budget > 0:
        import oracle
        rng = np.random.default_rng(0)
        pos_np = positions.cpu().numpy()
        n, total_t, done = 8, 0.0, 0
        while total_t < args.cpu_budget and done < B * N and n > 0:
            rows = [(int(rng.integers(B)), int(rng.integers(N))) for _ in range(n)]
            sub = np.stack([gen.bf16_bits(lg[b, i]) for b, i in rows])[:, None, :]
            t0 = time.perf_counter()
            oracle.sample_gumbel(sub, np.array([s.temperature[b] for b, _ in rows], np.float32),
                                 np.array([s.seed[b] for b, _ in rows], np.uint64),
                                 np.array([[pos_np[b, i]] for b, i in rows], np.int32))
            total_t += time.perf_counter() - t0
            done += n
            n = min(2 * n, 256, B * N - done)
        t_full = total_t * B * N / done
        cores = len(os.sched_getaffinity(0))
        omp = os.environ.get("OMP_NUM_THREADS")
        res["cpu_baseline"] = {"value": round(nbytes / t_full / 1e9, 4), "unit": "GB/s",
                               "cores": min(cores, int(omp)) if omp else cores, "kind": "oracle",
                               "sample": "%d of %d rows, %.1f s of fp64 oracle time, scaled to "
                                         "the whole step" % (done, B * N, total_t)}
    print(json.dumps(res), flush=True)


REJECTION_METRIC = "sampled tree verify by rejection: visited target rows GB/s"


def run_rejection(args):
    """Sampled verify by tree rejection sampling on the EAGLE-style verify
    shape: 32 requests x 64 rows (EAGLE top-8 trees), fp32 target rows over a
    128256-token vocabulary (1.05 GB).  One step is one verify_tree_rejection
    call; a request's walk reads the target rows of the nodes it visits, so
    the algorithmic bytes are sum_b accept_len[b] * V * 4 (twice that with
    the draft q rows).  The value is the median over K calls, each after a
    512 MiB write that evicts the last-level cache; the back-to-back time is
    reported beside it."""
    L = tav.lib()
    B, N, V = 32, 64, gen.SAMPLE_VOCAB
    with_q = args.rejection_q
    x = gen.make_rejection_inputs(B, N, V, args.seed, "cuda", tree="eagle", with_q=with_q)
    qptr, qstride = (x.draft_q.data_ptr(), x.draft_q.stride(1)) if with_q else (None, 0)
    t = lambda a, dt=torch.int32: torch.as_tensor(np.ascontiguousarray(a)).to(dt).to("cuda")
    draft, parents = t(x.draft), t(x.parents)
    score, coins, bu = t(x.draft_score, torch.float32), t(x.coins, torch.float32), \
        t(x.bonus_u, torch.float32)
    path = torch.empty((B, N), dtype=torch.int32, device="cuda")
    alen = torch.empty((B,), dtype=torch.int32, device="cuda")
    toks = torch.empty((B, N), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    probs = x.probs
    ws = torch.empty(tav.verify_tree_rejection_workspace_size(B, N, V), dtype=torch.uint8,
                     device="cuda")

    def run():
        assert L.verify_tree_rejection(probs.data_ptr(), probs.stride(1), V, qptr, qstride,
                                       draft.data_ptr(),
                                       parents.data_ptr(), score.data_ptr(), coins.data_ptr(),
                                       bu.data_ptr(), B, N, path.data_ptr(), alen.data_ptr(),
                                       toks.data_ptr(), ws.data_ptr(), ws.numel(), stream) == 0

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    start, end = mk(), mk()
    start.record()
    for _ in range(args.steps):
        run()
    end.record()
    torch.cuda.synchronize()
    ms_b2b = start.elapsed_time(end) / args.steps
    # the visited rows (tens of MB) stay in the last-level cache across back
    # to back calls; the flushed reps evict it before every call
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    evs = [(mk(), mk()) for _ in range(args.steps)]
    for i, (e0, e1) in enumerate(evs):
        flush.fill_(i & 0xff)
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    flushed_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    ms = float(np.median(flushed_ms))
    visited = int(alen.sum().item())
    nbytes = visited * V * 4 * (2 if with_q else 1)
    gbs = nbytes / (ms * 1e-3) / 1e9
    ntiles = (V + 255) // 256
    groups = min(-(-256 // B), -(-ntiles // 64))
    res = {"metric": REJECTION_METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": "rejection verify%s, %d requests x %d rows (EAGLE top-8 trees), "
                                  "vocabulary %d, fp32 target rows"
                                  % (" against the draft q" if with_q else "", B, N, V),
                      "mean_accept_len": round(visited / B, 3)},
           "rows_per_s": round(B * N / (ms * 1e-3), 1),
           "timing": {"mode": "flushed", "flush_bytes": FLUSH_BYTES, "call_ms": pct(flushed_ms),
                      "back_to_back_ms": round(ms_b2b, 4)},
           "roofline": {"kernel": "k_verify_rejection<%s>" % ("true" if with_q else "false"),
                        "bound": "hbm", "achieved": round(gbs, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "note": "%d workgroups per request share each row pass (%d in all); "
                                "a walk's passes follow one another" % (groups, groups * B)}}
    if args.cpu_budget > 0:
        import oracle
        host = {k: np.ascontiguousarray(getattr(x, k)) for k in
                ("draft", "parents", "draft_score", "coins", "bonus_u")}
        n, total_t, done = 1, 0.0, 0
        while total_t < args.cpu_budget and done < B:
            sl = slice(done, min(done + n, B))
            sub = np.ascontiguousarray(probs[sl].cpu().numpy())
            qsub = np.ascontiguousarray(x.draft_q[sl].cpu().numpy()) if with_q else None
            t0 = time.perf_counter()
            if with_q:
                oracle.verify_rejection_q(sub, qsub, host["draft"][sl], host["parents"][sl],
                                          host["coins"][sl], host["bonus_u"][sl],
                                          host["draft_score"][sl])
            else:
                oracle.verify_rejection(sub, host["draft"][sl], host["parents"][sl],
                                        host["coins"][sl], host["bonus_u"][sl],
                                        host["draft_score"][sl])
            total_t += time.perf_counter() - t0
            done = sl.stop
            n = min(2 * n, 8)
        t_full = total_t * B / done
        res["cpu_baseline"] = {"value": round(nbytes / t_full / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": "%d of %d requests, %.2f s of fp64 oracle time, scaled "
                                         "to the whole step" % (done, B, total_t)}
    print(json.dumps(res), flush=True)


def run_tree_build(args):
    """Tree construction on the EAGLE-style verify shape (32 requests, top-8
    beam over 6 expansion steps into a 328-candidate pool, N = 64): one step
    is the six tree_beam_step launches, tree_select_candidates (depth-first
    numbering) and tree_retrieve_links.  Latency-bound; reported in us."""
    L = tav.lib()
    B, K, S, N = 32, 8, 6, 64
    C = K + (S - 1) * K * K
    rng = np.random.default_rng(args.seed)
    t = lambda x, dt=torch.int32: torch.as_tensor(np.ascontiguousarray(x)).to(dt).to("cuda")
    steps = []
    for i in range(S):
        n_s = 1 if i == 0 else K
        steps.append((t(rng.dirichlet(np.ones(K), size=(B, n_s)).astype(np.float32), torch.float32),
                      t(rng.integers(0, gen.SAMPLE_VOCAB, size=(B, n_s, K)).astype(np.int32)), n_s))
    ps = torch.zeros((B, C), dtype=torch.float32, device="cuda")
    pp = torch.zeros((B, C), dtype=torch.int32, device="cuda")
    pt = torch.zeros((B, C), dtype=torch.int32, device="cuda")
    sc = torch.ones((B, K), dtype=torch.float32, device="cuda")
    si = torch.full((B, K), -1, dtype=torch.int32, device="cuda")
    roots = t(np.arange(B, dtype=np.int32))
    par = torch.empty((B, N), dtype=torch.int32, device="cuda")
    tok, sel, err = torch.empty_like(par), torch.empty_like(par), torch.empty((B,), dtype=torch.int32, device="cuda")
    nt, nsb = torch.empty_like(par), torch.empty_like(par)
    stream = torch.cuda.current_stream().cuda_stream

    def run():
        sc.fill_(1.0)
        si.fill_(-1)
        base = 0
        for p, tk, n_s in steps:
            assert L.tree_beam_step(sc.data_ptr(), si.data_ptr(), p.data_ptr(), tk.data_ptr(), B, n_s,
                                    K, C, base, ps.data_ptr(), pp.data_ptr(), pt.data_ptr(),
                                    sc.data_ptr(), si.data_ptr(), stream) == 0
            base += n_s * K
        assert L.tree_select_candidates(ps.data_ptr(), pp.data_ptr(), pt.data_ptr(), roots.data_ptr(),
                                        B, C, N, 1, par.data_ptr(), tok.data_ptr(), sel.data_ptr(),
                                        err.data_ptr(), stream) == 0
        assert L.tree_retrieve_links(par.data_ptr(), B, N, nt.data_ptr(), nsb.data_ptr(), stream) == 0

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        run()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    assert int(err.max()) == 0
    print(json.dumps({"metric": "tree construction latency (EAGLE top-8 x 6 steps, N 64)",
                      "value": round(ms * 1e3, 2), "unit": "us", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "ms_per_step": round(ms, 4),
                      "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
                      "dtype": "f32", "data": "synthetic",
                      "config": {"workload": "tree construction: B 32, topk 8, 6 steps, pool %d, "
                                             "N 64, depth-first numbering" % C},
                      "trees_per_s": round(B / (ms * 1e-3), 1)}), flush=True)


def run_mla(args):
    """The verify cascade over an MLA latent cache (tree_attention_mla: the
    split-K prefix and the window + merge) on one of the MLA workloads."""
    L = tav.lib()
    wl = gen.MLA_WORKLOADS[args.mla]
    log("workload", wl.describe())
    inp = gen.make_mla_inputs(wl, args.seed, "cuda")
    t = lambda x, dt=torch.int32: torch.as_tensor(np.ascontiguousarray(x)).to(dt).to("cuda")
    parents = t(inp.parents)
    m = tav.tree_build_masks(parents)
    masks = m["masks"]
    pt, pl = t(inp.page_table), t(inp.prefix_len)
    Dk = wl.Dc + wl.Dr
    ps = wl.page_size
    nbytes = tav.tree_attention_mla_workspace_size(wl.B, wl.R, wl.Hq, wl.Dc, wl.Dr, wl.P, ps)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.B, wl.R, wl.Hq, wl.Dc), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((wl.B, wl.R, wl.Hq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    fp8 = wl.kv == "fp8"
    code = tav.TAV_FP8_E4M3 if fp8 else tav.TAV_BF16

    def run():
        assert L.tree_attention_mla(inp.q.data_ptr(), inp.latent.data_ptr(), code, ps * Dk,
                                    Dk, inp.latent.shape[0], pt.data_ptr(), pt.shape[1], ps,
                                    pl.data_ptr(), wl.P, masks.data_ptr(), wl.W, wl.B, wl.R,
                                    wl.Hq, wl.Dc, wl.Dr, 0.0, out.data_ptr(), lse.data_ptr(),
                                    ws.data_ptr(), ws.numel(), stream) == 0, L.tav_last_error()

    # untimed calls back to back first, as for the verify step (--settle)
    settle_calls, t_s = 0, time.perf_counter()
    while time.perf_counter() - t_s < args.settle:
        for _ in range(20):
            run()
        torch.cuda.synchronize()
        settle_calls += 20
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        run()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    sustained = None
    if args.sustain > 0:
        n, t_s = 0, time.perf_counter()
        while time.perf_counter() - t_s < args.sustain:
            for _ in range(50):
                run()
            torch.cuda.synchronize()
            n += 50
        sustained = (time.perf_counter() - t_s) * 1e3 / n
        log("sustained: %d steps back to back, %.4f ms/step" % (n, sustained))
    masks_np = masks.cpu().numpy().view(np.uint64)
    pop = sum(bin(int(x)).count("1") for x in masks_np.reshape(-1))
    per_key = 2 * Dk + 2 * wl.Dc
    flops = per_key * wl.Hq * (wl.B * wl.R * wl.P + pop)
    kvb = wl.B * (wl.P + wl.W) * Dk * (1 if fp8 else 2)
    tfs = flops / (ms * 1e-3) / 1e12
    res = {"metric": "MLA tree-verify attention: latent KV GB/s and TFLOP/s", "value": round(kvb / (ms * 1e-3) / 1e9, 2),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": wl.describe()},
           "timing": {"settle_s": args.settle, "settle_calls": settle_calls},
           "rows_per_s": round(wl.B * wl.R / (ms * 1e-3), 1),
           # (under an FP8 latent cache the products run on the bf16 MFMA too:
           # E4M3 rows widened exactly, the query rounded to E4M3)
           "roofline": {"kernel": "k_mla_prefix + k_mla_window_merge", "bound": "mfma",
                        "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                        "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4), "algorithmic_flops": flops,
                        "flop_per_kv_byte": round(flops / kvb, 1), "traffic": None}}
    if sustained is not None:
        res["sustained_ms_per_step"] = round(sustained, 4)
    if args.cpu_budget > 0:
        import oracle as orc
        rng = np.random.default_rng(0)
        n_rows = wl.B * wl.R * wl.Hq
        n, total_t, done = 4, 0.0, 0
        qb, lb = gen.bf16_bits(inp.q), gen.bf16_bits(inp.latent)
        while total_t < args.cpu_budget and done < n_rows:
            rows = rng.integers(0, n_rows, n)
            t0 = time.perf_counter()
            orc.mla_attention(qb, lb, inp.strides, inp.page_table, ps, inp.prefix_len, masks_np,
                              wl.W, wl.Dc, wl.Dr, rows=rows)
            total_t += time.perf_counter() - t0
            done += n
            n = min(2 * n, 512, n_rows - done)
        t_full = total_t * n_rows / done
        cores = len(os.sched_getaffinity(0))
        omp = os.environ.get("OMP_NUM_THREADS")
        res["cpu_baseline"] = {"value": round(kvb / t_full / 1e9, 5), "unit": "GB/s",
                               "cores": min(cores, int(omp)) if omp else cores, "kind": "oracle",
                               "sample": "%d of %d (request, row, head) rows, %.1f s of fp64 oracle "
                                         "time, scaled to the whole step" % (done, n_rows, total_t)}
    print(json.dumps(res), flush=True)


def _smi_sample():
    """One amd-smi reading: (socket power W, mean GFX clock MHz), or None."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True,
                           timeout=20)
    except (OSError, subprocess.TimeoutExpired):
        return None
    pw = re.findall(r"SOCKET_POWER:\s*([0-9.]+)\s*W", r.stdout)
    clk = re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", r.stdout)
    if not pw:
        return None
    return float(pw[0]), (float(np.mean([float(c) for c in clk])) if clk else float("nan"))


def _sustained(run, seconds, per_sync=20, settle=4.0):
    """Runs `run` back to back for `seconds`; amd-smi is read every ~2 s
    after `settle` seconds.  -> (ms per call, [(W, MHz)])."""
    import threading
    samples, stop = [], threading.Event()

    def sampler():
        if stop.wait(settle):
            return
        while not stop.is_set():
            s = _smi_sample()
            if s is not None:
                samples.append(s)
            if stop.wait(2.0):
                return
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(per_sync):
            run()
        torch.cuda.synchronize()
        n += per_sync
    dt = time.perf_counter() - t0
    stop.set()
    th.join()
    return dt * 1e3 / n, samples


def run_power_model(args):
    """Board power and engine clock, sustained, for the pieces the
    long-context step is made of: idle; a bf16 GEMM on the MFMA (hipBLASLt
    through torch.matmul); an HBM copy; the long64 verify step; and the same
    step with every K/V page aliased onto 8 physical pages (the same
    arithmetic with the K/V stream served from the caches).  Energy per
    launch above idle follows from (W - idle W) x time; it prints one JSON
    line and the table of profiles/long64_power_model.md."""
    secs = args.power_seconds
    res = {"metric": "board power model of the long-context verify step", "rows": []}
    time.sleep(3.0)
    idle = [s for s in (_smi_sample() for _ in range(3)) if s is not None]
    idle_w = float(np.median([s[0] for s in idle])) if idle else float("nan")
    res["idle_w"] = idle_w

    def add(name, ms, samples, work):
        w = float(np.median([s[0] for s in samples])) if samples else float("nan")
        mhz = float(np.median([s[1] for s in samples])) if samples else float("nan")
        row = {"name": name, "ms_per_call": round(ms, 4), "power_w": w, "gfx_mhz": round(mhz),
               "energy_above_idle_mj": round((w - idle_w) * ms, 4), "samples": len(samples)}
        row.update(work)
        res["rows"].append(row)
        log("%-34s %.4f ms  %6.0f W  %5.0f MHz  %.3f mJ above idle  %s"
            % (name, ms, w, mhz, row["energy_above_idle_mj"], work))

    n = 8192
    a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
    b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    ms, smp = _sustained(lambda: torch.matmul(a, b, out=c), secs, per_sync=10)
    add("bf16 GEMM 8192^3 (torch.matmul)", ms, smp,
        {"tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1), "flops": 2.0 * n ** 3})
    del a, b, c
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms, smp = _sustained(lambda: dst.copy_(src), secs)
    add("HBM copy 1 GiB (read + write)", ms, smp,
        {"hbm_gbs": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1), "bytes": 2 * COPY_BYTES})
    del src, dst
    torch.cuda.empty_cache()
    wl = gen.WORKLOADS["long64"]
    inp = gen.make_inputs(wl, args.seed, "cuda")
    step = Step(wl, inp)
    kvb = kv_bytes(wl, wl.P)
    flops = 4.0 * wl.D * wl.Hq * wl.B * wl.R * wl.P
    ms, smp = _sustained(step.run, secs)
    add("long64 verify step", ms, smp, {"kv_gbs": round(kvb / (ms * 1e-3) / 1e9, 1),
                                          "bytes": kvb, "flops": flops})
    # every logical page of every request on one of 8 physical pages (the
    # first 8 pages of request 0, all inside its prefix, so finite): the
    # kernels do the same arithmetic while the K/V reads hit the caches
    pages8 = inp.page_table[0, :8]
    alias = pages8[np.arange(inp.page_table.size) % 8].reshape(inp.page_table.shape)
    step.page_table.copy_(torch.as_tensor(alias.astype(np.int32)))
    ms, smp = _sustained(step.run, secs)
    add("long64 step, K/V pages aliased (cached)", ms, smp, {"flops": flops})
    res["rows_note"] = ("energy_above_idle_mj = (median board power - idle power) x time per call")
    print(json.dumps(res), flush=True)


def summarize_power(json_path, cmd):
    """profiles/long64_power_model.md from the JSON line of --power-model."""
    d = json.loads(open(json_path).read().strip().splitlines()[-1])
    idle = d["idle_w"]
    rows = {r["name"]: r for r in d["rows"]}
    gemm = next(r for r in d["rows"] if r["name"].startswith("bf16 GEMM"))
    copy = next(r for r in d["rows"] if r["name"].startswith("HBM copy"))
    step = next(r for r in d["rows"] if r["name"] == "long64 verify step")
    alias = next(r for r in d["rows"] if "aliased" in r["name"])
    pj_flop = gemm["energy_above_idle_mj"] * 1e-3 / gemm["flops"] * 1e12
    j_gb = copy["energy_above_idle_mj"] * 1e-3 / (copy["bytes"] / 1e9)
    flops, kvb = step["flops"], step["bytes"]
    t_gemm = flops / (gemm["tflops"] * 1e12) * 1e6
    t70 = kvb / (0.7 * HBM_PEAK_GBS * 1e9) * 1e6
    out = os.path.join(PROFILES, "long64_power_model.md")
    with open(out, "w") as f:
        f.write("# Board power model of the long-context verify step\n\nCommand:\n\n    %s\n\n" % cmd)
        f.write("Each row runs back to back for 10 s; `amd-smi metric -p -c` is read every ~2 s "
                "after 4 s and the medians are shown.  Idle board power: %.0f W.  Energy above "
                "idle per call = (power - idle) x time per call.\n\n" % idle)
        f.write("| workload | ms per call | board W | GFX MHz | mJ above idle | rate |\n"
                "|---|---|---|---|---|---|\n")
        for r in d["rows"]:
            rate = ("%.0f TFLOP/s" % r["tflops"]) if "tflops" in r else \
                   ("%.0f GB/s" % r["hbm_gbs"]) if "hbm_gbs" in r else \
                   ("%.0f GB/s of K/V" % r["kv_gbs"]) if "kv_gbs" in r else \
                   ("%.0f TFLOP/s" % (r["flops"] / (r["ms_per_call"] * 1e-3) / 1e12))
            f.write("| %s | %.4f | %.0f | %.0f | %.1f | %s |\n"
                    % (r["name"], r["ms_per_call"], r["power_w"], r["gfx_mhz"],
                       r["energy_above_idle_mj"], rate))
        f.write("\nWhat bounds long64 (B 4, P 131072, N 64, Hq 32, Hkv 8, D 128, bf16: %.4g bytes "
                "of K/V and %.4g flops per step):\n\n" % (kvb, flops))
        f.write("- The vendor bf16 GEMM sustains %.0f TFLOP/s at the board's power cap, %.2f of the "
                "2.5 PFLOP/s dense peak.  At that rate the step's flops alone take %.0f us; 70%% "
                "of 8 TB/s needs the whole step in %.0f us.\n" % (gemm["tflops"],
                                                                   gemm["tflops"] / 2500, t_gemm, t70))
        f.write("- Energy above idle: the GEMM spends %.2f pJ per flop, the copy %.3f J per GB "
                "moved.  The step's flops at GEMM energy plus its bytes at copy energy come to "
                "%.0f mJ; the step measures %.0f mJ (%.0f mJ with its pages aliased onto cached "
                "ones, at a higher clock).\n" % (pj_flop, j_gb, pj_flop * flops * 1e-9 +
                                                  j_gb * kvb / 1e9 * 1e3,
                                                  step["energy_above_idle_mj"],
                                                  alias["energy_above_idle_mj"]))
        f.write("- At the cap (%.0f W above idle) that additive estimate takes %.0f us per step, "
                "and the step runs in %.0f us: it sits at the board's power bound.  Neither HBM "
                "bandwidth (the copy alone streams at %.0f GB/s) nor the MFMA issue rate (the "
                "compute alone runs at %.0f TFLOP/s) sets its time.\n"
                % (1400 - idle, (pj_flop * flops * 1e-12 + j_gb * kvb / 1e9) / (1400 - idle) * 1e6,
                   step["ms_per_call"] * 1e3, copy["hbm_gbs"],
                   flops / (alias["ms_per_call"] * 1e-3) / 1e12))
    print(open(out).read())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the board's power management settles within about 100 steps; the default
    # times the steady state that back-to-back verify rounds run in
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle", type=float, default=2.0, metavar="SECONDS",
                    help="untimed steps back to back for SECONDS before the warm-up, so that "
                         "the timed steps run at the board's steady clock (0 = none)")
    ap.add_argument("--workload", default="long64", choices=sorted(gen.WORKLOADS) + ["all"],
                    help="the verify workload to time; 'all' prints one line per "
                         "configuration, each with the last-level cache flushed before every step")
    ap.add_argument("--flush", action="store_true",
                    help="flush the last-level cache before every step and report medians")
    ap.add_argument("--seed", type=int, default=4)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle time for the CPU baseline (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB copy (calibrates FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--sampled", action="store_true",
                    help="time the sampled verify (Gumbel-max draws over a 128256-token "
                         "vocabulary, then the greedy walk) instead of the attention step")
    ap.add_argument("--rejection", action="store_true",
                    help="time the sampled verify by tree rejection sampling (fp32 target rows "
                         "over a 128256-token vocabulary) instead")
    ap.add_argument("--rejection-q", action="store_true",
                    help="the same, testing against the draft distributions (fp32 q rows too)")
    ap.add_argument("--mla", choices=sorted(gen.MLA_WORKLOADS),
                    help="time the cascade over an MLA latent cache on this workload instead")
    ap.add_argument("--tree-build", action="store_true",
                    help="time tree construction (beam steps, selection, links) instead")
    ap.add_argument("--sustain", type=float, default=0.0, metavar="SECONDS",
                    help="after the timed steps, run steps back to back for SECONDS (for board "
                         "power and clock readings taken meanwhile) and report their rate")
    ap.add_argument("--power-model", action="store_true",
                    help="sustained board power and clock of a bf16 GEMM, an HBM copy, the long64 "
                         "step and the long64 step over aliased (cached) pages")
    ap.add_argument("--power-seconds", type=float, default=10.0)
    ap.add_argument("--summarize-power", nargs=2, metavar=("JSON", "CMD"),
                    help="write profiles/long64_power_model.md from a --power-model JSON line")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "CMD"),
                    help="write profiles/<workload>_prefix_traffic.{json,md} from rocprofv3 CSVs")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_DIR", "CMD"),
                    help="write profiles/<workload>_kernel_stats.md from rocprofv3 --stats CSVs")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR_OR_CMD",
                    help="write profiles/<workload>_counters.md from rocprofv3 --pmc passes: "
                         "the pass directories, then the commands joined by ' ;; '")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(args.workload, *args.summarize_traffic)
        return
    if args.summarize_stats:
        summarize_stats(args.mla or args.workload, *args.summarize_stats, mla=bool(args.mla))
        return
    if args.summarize_power:
        summarize_power(*args.summarize_power)
        return
    if args.summarize_counters:
        summarize_counters(args.mla or args.workload, args.summarize_counters[:-1],
                           args.summarize_counters[-1], mla=bool(args.mla))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.power_model:
        run_power_model(args)
        return
    if args.sampled:
        run_sampled(args)
        return
    if args.tree_build:
        run_tree_build(args)
        return
    if args.rejection or args.rejection_q:
        run_rejection(args)
        return
    if args.mla:
        run_mla(args)
        return
    if args.workload == "all":
        for name in ALL_WORKLOADS:
            res = bench_workload(gen.WORKLOADS[name], args, flushed=True)
            print(json.dumps(res), flush=True)
        return
    res = bench_workload(gen.WORKLOADS[args.workload], args, flushed=args.flush)
    print(json.dumps(res), flush=True)


# every configuration of the verify path, one JSON line each under --workload all
ALL_WORKLOADS = ["worked", "random16", "eagle64", "long64", "lanes", "chain8", "long64_fp8",
                 "chain8_fp8", "long64_tp8"]
FLUSH_BYTES = 512 << 20       # > the 256 MB last-level cache (MALL)


def pct(xs):
    xs = np.asarray(xs, np.float64)
    return {"median": round(float(np.median(xs)), 4), "p10": round(float(np.percentile(xs, 10)), 4),
            "p90": round(float(np.percentile(xs, 90)), 4), "mean": round(float(xs.mean()), 4)}


def bench_workload(wl, args, flushed):
    """One JSON result for workload wl.  Unflushed (the default run): W warm-up
    steps, then K steps back to back between two events, each step's prefix
    launch also bracketed by its own events.  Flushed (--flush, and every line
    of --workload all): before every step a 512 MiB write evicts the
    last-level cache, and each step is timed by its own events (prefix launch,
    tree_attention = prefix + window/merge, whole step); the result reports
    median, p10 and p90 over the K steps and takes the medians as its value."""
    log("workload", wl)
    t0 = time.perf_counter()
    inp = gen.make_inputs(wl, args.seed, "cuda")
    torch.cuda.synchronize()
    log("inputs ready in %.1f s" % (time.perf_counter() - t0))
    step = Step(wl, inp)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda") if flushed else None
    # Untimed steps back to back for --settle seconds first: after an idle
    # moment the board runs the first launches at full clock, then clamps the
    # clock and relaxes it over about a hundred steps, so short warm-ups would
    # time that transient instead of the rate a serving loop sustains.
    settle_steps, t_s = 0, time.perf_counter()
    while time.perf_counter() - t_s < args.settle:
        for _ in range(20):
            step.run()
        torch.cuda.synchronize()
        settle_steps += 20
    if settle_steps:
        log("settled: %d untimed steps in %.1f s" % (settle_steps, time.perf_counter() - t_s))
    for i in range(args.warmup):
        if flush is not None:
            flush.fill_(i & 0xff)
        step.run()
    torch.cuda.synchronize()
    log("warmup done")

    mk = lambda: torch.cuda.Event(enable_timing=True)
    # flushed reps time every part of each step; back-to-back steps record
    # only the two events around the prefix launch (the roofline's timing),
    # so markers between the small kernels do not lengthen the step
    evs = [[mk() for _ in range(5)] if flushed else [None, mk(), mk(), None, None]
           for _ in range(args.steps)]
    start, end = mk(), mk()
    torch.cuda.synchronize()
    t_host = time.perf_counter()
    start.record()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0xff)
        step.run(evs[i])
    end.record()
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    prefix_ms = [e[1].elapsed_time(e[2]) for e in evs]
    if flushed:
        step_ms = [e[0].elapsed_time(e[4]) for e in evs]
        attn_ms = [e[1].elapsed_time(e[3]) for e in evs]
    else:
        step_ms = [start.elapsed_time(end) / args.steps]
        attn_ms = [float("nan")]
    if flushed:
        ms_step = float(np.median(step_ms))
        prefix_t = float(np.median(prefix_ms))
    else:
        ms_step = start.elapsed_time(end) / args.steps
        prefix_t = float(np.mean(prefix_ms))
    log("timed %d steps%s: %.4f ms/step (host %.3f ms/step incl. flushes), prefix kernel %s "
        "%.4f ms (min %.4f max %.4f)" % (args.steps, " (LLC flushed before each)" if flushed else "",
                                         ms_step, t_host * 1e3 / args.steps,
                                         "median" if flushed else "avg", prefix_t,
                                         min(prefix_ms), max(prefix_ms)))

    sustained = None
    if args.sustain > 0:
        n, t_s = 0, time.perf_counter()
        while time.perf_counter() - t_s < args.sustain:
            for _ in range(50):
                step.run()
            torch.cuda.synchronize()
            n += 50
        sustained = (time.perf_counter() - t_s) * 1e3 / n
        log("sustained: %d steps back to back, %.4f ms/step" % (n, sustained))

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    del flush

    masks_np = step.masks.cpu().numpy().view(np.uint64)
    P_vis = min(wl.P, wl.prefix_window) if wl.prefix_window else wl.P
    kvb = kv_bytes(wl, P_vis)
    rows = wl.B * wl.R
    value = kvb / (ms_step * 1e-3) / 1e9
    e = ELEM_BYTES[wl.dtype]
    prefix_bytes = kv_bytes(wl, P_vis, with_window=False) + wl.B * wl.R * wl.Hq * wl.D * e
    achieved = prefix_bytes / (prefix_t * 1e-3) / 1e9
    flops = attn_flops(wl, masks_np, P_vis)
    prefix_flops = 4.0 * wl.D * wl.Hq * wl.B * wl.R * P_vis
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.describe(),
                   "B": wl.B, "P": wl.P, "N": wl.N, "Hq": wl.Hq, "Hkv": wl.Hkv, "D": wl.D,
                   "page_size": wl.page_size, "parallelism": "1 GPU"},
        "rows_per_s": round(rows / (ms_step * 1e-3), 1),
        "head_rows_per_s": round(rows * wl.Hq / (ms_step * 1e-3), 1),
        "hbm_frac_of_step": round(value / HBM_PEAK_GBS, 4),
        "attention_tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "timing": {"llc_flushed": bool(flushed),
                   "flush_bytes": FLUSH_BYTES if flushed else 0,
                   "settle_s": args.settle, "settle_steps": settle_steps,
                   "step_ms": pct(step_ms),
                   "tree_attention_ms": pct(attn_ms) if flushed else None,
                   "prefix_ms": pct(prefix_ms),
                   "value_from": "median step" if flushed else
                                 "K back-to-back steps between two events"},
        "roofline": {"kernel": prefix_kernel_name(wl), "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes": prefix_bytes,
                     "avg_launch_ms": round(prefix_t, 4),
                     "mfma_tflops": round(prefix_flops / (prefix_t * 1e-3) / 1e12, 1),
                     "mfma_frac": round(prefix_flops / (prefix_t * 1e-3) / 1e12
                                        / MFMA_BF16_PEAK_TFS, 4)},
    }
    if flushed:
        res["roofline"]["launch_ms_statistic"] = "median over flushed reps"
    # shapes past the ridge (flop per byte above peak MFMA / peak HBM) are
    # MFMA-bound: report the prefix kernel against the bf16 MFMA peak instead
    # (FP8 caches too: their E4M3 keys and values are widened and multiplied
    # on the bf16 MFMA, so every product is exact)
    mfma_peak = MFMA_BF16_PEAK_TFS
    if wl.dtype == "bf16" and \
            prefix_flops / prefix_bytes > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9):
        rf = res["roofline"]
        tfs = prefix_flops / (prefix_t * 1e-3) / 1e12
        rf.update({"bound": "mfma", "achieved": round(tfs, 1), "peak": round(mfma_peak, 1),
                   "unit": "TFLOP/s", "frac": round(tfs / mfma_peak, 4),
                   "algorithmic_flops": prefix_flops, "hbm_gbs": round(achieved, 1)})
    if wl.dtype == "f32":
        res["roofline"]["note"] = "fp32 vector-ALU prefix on a 68 KB workload: launch-latency bound"
    if sustained is not None:
        res["sustained_ms_per_step"] = round(sustained, 4)
    t = traffic_for(wl.name)
    if t is not None:
        res["roofline"]["traffic"] = round(t["prefix_traffic_bytes"])
        res["roofline"]["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    budget = args.cpu_budget if args.workload != "all" else min(args.cpu_budget, 3.0)
    if budget > 0:
        log("cpu baseline (oracle), budget %.0f s" % budget)
        res["cpu_baseline"] = cpu_baseline(wl, inp, masks_np, budget)
    del step, inp
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
