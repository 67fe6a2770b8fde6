#!/usr/bin/env python3
"""Throughput of the KV-cache eviction hot path on one MI355X.

One step = one pass of the whole path over one row of synthetic cache already resident
in HBM:
    kv_score  (LSE pass -> LSE combine -> mass pass -> policy epilogue)
    kv_select (radix select of the budget)
    kv_compact_rerope (in-order gather of the kept tokens, all layers, exact re-RoPE)
Default workload: Qwen3-8B-shaped session, 36 layers, 32 Q / 8 KV heads, head_dim 128,
bf16 (144 KiB/token), N = 100,000 tokens, W = 64 window queries, budget 2,048 tokens
with 4 sinks + 128 recent pinned, H2O score plus a foresight bonus from 200 spans, PACE
renumbering under L = 8,192.

Prints one JSON line: metric/value (KV tokens scored+evicted+compacted per second), a
roofline entry for the dominant kernel (timed with HIP events on its launch stream) and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


class HipEvents:
    """hipEvent_t handles through the HIP runtime (timing on the library's own stream).

    The events are created with hipEventDisableSystemFence: they are only read after a full
    device synchronisation, and without the system-scope fence an event recorded between
    two launches holds the next launch back less (by kernel trace on this part: 4.9 us
    instead of 6.6 us)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE) == 0
            arr[i] = h
        return arr

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ev, stream) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "compaction_kv_score_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None when the
    kernel's source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("source_hash") != source_hash(*rec.get("sources", [])):
        return None
    return rec.get("bytes_per_launch")


# rocprofv3 kernel names -> the names used for the roofline, and their sources
TRAFFIC_KERNELS = {
    "lse_pass": ("lse_pass_kernel", ["kv_score.hip", "kv_internal.h"]),
    "mass_pass": ("mass_pass_kernel", ["kv_score.hip", "kv_internal.h"]),
    "compact_rerope": ("compact_kernel", ["kv_compact.hip", "kv_internal.h"]),
}


def pmc_summary(fetch_dir, write_dir, out_json):
    """HBM traffic per launch from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE),
    each holding the bench run (bench_counter_collection.csv) and the 1 GiB copy
    calibration run (copy_counter_collection.csv).  The counters are in KiB per
    dispatch; each is scaled by the factor that makes the copy read (write) exactly
    1 GiB.  Writes out_json and returns a markdown table."""
    import csv
    import glob

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return acc

    def find(d, stem):
        hits = glob.glob(os.path.join(d, "**", f"{stem}_counter_collection.csv"), recursive=True)
        if not hits:
            raise SystemExit(f"no {stem}_counter_collection.csv under {d}")
        return hits[0]

    res = {}
    calib = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        copy = per_kernel(find(d, "copy"), counter)
        cvals = [v for k, vs in copy.items() if "copyBuffer" in k for v in vs]
        if not cvals:
            raise SystemExit(f"{counter}: no copy kernel in the calibration run")
        scale = float(1 << 30) / (sum(cvals) / len(cvals))
        calib[counter] = scale
        bench = per_kernel(find(d, "bench"), counter)
        for name, (needle, _) in TRAFFIC_KERNELS.items():
            vals = [v for k, vs in bench.items() if needle in k for v in vs]
            if vals:
                res.setdefault(name, {})[counter] = sum(vals) / len(vals) * scale
    w = __import__("synth").workload("qwen3-8b-n100k")
    alg = {"lse_pass": w.n_layers * w.n_tokens * w.n_kv_heads * w.head_dim * 2
                       + w.n_layers * w.window * w.n_q_heads * w.head_dim * 2}
    alg["mass_pass"] = alg["lse_pass"]
    alg["compact_rerope"] = 2 * w.budget_tokens * w.kv_bytes_per_token
    out = {"_calibration": {"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30,
                            "fetch_scale": calib["FETCH_SIZE"], "write_scale": calib["WRITE_SIZE"]}}
    rows = ["| Kernel | FETCH (scaled, GB) | WRITE (scaled, GB) | Traffic (GB) | Algorithmic (GB) "
            "| Traffic / algorithmic |", "|---|---|---|---|---|---|"]
    for name, v in res.items():
        f, wr = v.get("FETCH_SIZE", 0.0), v.get("WRITE_SIZE", 0.0)
        srcs = TRAFFIC_KERNELS[name][1]
        out[name] = {"bytes_per_launch": f + wr, "fetch_bytes": f, "write_bytes": wr,
                     "algorithmic_bytes": alg[name], "sources": srcs, "source_hash": source_hash(*srcs)}
        rows.append(f"| {name} | {f / 1e9:.4f} | {wr / 1e9:.4f} | {(f + wr) / 1e9:.4f} | "
                    f"{alg[name] / 1e9:.4f} | {(f + wr) / alg[name]:.3f} |")
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)
    return "\n".join(rows) + (f"\n\nscales: FETCH_SIZE x{calib['FETCH_SIZE']:.4f}, "
                              f"WRITE_SIZE x{calib['WRITE_SIZE']:.4f}")


def measured_mfma_busy():
    """Executed MFMA busy share of the two scoring passes (SQ_VALU_MFMA_BUSY_CYCLES over the
    cycles of all SIMDs) from the committed rocprofv3 counter run, per pass, or None for a
    pass whose source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "mfma_busy.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        recs = json.load(f)
    out = {}
    for name in ("lse_pass", "mass_pass"):
        rec = recs.get(name)
        ok = rec and rec.get("source_hash") == source_hash(*rec.get("sources", []))
        out[name] = round(rec["mfma_busy"], 4) if ok else None
    return out


def clock_summary(pmc_dir, out_json=None):
    """Effective core clock and MFMA busy share per kernel from a rocprofv3 --pmc run with
    GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES.  rocprofv3 sums GRBM_GUI_ACTIVE over the
    8 XCDs of the MI355X (a memory-only kernel reads 2.4 GHz with this factor); the MFMA
    busy share divides by the cycles of all 1,024 SIMDs.  Writes the scoring passes' shares
    to out_json (with the source hash they were measured on) and returns a markdown table."""
    import csv
    import glob
    hits = glob.glob(os.path.join(pmc_dir, "**", "*_counter_collection.csv"), recursive=True)
    if not hits:
        raise SystemExit(f"no *_counter_collection.csv under {pmc_dir}")
    per = {}
    for r in csv.DictReader(open(hits[0])):
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        d = per.setdefault(key, {"dur_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    rows = ["| Kernel | Dispatches | Average (us) | Effective clock (GHz) | MFMA busy |",
            "|---|---|---|---|---|"]
    busy = {}
    for needle in ("lse_pass_kernel", "mass_pass_kernel", "compact_kernel", "select_hist_kernel",
                   "epilogue_kernel", "lse_combine_kernel"):
        ds = [d for (k, _), d in per.items() if needle in k and "GRBM_GUI_ACTIVE" in d]
        if not ds:
            continue
        dur = sum(d["dur_ns"] for d in ds) / len(ds)
        cyc = sum(d["GRBM_GUI_ACTIVE"] for d in ds) / len(ds) / 8.0
        mfma = sum(d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for d in ds) / len(ds)
        rows.append(f"| {needle} | {len(ds)} | {dur / 1e3:.1f} | {cyc / dur:.2f} | "
                    f"{mfma / (1024.0 * cyc):.1%} |")
        name = {"lse_pass_kernel": "lse_pass", "mass_pass_kernel": "mass_pass"}.get(needle)
        if name:
            srcs = TRAFFIC_KERNELS[name][1]
            busy[name] = {"mfma_busy": mfma / (1024.0 * cyc), "clock_ghz": cyc / dur, "avg_us": dur / 1e3,
                          "dispatches": len(ds), "sources": srcs, "source_hash": source_hash(*srcs)}
    if out_json and busy:
        with open(out_json, "w") as fh:
            json.dump(busy, fh, indent=1)
    return "\n".join(rows)


def extras(steps=5, warmup=2, oracle=True):
    """Timings of the rows beyond the headline step, each on one GPU with inputs resident
    in HBM, HIP events on the launch stream, mean over `steps` runs after `warmup`:
      f1: single-pass scoring with a supplied LSE (sum and group maximum), Qwen3-8B 100K;
      f2: compaction + re-rotation of 2,048 kept tokens through the reference store;
      f3: LRFU keep-score update over 100K entries, in-place tail compaction of 2,048;
      f4: gather of 16,384 evicted rows on the device, and offload of 16,384 rows to
          pinned host memory (PCIe-bound, chunks of 1,024);
      Mistral-7B 131,072-token in-place segment eviction + re-rotation;
      Qwen3-8B at 1,000,000 tokens: the full step (MemDecay page scoring, select, compaction);
      the two Qwen2.5-1.5B-shaped workloads (512 and 2,048 tokens): the full step in us;
      f4 swap-in: 16,384 rows loaded back from pinned host memory, and Penelope's chunked
          swap of 16,384 rows through a 1,024-row buffer.
    Prints one JSON line, then (unless oracle=False) a second one with the CPU oracle timed
    on the 512- and 2,048-token workloads, the Mistral segment case and the 1M-token step
    (layer samples scaled to all layers)."""
    import numpy as np
    import compaction_kv_score_amd as kv
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    hip = HipEvents()
    out = {}

    def timed(fn, n=steps, w=warmup):
        for _ in range(w):
            fn()
        evs = [hip.create(2) for _ in range(n)]
        for e in evs:
            hip.record(e[0], sh)
            fn()
            hip.record(e[1], sh)
        torch.cuda.synchronize()
        return sum(hip.ms(e[0], e[1]) for e in evs) / n

    def log(msg):
        print(f"[extras] {msg}", file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- Qwen3-8B 100K
    w = synth.workload("qwen3-8b-n100k")
    N, NL, HKV, D, W, B = w.n_tokens, w.n_layers, w.n_kv_heads, w.head_dim, w.window, w.budget_tokens
    kvb = w.kv_bytes_per_token
    log("qwen3-8b-n100k inputs")
    k, v, _ = synth.kv_cache(w, seed=0, device=dev)
    q = synth.window_queries(w, seed=0, device=dev)
    src = kv.PagedCache(k, v, N)
    acc = torch.zeros(N, device=dev)
    item_score = torch.zeros(N, device=dev)
    item_pinned = torch.zeros(N, dtype=torch.uint8, device=dev)
    mass = torch.zeros(N, device=dev)
    lse = torch.zeros((NL, w.n_q_heads, W), device=dev)
    kw = dict(policy="h2o", window=W, item_tokens=1, accum=acc, item_score=item_score,
              item_pinned=item_pinned, mass=mass)
    ws = torch.empty(kv.kv_score_workspace_size(src, q, **kw), dtype=torch.uint8, device=dev)
    kv.kv_score(src, q, workspace=ws, lse=lse, **kw)
    k_bytes = NL * N * HKV * D * 2
    for agg in ("sum", "max_group"):
        ev = hip.create(5)
        evp = ctypes.cast(ev, ctypes.c_void_p)
        runs = []
        for i in range(warmup + steps):
            kv.kv_score(src, q, workspace=ws, lse_in=lse, aggregate=agg, stage_events=evp, **kw)
            torch.cuda.synchronize()
            if i >= warmup:
                runs.append((hip.ms(ev[0], ev[4]), hip.ms(ev[2], ev[3])))
        tot = sum(r[0] for r in runs) / len(runs)
        mp = sum(r[1] for r in runs) / len(runs)
        out[f"f1_single_pass_{agg}"] = {"score_ms": round(tot, 4), "mass_pass_ms": round(mp, 4),
                                        "mass_pass_GBps": round(k_bytes / (mp * 1e-3) / 1e9, 1)}
        log(f"f1 {agg}: {out[f'f1_single_pass_{agg}']}")
    del ws

    g = torch.Generator().manual_seed(5)
    keep = torch.sort(torch.randperm(N, generator=g)[:B])[0].to(torch.int32).to(dev)
    old_pos = (torch.arange(N, dtype=torch.int32) + 10_000).to(dev)
    dk = torch.zeros((NL, B // 16, 16, HKV, D), dtype=torch.bfloat16, device=dev)
    dv = torch.zeros_like(dk)
    dst = kv.PagedCache(dk, dv, B)
    # every kept token holds a valid entry (the stored key equals the cached key at its position)
    ref_src = kv.RefStore(k.reshape(NL, -1, HKV, D)[:, :N].contiguous(), old_pos.clone())
    ref_dst = kv.RefStore.empty(NL, B, HKV, dev)
    newp = torch.zeros(B, dtype=torch.int32, device=dev)
    rope = kv.kv_rope("default", base=w.rope_theta)
    t_plain = timed(lambda: kv.kv_compact_rerope(src, dst, keep, None, B, old_pos, newp, renumber_base=0,
                                                 rope_theta=w.rope_theta))
    t_store = timed(lambda: kv.kv_compact_rerope(src, dst, keep, None, B, old_pos, newp, renumber_base=0,
                                                 rope=rope, ref_src=ref_src, ref_dst=ref_dst))
    assert int((ref_dst.pos != kv.KV_REF_NONE).sum()) == B
    kb = kvb // 2
    out["f2_store_compaction"] = {
        "ms": round(t_store, 4), "plain_ms": round(t_plain, 4), "kept": B,
        "bytes": 6 * B * kb, "GBps": round(6 * B * kb / (t_store * 1e-3) / 1e9, 1),
        "note": "reads cached K, stored K, V; writes K, V, stored K (72 KiB each per token)"}
    log(f"f2: {out['f2_store_compaction']}")
    del ref_src, ref_dst

    scores = torch.rand(N, generator=g).pow(8).to(dev)
    ks = torch.zeros(N, device=dev)
    ws_l = torch.empty(kv.kv_lrfu_workspace_size(N), dtype=torch.uint8, device=dev)
    t_lrfu = timed(lambda: kv.kv_lrfu_update(scores, ks, top_p=0.9, decay=0.5, workspace=ws_l))
    out["f3_lrfu_update"] = {"ms": round(t_lrfu, 4), "entries": N}
    keeps = [torch.sort(torch.randperm(N, generator=g)[:B])[0].to(torch.int32).to(dev)
             for _ in range(warmup + steps)]
    it = iter(keeps)
    moved = [int(((kk < (16 * -(-N // 16) - 16 * -(-B // 16))) | (kk >= 16 * -(-N // 16) - 16 * -(-B // 16) + B))
                 .sum()) for kk in keeps]
    t_tail = timed(lambda: kv.kv_compact_tail_inplace(src, next(it), None, B, B))
    mv = sum(moved[warmup:]) / steps
    out["f3_tail_compaction"] = {"ms": round(t_tail, 4), "moved_tokens": round(mv, 1),
                                 "GBps": round(2 * mv * kvb / (t_tail * 1e-3) / 1e9, 1)}
    log(f"f3: {out['f3_lrfu_update']} {out['f3_tail_compaction']}")

    n_ev = 16384
    stage_k = torch.zeros((NL, n_ev // 16, 16, HKV, D), dtype=torch.bfloat16, device=dev)
    stage_v = torch.zeros_like(stage_k)
    t_gather = timed(lambda: kv.kv_gather_evicted(src, keep, B, 0, n_ev, kv.PagedCache(stage_k, stage_v, n_ev)))
    keep_off = torch.sort(torch.randperm(N, generator=g)[:N - n_ev])[0].to(torch.int32).to(dev)
    hk = torch.empty((NL, n_ev, HKV, D), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk).pin_memory()
    ws_o = None

    def off():
        nonlocal ws_o
        ws_o = kv.kv_offload_evicted(src, keep_off, N - n_ev, hk, hv, chunk=1024, workspace=ws_o)

    t_off = timed(off, n=3, w=1)
    out["f4_gather_evicted"] = {"ms": round(t_gather, 4), "tokens": n_ev,
                                "GBps": round(2 * n_ev * kvb / (t_gather * 1e-3) / 1e9, 1)}
    out["f4_offload_to_host"] = {"ms": round(t_off, 3), "tokens": n_ev, "bytes": n_ev * kvb,
                                 "GBps": round(n_ev * kvb / (t_off * 1e-3) / 1e9, 2),
                                 "note": "device gather then device-to-host copies into pinned memory"}
    log(f"f4: {out['f4_gather_evicted']} {out['f4_offload_to_host']}")
    # swap-in: the same 16,384 rows loaded back from pinned host memory into their slots,
    # then Penelope's both-tiers-full swap of 16,384 rows through a 1,024-row buffer
    ht_slots = torch.from_numpy(
        __import__("oracle").evicted_tokens(N, keep_off.cpu().numpy()).astype("int32")).to(dev)
    ws_l = None

    def load():
        nonlocal ws_l
        ws_l = kv.kv_load_rows(src, ht_slots, hk, hv, chunk=1024, workspace=ws_l)

    t_load = timed(load, n=3, w=1)
    pool_rows = n_ev + 1024
    pk = torch.empty((NL, pool_rows, HKV, D), dtype=torch.bfloat16, pin_memory=True)
    pv = torch.empty_like(pk).pin_memory()
    swap_slots = torch.sort(torch.randperm(N, generator=g)[:n_ev])[0].to(torch.int32).to(dev)
    ws_s = None
    in_stream = torch.cuda.Stream(dev)

    def swap(two):
        nonlocal ws_s
        _, _, ws_s = kv.kv_swap_chunked(src, swap_slots, pk, pv, 0, n_ev, chunk=1024, workspace=ws_s,
                                        in_stream=in_stream if two else None)

    t_swap1 = timed(lambda: swap(False), n=3, w=1)
    t_swap = timed(lambda: swap(True), n=3, w=1)
    out["f4_load_from_host"] = {"ms": round(t_load, 3), "tokens": n_ev, "bytes": n_ev * kvb,
                                "GBps": round(n_ev * kvb / (t_load * 1e-3) / 1e9, 2),
                                "note": "host-to-device copies into staging, then a scatter into the slots"}
    out["f4_swap_chunked"] = {"ms": round(t_swap, 3), "one_stream_ms": round(t_swap1, 3), "tokens": n_ev,
                              "chunk": 1024, "bytes": 2 * n_ev * kvb,
                              "GBps_both_directions": round(2 * n_ev * kvb / (t_swap * 1e-3) / 1e9, 2),
                              "note": "per chunk: gather + device-to-host into the buffer on one stream, "
                                      "host-to-device + scatter on a second one; one_stream_ms: all in order"}
    log(f"f4: {out['f4_load_from_host']} {out['f4_swap_chunked']}")
    del k, v, src, dk, dv, stage_k, stage_v, hk, hv, ws_o, ws_l, ws_s, pk, pv
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- Mistral-7B segment
    log("mistral-7b-n131072 inputs")
    out["mistral7b_n131072_segment_inplace"] = segment_case(steps=3, warmup=1)
    log(f"segment: {out['mistral7b_n131072_segment_inplace']}")
    torch.cuda.empty_cache()
    out["mistral7b_n131072_segment_remap"] = segment_remap_case(steps=3, warmup=1)
    log(f"segment remap: {out['mistral7b_n131072_segment_remap']}")
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- Qwen3-8B 1M tokens
    w5 = synth.workload("qwen3-8b-n1m")
    N5, B5 = w5.n_tokens, w5.budget_tokens
    log("qwen3-8b-n1m inputs (147 GB)")
    k5, v5, _ = synth.kv_cache(w5, seed=0, device=dev,
                               progress=lambda l: torch.cuda.synchronize() or log(f"layer {l} generated"))
    q5 = synth.window_queries(w5, seed=0, device=dev)
    c5 = kv.PagedCache(k5, v5, N5)
    ewma, clock = synth.memdecay_state(w5, seed=0)
    b_r, lam = synth.region_params(0)
    region = synth.regions(w5, seed=0)
    sid, sbonus = synth.spans(w5, seed=0)
    n_items = -(-N5 // 16)
    st5 = dict(region=region.to(dev), base_prio=b_r.to(dev), decay_rate=lam.to(dev), ewma=ewma.to(dev),
               clock=clock.to(dev), span_id=sid.to(dev), span_bonus=sbonus.to(dev),
               n_sink=w5.n_sink, n_recent=w5.n_recent, pinned_regions=1,
               item_score=torch.zeros(n_items, device=dev),
               item_pinned=torch.zeros(n_items, dtype=torch.uint8, device=dev))
    kw5 = dict(policy="memdecay", window=w5.window, item_tokens=16, rho=w5.rho, alpha=w5.alpha, tau=w5.tau,
               dt_steps=1, **st5)
    ws5 = torch.empty(kv.kv_score_workspace_size(c5, q5, **kw5), dtype=torch.uint8, device=dev)
    keep5 = torch.zeros(N5, dtype=torch.int32, device=dev)
    nk5 = torch.zeros(1, dtype=torch.int64, device=dev)
    status5 = torch.zeros(1, dtype=torch.int32, device=dev)
    ws_s5 = torch.empty(kv.kv_select_workspace_size(n_items), dtype=torch.uint8, device=dev)
    cap5 = 2 * B5 + 4096
    dk5 = torch.zeros((w5.n_layers, cap5 // 16, 16, w5.n_kv_heads, w5.head_dim), dtype=torch.bfloat16, device=dev)
    dv5 = torch.zeros_like(dk5)
    old5 = torch.arange(N5, dtype=torch.int32, device=dev)
    new5 = torch.zeros(cap5, dtype=torch.int32, device=dev)
    ev5 = hip.create(5)
    ev5p = ctypes.cast(ev5, ctypes.c_void_p)
    stage = {"score": 0.0, "lse_pass": 0.0, "mass_pass": 0.0, "select": 0.0, "compact": 0.0}
    tsteps = []
    for i in range(1 + 3):
        e_sel, e_cmp = hip.create(2), hip.create(2)
        t0 = time.perf_counter()
        kv.kv_score(c5, q5, workspace=ws5, stage_events=ev5p, **kw5)
        hip.record(e_sel[0], sh)
        kv.kv_select(st5["item_score"], st5["item_pinned"], 16, N5, B5 // 16, keep5, nk5, status5, workspace=ws_s5)
        hip.record(e_sel[1], sh)
        hip.record(e_cmp[0], sh)
        kv.kv_compact_rerope(c5, kv.PagedCache(dk5, dv5, cap5), keep5, nk5, cap5, old5, new5, renumber_base=0,
                             rope_theta=w5.rope_theta, limit=w5.limit)
        hip.record(e_cmp[1], sh)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if i >= 1:
            tsteps.append((t1 - t0) * 1e3)
            stage["score"] += hip.ms(ev5[0], ev5[4]) / 3
            stage["lse_pass"] += hip.ms(ev5[0], ev5[1]) / 3
            stage["mass_pass"] += hip.ms(ev5[2], ev5[3]) / 3
            stage["select"] += hip.ms(e_sel[0], e_sel[1]) / 3
            stage["compact"] += hip.ms(e_cmp[0], e_cmp[1]) / 3
    ms5 = sum(tsteps) / len(tsteps)
    # the same compaction by relinking the kept pages (the row behind an identity block
    # table): keys re-rotated in their slots, values untouched
    c5p = kv.PagedCache(k5, v5, N5, torch.arange(n_items, dtype=torch.int32, device=dev))
    bt5_out = torch.zeros(-(-cap5 // 16), dtype=torch.int32, device=dev)
    t_relink = []
    for i in range(4):
        e = hip.create(2)
        hip.record(e[0], sh)
        kv.kv_compact_pages_remap(c5p, keep5, nk5, cap5, bt5_out, old5, new5, renumber_base=0,
                                  rope_theta=w5.rope_theta, limit=w5.limit)
        hip.record(e[1], sh)
        torch.cuda.synchronize()
        if i >= 1:
            t_relink.append(hip.ms(e[0], e[1]))
    kb5 = w5.n_layers * N5 * w5.n_kv_heads * w5.head_dim * 2
    out["qwen3_8b_n1m_full_step"] = {"workload": w5.name, "ms_per_step": round(ms5, 3),
                             "KV_tokens_per_s": round(N5 / (ms5 * 1e-3), 1), "n_keep": int(nk5.item()),
                             "status": int(status5.item()),
                             "stages_ms": {a: round(b, 3) for a, b in stage.items()},
                             "compact_by_relinking_pages_ms": round(sum(t_relink) / len(t_relink), 3),
                             "scoring_pass_GBps": {
                                 "lse_pass": round(kb5 / (stage["lse_pass"] * 1e-3) / 1e9, 1),
                                 "mass_pass": round(kb5 / (stage["mass_pass"] * 1e-3) / 1e9, 1)}}
    log(f"1M step: {out['qwen3_8b_n1m_full_step']}")
    del k5, v5, c5, dk5, dv5, ws5
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- small configs
    for name in ("qwen2.5-1.5b-1layer-n512", "qwen2.5-1.5b-n2048"):
        out[f"step_{name}"] = small_config_step(name)
        log(f"{name}: {out[f'step_{name}']}")
    print(json.dumps({"extras": out, "n_gpus": 1, "data": "synthetic"}), flush=True)

    # ---------------------------------------------------------------- oracle baselines
    if oracle:
        base = {}
        for name, layers, rep in (("qwen2.5-1.5b-1layer-n512", None, 3), ("qwen2.5-1.5b-n2048", None, 3),
                                  ("mistral-7b-n131072-segment", 2, 1), ("qwen3-8b-n1m", 2, 1)):
            log(f"oracle baseline {name} ({layers or 'all'} layers)")
            base[name] = oracle_baseline(name, layers, rep)
            log(f"oracle {name}: {base[name]}")
        print(json.dumps({"oracle_baselines": base, "data": "synthetic"}), flush=True)


def segment_case(steps=3, warmup=1):
    """Mistral-7B shape, 131,072 tokens: in-place front-of-history segment eviction of 30%
    (16,384-token prefix kept) with re-rotation of the moved suffix, all 32 layers.  Runs
    are enqueued back to back on one stream; mean HIP-event time per run."""
    import compaction_kv_score_amd as kv
    import synth
    dev = torch.device("cuda:0")
    sh = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    hip = HipEvents()
    w4 = synth.workload("mistral-7b-n131072-segment")
    k4, v4, _ = synth.kv_cache(w4, seed=0, device=dev)
    c4 = kv.PagedCache(k4, v4, w4.n_tokens)
    n_keep4, e4 = kv.kv_select_segment(w4.n_tokens, w4.segment_prefix, int(w4.segment_frac * w4.n_tokens), 16)
    pos4 = torch.arange(w4.n_tokens, dtype=torch.int32, device=dev)
    run = lambda: kv.kv_compact_segment_inplace(c4, w4.segment_prefix, e4, pos4, renumber_base=0,  # noqa: E731
                                                rope_theta=w4.rope_theta)
    for _ in range(warmup):
        run()
    evs = [hip.create(2) for _ in range(steps)]
    for e in evs:
        hip.record(e[0], sh)
        run()
        hip.record(e[1], sh)
    torch.cuda.synchronize()
    t4 = sum(hip.ms(e[0], e[1]) for e in evs) / steps
    moved4 = n_keep4 - w4.segment_prefix
    b4 = 2 * moved4 * w4.kv_bytes_per_token
    return {"workload": w4.name, "ms": round(t4, 3), "evicted": e4, "moved_tokens": moved4, "bytes": b4,
            "GBps": round(b4 / (t4 * 1e-3) / 1e9, 1), "hbm_frac": round(b4 / (t4 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def segment_remap_case(steps=3, warmup=1):
    """The same Mistral-7B segment eviction through the page-table form: a shuffled block
    table, the suffix relinked instead of moved, its keys re-rotated in place (renumbered
    from 0), values untouched; and the same without renumbering (only the table changes).
    Mean HIP-event time per run, runs back to back on one stream."""
    import compaction_kv_score_amd as kv
    import synth
    dev = torch.device("cuda:0")
    sh = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    hip = HipEvents()
    w4 = synth.workload("mistral-7b-n131072-segment")
    N = w4.n_tokens
    k4, v4, bt4 = synth.kv_cache(w4, seed=0, device=dev, paged_shuffle=True, extra_pages=4)
    c4 = kv.PagedCache(k4, v4, N, bt4)
    n_keep4, e4 = kv.kv_select_segment(N, w4.segment_prefix, int(w4.segment_frac * N), 16)
    old = torch.arange(N, dtype=torch.int32, device=dev)
    new = torch.zeros(n_keep4, dtype=torch.int32, device=dev)
    bt_out = torch.zeros(-(-n_keep4 // 16), dtype=torch.int32, device=dev)
    freed = torch.zeros(e4 // 16, dtype=torch.int32, device=dev)
    out = {}
    for base in (0, -1):
        run = lambda: kv.kv_compact_segment_remap(c4, w4.segment_prefix, e4, bt_out, old, new,  # noqa: E731
                                                  freed_pages=freed, renumber_base=base, rope_theta=w4.rope_theta)
        for _ in range(warmup):
            run()
        evs = [hip.create(2) for _ in range(steps)]
        for e in evs:
            hip.record(e[0], sh)
            run()
            hip.record(e[1], sh)
        torch.cuda.synchronize()
        out[base] = sum(hip.ms(e[0], e[1]) for e in evs) / steps
    moved4 = n_keep4 - w4.segment_prefix
    b4 = moved4 * w4.kv_bytes_per_token            # the suffix's keys read and written
    return {"workload": w4.name, "ms": round(out[0], 3), "evicted": e4, "rotated_tokens": moved4, "bytes": b4,
            "GBps": round(b4 / (out[0] * 1e-3) / 1e9, 1),
            "hbm_frac": round(b4 / (out[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "no_renumber_us": round(out[-1] * 1e3, 1),
            "note": "block table relinked; keys re-rotated in place, values not touched"}


def small_config_step(name, steps=20, warmup=3):
    """One full step of a small workload (Qwen2.5-1.5B head shape): MemDecay page scoring,
    page selection, compaction of the kept pages with renumbering.  Median over `steps`
    HIP-event-timed steps after `warmup`, with the MemDecay state restored from a copy
    before every step, outside its events."""
    import compaction_kv_score_amd as kv
    import synth
    dev = torch.device("cuda:0")
    sh = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    hip = HipEvents()
    w = synth.workload(name)
    N, pg = w.n_tokens, w.page_size
    k, v, bt = synth.kv_cache(w, seed=0, device=dev, paged_shuffle=True, extra_pages=2)
    q = synth.window_queries(w, seed=0, device=dev)
    ewma0, clock0 = synth.memdecay_state(w, seed=0)
    b_r, lam = synth.region_params(0)
    ewma, clock = ewma0.to(dev), clock0.to(dev)
    ewma0, clock0 = ewma.clone(), clock.clone()
    n_items = w.n_pages
    item_score = torch.zeros(n_items, device=dev)
    item_pinned = torch.zeros(n_items, dtype=torch.uint8, device=dev)
    src = kv.PagedCache(k, v, N, bt)
    kw = dict(policy="memdecay", window=w.window, item_tokens=pg, region=synth.regions(w, seed=0).to(dev),
              base_prio=b_r.to(dev), decay_rate=lam.to(dev), rho=w.rho, alpha=w.alpha, tau=w.tau, dt_steps=1,
              ewma=ewma, clock=clock, pinned_regions=1, item_score=item_score, item_pinned=item_pinned)
    ws = torch.empty(kv.kv_score_workspace_size(src, q, **kw), dtype=torch.uint8, device=dev)
    ws_sel = torch.empty(kv.kv_select_workspace_size(n_items), dtype=torch.uint8, device=dev)
    B = w.budget_tokens
    keep = torch.zeros(B, dtype=torch.int32, device=dev)
    nk = torch.zeros(1, dtype=torch.int64, device=dev)
    dk = torch.zeros((w.n_layers, B // pg, pg, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    dv = torch.zeros_like(dk)
    dst = kv.PagedCache(dk, dv, B)
    pos = torch.arange(N, dtype=torch.int32, device=dev)
    newp = torch.zeros(B, dtype=torch.int32, device=dev)
    def step():
        kv.kv_score(src, q, workspace=ws, **kw)
        kv.kv_select(item_score, item_pinned, pg, N, w.budget_items, keep, nk, workspace=ws_sel)
        kv.kv_compact_rerope(src, dst, keep, nk, B, pos, newp, renumber_base=0, rope_theta=w.rope_theta)

    def timed(run):
        times = []
        for i in range(warmup + steps):
            ewma.copy_(ewma0)
            clock.copy_(clock0)
            e = hip.create(2)
            hip.record(e[0], sh)
            run()
            hip.record(e[1], sh)
            torch.cuda.synchronize()
            if i >= warmup:
                times.append(hip.ms(e[0], e[1]))
        return sorted(times)

    # eager: the three calls from Python, so the host's enqueue time is part of the step
    times = timed(step)
    ref = [t.clone() for t in (keep, nk, dk, dv, newp, item_score)]
    # the same step captured once in a HIP graph (the library records no memset and
    # allocates nothing) and replayed: the device-side time without the Python calls
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cap):
        ewma.copy_(ewma0)
        clock.copy_(clock0)
        step()
    torch.cuda.current_stream(dev).wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    gtimes = timed(g.replay)
    same = all(torch.equal(a, b) for a, b in zip(ref, (keep, nk, dk, dv, newp, item_score)))
    if not same:
        raise RuntimeError(f"{name}: the graph replay differs from the eager step")
    med, gmed = times[len(times) // 2], gtimes[len(gtimes) // 2]
    return {"workload": name, "step_us_median": round(1e3 * med, 1), "step_us_min": round(1e3 * times[0], 1),
            "steps": steps, "KV_tokens_per_s": round(N / (med * 1e-3), 1),
            "graph_step_us_median": round(1e3 * gmed, 1), "graph_step_us_min": round(1e3 * gtimes[0], 1),
            "graph_KV_tokens_per_s": round(N / (gmed * 1e-3), 1),
            "note": "step_us: eager calls from Python (host enqueue included); graph_step_us: the same "
                    "launches replayed from one captured HIP graph, outputs identical"}


def oracle_baseline(name, layers=None, repeats=1):
    """The CPU oracle, untuned, on one workload: score (when the workload scores), select
    and compact, timed with perf_counter (best of `repeats`).  With `layers` only that many
    layers are scored and compacted and those parts are scaled to all layers."""
    import numpy as np
    import oracle as O
    import synth
    full = synth.workload(name)
    nl = layers or full.n_layers
    w = synth.workload(name, n_layers=nl)
    N = w.n_tokens
    k, v, bt = synth.kv_cache(w, seed=0)
    kl = k.float().double().numpy().reshape(nl, -1, w.n_kv_heads, w.head_dim)[:, :N]
    vl = v.float().double().numpy().reshape(nl, -1, w.n_kv_heads, w.head_dim)[:, :N]
    scale = full.n_layers / nl
    best = None
    for _ in range(repeats):
        t = {}
        t0 = time.perf_counter()
        if w.policy == "segment":
            keep = O.select_segment(N, w.segment_prefix, int(w.segment_frac * N), w.page_size)
            t1 = t0
        else:
            q = synth.window_queries(w, seed=0).float().double().numpy()
            kw = {}
            if w.policy == "memdecay":
                ewma, clock = synth.memdecay_state(w, seed=0)
                b_r, lam = synth.region_params(0)
                kw = dict(region=synth.regions(w, seed=0).numpy(), base_prio=b_r.double().numpy(),
                          decay_rate=lam.double().numpy(), rho=w.rho, alpha=w.alpha, tau=w.tau,
                          dt_steps=w.dt_steps, ewma=ewma.double().numpy(), clock=clock.numpy(),
                          pinned_regions=1)
            else:
                kw = dict(accum=np.zeros(N))
            if w.n_spans:
                sid, sbonus = synth.spans(w, seed=0)
                kw.update(span_id=sid.numpy(), span_bonus=sbonus.numpy())
            t0 = time.perf_counter()
            out = O.score_step(q, kl, policy=w.policy, n_sink=w.n_sink, n_recent=w.n_recent,
                               item_tokens=w.item_tokens, **kw)
            t1 = time.perf_counter()
            items, _ = O.select_items(out["item_score"], out["item_pinned"], w.budget_items)
            keep = O.expand_items(items, w.item_tokens, N)
        t2 = time.perf_counter()
        O.compact_rerope(kl, vl, keep, np.arange(N), 0, w.rope_theta)
        t3 = time.perf_counter()
        t = {"score_s": (t1 - t0) * scale, "select_s": t2 - t1, "compact_s": (t3 - t2) * scale}
        if best is None or sum(t.values()) < sum(best.values()):
            best = t
    total = sum(best.values())
    return {"workload": name, "kind": "oracle", "total_s": round(total, 4),
            "KV_tokens_per_s": round(N / total, 1),
            "parts_s": {a: round(b, 4) for a, b in best.items()},
            "sample": (f"{nl} of {full.n_layers} layers, score and compaction scaled x{scale:g}"
                       if nl != full.n_layers else "all layers") + f", best of {repeats}",
            "host_cpus": os.cpu_count()}


def cpu_baseline(w, layers):
    """The CPU oracle, untuned, on a bounded sample of the workload: attention mass and
    epilogue for `layers` of the 36 layers at full N, selection at full N, compaction of
    the full budget for the same layers; scaled to all layers."""
    import numpy as np
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    ws = synth.workload("qwen3-8b-n100k", n_layers=layers)
    k, v, _ = synth.kv_cache(ws, seed=0)
    q = synth.window_queries(ws, seed=0)
    span_id, span_bonus = synth.spans(ws, seed=0)
    kl = k.float().double().numpy().reshape(layers, -1, ws.n_kv_heads, ws.head_dim)[:, : ws.n_tokens]
    vl = v.float().double().numpy().reshape(layers, -1, ws.n_kv_heads, ws.head_dim)[:, : ws.n_tokens]
    t0 = time.perf_counter()
    out = O.score_step(q.float().double().numpy(), kl, policy="h2o", accum=np.zeros(ws.n_tokens),
                       span_id=span_id.numpy(), span_bonus=span_bonus.numpy(), n_sink=ws.n_sink,
                       n_recent=ws.n_recent)
    t1 = time.perf_counter()
    kept, _ = O.select_items(out["item_score"], out["item_pinned"], ws.budget_items)
    t2 = time.perf_counter()
    O.compact_rerope(kl, vl, kept, np.arange(ws.n_tokens), 0, ws.rope_theta)
    t3 = time.perf_counter()
    scale = w.n_layers / layers
    total = (t1 - t0) * scale + (t2 - t1) + (t3 - t2) * scale
    return {
        "value": w.n_tokens / total,
        "unit": "KV tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{layers} of {w.n_layers} layers at N={w.n_tokens} (score + compaction "
                   f"scaled x{scale:g}), selection at full N; measured {t3 - t0:.1f} s "
                   f"on {os.cpu_count()} host CPUs ({platform.processor() or platform.machine()})"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3-8b-n100k", help="workload name (the bench line: qwen3-8b-n100k)")
    ap.add_argument("--cpu-layers", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the rocprofv3 FETCH_SIZE / WRITE_SIZE runs (bench + copy calibration "
                         "in each directory) into profiles/traffic.json and print a table")
    ap.add_argument("--clock-summary", metavar="PMC_DIR",
                    help="print effective clock and MFMA busy share per kernel from a "
                         "rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES run, write the "
                         "scoring passes' shares to profiles/mfma_busy.json and exit")
    ap.add_argument("--extras", action="store_true",
                    help="time the rows beyond the headline step (single-pass and group-maximum "
                         "scoring, reference store, LRFU, tail compaction, offload, the Mistral "
                         "segment case and the 1M-token step) and print one JSON line")
    ap.add_argument("--segment", action="store_true",
                    help="only the Mistral-7B 131,072-token in-place segment case (5 runs after 1 "
                         "warm-up), one JSON line")
    ap.add_argument("--segment-remap", action="store_true",
                    help="only the same segment eviction through the page table (kv_compact_segment_remap, "
                         "with and without renumbering; 5 runs after 1 warm-up), one JSON line")
    ap.add_argument("--small", action="store_true",
                    help="only the two Qwen2.5-1.5B-shaped steps (eager and graph-replayed), one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reads 1 GiB, writes 1 GiB) three "
                         "times, to calibrate the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.pmc_summary:
        print(pmc_summary(args.pmc_summary[0], args.pmc_summary[1],
                          os.path.join(ROOT, "profiles", "traffic.json")))
        return
    if args.clock_summary:
        print(clock_summary(args.clock_summary, os.path.join(ROOT, "profiles", "mfma_busy.json")))
        return
    if args.extras:
        extras(oracle=not args.no_cpu)
        return
    if args.segment:
        print(json.dumps({"segment": segment_case(steps=5, warmup=1)}), flush=True)
        return
    if args.segment_remap:
        print(json.dumps({"segment_remap": segment_remap_case(steps=5, warmup=1)}), flush=True)
        return
    if args.small:
        print(json.dumps({f"step_{n}": small_config_step(n)
                          for n in ("qwen2.5-1.5b-1layer-n512", "qwen2.5-1.5b-n2048")}), flush=True)
        return
    if args.copy_calibration:
        a = torch.ones(1 << 29, dtype=torch.int16, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": a.numel() * 2, "launches": 3}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(across GPUs the per-token mass would be all-reduced over ranks)", file=sys.stderr)
        sys.exit(2)
    if args.workload != "qwen3-8b-n100k":
        print("only the qwen3-8b-n100k workload (Qwen3-8B, N=100K) is a bench line", file=sys.stderr)
        sys.exit(2)

    import compaction_kv_score_amd as kv
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.workload(args.workload)
    N, NL, HKV, HQ, D, W = w.n_tokens, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim, w.window
    B = w.budget_tokens
    print(f"[bench] generating {w.name}: {N} tokens x {w.kv_bytes_per_token} B", file=sys.stderr, flush=True)
    k, v, _ = synth.kv_cache(w, seed=0, device=dev)
    q = synth.window_queries(w, seed=0, device=dev)
    span_id, span_bonus = synth.spans(w, seed=0)
    span_id, span_bonus = span_id.to(dev), span_bonus.to(dev)
    accum = torch.zeros(N, device=dev)
    item_score = torch.zeros(N, device=dev)
    item_pinned = torch.zeros(N, dtype=torch.uint8, device=dev)
    keep = torch.zeros(B, dtype=torch.int32, device=dev)
    n_keep = torch.zeros(1, dtype=torch.int64, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    old_pos = torch.arange(N, dtype=torch.int32, device=dev)
    new_pos = torch.zeros(B, dtype=torch.int32, device=dev)
    dst_k = torch.zeros((NL, B // w.page_size, w.page_size, HKV, D), dtype=torch.bfloat16, device=dev)
    dst_v = torch.zeros_like(dst_k)
    dst_accum = torch.zeros(B, device=dev)
    dst_span = torch.zeros(B, dtype=torch.int32, device=dev)
    src = kv.PagedCache(k, v, N)
    dst = kv.PagedCache(dst_k, dst_v, B)
    score_kw = dict(policy="h2o", window=W, item_tokens=1, accum=accum, span_id=span_id,
                    span_bonus=span_bonus, n_sink=w.n_sink, n_recent=w.n_recent,
                    item_score=item_score, item_pinned=item_pinned)
    ws_score = torch.empty(kv.kv_score_workspace_size(src, q, **score_kw), dtype=torch.uint8, device=dev)
    ws_sel = torch.empty(kv.kv_select_workspace_size(N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    hip = HipEvents()
    n_ev = 8

    def step(ev=None, edge=None):
        """One step.  ev: 7 events recorded between the stages (kv_score records the first
        five), for the per-kernel times.  edge: 2 events recorded before and after the step
        only; every event recorded between two launches holds the next one back by about
        5 us, so the step time is taken from steps that record none inside."""
        if edge is not None:
            hip.record(edge[0], sh)
        kv.kv_score(src, q, workspace=ws_score,
                    stage_events=None if ev is None else ctypes.cast(ev, ctypes.c_void_p), **score_kw)
        kv.kv_select(item_score, item_pinned, 1, N, B, keep, n_keep, status, workspace=ws_sel)
        if ev is not None:
            hip.record(ev[5], sh)
        kv.kv_compact_rerope(src, dst, keep, n_keep, B, old_pos, new_pos, renumber_base=0,
                             rope_theta=w.rope_theta, limit=w.limit,
                             meta=[(accum, dst_accum), (span_id, dst_span)])
        if ev is not None:
            hip.record(ev[6], sh)
        if edge is not None:
            hip.record(edge[1], sh)

    def median(xs):
        xs = sorted(xs)
        m = len(xs) // 2
        return xs[m] if len(xs) % 2 else 0.5 * (xs[m - 1] + xs[m])

    # every step scores the same state: the H2O accumulator is restored from a copy before
    # each step, outside the step's events
    accum0 = accum.clone()
    warm = hip.create(n_ev)
    for _ in range(args.warmup):
        accum.copy_(accum0)
        step(ev=warm)
    torch.cuda.synchronize()
    edges = [hip.create(2) for _ in range(args.steps)]
    events = [hip.create(n_ev) for _ in range(args.steps)]
    torch.cuda.synchronize()
    # the timed steps (events only around each step), each followed by one step with events
    # between the stages for the per-kernel times, so that both see the same conditions
    t0 = time.perf_counter()
    for s in range(args.steps):
        accum.copy_(accum0)
        step(edge=edges[s])
        accum.copy_(accum0)
        step(ev=events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_wall = (t1 - t0) * 1e3 / args.steps / 2
    step_ms = sorted(hip.ms(e[0], e[1]) for e in edges)
    ms_step = median(step_ms)
    staged_ms = median([hip.ms(e[0], e[6]) for e in events])
    assert int(status.item()) == 0 and int(n_keep.item()) == B

    def avg(a, b):
        return sum(hip.ms(e[a], e[b]) for e in events) / len(events)

    t_lse, t_comb, t_mass, t_epi = avg(0, 1), avg(1, 2), avg(2, 3), avg(3, 4)
    t_sel, t_cmp = avg(4, 5), avg(5, 6)
    k_bytes = NL * N * HKV * D * 2
    q_bytes = NL * W * HQ * D * 2
    flops = 2.0 * NL * HQ * W * N * D
    cmp_bytes = 2 * B * w.kv_bytes_per_token
    kern = {
        "lse_pass": {"ms": t_lse, "bytes": k_bytes + q_bytes, "flops": flops},
        "mass_pass": {"ms": t_mass, "bytes": k_bytes + q_bytes, "flops": flops},
        "compact_rerope": {"ms": t_cmp, "bytes": cmp_bytes, "flops": 0.0},
    }
    for name, r in kern.items():
        r["gbs"] = r["bytes"] / (r["ms"] * 1e-3) / 1e9
        r["hbm_frac"] = r["gbs"] / HBM_PEAK_GBS
        r["mfma_frac"] = r["flops"] / (r["ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS
    dom = max(("lse_pass", "mass_pass"), key=lambda n: kern[n]["ms"])
    traffic = measured_traffic(dom)
    result = {
        "metric": "KV tokens scored+evicted+compacted/sec (all layers)",
        "value": N / (ms_step * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_note": "median over the timed steps of each step's HIP-event time (events before "
                            "and after the step only, one stream); state restored before every step, "
                            "outside it. Each timed step is followed by one with events between the "
                            "stages, which add about 5 us per stage boundary: stages_ms, roofline and "
                            "ms_per_step_staged come from those",
        "ms_per_step_wall_mean": ms_wall,
        "ms_per_step_wall_note": "wall clock over the timed and the staged steps, per step",
        "ms_per_step_min_max": [step_ms[0], step_ms[-1]],
        "ms_per_step_staged": staged_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "n_layers": NL, "q_heads": HQ, "kv_heads": HKV, "head_dim": D,
                   "n_tokens": N, "window": W, "budget_tokens": B, "page_size": w.page_size,
                   "policy": "h2o+foresight", "renumber_limit": w.limit},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(kern[dom]["gbs"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kern[dom]["hbm_frac"], 4),
                     "traffic": traffic,
                     "mfma_tflops": round(kern[dom]["flops"] / (kern[dom]["ms"] * 1e-3) / 1e12, 1),
                     "mfma_frac": round(kern[dom]["mfma_frac"], 4),
                     "mfma_busy_counter": measured_mfma_busy()},
        "stages_ms": {"lse_pass": round(t_lse, 4), "lse_combine": round(t_comb, 4),
                      "mass_pass": round(t_mass, 4), "epilogue": round(t_epi, 4),
                      "select": round(t_sel, 4), "compact_rerope": round(t_cmp, 4)},
        "compact_rerope": {"achieved": round(kern["compact_rerope"]["gbs"], 1), "unit": "GB/s",
                           "frac": round(kern["compact_rerope"]["hbm_frac"], 4)},
        # the two stated targets, checked on this run's own figures
        "targets": {
            "compaction_hbm_frac": {"min": 0.70, "value": round(kern["compact_rerope"]["hbm_frac"], 4),
                                    "met": kern["compact_rerope"]["hbm_frac"] >= 0.70},
            "scoring_mfma_frac": {"min": 0.50,
                                  "value": round(min(kern["lse_pass"]["mfma_frac"], kern["mass_pass"]["mfma_frac"]), 4),
                                  "met": min(kern["lse_pass"]["mfma_frac"], kern["mass_pass"]["mfma_frac"]) >= 0.50,
                                  "note": "useful MFMA flops per scoring pass over the 2.5 PF bf16 peak"},
        },
    }
    print(f"[bench] {ms_step:.3f} ms/step ({staged_ms:.3f} with stage events); stages {result['stages_ms']}",
          file=sys.stderr, flush=True)
    del k, v, dst_k, dst_v, ws_score
    torch.cuda.empty_cache()
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_layers)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
