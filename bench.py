#!/usr/bin/env python3
"""Benchmark of indexer-selected sparse attention on one MI355X.

One step = one causal prefill of a 131072-token sequence (indexer scores of every causal
pair, per-query top-2048, attention over the selected rows) plus one decode step of 64
sequences at 131072 tokens of paged context (indexer over the whole context, top-2048,
attention over the selected rows of the paged cache).  Inputs are seeded synthetic data
resident in HBM before timing starts.

Prints one JSON line: `value` is prefill tokens/s at 128K context; decode tokens/s, the
per-kernel times (HIP events the library records around each launch on the launch stream),
the roofline of the dominant kernel (the fused prefill indexer / top-k) and of the decode
kernels, the index projections, the two-tier (block -> token) selection variant of both
steps, a chunked prefill against the paged caches, the acceptance-rate statistic, the RL-rollout
decode sweep (256 sequences, context 1K..32K, per-sequence budgets), cold-cache medians of both calls
(a 512 MiB write before each timed call), and the CPU oracle's throughput on a bounded sample ride along.

HBM traffic per launch comes from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this script,
calibrated on the 1 GiB copy it performs after the warm-up, and stored in
profiles/traffic.json together with a hash of the kernel sources; it is reported only while
the sources still match.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "decode tokens/s and prefill tokens/s at 128K ctx, top-k=2048; % of MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CALIBRATION_BYTES = 1 << 30  # the plain copy whose counters calibrate FETCH_SIZE / WRITE_SIZE
CSRC = os.path.join(ROOT, "indexer_selected_sparse_scores_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prefill-len", type=int, default=131072)
    ap.add_argument("--decode-batch", type=int, default=64)
    ap.add_argument("--decode-ctx", type=int, default=131072)
    ap.add_argument("--topk", type=int, default=2048)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample (0 disables it)")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event timing")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak microbenchmarks")
    ap.add_argument("--no-projections", action="store_true", help="skip the index-projection measurement")
    ap.add_argument("--no-two-tier", action="store_true", help="skip the two-tier (block -> token) measurement")
    ap.add_argument("--no-chunk", action="store_true", help="skip the chunked-prefill (paged query rows) measurement")
    ap.add_argument("--no-acceptance", action="store_true", help="skip the acceptance-rate measurement")
    ap.add_argument("--no-rl-sweep", action="store_true", help="skip the RL-rollout decode sweep")
    ap.add_argument("--no-graph", action="store_true", help="skip the decode step replayed from a HIP graph")
    ap.add_argument("--no-c1", action="store_true", help="skip the 8192-token prefill workload")
    ap.add_argument("--no-c2", action="store_true", help="skip the ragged decode workload (contexts 16K..64K)")
    ap.add_argument("--main-only", action="store_true",
                    help="time the step alone (no projections, two-tier, chunked-prefill or acceptance legs)")
    ap.add_argument("--ingest-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from rocprofv3 FETCH_SIZE and WRITE_SIZE counter files of a "
                         "--main-only run (no GPU needed)")
    ap.add_argument("--chunk", type=int, default=4096, help="chunked prefill: new tokens at the end of the context")
    ap.add_argument("--block-size", type=int, default=64, help="two-tier selection: tokens per block")
    ap.add_argument("--n-blocks", type=int, default=64, help="two-tier selection: blocks kept per query")
    return ap.parse_args()


def source_hash(files):
    """sha256 over the code of `files` (line comments, trailing blanks and empty lines
    dropped, so that an edit of comments alone keeps stored counters valid)."""
    h = hashlib.sha256()
    for f in sorted(files):
        with open(os.path.join(CSRC, f)) as fh:
            code = [ln.split("//", 1)[0].rstrip() for ln in fh]
        h.update(f.encode() + b"\0" + "\n".join(ln for ln in code if ln).encode())
    return h.hexdigest()


def stored_traffic(kernel: str):
    """Calibrated HBM bytes per launch of `kernel` from profiles/traffic.json, or None when
    absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh).get(kernel)
    if not rec or rec.get("source_sha256") != source_hash(rec["sources"]):
        return None
    return rec["bytes_per_launch"]


# Kernel -> the source files its code comes from (the stored traffic is valid while they are unchanged).
KERNEL_SOURCES = {
    "indexer_topk_prefill_kernel": ["prefill_topk.hip", "topk_device.hpp", "sa_device.hpp", "sa_internal.hpp"],
    "attn_latent_mfma_kernel": ["attention.hip", "sa_device.hpp", "sa_internal.hpp"],
    "indexer_decode_kernel": ["decode.hip", "topk_device.hpp", "sa_device.hpp", "sa_internal.hpp"],
    "decode_topk_kernel": ["decode.hip", "topk_device.hpp", "sa_device.hpp", "sa_internal.hpp"],
    "attn_decode_lds_kernel": ["attention.hip", "sa_device.hpp", "sa_internal.hpp"],
    "attn_merge_kernel": ["attention.hip", "sa_device.hpp", "sa_internal.hpp"],
}


def ingest_traffic(fetch_csv: str, write_csv: str):
    """profiles/traffic.json from the FETCH_SIZE and WRITE_SIZE counter files of two `--main-only`
    runs: each counter (KiB per dispatch) is divided by what it reads for the 1 GiB calibration copy
    (the dispatch right after the 1 GiB fill that creates its source), then averaged per kernel."""
    import csv
    import re

    def load(path):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        cal = None
        for i, r in enumerate(rows):
            if "FillFunctor<unsigned char>" in r["Kernel_Name"] and int(r["Grid_Size"]) * 16 >= CALIBRATION_BYTES:
                cal = float(rows[i + 1]["Counter_Value"]) * 1024 / CALIBRATION_BYTES
        if cal is None:
            raise SystemExit(f"{path}: no calibration copy found")
        per = {}
        for r in rows:
            m = re.search(r"sa::\(anonymous namespace\)::(\w+)", r["Kernel_Name"])
            if m and m.group(1) in KERNEL_SOURCES:
                per.setdefault(m.group(1), []).append(float(r["Counter_Value"]))
        return cal, {k: sum(v) / len(v) for k, v in per.items()}

    f_cal, fetch = load(fetch_csv)
    w_cal, write = load(write_csv)
    out = {}
    for k in KERNEL_SOURCES:
        if k not in fetch or k not in write:
            continue
        rd = fetch[k] * 1024 / f_cal
        wr = write[k] * 1024 / w_cal
        out[k] = {"sources": KERNEL_SOURCES[k], "source_sha256": source_hash(KERNEL_SOURCES[k]),
                  "fetch_size_kib": fetch[k], "write_size_kib": write[k], "read_bytes": int(rd),
                  "write_bytes": int(wr), "bytes_per_launch": int(rd + wr),
                  "calibration": {"copy_bytes": CALIBRATION_BYTES, "fetch_factor": f_cal, "write_factor": w_cal}}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    for k, v in out.items():
        print(f"{k}: read {v['read_bytes'] / 1e9:.4g} GB, write {v['write_bytes'] / 1e9:.4g} GB per launch")
    print(f"wrote {path}")


def main():
    args = parse()
    if args.ingest_traffic:
        ingest_traffic(*args.ingest_traffic)
        return
    if args.main_only:
        args.no_projections = args.no_two_tier = args.no_chunk = args.no_acceptance = args.no_rl_sweep = True
        args.no_graph = args.no_c1 = args.no_c2 = True
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build runs the per-GPU share of the path and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import indexer_selected_sparse_scores_amd as sa
    from indexer_selected_sparse_scores_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = "cuda"
    L, B, N, K = args.prefill_len, args.decode_batch, args.decode_ctx, args.topk

    pre_wl = inputs.small(inputs.WORKLOADS["prefill_128k"], L=L, topk=K)
    dec_wl = inputs.small(inputs.WORKLOADS["decode_b64_128k"], B=B, ctx_range=(N, N), topk=K)
    cfg = inputs.library_config(pre_wl, max_topk=K)

    log(f"[bench] generating prefill inputs L={L}")
    P = inputs.prefill_inputs(pre_wl, dev)
    log(f"[bench] generating decode inputs B={B} ctx={N}")
    D = inputs.decode_inputs(dec_wl, dev)
    torch.cuda.synchronize()

    h_pre = sa.Handle(cfg)
    h_dec = sa.Handle(cfg)
    s = cfg
    out_p = torch.empty((L, s.n_heads, s.d_v), device=dev)
    lse_p = torch.empty((L, s.n_heads), device=dev)
    idx_p = torch.empty((L, K), device=dev, dtype=torch.int32)
    ws_p = sa.workspace(h_pre, sa.SA_OP_PREFILL, L)
    out_d = torch.empty((B, s.n_heads, s.d_v), device=dev)
    lse_d = torch.empty((B, s.n_heads), device=dev)
    idx_d = torch.empty((B, K), device=dev, dtype=torch.int32)
    ws_d = sa.workspace(h_dec, sa.SA_OP_DECODE, B, D["max_ctx"])

    def prefill():
        sa.sparse_attn_prefill(h_pre, P["q"], P["k"], None, P["q_idx"], P["w"], P["k_idx"], K,
                               out_p, lse_p, idx_p, ws_p)

    def decode():
        sa.sparse_attn_decode(h_dec, D["q"], D["q_idx"], D["w"], D["kv_pages"], None, D["kidx_pages"],
                              D["block_table"], D["ctx_len"], D["topk"], D["max_ctx"], out_d, lse_d,
                              idx_d, ws_d)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()
    sa.sparse_attn_check(h_pre)
    sa.sparse_attn_check(h_dec)

    # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE calibrate the traffic counters
    cal_src = torch.ones(CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    peaks = None if args.no_peaks else measured_peaks(h_pre, torch)

    # K timed steps, each after a 512 MiB write that evicts the L2 and Infinity Cache (the write is outside
    # the timed span): per-step prefill and decode times from events on the stream, and per-kernel times of
    # the step from the events the library records around each launch.  Medians over the K steps.
    profile = not args.no_profile
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps)]
    step_kern = []
    log(f"[bench] timing {args.steps} steps (each after a {FLUSH_BYTES >> 20} MiB cache flush)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush_buf.fill_(i & 0xFF)
        if profile:
            sa.sparse_attn_profile(h_pre, True)
            sa.sparse_attn_profile(h_dec, True)
        ev[3 * i].record()
        prefill()
        ev[3 * i + 1].record()
        decode()
        ev[3 * i + 2].record()
        if profile:
            step_kern.append((sa.sparse_attn_profile_read(h_pre), sa.sparse_attn_profile_read(h_dec)))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if profile:
        sa.sparse_attn_profile(h_pre, False)
        sa.sparse_attn_profile(h_dec, False)
    pre_steps = [ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(args.steps)]
    dec_steps = [ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(args.steps)]
    pre_ms, dec_ms = median(pre_steps), median(dec_steps)
    step_ms = median([a + b for a, b in zip(pre_steps, dec_steps)])
    sa.sparse_attn_check(h_pre)
    sa.sparse_attn_check(h_dec)
    log(f"[bench] cold-step medians: prefill {pre_ms:.3f} ms, decode {dec_ms:.4f} ms (wall {wall:.2f} s)")

    # the same steps back to back, without flushes (warm caches), for comparison
    ev_w = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev_w[0].record()
    for _ in range(args.steps):
        prefill()
    ev_w[1].record()
    for _ in range(args.steps):
        decode()
    ev_w[2].record()
    torch.cuda.synchronize()
    warm = {"prefill_ms_mean": round(ev_w[0].elapsed_time(ev_w[1]) / args.steps, 4),
            "decode_ms_mean": round(ev_w[1].elapsed_time(ev_w[2]) / args.steps, 4)}
    del flush_buf

    # algorithmic work (per step)
    pairs = L * (L + 1) // 2
    flop_per_pair = 2 * s.n_idx_heads * s.d_idx
    idx_flops = pairs * flop_per_pair
    ctx_total = int(D["ctx_np"].sum())
    key_bytes = s.d_idx * 2
    dec_idx_bytes = ctx_total * key_bytes
    sel_rows = int(np.minimum(D["ctx_np"], K).sum())
    row_bytes = s.d_qk * 2
    dec_gather_bytes = sel_rows * row_bytes

    kernels = {}
    roofline = roofline_dec_idx = roofline_dec_attn = None
    if profile:
        kern_med = {}
        for j, name in enumerate(("prefill", "decode")):
            for kind in sa.KERNEL_KINDS:
                per_step = [k[j].get(kind, (0.0, 0)) for k in step_kern]
                if per_step and per_step[0][1]:
                    kern_med[(name, kind)] = median([ms for ms, _ in per_step])
                    kernels[f"{name}.{kind}"] = {"launches_per_step": per_step[0][1],
                                                 "ms_per_step_median": round(kern_med[(name, kind)], 5)}
        launches = lambda name, kind: kernels[f"{name}.{kind}"]["launches_per_step"]
        if ("prefill", "indexer") in kern_med:
            ms = kern_med[("prefill", "indexer")] / launches("prefill", "indexer")
            roofline = mfma_roofline("indexer_topk_prefill_kernel", idx_flops, ms,
                                     f"{idx_flops:.4g} flop = {pairs} causal (t,s) pairs x {flop_per_pair} flop "
                                     f"(2 H_I d_I)", peaks)
            roofline["traffic"] = stored_traffic("indexer_topk_prefill_kernel")
        if ("decode", "indexer") in kern_med:
            ms = kern_med[("decode", "indexer")] / launches("decode", "indexer")
            roofline_dec_idx = hbm_roofline("indexer_decode_kernel", dec_idx_bytes, ms,
                                            f"{dec_idx_bytes} B = {ctx_total} cached tokens x {key_bytes} B of "
                                            f"index key", peaks)
            roofline_dec_idx["traffic"] = stored_traffic("indexer_decode_kernel")
        if ("decode", "attention") in kern_med:
            ms = kern_med[("decode", "attention")] / launches("decode", "attention")
            roofline_dec_attn = hbm_roofline("attn_decode_lds_kernel (paged decode gather)", dec_gather_bytes, ms,
                                             f"{dec_gather_bytes} B = {sel_rows} selected rows x {row_bytes} B "
                                             f"latent row", peaks)
            roofline_dec_attn["traffic"] = stored_traffic("attn_decode_lds_kernel")
        # the whole decode step against HBM: index keys + selected rows over the step's median time
        dec_all = dec_idx_bytes + dec_gather_bytes
        decode_step_roofline = hbm_roofline("whole decode step (reset, paged indexer, top-k, gather, merge)", dec_all,
                                            dec_ms, f"{dec_all} B = index keys of every cached token + the "
                                                    f"selected latent rows", peaks)
    else:
        decode_step_roofline = None

    graph = None if args.no_graph else measure_decode_graph(decode, args.steps, torch)
    c1 = None if args.no_c1 else measure_prefill_8k(cfg, args, peaks, torch)
    c2 = None if args.no_c2 else measure_decode_ragged(cfg, args, peaks, torch)

    projections = None if args.no_projections else measure_projections(h_pre, P, L, args.steps, torch)
    two_tier = None if args.no_two_tier else measure_two_tier(cfg, P, D, L, K, args, torch)
    chunk = None if args.no_chunk else measure_chunk(cfg, P, D, K, args, torch)
    acceptance = None if args.no_acceptance else measure_acceptance(cfg, args, torch)
    rl_sweep = None if args.no_rl_sweep else measure_rl_sweep(args, torch)

    cpu = cpu_dec = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(P, pre_wl, K, args.cpu_seconds)
        cpu_dec = cpu_baseline_decode(D, dec_wl, K, args.cpu_seconds / 3)

    result = {
        "metric": METRIC,
        "value": round(L / (pre_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"prefill L={L} (prefill_128k) + paged decode B={B} at ctx={N} "
                               f"(decode_b64_128k)", "topk": K,
                   "index_heads": s.n_idx_heads, "d_index": s.d_idx, "heads": s.n_heads,
                   "d_qk": s.d_qk, "d_v": s.d_v, "page_size": s.page_size,
                   "timing": f"median over {args.steps} steps, each after a {FLUSH_BYTES >> 20} MiB cache flush"},
        "prefill_tokens_per_s": round(L / (pre_ms * 1e-3), 1),
        "decode_tokens_per_s": round(B / (dec_ms * 1e-3), 1),
        "prefill_ms": round(pre_ms, 4),
        "decode_ms": round(dec_ms, 4),
        "roofline": roofline,
        "roofline_decode_indexer": roofline_dec_idx,
        "roofline_decode_gather": roofline_dec_attn,
        "roofline_decode_step": decode_step_roofline,
        "kernels": kernels,
        "warm_cache": warm,
        "decode_graph": graph,
        "prefill_8k": c1,
        "decode_ragged": c2,
        "peaks_measured": peaks,
        "projections": projections,
        "two_tier": two_tier,
        "chunked_prefill": chunk,
        "acceptance": acceptance,
        "rl_sweep": rl_sweep,
        "cpu_baseline": cpu,
        "cpu_baseline_decode": cpu_dec,
    }
    print(json.dumps(result), flush=True)
    h_pre.close()
    h_dec.close()


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def mfma_roofline(kernel, flops, ms, what, peaks):
    tf = flops / (ms * 1e-3) / 1e12
    rf = {"kernel": kernel, "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
          "frac": round(tf / PEAK_BF16_TFLOPS, 4), "ms": round(ms, 5), "algorithmic_per_launch": what}
    if peaks and peaks.get("mfma_loop_tflops"):
        rf["frac_of_measured"] = round(tf / peaks["mfma_loop_tflops"], 4)
        rf["measured_peak"] = "mfma_loop_tflops"
    return rf


def hbm_roofline(kernel, nbytes, ms, what, peaks):
    gbs = nbytes / (ms * 1e-3) / 1e9
    rf = {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
          "frac": round(gbs / PEAK_HBM_GBS, 4), "ms": round(ms, 5), "algorithmic_per_launch": what}
    if peaks and peaks.get("stream_read_gbs"):
        rf["frac_of_measured"] = round(gbs / peaks["stream_read_gbs"], 4)
        rf["measured_peak"] = "stream_read_gbs"
    return rf


def cold_runs(fn, reps, torch, profile_handle=None):
    """fn timed `reps` times, each alone after a 512 MiB write that evicts the L2 and Infinity Cache (the write
    is outside the timed span); returns the per-call times and, with a handle, its per-kernel times per call."""
    import indexer_selected_sparse_scores_amd as sa
    buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    times, kerns = [], []
    for i in range(reps):
        buf.fill_(i & 0xFF)
        if profile_handle is not None:
            sa.sparse_attn_profile(profile_handle, True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
        if profile_handle is not None:
            kerns.append(sa.sparse_attn_profile_read(profile_handle))
    if profile_handle is not None:
        sa.sparse_attn_profile(profile_handle, False)
    del buf
    return times, kerns


def kernel_medians(kerns):
    """{kind: median ms per call} over calls (each call's summed launches of that kind)."""
    out = {}
    for kind in (kerns[0] if kerns else {}):
        if kerns[0][kind][1]:
            out[kind] = median([k[kind][0] for k in kerns])
    return out


def measure_decode_graph(decode, reps, torch):
    """The benchmark's decode step captured once in a HIP graph and replayed (not part of `value`): the same
    kernels without the per-launch host work between them; median of cold replays."""
    log("[bench] decode step replayed from a HIP graph")
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        decode()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=st):
        decode()
    g.replay()
    torch.cuda.synchronize()
    times, _ = cold_runs(g.replay, max(reps, 5), torch)
    del g
    return {"ms_median": round(median(times), 4), "reps": len(times),
            "note": "one replay per timed call, each after a 512 MiB cache flush"}


def measure_prefill_8k(cfg, args, peaks, torch):
    """The 8192-token prefill workload (prefill_8k: one sequence, k = 2048; not part of `value`), cold median
    over the steps, with the roofline of the fused indexer."""
    import indexer_selected_sparse_scores_amd as sa
    from indexer_selected_sparse_scores_amd import inputs
    wl = inputs.WORKLOADS["prefill_8k"]
    L, K = wl.L, wl.topk
    log(f"[bench] prefill_8k L={L}")
    P8 = inputs.prefill_inputs(wl, "cuda")
    s = cfg
    with sa.Handle(inputs.library_config(wl, max_topk=K)) as h:
        out = torch.empty((L, s.n_heads, s.d_v), device="cuda")
        idx = torch.empty((L, K), device="cuda", dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_PREFILL, L)
        run = lambda: sa.sparse_attn_prefill(h, P8["q"], P8["k"], None, P8["q_idx"], P8["w"], P8["k_idx"], K, out,
                                             None, idx, ws)
        for _ in range(2):
            run()
        torch.cuda.synchronize()
        sa.sparse_attn_check(h)
        times, kerns = cold_runs(run, max(args.steps, 5), torch, h)
        sa.sparse_attn_check(h)
        km = kernel_medians(kerns)
        del out, idx, ws
    del P8
    torch.cuda.empty_cache()
    pairs = L * (L + 1) // 2
    flops = pairs * 2 * s.n_idx_heads * s.d_idx
    ms = median(times)
    res = {"workload": f"prefill_8k: one sequence, L={L}, top-{K}", "ms_median": round(ms, 4),
           "tokens_per_s": round(L / (ms * 1e-3), 1), "kernels_ms_median": {k: round(v, 5) for k, v in km.items()}}
    if km.get("indexer"):
        res["roofline"] = mfma_roofline("indexer_topk_prefill_kernel", flops, km["indexer"],
                                        f"{flops:.4g} flop = {pairs} causal pairs x {2 * s.n_idx_heads * s.d_idx} flop",
                                        peaks)
    return res


def measure_decode_ragged(cfg, args, peaks, torch):
    """The ragged decode workload (decode_b64: 64 sequences, contexts uniform in [16K, 64K], k = 2048; not part of
    `value`), cold median over the steps, with the rooflines of the decode indexer, the gather and the step."""
    import numpy as np

    import indexer_selected_sparse_scores_amd as sa
    from indexer_selected_sparse_scores_amd import inputs
    wl = inputs.WORKLOADS["decode_b64"]
    log("[bench] decode_b64: B=64, contexts uniform in [16384, 65536]")
    D2 = inputs.decode_inputs(wl, "cuda")
    B, K = D2["q"].shape[0], wl.topk
    s = cfg
    with sa.Handle(inputs.library_config(wl, max_topk=K)) as h:
        out = torch.empty((B, s.n_heads, s.d_v), device="cuda")
        idx = torch.empty((B, K), device="cuda", dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_DECODE, B, D2["max_ctx"])
        run = lambda: sa.sparse_attn_decode(h, D2["q"], D2["q_idx"], D2["w"], D2["kv_pages"], None, D2["kidx_pages"],
                                            D2["block_table"], D2["ctx_len"], D2["topk"], D2["max_ctx"], out, None,
                                            idx, ws)
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        sa.sparse_attn_check(h)
        times, kerns = cold_runs(run, max(args.steps, 9), torch, h)
        sa.sparse_attn_check(h)
        km = kernel_medians(kerns)
        del out, idx, ws
    ctx = D2["ctx_np"].astype(np.int64)
    del D2
    torch.cuda.empty_cache()
    idx_bytes = int(ctx.sum()) * s.d_idx * 2
    gather_bytes = int(np.minimum(ctx, K).sum()) * s.d_qk * 2
    ms = median(times)
    res = {"workload": f"decode_b64: {B} sequences, contexts {int(ctx.min())}..{int(ctx.max())} (uniform in "
                       f"[16384, 65536]), top-{K}, paged 64-token blocks", "ms_median": round(ms, 4),
           "tokens_per_s": round(B / (ms * 1e-3), 1), "kernels_ms_median": {k: round(v, 5) for k, v in km.items()},
           "roofline_step": hbm_roofline("whole decode step", idx_bytes + gather_bytes, ms,
                                         f"{idx_bytes + gather_bytes} B = index keys of every cached token + the "
                                         f"selected latent rows", peaks)}
    if km.get("indexer"):
        res["roofline_indexer"] = hbm_roofline("indexer_decode_kernel", idx_bytes, km["indexer"],
                                               f"{idx_bytes} B of index keys", peaks)
    if km.get("attention"):
        res["roofline_gather"] = hbm_roofline("attn_decode_lds_kernel", gather_bytes, km["attention"],
                                              f"{gather_bytes} B of selected latent rows", peaks)
    return res


FLUSH_BYTES = 512 << 20  # twice the MI355X's 256 MB Infinity Cache


def measure_projections(h, P, L, steps, torch):
    """The index projections at the prefill shape (not part of `value`): q_idx and w from the L
    attention query rows (one MFMA GEMM over [W_iq; W_w]) and k_idx from the L latent rows, with
    synthetic N(0, 1/width) bf16 weights."""
    import indexer_selected_sparse_scores_amd as sa
    dev = "cuda"
    s = h.cfg
    kq = s.n_heads * s.d_qk
    kk = s.n_kv_heads * s.d_qk
    g = torch.Generator(device=dev).manual_seed(20261202)
    W_iq = (torch.randn((s.n_idx_heads * s.d_idx, kq), generator=g, device=dev) * kq ** -0.5).to(torch.bfloat16)
    W_w = (torch.randn((s.n_idx_heads, kq), generator=g, device=dev) * kq ** -0.5).to(torch.bfloat16)
    W_ik = (torch.randn((s.d_idx, kk), generator=g, device=dev) * kk ** -0.5).to(torch.bfloat16)
    q_idx = torch.empty((L, s.n_idx_heads, s.d_idx), dtype=torch.bfloat16, device=dev)
    w = torch.empty((L, s.n_idx_heads), dtype=torch.float32, device=dev)
    k_idx = torch.empty((L, s.d_idx), dtype=torch.bfloat16, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    log(f"[bench] index projections L={L}")
    q_ms = timed(lambda: sa.indexer_project_q(h, P["q"], W_iq, W_w, q_idx, w))
    k_ms = timed(lambda: sa.indexer_project_k(h, P["k"], W_ik, k_idx))
    sa.sparse_attn_check(h)
    q_flop = 2.0 * L * kq * (s.n_idx_heads * s.d_idx + s.n_idx_heads)
    k_bytes = L * (2 * kk + 2 * s.d_idx) + 2 * s.d_idx * kk
    q_tf = q_flop / (q_ms * 1e-3) / 1e12
    k_gbs = k_bytes / (k_ms * 1e-3) / 1e9
    return {
        "query": {"ms": round(q_ms, 4), "bound": "mfma", "achieved": round(q_tf, 2), "peak": PEAK_BF16_TFLOPS,
                  "unit": "TFLOP/s", "frac": round(q_tf / PEAK_BF16_TFLOPS, 4),
                  "algorithmic_per_launch": f"{q_flop:.4g} flop = {L} rows x 2 x {kq} x "
                                            f"({s.n_idx_heads * s.d_idx} + {s.n_idx_heads}) (q_idx and w)"},
        "key": {"ms": round(k_ms, 4), "bound": "hbm", "achieved": round(k_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(k_gbs / PEAK_HBM_GBS, 4),
                "algorithmic_per_launch": f"{k_bytes} B = {L} rows x ({2 * kk} B latent row read + "
                                          f"{2 * s.d_idx} B index key written) + W_ik"},
    }


def measure_two_tier(cfg, P, D, L, K, args, torch):
    """The two-tier (block -> token) selection on the same inputs (not part of `value`): blocks of
    --block-size tokens, --n-blocks kept per query, top-K inside them.  Decode: the paged indexer,
    then one selection workgroup per sequence over its scores (4 B per cached token read back), then
    the same attention.  Prefill (blocks of >= 64 tokens): the fused indexer writes each row's best score
    per 64-key tile, one workgroup per row keeps the best blocks and rescores only their tokens, then the
    same attention."""
    import numpy as np

    import indexer_selected_sparse_scores_amd as sa
    dev = "cuda"
    bs, nb = args.block_size, args.n_blocks
    s = cfg
    B = D["q"].shape[0]
    res = {"block_size": bs, "n_blocks": nb, "topk": K}

    def timed(h, fn, reps):
        fn()
        torch.cuda.synchronize()
        sa.sparse_attn_check(h)
        sa.sparse_attn_profile(h, True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        kern = sa.sparse_attn_profile_read(h)
        sa.sparse_attn_profile(h, False)
        sa.sparse_attn_check(h)
        per = {k: round(ms / reps, 4) for k, (ms, n) in kern.items() if n}
        return e0.elapsed_time(e1) / reps, per

    with sa.Handle(cfg) as h:
        out = torch.empty((B, s.n_heads, s.d_v), device=dev)
        idx = torch.empty((B, K), device=dev, dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_DECODE_BLOCKS, B, D["max_ctx"])
        log(f"[bench] two-tier decode B={B} block={bs} n_blocks={nb}")
        ms, per = timed(h, lambda: sa.sparse_attn_decode_blocks(
            h, D["q"], D["q_idx"], D["w"], D["kv_pages"], None, D["kidx_pages"], D["block_table"], D["ctx_len"],
            D["topk"], D["max_ctx"], bs, nb, out, None, idx, ws), args.steps)
        ctx = D["ctx_np"].astype(np.int64)
        # per sequence: one page-maximum key per 64 tokens (bs >= 64; else every score), the scores of
        # the kept blocks' tokens, and the k index slots written
        span = 64 if bs >= 64 else 1
        cand = np.minimum(ctx, nb * bs)
        sel_bytes = int((-(-ctx // span) * 4 + cand * 4 + K * 4).sum())
        sel_ms = per.get("topk")
        res["decode"] = {"ms": round(ms, 4), "tokens_per_s": round(B / (ms * 1e-3), 1), "kernels_ms": per}
        if sel_ms:
            gbs = sel_bytes / (sel_ms * 1e-3) / 1e9
            # a few KB per sequence through dependent phases (block keys, radix selects): bound by their
            # latency, not by bandwidth; the rate against the HBM peak is given for scale only
            res["decode"]["selection_roofline"] = {
                "kernel": "block_topk_rows_kernel", "bound": "latency", "achieved": round(gbs, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                "algorithmic_per_launch": f"{sel_bytes} B = per sequence ceil(n/{span}) block-maximum keys + "
                                          f"min(n, {nb * bs}) candidate scores read + {K} indices written"}
        del out, idx, ws
    with sa.Handle(cfg) as h:
        out = torch.empty((L, s.n_heads, s.d_v), device=dev)
        idx = torch.empty((L, K), device=dev, dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_PREFILL_BLOCKS, L)
        log(f"[bench] two-tier prefill L={L} block={bs} n_blocks={nb}")
        ms, per = timed(h, lambda: sa.sparse_attn_prefill_blocks(
            h, P["q"], P["k"], None, P["q_idx"], P["w"], P["k_idx"], K, bs, nb, out, None, idx, ws),
            max(1, min(args.steps, 2)))
        res["prefill"] = {"ms": round(ms, 4), "tokens_per_s": round(L / (ms * 1e-3), 1), "kernels_ms": per}
        if per.get("indexer") and bs >= 64:
            pairs = L * (L + 1) // 2
            flops = pairs * 2 * s.n_idx_heads * s.d_idx
            tf = flops / (per["indexer"] * 1e-3) / 1e12
            res["prefill"]["block_key_roofline"] = {
                "kernel": "indexer_topk_prefill_kernel (block-key mode)", "bound": "mfma", "achieved": round(tf, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                "algorithmic_per_launch": f"{flops:.4g} flop = {pairs} causal pairs x {2 * s.n_idx_heads * s.d_idx} flop"}
        del out, idx, ws
    torch.cuda.empty_cache()
    return res


def measure_chunk(cfg, P, D, K, args, torch):
    """Chunked prefill (not part of `value`): the last --chunk positions of sequence 0 of the decode
    caches as query rows, each over its own causal prefix of the paged caches, through
    sparse_attn_prefill_chunk (fused row tiles) and through sparse_attn_prefill_paged (rows naming their own
    sequence and position, cut into row tiles on the device);
    the query rows are the first rows of the prefill inputs (synthetic, same distribution)."""
    import numpy as np

    import indexer_selected_sparse_scores_amd as sa
    dev = "cuda"
    s = cfg
    n = int(D["ctx_np"][0])
    C = min(args.chunk, n, P["q"].shape[0])
    pos = np.arange(n - C, n)
    row_seq = torch.zeros(C, dtype=torch.int32, device=dev)
    row_pos = torch.from_numpy(pos.astype(np.int32)).to(dev)
    with sa.Handle(cfg) as h:
        out = torch.empty((C, s.n_heads, s.d_v), device=dev)
        idx = torch.empty((C, K), device=dev, dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_PREFILL_PAGED, C, n)

        ws_c = sa.workspace(h, sa.SA_OP_PREFILL_CHUNK, C, n)
        table_row = D["block_table"][0].contiguous()

        def run_rows():   # each row names its (sequence, position): row tiles sorted on the device
            sa.sparse_attn_prefill_paged(h, P["q"][:C], P["q_idx"][:C], P["w"][:C], D["kv_pages"], None,
                                         D["kidx_pages"], D["block_table"][:1], row_seq, row_pos, n, K, out, None,
                                         idx, ws)

        def run_chunk():  # the chunk known on the host: fused row tiles over the pages
            sa.sparse_attn_prefill_chunk(h, P["q"][:C], P["q_idx"][:C], P["w"][:C], D["kv_pages"], None,
                                         D["kidx_pages"], table_row, n - C, K, out, None, idx, ws_c)

        def timed(run):
            run()
            torch.cuda.synchronize()
            sa.sparse_attn_check(h)
            sa.sparse_attn_profile(h, True)
            reps = max(1, min(args.steps, 3))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                run()
            e1.record()
            torch.cuda.synchronize()
            kern = sa.sparse_attn_profile_read(h)
            sa.sparse_attn_profile(h, False)
            sa.sparse_attn_check(h)
            return e0.elapsed_time(e1) / reps, {k: round(v / reps, 4) for k, (v, c) in kern.items() if c}

        # a varlen batch of the same size: 8 sequences, C / 8 new tokens at the end of each context
        n_seq = 8
        per = C // n_seq
        cu = torch.arange(0, n_seq + 1, dtype=torch.int32, device=dev) * per
        ws_v = sa.workspace(h, sa.SA_OP_PREFILL_VARLEN, n_seq * per, n)

        def run_varlen():  # the layout known only on the device: fused row tiles per sequence
            sa.sparse_attn_prefill_varlen(h, P["q"][:n_seq * per], P["q_idx"][:n_seq * per], P["w"][:n_seq * per],
                                          D["kv_pages"], None, D["kidx_pages"], D["block_table"][:n_seq], cu,
                                          D["ctx_len"][:n_seq], n, K, out[:n_seq * per], None, idx[:n_seq * per], ws_v)

        log(f"[bench] chunked prefill: {C} new tokens at positions {n - C}..{n - 1}")
        ms_c, per_c = timed(run_chunk)
        ms_r, per_r = timed(run_rows)
        log(f"[bench] varlen prefill: {n_seq} sequences x {per} new tokens at the end of their contexts")
        ms_v, per_v = timed(run_varlen)
        del out, idx, ws, ws_c, ws_v
    torch.cuda.empty_cache()
    pairs = int((pos + 1).sum())
    flops = pairs * 2 * s.n_idx_heads * s.d_idx

    def roof(kernel, ms):
        tf = flops / (ms * 1e-3) / 1e12
        return {"kernel": kernel, "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                "algorithmic_per_launch": f"{flops:.4g} flop = {pairs} causal pairs x "
                                          f"{2 * s.n_idx_heads * s.d_idx} flop"}

    res = {"workload": f"{C} new tokens of one sequence at positions {n - C}..{n - 1} over its paged caches",
           "ms": round(ms_c, 4), "tokens_per_s": round(C / (ms_c * 1e-3), 1), "kernels_ms": per_c,
           "paged_rows_call": {"ms": round(ms_r, 4), "tokens_per_s": round(C / (ms_r * 1e-3), 1), "kernels_ms": per_r,
                               "call": "sparse_attn_prefill_paged (rows naming their own sequence and position)"}}
    if per_c.get("indexer"):
        res["indexer_roofline"] = roof("indexer_topk_prefill_kernel (paged row tiles)", per_c["indexer"])
    if per_r.get("indexer"):
        res["paged_rows_call"]["indexer_roofline"] = roof("indexer_topk_prefill_kernel (row tiles sorted by sequence "
                                                          "and position on the device)", per_r["indexer"])
    ctx8 = D["ctx_np"][:n_seq].astype(np.int64)
    vpairs = int(sum((np.arange(c - per, c) + 1).sum() for c in ctx8))
    vtf = vpairs * 2 * s.n_idx_heads * s.d_idx / (per_v["indexer"] * 1e-3) / 1e12 if per_v.get("indexer") else None
    res["varlen"] = {"workload": f"{n_seq} sequences x {per} new tokens at the end of their {int(ctx8.max())}-token "
                                 f"paged contexts (sparse_attn_prefill_varlen)",
                     "ms": round(ms_v, 4), "tokens_per_s": round(n_seq * per / (ms_v * 1e-3), 1), "kernels_ms": per_v,
                     "indexer_tflops": round(vtf, 2) if vtf else None}
    return res


def measure_rl_sweep(args, torch):
    """The RL-rollout decode sweep (not part of `value`): 256 sequences whose context grows from 1K to 32K in
    steps of 1K, each sequence with its own budget k_b(n) = min(n, max(256, floor(rho_b n))), rho_b ~ U(0.05,
    0.25); one decode step at each n = 1024 i, i = 1..32 (8192 generated tokens in all).  The paged caches are
    generated once for 32K tokens per sequence and each step sees its first n."""
    import numpy as np

    import indexer_selected_sparse_scores_amd as sa
    from indexer_selected_sparse_scores_amd import inputs
    dev = "cuda"
    wl = inputs.WORKLOADS["decode_rl_sweep"]
    n_max = wl.ctx_range[1]
    B = wl.B
    log(f"[bench] RL-rollout decode sweep B={B}, n = 1024 .. {n_max}")
    D = inputs.decode_inputs(wl, dev, ctx=np.full(B, n_max))
    cfg = inputs.library_config(wl, max_topk=8192)
    s = cfg
    steps = list(range(1024, n_max + 1, 1024))
    with sa.Handle(cfg) as h:
        out = torch.empty((B, s.n_heads, s.d_v), device=dev)
        idx = torch.empty((B, s.max_topk), device=dev, dtype=torch.int32)
        ws = sa.workspace(h, sa.SA_OP_DECODE, B, n_max)
        plan = []
        for n in steps:
            k = inputs.rl_budget(n, D["rho"])
            plan.append((n, torch.full((B,), n, dtype=torch.int32, device=dev),
                         torch.from_numpy(k.astype(np.int32)).to(dev), k))

        def step(p):
            n, ctx, topk, _ = p
            sa.sparse_attn_decode(h, D["q"], D["q_idx"], D["w"], D["kv_pages"], None, D["kidx_pages"],
                                  D["block_table"], ctx, topk, n, out, None, idx, ws)

        for p in plan:  # warm-up pass
            step(p)
        torch.cuda.synchronize()
        sa.sparse_attn_check(h)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(plan) + 1)]
        ev[0].record()
        for i, p in enumerate(plan):
            step(p)
            ev[i + 1].record()
        torch.cuda.synchronize()
        sa.sparse_attn_check(h)
        per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(plan))]
        del out, idx, ws
    del D
    torch.cuda.empty_cache()
    total_ms = sum(per_step)
    tokens = B * len(steps)
    nbytes = sum(B * n * s.d_idx * 2 + int(k.sum()) * s.d_qk * 2 for n, _, _, k in plan)
    gbs = nbytes / (total_ms * 1e-3) / 1e9
    return {"workload": f"{B} sequences, one decode step at each context n = 1024 i (i = 1..{len(steps)}), "
                        "per-sequence top-k min(n, max(256, floor(rho n))), rho ~ U(0.05, 0.25)",
            "steps": len(steps), "tokens": tokens, "ms_total": round(total_ms, 4),
            "tokens_per_s": round(tokens / (total_ms * 1e-3), 1),
            "ms_first_last_step": [round(per_step[0], 4), round(per_step[-1], 4)],
            "roofline": {"kernel": "whole decode step (paged indexer, top-k, gather-attention, merge)", "bound": "hbm",
                         "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "algorithmic_per_launch": f"{nbytes} B over the sweep = sum over steps of B n x 256 B index "
                                                   f"keys + sum_b k_b x 1152 B selected latent rows"}}


def measure_acceptance(cfg, args, torch, T=4096, V=151936):
    """The per-token acceptance rate between dense and sparse next-token logits and its 5-percentile
    per bin of 2048 positions (not part of `value`): T tokens over a vocabulary of V, fp32 logits
    (synthetic, inputs.acceptance_inputs)."""
    import indexer_selected_sparse_scores_amd as sa
    from indexer_selected_sparse_scores_amd import inputs
    dev = "cuda"
    d = inputs.acceptance_inputs(T, V, dev)
    n_bins = (T + 2047) // 2048
    alpha = torch.empty(T, dtype=torch.float32, device=dev)
    count = torch.empty(n_bins, dtype=torch.int32, device=dev)
    mean = torch.empty(n_bins, dtype=torch.float32, device=dev)
    pct = torch.empty(n_bins, dtype=torch.float32, device=dev)
    log(f"[bench] acceptance rate T={T} V={V}")
    with sa.Handle(cfg) as h:
        ws = sa.workspace(h, sa.SA_OP_ACCEPT, T, V)  # the single-read path

        def run():
            sa.acceptance_rate(h, d["logits_p"], d["logits_q"], alpha, ws=ws)
            sa.acceptance_bin_stats(h, alpha, d["pos"], 2048, n_bins, 5.0, count, mean, pct)

        run()
        torch.cuda.synchronize()
        sa.sparse_attn_check(h)
        reps = max(1, args.steps)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        for _ in range(reps):
            sa.acceptance_rate(h, d["logits_p"], d["logits_q"], alpha, ws=ws)
        ev[1].record()
        for _ in range(reps):
            sa.acceptance_bin_stats(h, alpha, d["pos"], 2048, n_bins, 5.0, count, mean, pct)
        ev[2].record()
        alpha2 = torch.empty_like(alpha)
        for _ in range(reps):
            sa.acceptance_rate(h, d["logits_p"], d["logits_q"], alpha2)  # two passes over the logits
        ev[3].record()
        torch.cuda.synchronize()
        sa.sparse_attn_check(h)
        a_ms = ev[0].elapsed_time(ev[1]) / reps
        b_ms = ev[1].elapsed_time(ev[2]) / reps
        two_ms = ev[2].elapsed_time(ev[3]) / reps
        two_diff = float((alpha - alpha2).abs().max())
    nbytes = 2 * T * V * 4
    gbs = nbytes / (a_ms * 1e-3) / 1e9
    res = {"workload": f"{T} tokens x {V} vocabulary, fp32 logits, 5-percentile per 2048 positions",
           "alpha_ms": round(a_ms, 4), "bin_stats_ms": round(b_ms, 4),
           "tokens_per_s": round(T / ((a_ms + b_ms) * 1e-3), 1),
           "two_pass": {"alpha_ms": round(two_ms, 4), "max_abs_diff": two_diff,
                        "note": "the same call without a workspace: each logit read twice"},
           "roofline": {"kernel": "acceptance_once_kernel (with its fill and sum launches)", "bound": "hbm",
                        "achieved": round(gbs, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "algorithmic_per_launch": f"{nbytes} B = {T} tokens x 2 rows x {V} x 4 B (each logit "
                                                  f"read once)"},
           "pct_5": [round(float(x), 5) for x in pct.cpu()], "mean": [round(float(x), 5) for x in mean.cpu()]}
    del d
    torch.cuda.empty_cache()
    return res


def measured_peaks(h, torch):
    """Rates measured on this machine, references beside the spec peaks: the library's bf16 MFMA loop on random
    operands (the fused indexer's instruction and occupancy; with the shader clock it ran at, from the
    s_memtime / s_memrealtime counters it reads), its streaming read and copy kernels over 4 GiB, and for
    context a large bf16 GEMM (hipBLASLt through torch)."""
    import indexer_selected_sparse_scores_amd as sa
    dev = "cuda"
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    g = torch.Generator(device=dev).manual_seed(20261202)
    operands = torch.randn(1 << 19, generator=g, device=dev).to(torch.bfloat16)  # 1 MiB of random bf16
    clocks = torch.zeros(256, dtype=torch.int64, device=dev)
    sink = torch.zeros(1, device=dev)
    iters = 40000                      # about 20 ms per launch; 6 launches ~ the fused indexer's 0.1 s
    flop_per_launch = n_cu * 8 * iters * 8 * 32768
    for _ in range(2):
        sa.sparse_attn_peak_mfma(h, operands, iters, clocks, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 6
    e0.record()
    for _ in range(reps):
        sa.sparse_attn_peak_mfma(h, operands, iters, clocks, sink)
    e1.record()
    torch.cuda.synchronize()
    mfma_ms = e0.elapsed_time(e1) / reps
    mfma_tflops = flop_per_launch / (mfma_ms * 1e-3) / 1e12
    c = clocks.view(-1, 4).cpu().numpy()[:min(n_cu, 64)].astype("float64")
    ghz = sorted(((c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / 100e6) / 1e9).tolist())  # s_memrealtime: 100 MHz
    clock_ghz = ghz[len(ghz) // 2]
    del operands, clocks
    nbytes = 1 << 32
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty(nbytes // 2, dtype=torch.uint8, device=dev)

    def timed(fn, n=5):
        fn()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    read_ms = timed(lambda: sa.sparse_attn_peak_stream(h, src, None, nbytes, sink))
    copy_ms = timed(lambda: sa.sparse_attn_peak_stream(h, src[:nbytes // 2], dst, nbytes // 2))
    sa.sparse_attn_check(h)
    del src, dst
    n = 8192
    a = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    b = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    gemm_ms = timed(lambda: torch.matmul(a, b), 10)
    del a, b
    torch.cuda.empty_cache()
    return {"mfma_loop_tflops": round(mfma_tflops, 1), "mfma_loop_clock_ghz": round(clock_ghz, 3),
            "mfma_loop": f"{n_cu} workgroups x 8 waves, v_mfma_f32_32x32x16_bf16 on eight random bf16 fragment "
                         f"pairs per wave, {reps} launches of {mfma_ms:.2f} ms; clock = median over workgroups of "
                         f"shader cycles / (reference ticks / 100 MHz)",
            "stream_read_gbs": round(nbytes / (read_ms * 1e-3) / 1e9, 1),
            "stream_copy_read_plus_write_gbs": round(nbytes / (copy_ms * 1e-3) / 1e9, 1),
            "stream": "4 GiB read once (16-byte non-temporal loads), and 2 GiB copied, by the library's stream kernel",
            "bf16_gemm_8192_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1)}


def cpu_baseline(P, wl, K, seconds):
    """The oracle as it stands, on a bounded sample of the prefill workload: uniformly drawn
    query rows, each scored against all of its preceding keys, top-k selected and attended.
    Uniform rows have the average causal length, so rows/s estimates prefill tokens/s."""
    import numpy as np
    import torch

    import oracle

    L = P["q"].shape[0]
    d_qk = P["q"].shape[-1]
    d_v = 512 if wl.shapes.latent else wl.shapes.d_v
    rng = np.random.default_rng(20261202)
    k_idx = P["k_idx"].float().cpu().numpy()
    kv = P["k"].float().cpu().numpy()
    threads = oracle.num_threads()

    def run(n):
        rows = np.sort(rng.integers(0, L, n))
        sel = torch.as_tensor(rows, device=P["q"].device)
        q_idx = P["q_idx"][sel].float().cpu().numpy()
        w = P["w"][sel].float().cpu().numpy()
        q = P["q"][sel].float().cpu().numpy()
        t0 = time.perf_counter()
        sc = oracle.indexer_scores(q_idx, w, k_idx, rows + 1)
        idx = oracle.topk(sc, rows + 1, K)
        oracle.attention_rows(q, kv, None, idx, oracle.default_scale(d_qk), d_v=d_v)
        return time.perf_counter() - t0

    log(f"[bench] cpu baseline: oracle on sampled rows (~{seconds:.0f} s, {threads} threads)")
    n0 = max(2, threads // 2)
    t0 = run(n0)
    n = int(min(4096, max(n0, n0 * seconds / max(t0, 1e-3))))
    t = run(n)
    # the same oracle on one thread, on a smaller sample of the same rows' distribution
    oracle.set_num_threads(1)
    try:
        n1 = max(1, int(n * (seconds / 3) / max(t, 1e-3) / threads))
        t1 = run(n1)
    finally:
        oracle.set_num_threads(threads)
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(n / t, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle", "cpu": cpu_model,
            "sample": f"{n} uniformly drawn query rows of the L={L} prefill (indexer over all "
                      f"preceding keys, top-{K}, attention), {t:.1f} s on {threads} threads",
            "one_thread": {"value": round(n1 / t1, 4), "unit": "tokens/s", "cores": 1,
                           "sample": f"{n1} uniformly drawn query rows, {t1:.1f} s on 1 thread"}}


def cpu_baseline_decode(D, wl, K, seconds):
    """The oracle's decode step on a bounded sample of the decode workload: whole sequences (index
    keys of every cached token scored, top-k, attention over the selected latent rows), their pages
    copied to the host beforehand and only the oracle call timed.  Sequences/s = decode tokens/s."""
    import numpy as np
    import torch

    import oracle

    page = D["kv_pages"].shape[1]
    threads = oracle.num_threads()

    def host_seqs(seqs):
        tabs, kv, ki = [], [], []
        base = 0
        for b in seqs:
            n_pg = -(-int(D["ctx_np"][b]) // page)
            pages = D["block_table"][b, :n_pg].long()
            kv.append(D["kv_pages"][pages].float().cpu().numpy())
            ki.append(D["kidx_pages"][pages].float().cpu().numpy())
            tabs.append(np.arange(base, base + n_pg, dtype=np.int32))
            base += n_pg
        width = max(len(t) for t in tabs)
        table = np.full((len(seqs), width), -1, dtype=np.int32)
        for i, t in enumerate(tabs):
            table[i, :len(t)] = t
        sel = torch.as_tensor(np.asarray(seqs), device=D["q"].device)
        pick = lambda t: t[sel].float().cpu().numpy()
        return (pick(D["q"]), pick(D["q_idx"]), pick(D["w"]), np.concatenate(kv), np.concatenate(ki), table,
                D["ctx_np"][seqs], D["topk"][sel].cpu().numpy())

    def run(seqs):
        q, q_idx, w, kv, ki, table, ctx, topk = host_seqs(seqs)
        t0 = time.perf_counter()
        oracle.decode(q, q_idx, w, kv, None, ki, table, ctx, topk, k_max=K, d_v=512)
        return time.perf_counter() - t0

    B = D["q"].shape[0]
    log(f"[bench] cpu baseline: oracle decode on sampled sequences (~{seconds:.0f} s, {threads} threads)")
    t1 = run([0])
    n = int(min(B, 16, max(1, seconds / max(t1, 1e-3))))  # at most 16 sequences' pages on the host
    seqs = list(range(1, 1 + n)) if n < B else list(range(B))
    t = run(seqs)
    oracle.set_num_threads(1)
    try:
        t1 = run([0])
    finally:
        oracle.set_num_threads(threads)
    return {"value": round(len(seqs) / t, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(seqs)} of the B={B} sequences of the decode step at ctx={int(D['ctx_np'].max())} "
                      f"(indexer over every cached token, top-{K}, attention), {t:.1f} s on {threads} threads",
            "one_thread": {"value": round(1 / t1, 4), "unit": "tokens/s", "cores": 1,
                           "sample": f"sequence 0 of the step, {t1:.1f} s on 1 thread"}}


if __name__ == "__main__":
    main()
